// Main-kernel instantiations for kernel head dim 32 (see main_launch.h).
#include "main_launch.h"

template hipError_t sdpa::launch_main_dqk<32>(const MainParams&, DqMode, bool, int, int, int,
                                             hipStream_t, bool);
