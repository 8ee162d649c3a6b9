// Main-kernel instantiations for kernel head dim 64 (see main_launch.h).
#include "main_launch.h"

template hipError_t sdpa::launch_main_dqk<64>(const MainParams&, DqMode, bool, int, int, int,
                                              hipStream_t, bool);
