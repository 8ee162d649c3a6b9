// Main-kernel instantiations built with the latency-oriented instruction scheduler
// (-mllvm -amdgpu-sched-strategy=iterative-ilp, set for this file by build.py); the set is
// IlpSched in main_launch.h, and every other instantiation lives in main_d<DQK>.hip.
#include "main_launch.h"

namespace sdpa {

template <class C>
hipError_t launch_main_cfg_ilp(const MainParams& mp, int grid, hipStream_t s) {
  static_assert(IlpSched<C>::value, "instantiated here only for the IlpSched set");
  const hipError_t e = lds_limit_once<C>(bwd_main_kernel<C>, C::LDS_BYTES);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_main_kernel<C>, dim3(grid), dim3(C::NT), C::LDS_BYTES, s, mp);
  return hipGetLastError();
}

#define SDPA_ILP(DQK, NW, MODE, F16)                                                               \
  template hipError_t launch_main_cfg_ilp<MainCfg<DQK, DQK, 32, NW, MODE, F16>>(const MainParams&, \
                                                                                int, hipStream_t);
SDPA_ILP(256, 4, DQ_ATOMIC, false)
SDPA_ILP(256, 4, DQ_ATOMIC, true)
SDPA_ILP(256, 4, DQ_DS, false)
SDPA_ILP(256, 4, DQ_DS, true)
SDPA_ILP(256, 4, DQ_PARTIAL, false)
SDPA_ILP(256, 4, DQ_PARTIAL, true)
SDPA_ILP(128, 8, DQ_DS, false)
SDPA_ILP(128, 8, DQ_DS, true)
#undef SDPA_ILP
template hipError_t launch_main_cfg_ilp<MainCfg<128, 128, 32, 4, DQ_DS, false, 0, false, true>>(
    const MainParams&, int, hipStream_t);  // NVFP4 QAT

}  // namespace sdpa
