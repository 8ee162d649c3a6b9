// Shared part of the main-kernel units built with the latency-oriented instruction scheduler
// (main_ilp_d128.hip, main_ilp_d256.hip; -mllvm -amdgpu-sched-strategy=iterative-ilp, set by
// build.py): the launch of one instantiation of the IlpSched set (main_launch.h).
#pragma once
#include "main_launch.h"

namespace sdpa {

template <class C>
hipError_t launch_main_cfg_ilp(const MainParams& mp, int grid, hipStream_t s) {
  static_assert(IlpSched<C>::value, "instantiated only for the IlpSched set");
  const hipError_t e = lds_limit_once<C>(bwd_main_kernel<C>, C::LDS_BYTES);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_main_kernel<C>, dim3(grid), dim3(C::NT), C::LDS_BYTES, s, mp);
  return hipGetLastError();
}

}  // namespace sdpa

// one instantiation, and the same for exact and padded head dims and for bf16 and fp16
#define SDPA_ILP(D, NW, MODE, F16, BIAS, PAD, QAT)                                                 \
  template hipError_t sdpa::launch_main_cfg_ilp<                                                   \
      sdpa::MainCfg<D, D, 32, NW, sdpa::MODE, F16, BIAS, PAD, QAT>>(const sdpa::MainParams&, int, \
                                                                     hipStream_t);
#define SDPA_ILP_PF(D, NW, MODE, BIAS)                                                             \
  SDPA_ILP(D, NW, MODE, false, BIAS, false, false)                                                 \
  SDPA_ILP(D, NW, MODE, false, BIAS, true, false)                                                  \
  SDPA_ILP(D, NW, MODE, true, BIAS, false, false)                                                  \
  SDPA_ILP(D, NW, MODE, true, BIAS, true, false)
