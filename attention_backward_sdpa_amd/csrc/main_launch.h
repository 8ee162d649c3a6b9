// Launch of the fused main kernel (bwd_main.h) for one kernel head dim.  Each head dim's
// instantiations (4 dQ modes x bf16/fp16 x bias none/bias/dBias x exact/padded head dims) live in
// a translation unit of their own (main_d<DQK>.hip), so the library's objects compile in
// parallel; the host side (sdpa_bwd.hip) calls launch_main_dqk<DQK>.
#pragma once
#include <atomic>

#include "bwd_main.h"

namespace sdpa {

// Tile geometry of the main kernel for a kernel head dim: 8 waves (256 registers each, 256-key
// tiles) for DQK <= 192 without a bias, and for DQK <= 128 with an io-type bias staged in LDS;
// 4 waves (512 registers, 128-key tiles) for DQK = 256 and for the other biases, whose next-tile
// values are held in registers.
template <int DQK>
struct MainShape {
  static constexpr int DV = DQK == 192 ? 128 : DQK;
  static constexpr int KPW = 32;
  static constexpr int nw(bool bias) { return DQK == 256 || bias ? 4 : 8; }
};

// bias: 0 none, 1 additive bias, 2 bias and dBias.  `bc` is the key tile the caller's workspace
// carve and grid assume; a mismatch with the kernel's is hipErrorInvalidValue.
template <int DQK>
hipError_t launch_main_dqk(const MainParams& mp, DqMode mode, bool f16, int bias, int grid, int bc,
                           hipStream_t s, bool qat = false);

// Raise a kernel's dynamic-LDS limit to `bytes`, once per device (the attribute is set for the
// current device); Tag names the kernel instantiation.
template <class Tag, class F>
hipError_t lds_limit_once(F* kernel, int bytes) {
  static std::atomic<uint64_t> done{0};  // bit d: set on device d (devices >= 64: every call)
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t{1} << dev) : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

// Instantiations compiled with the backend's latency-oriented scheduler (main_ilp_d<DQK>.hip,
// built with -amdgpu-sched-strategy=iterative-ilp): with every register of a one-wave-per-SIMD
// kernel taken (head dim 256) the default scheduler issued each GEMM1/GEMM2 operand read one MFMA
// ahead and waited on it, an LDS round trip per MFMA with no other wave to hide it.  The set is
// what measured faster or the same under it without spilling: every bias-free head-dim-256
// kernel (the bias variants spill), and every head-dim-128 kernel but the 8-wave dQ-partial ones
// (slower under it).  The other head dims stay on the default schedule (192 spills, 32 does not
// compile under it, 64 gains nothing).
template <class C>
struct IlpSched {
  static constexpr bool value =
      C::KPW == 32 && C::DQK == C::DV && !C::BIAS_LDS && !(C::QAT && C::NW == 8) &&
      ((C::DQK == 256 && C::NW == 4 && C::BIAS == 0 && !C::QAT) ||
       (C::DQK == 128 && !(C::NW == 8 && C::MODE == DQ_PARTIAL)));
};

template <class C>
hipError_t launch_main_cfg_ilp(const MainParams& mp, int grid, hipStream_t s);  // main_ilp_d*.hip

template <class C>
hipError_t launch_main_cfg(const MainParams& mp, int grid, hipStream_t s) {
  if constexpr (IlpSched<C>::value) {
    return launch_main_cfg_ilp<C>(mp, grid, s);
  } else {
    const hipError_t e = lds_limit_once<C>(bwd_main_kernel<C>, C::LDS_BYTES);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_main_kernel<C>, dim3(grid), dim3(C::NT), C::LDS_BYTES, s, mp);
    return hipGetLastError();
  }
}

template <int DQK, int DV, int KPW, int NW, bool F16, int BIAS, bool PAD, bool QAT = false>
hipError_t launch_main_mode(const MainParams& mp, DqMode mode, int grid, hipStream_t s) {
  if (mode == DQ_DS)
    return launch_main_cfg<MainCfg<DQK, DV, KPW, NW, DQ_DS, F16, BIAS, PAD, QAT>>(mp, grid, s);
  if (mode == DQ_PARTIAL)
    return launch_main_cfg<MainCfg<DQK, DV, KPW, NW, DQ_PARTIAL, F16, BIAS, PAD, QAT>>(mp, grid, s);
  if (mode == DQ_RELAY) {
    // the relay keeps a bias and the QAT variant on the 4-wave layout (their 8-wave kernels do
    // not fit in 256 registers); the host never asks for them
    if constexpr ((BIAS > 0 || QAT) && NW == 8)
      return hipErrorInvalidValue;
    else
      return launch_main_cfg<MainCfg<DQK, DV, KPW, NW, DQ_RELAY, F16, BIAS, PAD, QAT>>(mp, grid, s);
  }
  return launch_main_cfg<MainCfg<DQK, DV, KPW, NW, DQ_ATOMIC, F16, BIAS, PAD, QAT>>(mp, grid, s);
}

template <int DQK, int NW, int BIAS>
hipError_t launch_main_nw(const MainParams& mp, DqMode mode, bool f16, int grid, int bc,
                          hipStream_t s) {
  constexpr int DV = MainShape<DQK>::DV, KPW = MainShape<DQK>::KPW;
  if (MainCfg<DQK, DV, KPW, NW, DQ_ATOMIC>::BC != bc) return hipErrorInvalidValue;
  // head dims below the kernel's take the variant that zero-pads the operands
  const bool pad = mp.dqk_act != DQK || mp.dv_act != DV;
  if (f16)
    return pad ? launch_main_mode<DQK, DV, KPW, NW, true, BIAS, true>(mp, mode, grid, s)
               : launch_main_mode<DQK, DV, KPW, NW, true, BIAS, false>(mp, mode, grid, s);
  return pad ? launch_main_mode<DQK, DV, KPW, NW, false, BIAS, true>(mp, mode, grid, s)
             : launch_main_mode<DQK, DV, KPW, NW, false, BIAS, false>(mp, mode, grid, s);
}

template <int DQK>
hipError_t launch_main_dqk(const MainParams& mp, DqMode mode, bool f16, int bias, int grid, int bc,
                           hipStream_t s, bool qat) {
  constexpr int NW0 = MainShape<DQK>::nw(false), NW1 = MainShape<DQK>::nw(true);
  if (qat) {  // NVFP4 QAT: head dim 128, bf16, no bias, exact head dims; 8 waves but on the relay
    if constexpr (DQK == 128) {
      if (f16 || bias || mp.dqk_act != 128 || mp.dv_act != 128) return hipErrorInvalidValue;
      if (MainCfg<128, 128, 32, NW0, DQ_ATOMIC>::BC == bc)
        return launch_main_mode<128, 128, 32, NW0, false, 0, false, true>(mp, mode, grid, s);
      if (MainCfg<128, 128, 32, NW1, DQ_ATOMIC>::BC != bc || mode != DQ_RELAY)
        return hipErrorInvalidValue;
      return launch_main_cfg<MainCfg<128, 128, 32, NW1, DQ_RELAY, false, 0, false, true>>(mp, grid, s);
    } else {
      return hipErrorInvalidValue;
    }
  }
  if (bias) {
    // an io-type bias at head dims up to 128 may run the 8-wave layout with the bias tile staged
    // in LDS (the host chose it through the key tile); otherwise the 4-wave layout
    if constexpr (DQK <= 128 && NW0 == 8) {
      if (bc == MainCfg<DQK, MainShape<DQK>::DV, 32, NW0, DQ_ATOMIC>::BC)
        return bias == 1 ? launch_main_nw<DQK, NW0, 1>(mp, mode, f16, grid, bc, s)
                         : launch_main_nw<DQK, NW0, 2>(mp, mode, f16, grid, bc, s);
    }
    return bias == 1 ? launch_main_nw<DQK, NW1, 1>(mp, mode, f16, grid, bc, s)
                     : launch_main_nw<DQK, NW1, 2>(mp, mode, f16, grid, bc, s);
  }
  return launch_main_nw<DQK, NW0, 0>(mp, mode, f16, grid, bc, s);
}

// instantiated once each, in main_d<DQK>.hip
#define SDPA_MAIN_DQK(D)                                                                           \
  extern template hipError_t launch_main_dqk<D>(const MainParams&, DqMode, bool, int, int, int,    \
                                                hipStream_t, bool);
SDPA_MAIN_DQK(32)
SDPA_MAIN_DQK(64)
SDPA_MAIN_DQK(128)
SDPA_MAIN_DQK(192)
SDPA_MAIN_DQK(256)
#undef SDPA_MAIN_DQK

}  // namespace sdpa
