// Deterministic dQ kernel of the two-kernel route ("SDPA Backward (SM120)", sections
// "Determinism" and "Deterministic vs. non-deterministic dQ"): dQ = scale * dS K, one workgroup per
// q tile of one query head, accumulating in registers over an ascending walk of exactly the KV
// tiles the main kernel stored for that q tile, then a single bf16 store.  No atomics, fixed
// order, so the result is bitwise reproducible.
//
// The workspace holds each stored (q tile, KV tile) block as dS^T (keys x q, q contiguous), the
// layout the main kernel produces it in; both tiles are staged row-major in LDS and read as MFMA
// operands with the transpose instruction.
#pragma once
#include "common.h"
#include "masks.h"

namespace sdpa {

struct Dq2kParams {
  const bf16_t* ds_ws;        // (B, Hq, skv_pad, sq_pad)
  const bf16_t* k;            // (B, Hkv, Skv, Dqk)
  bf16_t* dq;                 // (B, Hq, Sq, Dqk)
  const int* seq_q_lens;
  const int* seq_kv_lens;
  int B, Hq, Hkv, Sq, Skv, group;
  int causal, window_left, window_right, bottom_right;
  int n_kv_tiles, n_q_tiles;
  int sq_pad, skv_pad;
  float scale;
};

template <int DQK_, int BR_, int BC_>
struct Dq2kCfg {
  static constexpr int DQK = DQK_, BR = BR_, BC = BC_;
  static constexpr int NW = 4, NT = 256;
  static constexpr int DW = DQK / NW;                 // d columns per wave
  static constexpr int MT = (DW % 32 == 0) ? 32 : 16;
  using M = Mfma<MT>;
  static constexpr int KT = M::KT, NACC = M::NACC;
  static constexpr int N_RT = BR / MT, N_DT = DW / MT, N_K = BC / KT;
  static constexpr int STROWB = BR * 2, KROWB = DQK * 2;
  static constexpr int OFF_ST = 0, OFF_K = BC * STROWB;
  static constexpr int LDS_BYTES = OFF_K + BC * KROWB;
  static constexpr int SCH = BC * BR / 8 / NT, KCH = BC * DQK / 8 / NT;
  static_assert(SCH * NT * 8 == BC * BR && KCH * NT * 8 == BC * DQK, "tile/thread mismatch");
  static_assert(DW % MT == 0 && BR % MT == 0 && BC % KT == 0, "tile shapes");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

template <int MT, int ROWB>
__device__ __forceinline__ bf16x8 tr_operand2(const char* base, int n_base, int k0a, int k0b,
                                              int lane) {
  const int i = lane & 15;
  const int col = n_base + ((lane % MT) & ~15) + 4 * (i & 3);
  return concat(lds_read_tr(base, lds_off<ROWB>(k0a + (i >> 2), col)),
                lds_read_tr(base, lds_off<ROWB>(k0b + (i >> 2), col)));
}

template <class C>
__global__ void __launch_bounds__(C::NT, 1) dq2k_kernel(Dq2kParams p) {
  using M = typename C::M;
  using acc_t = typename M::acc_t;
  constexpr int MT = C::MT, BR = C::BR, BC = C::BC, DQK = C::DQK, NT = C::NT, KT = C::KT;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* sST = smem + C::OFF_ST;
  char* sK = smem + C::OFF_K;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane / MT, lc = lane % MT;

  const int nbh = p.B * p.Hq;
  const int bh = blockIdx.x % nbh;
  const int i = blockIdx.x / nbh;
  const int h = bh % p.Hq, b = bh / p.Hq;
  const int kvh = h / p.group;
  const int q0 = i * BR;

  MaskGeom mg;
  mg.Lq = p.seq_q_lens ? min(max(p.seq_q_lens[b], 0), p.Sq) : p.Sq;
  mg.Lkv = p.seq_kv_lens ? min(max(p.seq_kv_lens[b], 0), p.Skv) : p.Skv;
  mg.diag = p.bottom_right ? mg.Lkv - mg.Lq : 0;
  mg.causal = p.causal;
  mg.W = p.window_left;
  mg.R = p.window_right;

  // The KV tiles whose stored band contains this q tile form one contiguous run [j_first, j_last]
  // (both ends of q_tile_range are non-decreasing in the KV tile index).
  int j_first = p.n_kv_tiles, j_last = -1;
  for (int j = 0; j < p.n_kv_tiles; ++j) {
    int lo, hi;
    q_tile_range(mg, j * BC, BC, BR, &lo, &hi);
    if (lo <= i && i <= hi) {
      j_first = j < j_first ? j : j_first;
      j_last = j;
    }
  }

  const bf16_t* wsb = p.ds_ws + (int64_t)(b * p.Hq + h) * p.skv_pad * p.sq_pad + q0;
  const bf16_t* Kb = p.k + (int64_t)(b * p.Hkv + kvh) * p.Skv * DQK;

  acc_t acc[C::N_RT * C::N_DT];
#pragma unroll
  for (int t = 0; t < C::N_RT * C::N_DT; ++t) acc[t] = acc_t{};

  u32x4 ps[C::SCH], pk[C::KCH];
  auto prefetch = [&](int j) {
    const int k0 = j * BC;
#pragma unroll
    for (int n = 0; n < C::SCH; ++n) {
      const int c = tid + n * NT, row = c / (BR / 8), col = (c % (BR / 8)) * 8;
      ps[n] = *reinterpret_cast<const u32x4*>(wsb + (int64_t)(k0 + row) * p.sq_pad + col);
    }
#pragma unroll
    for (int n = 0; n < C::KCH; ++n) {
      const int c = tid + n * NT, row = c / (DQK / 8), col = (c % (DQK / 8)) * 8;
      pk[n] = (k0 + row < p.Skv) ? *reinterpret_cast<const u32x4*>(Kb + (int64_t)(k0 + row) * DQK + col)
                                 : u32x4{0, 0, 0, 0};
    }
  };

  if (j_first <= j_last) prefetch(j_first);
  for (int j = j_first; j <= j_last; ++j) {  // ascending KV order
    __syncthreads();
#pragma unroll
    for (int n = 0; n < C::SCH; ++n) {
      const int c = tid + n * NT, row = c / (BR / 8), col = (c % (BR / 8)) * 8;
      *reinterpret_cast<u32x4*>(sST + lds_off<C::STROWB>(row, col)) = ps[n];
    }
#pragma unroll
    for (int n = 0; n < C::KCH; ++n) {
      const int c = tid + n * NT, row = c / (DQK / 8), col = (c % (DQK / 8)) * 8;
      *reinterpret_cast<u32x4*>(sK + lds_off<C::KROWB>(row, col)) = pk[n];
    }
    __syncthreads();
    if (j < j_last) prefetch(j + 1);
#pragma unroll
    for (int t = 0; t < C::N_K; ++t) {
      const int ka = t * KT + 8 * g;
      bf16x8 bk[C::N_DT];
#pragma unroll
      for (int dt = 0; dt < C::N_DT; ++dt)
        bk[dt] = tr_operand2<MT, C::KROWB>(sK, w * C::DW + dt * MT, ka, ka + 4, lane);
#pragma unroll
      for (int rt = 0; rt < C::N_RT; ++rt) {
        bf16x8 a = tr_operand2<MT, C::STROWB>(sST, rt * MT, ka, ka + 4, lane);
#pragma unroll
        for (int dt = 0; dt < C::N_DT; ++dt)
          acc[rt * C::N_DT + dt] = M::mma(a, bk[dt], acc[rt * C::N_DT + dt]);
      }
    }
  }

  // dQ = scale * acc, rows past the buffer are not stored; rows past len_q are exactly zero
  bf16_t* dqb = p.dq + (int64_t)(b * p.Hq + h) * p.Sq * DQK;
#pragma unroll
  for (int rt = 0; rt < C::N_RT; ++rt)
#pragma unroll
    for (int dt = 0; dt < C::N_DT; ++dt)
#pragma unroll
      for (int r = 0; r < C::NACC; ++r) {
        const int q = q0 + rt * MT + acc_row<MT>(r, g);
        if (q < p.Sq)
          dqb[(int64_t)q * DQK + w * C::DW + dt * MT + lc] =
              float_to_bf16(acc[rt * C::N_DT + dt][r] * p.scale);
      }
}

}  // namespace sdpa
