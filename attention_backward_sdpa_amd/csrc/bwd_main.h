// Fused five-GEMM attention-backward main kernel for gfx950.
//
// "SDPA Backward (SM120)", section "Main-kernel pipeline: KV-stationary, five chained GEMMs": one
// workgroup owns one KV tile of one query head (its KV head is q_head / group), loads K and V once
// and walks the visible q tiles in descending order.  Per q tile:
//     GEMM1  S  = Q K^T                       P  = exp2(S * scale * log2e - LSE * log2e)
//     GEMM2  dP = dO V^T                      dS = P * (dP - delta)
//     GEMM3  dV += P^T dO      (bf16 P)
//     GEMM5  dK += dS^T Q      (bf16 dS)
//     GEMM4  dQ  = dS K  -> fp32 atomic add into dq_accum
// dK/dV stay in registers for the whole pass and are written once (dK scaled by the softmax
// scale).  On the deterministic route ("Deterministic vs. non-deterministic dQ") GEMM4 and the
// atomics are replaced by a store of the unscaled bf16 dS tile to a workspace that the dq2k
// kernel reduces in ascending KV order.
//
// MI355X mapping (differs from the pages' SM120 warp-specialised design):
//   * 4 waves of 64 lanes; wave w owns key columns [w*MT, (w+1)*MT) of the BC = 4*MT key tile.
//     S and dP are computed with q as the MFMA row index and keys as the column index, so each
//     wave's P and dS accumulators are already the B operand of GEMM3/GEMM5 (contraction over q)
//     and the wave's dK^T/dV^T partials complete inside the wave.
//   * The wave's K and V slices are held in registers as the B operands of GEMM1/GEMM2.
//   * Q and dO tiles are staged row-major in LDS; GEMM3/GEMM5 read them transposed with
//     ds_read_b64_tr_b16, so no transposed copy is stored.
//   * dS is written to LDS as dS^T (keys x q, 8-byte stores from the accumulator layout) and read
//     back transposed as the A operand of GEMM4; K is kept in LDS as GEMM4's B operand.
//   * The next q tile's Q/dO/LSE/delta are prefetched into registers while the current one runs.
#pragma once
#include "common.h"
#include "masks.h"

namespace sdpa {

struct MainParams {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  const bf16_t* dO;
  const float* lse;
  const float* delta;
  float* dq_accum;          // (B, Hq, Sq, Dqk) fp32, non-deterministic route
  bf16_t* ds_ws;            // (B, Hq, Skv_pad, Sq_pad) bf16 dS^T tiles, deterministic route
  bf16_t* dk_out;           // (B, out_heads, Skv, Dqk)
  bf16_t* dv_out;           // (B, out_heads, Skv, Dv)
  const int* seq_q_lens;    // (B,) or null
  const int* seq_kv_lens;   // (B,) or null
  int B, Hq, Hkv, Sq, Skv, group, out_heads;
  int causal, window_left, window_right, bottom_right;
  int n_kv_tiles;
  int sq_pad, skv_pad;      // dS workspace extents
  float scale;              // softmax scale
  float scale_log2;         // scale * log2(e)
};

template <int DQK_, int DV_, int MT_, int BR_, bool DET_>
struct MainCfg {
  static constexpr int DQK = DQK_, DV = DV_, MT = MT_, BR = BR_;
  static constexpr bool DET = DET_;
  static constexpr int NW = 4;
  static constexpr int NT = NW * 64;
  static constexpr int BC = NW * MT;
  using M = Mfma<MT>;
  static constexpr int KT = M::KT, NG = M::NG, NACC = M::NACC;
  static constexpr int QROWB = DQK * 2, OROWB = DV * 2, KROWB = DQK * 2, STROWB = BR * 2;
  static constexpr int SQ_BYTES = BR * QROWB;
  static constexpr int SO_BYTES = BR * OROWB;
  static constexpr int SK_BYTES = DET ? 0 : BC * KROWB;
  static constexpr int SST_BYTES = BC * STROWB;
  static constexpr int OFF_Q = 0;
  static constexpr int OFF_O = OFF_Q + SQ_BYTES;
  static constexpr int OFF_K = OFF_O + SO_BYTES;
  static constexpr int OFF_ST = OFF_K + SK_BYTES;
  static constexpr int OFF_LSE = OFF_ST + SST_BYTES;
  static constexpr int OFF_DELTA = OFF_LSE + BR * 4;
  static constexpr int LDS_BYTES = OFF_DELTA + BR * 4;
  // register-prefetched 16-byte chunks per thread
  static constexpr int QCH = BR * DQK / 8 / NT;
  static constexpr int OCH = BR * DV / 8 / NT;
  static constexpr int N_RT = BR / MT;           // S/dP row tiles per wave
  static constexpr int N_DQT = DQK / MT;         // d tiles of dK^T / dQ
  static constexpr int N_DVT = DV / MT;          // d tiles of dV^T
  static constexpr int N_KQ = DQK / KT;          // GEMM1 contraction steps
  static constexpr int N_KV = DV / KT;           // GEMM2 contraction steps
  static constexpr int N_KB = BR / KT;           // GEMM3/5 contraction steps (over q)
  static constexpr int N_KC = BC / KT;           // GEMM4 contraction steps (over keys)
  static_assert(QCH * NT * 8 == BR * DQK && OCH * NT * 8 == BR * DV, "tile/thread mismatch");
  static_assert(BR % MT == 0 && BR % KT == 0 && DQK % KT == 0 && DV % KT == 0, "tile shapes");
  static_assert(DQK % MT == 0 && DV % MT == 0, "head dims must be multiples of the MFMA tile");
  static_assert(2 * BR <= NT, "lse/delta loaders");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// Operand whose contraction index runs down the rows of a swizzled row-major LDS tile, read with
// the transpose instruction: lane l gets column n_base + (l % MT) and rows k0a..k0a+3 (slots 0-3)
// and k0b..k0b+3 (slots 4-7).
template <int MT, int ROWB>
__device__ __forceinline__ bf16x8 tr_operand(const char* base, int n_base, int k0a, int k0b,
                                             int lane) {
  const int i = lane & 15;
  const int col = n_base + ((lane % MT) & ~15) + 4 * (i & 3);
  bf16x4 a = lds_read_tr(base, lds_off<ROWB>(k0a + (i >> 2), col));
  bf16x4 b = lds_read_tr(base, lds_off<ROWB>(k0b + (i >> 2), col));
  return concat(a, b);
}

template <class C>
__global__ void __launch_bounds__(C::NT, 1) bwd_main_kernel(MainParams p) {
  using M = typename C::M;
  using acc_t = typename M::acc_t;
  constexpr int MT = C::MT, BR = C::BR, BC = C::BC, DQK = C::DQK, DV = C::DV;
  constexpr int NT = C::NT, KT = C::KT, NG = C::NG, NACC = C::NACC;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* sQ = smem + C::OFF_Q;
  char* sO = smem + C::OFF_O;
  char* sK = smem + C::OFF_K;
  char* sST = smem + C::OFF_ST;
  float* sLse = reinterpret_cast<float*>(smem + C::OFF_LSE);
  float* sDelta = reinterpret_cast<float*>(smem + C::OFF_DELTA);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane / MT, lc = lane % MT;

  // Longest-first order: all heads of key tile 0 first (causal tiles near the start see the most
  // q tiles).  Consecutive blocks are different heads, so the 8 XCDs split the heads.
  const int nbh = p.B * p.Hq;
  const int bh = blockIdx.x % nbh;
  const int j = blockIdx.x / nbh;
  const int h = bh % p.Hq, b = bh / p.Hq;
  const int kvh = h / p.group;

  MaskGeom mg;
  mg.Lq = p.seq_q_lens ? min(max(p.seq_q_lens[b], 0), p.Sq) : p.Sq;
  mg.Lkv = p.seq_kv_lens ? min(max(p.seq_kv_lens[b], 0), p.Skv) : p.Skv;
  mg.diag = p.bottom_right ? mg.Lkv - mg.Lq : 0;
  mg.causal = p.causal;
  mg.W = p.window_left;
  mg.R = p.window_right;
  const int k0 = j * BC;
  int i_lo, i_hi;
  q_tile_range(mg, k0, BC, BR, &i_lo, &i_hi);

  const int64_t kv_row0 = (int64_t)(b * p.Hkv + kvh) * p.Skv;
  const int64_t q_row0 = (int64_t)(b * p.Hq + h) * p.Sq;
  const bf16_t* Kb = p.k + kv_row0 * DQK;
  const bf16_t* Vb = p.v + kv_row0 * DV;
  const bf16_t* Qb = p.q + q_row0 * DQK;
  const bf16_t* dOb = p.dO + q_row0 * DV;
  const float* lseb = p.lse + q_row0;
  const float* deltab = p.delta + q_row0;

  acc_t accK[C::N_DQT], accV[C::N_DVT];
#pragma unroll
  for (int t = 0; t < C::N_DQT; ++t) accK[t] = acc_t{};
#pragma unroll
  for (int t = 0; t < C::N_DVT; ++t) accV[t] = acc_t{};

  const int my_key = k0 + w * MT + lc;  // this lane's key (column of S, dP, P, dS)

  if (i_lo <= i_hi) {
    // ---- K/V slices into registers (B operands of GEMM1/GEMM2) --------------------------------
    bf16x8 kreg[C::N_KQ], vreg[C::N_KV];
    {
      const bool ok = my_key < p.Skv;
      const bf16_t* kr = Kb + (int64_t)(ok ? my_key : 0) * DQK + g * 8;
      const bf16_t* vr = Vb + (int64_t)(ok ? my_key : 0) * DV + g * 8;
#pragma unroll
      for (int t = 0; t < C::N_KQ; ++t)
        kreg[t] = ok ? *reinterpret_cast<const bf16x8*>(kr + t * KT) : bf16x8{};
#pragma unroll
      for (int t = 0; t < C::N_KV; ++t)
        vreg[t] = ok ? *reinterpret_cast<const bf16x8*>(vr + t * KT) : bf16x8{};
    }
    // ---- K tile into LDS (B operand of GEMM4) --------------------------------------------------
    if constexpr (!C::DET) {
      constexpr int KCH = BC * DQK / 8;
      for (int c = tid; c < KCH; c += NT) {
        const int row = c / (DQK / 8), col = (c % (DQK / 8)) * 8;
        u32x4 val = u32x4{0, 0, 0, 0};
        if (k0 + row < p.Skv) val = *reinterpret_cast<const u32x4*>(Kb + (int64_t)(k0 + row) * DQK + col);
        *reinterpret_cast<u32x4*>(sK + lds_off<C::KROWB>(row, col)) = val;
      }
    }

    // ---- prefetch registers for one q tile ------------------------------------------------------
    u32x4 pq[C::QCH], po[C::OCH];
    float pstat = 0.f;
    auto prefetch = [&](int i) {
      const int q0 = i * BR;
#pragma unroll
      for (int n = 0; n < C::QCH; ++n) {
        const int c = tid + n * NT, row = c / (DQK / 8), col = (c % (DQK / 8)) * 8;
        pq[n] = (q0 + row < p.Sq) ? *reinterpret_cast<const u32x4*>(Qb + (int64_t)(q0 + row) * DQK + col)
                                  : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int n = 0; n < C::OCH; ++n) {
        const int c = tid + n * NT, row = c / (DV / 8), col = (c % (DV / 8)) * 8;
        po[n] = (q0 + row < p.Sq) ? *reinterpret_cast<const u32x4*>(dOb + (int64_t)(q0 + row) * DV + col)
                                  : u32x4{0, 0, 0, 0};
      }
      if (tid < BR) {
        const int q = q0 + tid;
        float l = (q < mg.Lq) ? lseb[q] : -INFINITY;
        // fully masked rows (LSE = -inf) replay as P = 0: use +inf in the exponent
        pstat = (l == -INFINITY) ? INFINITY : l * kLog2e;
      } else if (tid < 2 * BR) {
        const int q = q0 + tid - BR;
        pstat = (q < p.Sq) ? deltab[q] : 0.f;
      }
    };
    prefetch(i_hi);

    for (int i = i_hi; i >= i_lo; --i) {
      const int q0 = i * BR;
      __syncthreads();  // previous tile's readers of sQ/sO/sST/stats are done
#pragma unroll
      for (int n = 0; n < C::QCH; ++n) {
        const int c = tid + n * NT, row = c / (DQK / 8), col = (c % (DQK / 8)) * 8;
        *reinterpret_cast<u32x4*>(sQ + lds_off<C::QROWB>(row, col)) = pq[n];
      }
#pragma unroll
      for (int n = 0; n < C::OCH; ++n) {
        const int c = tid + n * NT, row = c / (DV / 8), col = (c % (DV / 8)) * 8;
        *reinterpret_cast<u32x4*>(sO + lds_off<C::OROWB>(row, col)) = po[n];
      }
      if (tid < BR) sLse[tid] = pstat;
      else if (tid < 2 * BR) sDelta[tid - BR] = pstat;
      __syncthreads();
      if (i > i_lo) prefetch(i - 1);

      // ---- GEMM1 / GEMM2 ------------------------------------------------------------------------
      acc_t S[C::N_RT], dP[C::N_RT];
#pragma unroll
      for (int rt = 0; rt < C::N_RT; ++rt) {
        S[rt] = acc_t{};
        dP[rt] = acc_t{};
#pragma unroll
        for (int t = 0; t < C::N_KQ; ++t) {
          bf16x8 a = lds_read_b128(sQ, lds_off<C::QROWB>(rt * MT + lc, t * KT + g * 8));
          S[rt] = M::mma(a, kreg[t], S[rt]);
        }
#pragma unroll
        for (int t = 0; t < C::N_KV; ++t) {
          bf16x8 a = lds_read_b128(sO, lds_off<C::OROWB>(rt * MT + lc, t * KT + g * 8));
          dP[rt] = M::mma(a, vreg[t], dP[rt]);
        }
      }

      // ---- softmax replay and dS ---------------------------------------------------------------
      const bool edge = tile_needs_mask(mg, q0, BR, k0, BC);
      uint32_t pb[C::N_RT * NACC / 2], sb[C::N_RT * NACC / 2];
#pragma unroll
      for (int rt = 0; rt < C::N_RT; ++rt) {
#pragma unroll
        for (int r0 = 0; r0 < NACC; r0 += 4) {
          const int qloc = rt * MT + acc_row<MT>(r0, g);
          const floatx4 l4 = *reinterpret_cast<const floatx4*>(sLse + qloc);
          const floatx4 d4 = *reinterpret_cast<const floatx4*>(sDelta + qloc);
          float pv[4], dv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float pe = __builtin_amdgcn_exp2f(S[rt][r0 + e] * p.scale_log2 - l4[e]);
            if (edge && !mask_visible(mg, q0 + qloc + e, my_key)) pe = 0.f;
            pv[e] = pe;
            dv[e] = pe * (dP[rt][r0 + e] - d4[e]);
          }
          const int v = rt * NACC + r0;
          pb[v / 2] = pack_bf16x2(pv[0], pv[1]);
          pb[v / 2 + 1] = pack_bf16x2(pv[2], pv[3]);
          sb[v / 2] = pack_bf16x2(dv[0], dv[1]);
          sb[v / 2 + 1] = pack_bf16x2(dv[2], dv[3]);
          // dS^T tile in LDS: row = key, 4 consecutive q
          *reinterpret_cast<u32x2*>(sST + lds_off<C::STROWB>(w * MT + lc, qloc)) =
              u32x2{sb[v / 2], sb[v / 2 + 1]};
        }
      }

      // ---- GEMM3 (dV^T += dO^T P) and GEMM5 (dK^T += Q^T dS) ----------------------------------
#pragma unroll
      for (int tb = 0; tb < C::N_KB; ++tb) {
        const bf16x8 bP = __builtin_bit_cast(bf16x8, u32x4{pb[4 * tb], pb[4 * tb + 1], pb[4 * tb + 2], pb[4 * tb + 3]});
        const bf16x8 bS = __builtin_bit_cast(bf16x8, u32x4{sb[4 * tb], sb[4 * tb + 1], sb[4 * tb + 2], sb[4 * tb + 3]});
        const int ka = 8 * NG * tb + 4 * g, kb = ka + 4 * NG;
#pragma unroll
        for (int dt = 0; dt < C::N_DVT; ++dt) {
          bf16x8 a = tr_operand<MT, C::OROWB>(sO, dt * MT, ka, kb, lane);
          accV[dt] = M::mma(a, bP, accV[dt]);
        }
#pragma unroll
        for (int dt = 0; dt < C::N_DQT; ++dt) {
          bf16x8 a = tr_operand<MT, C::QROWB>(sQ, dt * MT, ka, kb, lane);
          accK[dt] = M::mma(a, bS, accK[dt]);
        }
      }
      __syncthreads();  // dS^T tile complete

      if constexpr (!C::DET) {
        // ---- GEMM4: dQ (q x d) = dS K over this tile's keys; fp32 atomics into dq_accum -------
        constexpr int NTILES = C::N_RT * C::N_DQT;
        float* dqb = p.dq_accum + q_row0 * DQK;
#pragma unroll
        for (int tt = w; tt < NTILES; tt += C::NW) {
          const int rt = tt / C::N_DQT, dt = tt % C::N_DQT;
          acc_t acc = acc_t{};
#pragma unroll
          for (int t = 0; t < C::N_KC; ++t) {
            const int ka = t * KT + 8 * g;
            bf16x8 a = tr_operand<MT, C::STROWB>(sST, rt * MT, ka, ka + 4, lane);
            bf16x8 bk = tr_operand<MT, C::KROWB>(sK, dt * MT, ka, ka + 4, lane);
            acc = M::mma(a, bk, acc);
          }
#pragma unroll
          for (int r = 0; r < NACC; ++r) {
            const int q = q0 + rt * MT + acc_row<MT>(r, g);
            if (q < mg.Lq)
              __hip_atomic_fetch_add(dqb + (int64_t)q * DQK + dt * MT + lc, acc[r], __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      } else {
        // ---- deterministic route: store the bf16 dS^T tile (keys x q) to the workspace ---------
        bf16_t* wsb = p.ds_ws + ((int64_t)(b * p.Hq + h) * p.skv_pad + k0) * p.sq_pad + q0;
        constexpr int SCH = BC * BR / 8;
        for (int c = tid; c < SCH; c += NT) {
          const int row = c / (BR / 8), col = (c % (BR / 8)) * 8;
          *reinterpret_cast<u32x4*>(wsb + (int64_t)row * p.sq_pad + col) =
              *reinterpret_cast<const u32x4*>(sST + lds_off<C::STROWB>(row, col));
        }
      }
    }
  }

  // ---- epilogue: dK (scaled) and dV, written once; rows past the sequence are zero -------------
  if (my_key < p.Skv) {
    const int oh = (p.out_heads == p.Hq) ? h : kvh;
    const int64_t orow = ((int64_t)(b * p.out_heads + oh) * p.Skv + my_key);
    bf16_t* dkr = p.dk_out + orow * DQK;
    bf16_t* dvr = p.dv_out + orow * DV;
#pragma unroll
    for (int dt = 0; dt < C::N_DQT; ++dt)
#pragma unroll
      for (int r0 = 0; r0 < NACC; r0 += 4) {
        const int d = dt * MT + acc_row<MT>(r0, g);
        *reinterpret_cast<u32x2*>(dkr + d) =
            u32x2{pack_bf16x2(accK[dt][r0] * p.scale, accK[dt][r0 + 1] * p.scale),
                  pack_bf16x2(accK[dt][r0 + 2] * p.scale, accK[dt][r0 + 3] * p.scale)};
      }
#pragma unroll
    for (int dt = 0; dt < C::N_DVT; ++dt)
#pragma unroll
      for (int r0 = 0; r0 < NACC; r0 += 4) {
        const int d = dt * MT + acc_row<MT>(r0, g);
        *reinterpret_cast<u32x2*>(dvr + d) =
            u32x2{pack_bf16x2(accV[dt][r0], accV[dt][r0 + 1]),
                  pack_bf16x2(accV[dt][r0 + 2], accV[dt][r0 + 3])};
      }
  }
}

}  // namespace sdpa
