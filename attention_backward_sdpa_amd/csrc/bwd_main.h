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
//   * 4 waves of 64 lanes, one per SIMD; wave w owns KPW keys (64 at head dim <= 128, else 32),
//     so the key tile is BC = 4 * KPW.  S and dP are computed with q as the MFMA row index and
//     keys as the column index (v_mfma_f32_32x32x16_bf16), so each wave's P and dS accumulators
//     are already the B operand of GEMM3/GEMM5 (contraction over q) and its dK^T/dV^T partials
//     complete inside the wave.
//   * LDS holds every shared operand as ready-made MFMA fragments (1 KiB each, lane-major), so
//     every operand read is one linear, bank-conflict-free ds_read_b128 at a per-lane base plus an
//     immediate offset: LDS issue rate, not bytes, bounds this kernel on gfx950, and a 16-byte
//     read costs the same issue slot as the half-as-wide transpose read.
//       - Q and dO tiles (32 q rows) as A fragments of GEMM1/GEMM2, gathered straight from Q/dO
//         with 16-byte global_load_lds;
//       - Q^T and dO^T as A fragments of GEMM5/GEMM3, written once per q tile by the preprocess
//         kernel and copied linearly;
//       - the key tile K as B fragments of GEMM1 (registers instead at head dim >= 192).
//     The q-tile buffers are double-buffered and filled one tile ahead of the compute.
//   * The wave's V slice is held in registers as the B operand of GEMM2.
//   * Deterministic route: each lane stores its bf16 dS values straight from registers (512
//     contiguous bytes per instruction); no LDS round trip.
//   * fp32-atomic route: dS is written to LDS in the same register order and GEMM4 reads it (and
//     K) with ds_read_b64_tr_b16.  GEMM4 of q tile i runs at the start of the next iteration so
//     its atomics drain while that iteration computes.
//   * The preprocess kernel supplies LSE * log2(e) per row (+inf for rows without keys), so the
//     replay is one FMA and one v_exp_f32 per element.
#pragma once
#include "common.h"
#include "masks.h"

namespace sdpa {

struct MainParams {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  const bf16_t* dO;
  const float* stats;       // (B*Hq, sq_pad, 2): [LSE*log2e or +inf, delta] per q row
  const bf16_t* qt;         // (B*Hq, sq_pad/32) tiles of Q^T fragments
  const bf16_t* dot;        // (B*Hq, sq_pad/32) tiles of dO^T fragments
  float* dq_accum;          // (B, Hq, Sq, Dqk) fp32, non-deterministic route
  bf16_t* ds_ws;            // (B*Hq, n_kv_tiles, sq_pad/32) blocks of BC x 32 bf16 dS
  bf16_t* dk_out;           // (B, out_heads, Skv, Dqk)
  bf16_t* dv_out;           // (B, out_heads, Skv, Dv)
  const int* seq_q_lens;    // (B,) or null
  const int* seq_kv_lens;   // (B,) or null
  int B, Hq, Hkv, Sq, Skv, group, out_heads;
  int causal, window_left, window_right, bottom_right;
  int n_kv_tiles;
  int sq_pad, skv_pad;      // statistics / dS workspace extents
  float scale;              // softmax scale
  float scale_log2;         // scale * log2(e)
};

template <int DQK_, int DV_, int KPW_, bool DET_>
struct MainCfg {
  static constexpr int DQK = DQK_, DV = DV_, KPW = KPW_;
  static constexpr bool DET = DET_;
  static constexpr int NW = 4, NT = 256, MT = 32, BR = 32, FRAG = 1024;
  static constexpr int BC = NW * KPW;
  static constexpr int NKT = KPW / 32;         // 32-key MFMA tiles per wave
  static constexpr bool KREG = DQK >= 192;     // GEMM1's K operand from registers
  static constexpr bool KLDS = !KREG || !DET;  // K fragments in LDS (GEMM1 and/or GEMM4)
  using M = Mfma<32>;
  static constexpr int N_DQT = DQK / MT, N_DVT = DV / MT;
  static constexpr int N_KQ = DQK / 16, N_KV = DV / 16;
  // q-tile buffer: [Q A-frags | Q^T frags | dO A-frags | dO^T frags | stats]
  static constexpr int T_QA = 0;
  static constexpr int T_QT = T_QA + N_KQ * FRAG;
  static constexpr int T_OA = T_QT + N_DQT * 2 * FRAG;
  static constexpr int T_OT = T_OA + N_KV * FRAG;
  static constexpr int T_ST = T_OT + N_DVT * 2 * FRAG;
  static constexpr int TILE_BYTES = T_ST + 2 * BR * 4;
  static constexpr int SK_BYTES = KLDS ? BC * DQK * 2 : 0;
  static constexpr int SST_BYTES = DET ? 0 : BC * BR * 2;
  static constexpr int NBUF = (SK_BYTES + 2 * TILE_BYTES + SST_BYTES <= 160 * 1024) ? 2 : 1;
  static constexpr int OFF_K = 0;
  static constexpr int OFF_T = OFF_K + SK_BYTES;
  static constexpr int OFF_ST = OFF_T + NBUF * TILE_BYTES;
  static constexpr int LDS_BYTES = OFF_ST + SST_BYTES;
  static_assert(KPW % 32 == 0, "keys per wave");
  static_assert(DQK % 64 == 0 && DV % 64 == 0, "head dims must be multiples of 64");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ void g2lds4(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)lds_wave_base, 4, 0, 0);
}
__device__ __forceinline__ void g2lds16(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}
// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima)
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Gather `nfrag` MFMA fragments of a row-major (.., D) bf16 matrix into LDS, one 16-byte
// global_load_lds per fragment and wave: fragment (rt, t) of rows row0 + 32*rt .. +31 holds, for
// lane l, row 32*rt + l % 32 and columns 16*t + 8*(l / 32) .. +7.  Fragment f = rt*(D/16) + t
// lands at lds + f * 1 KiB.  Rows at or past rows_valid re-read row rows_valid - 1 (finite data
// that every product masks out).  Fragments are spread over the 4 waves.
template <int D>
__device__ __forceinline__ void gather_frags(const bf16_t* gbase, int row0, int rows_valid,
                                             int nfrag, char* lds, int w, int lane) {
  for (int f = w; f < nfrag; f += 4) {
    const int rt = f / (D / 16), t = f % (D / 16);
    int row = row0 + 32 * rt + (lane & 31);
    row = row < rows_valid ? row : rows_valid - 1;
    g2lds16(gbase + (int64_t)row * D + 16 * t + 8 * (lane >> 5), lds + f * 1024);
  }
}

// Linear copy of `nfrag` consecutive 1 KiB fragments from global memory into LDS.
__device__ __forceinline__ void copy_frags(const bf16_t* gsrc, int nfrag, char* lds, int w,
                                           int lane) {
  for (int f = w; f < nfrag; f += 4) g2lds16(gsrc + f * 512 + lane * 8, lds + f * 1024);
}

__device__ __forceinline__ bf16x8 frag(const char* base, int f, int lane) {
  return *reinterpret_cast<const bf16x8*>(base + f * 1024 + lane * 16);
}

// Softmax replay and dS for one 32-key MFMA tile (keys key_col .. of this lane's column):
// P = exp2(S * scale * log2e - LSE * log2e) (0 on masked pairs), dS = P * (dP - delta); both are
// packed to bf16 pairs in accumulator order (pb/sb[v/2] holds registers v, v+1).
template <bool MASK>
__device__ __forceinline__ void softmax_ds(const floatx16& S, const floatx16& dP,
                                           const float* sStat, int g, float scale_log2,
                                           const MaskGeom& mg, int q_lane, int key_col,
                                           uint32_t (&pb)[8], uint32_t (&sb)[8]) {
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    // rows of accumulator registers 4x..4x+3 of this lane: g*4 + 8x + 0..3
    const floatx4 a = *reinterpret_cast<const floatx4*>(sStat + 2 * (g * 4 + 8 * x));
    const floatx4 c = *reinterpret_cast<const floatx4*>(sStat + 2 * (g * 4 + 8 * x) + 4);
    const float l4[4] = {a[0], a[2], c[0], c[2]};
    const float d4[4] = {a[1], a[3], c[1], c[3]};
    float pv[4], dv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(S[4 * x + e], scale_log2, -l4[e]));
      if constexpr (MASK) {
        if (!mask_visible(mg, q_lane + 8 * x + e, key_col)) pe = 0.f;
      }
      pv[e] = pe;
      dv[e] = pe * (dP[4 * x + e] - d4[e]);
    }
    pb[2 * x] = pack_bf16x2(pv[0], pv[1]);
    pb[2 * x + 1] = pack_bf16x2(pv[2], pv[3]);
    sb[2 * x] = pack_bf16x2(dv[0], dv[1]);
    sb[2 * x + 1] = pack_bf16x2(dv[2], dv[3]);
  }
}

// GEMM4 of the fp32-atomic route for one q tile: dQ (32 q x Dqk) = dS K over the tile's keys,
// added into dq_accum with fp32 atomics.  dS sits in sST in register order (block (w,kt,x) of
// 64 lanes x 4 q, see the writer) and K in sK as B fragments of GEMM1; both are read with the
// transpose instruction.  Wave w handles the 32-column d tiles w, w + 4, ...
template <class C>
__device__ __forceinline__ void gemm4_atomic(const char* sST, const char* sK, float* dqb, int q0,
                                             int Lq, int w, int lane) {
  using M = typename C::M;
  using acc_t = typename M::acc_t;
  constexpr int DQK = C::DQK;
  const int i = lane & 15, g = lane >> 5, lc = lane & 31;
  const int jj = i >> 2, cc = i & 3;
  const int q4 = ((lane & 16) >> 2) + cc;  // q / 4 of the 4 values this lane's address covers
  // dS (A operand): key = 16 t + 8 g + jj (+4), q = 4 q4 .. +3
  const int a_base = (q4 >> 1) * 512 + (8 * g + jj + 32 * (q4 & 1)) * 8;
  // K (B operand): key as above, d = 32 dt + (lane & 16) + 4 cc .. +3
  const int b_base = (2 * 0 + ((lane & 16) >> 4)) * 1024 + (8 * g + jj + 32 * (cc >> 1)) * 16 +
                     8 * (cc & 1);
  const bool full = q0 + C::BR <= Lq;
  for (int dt = w; dt < C::N_DQT; dt += C::NW) {
    acc_t acc = acc_t{};
#pragma unroll
    for (int t = 0; t < C::BC / 16; ++t) {
      const int ka = (t >> 1) * 2048 + (t & 1) * 128;                      // + 32 for keys +4
      const int kb = ((t >> 1) * (DQK / 16) + 2 * dt) * 1024 + (t & 1) * 256;  // + 64 for keys +4
      const bf16x8 a = concat(lds_read_tr(sST, a_base + ka), lds_read_tr(sST, a_base + ka + 32));
      const bf16x8 bk = concat(lds_read_tr(sK, b_base + kb), lds_read_tr(sK, b_base + kb + 64));
      acc = M::mma(a, bk, acc);
    }
    float* dst = dqb + dt * 32 + lc;
    if (full) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        __hip_atomic_fetch_add(dst + acc_row<32>(r, g) * DQK, acc[r], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = acc_row<32>(r, g);
        if (q0 + row < Lq)
          __hip_atomic_fetch_add(dst + row * DQK, acc[r], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

template <class C>
__global__ void __launch_bounds__(C::NT, 1) bwd_main_kernel(MainParams p) {
  using M = typename C::M;
  using acc_t = typename M::acc_t;
  constexpr int BR = C::BR, BC = C::BC, DQK = C::DQK, DV = C::DV, KPW = C::KPW, NKT = C::NKT;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* sK = smem + C::OFF_K;
  char* sST = smem + C::OFF_ST;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform per wave
  const int g = lane >> 5, lc = lane & 31;

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

  const int n_q_tiles = p.sq_pad / BR;
  const int64_t kv_row0 = (int64_t)(b * p.Hkv + kvh) * p.Skv;
  const int64_t q_row0 = (int64_t)(b * p.Hq + h) * p.Sq;
  const bf16_t* Kb = p.k + kv_row0 * DQK;
  const bf16_t* Vb = p.v + kv_row0 * DV;
  const bf16_t* Qb = p.q + q_row0 * DQK;
  const bf16_t* dOb = p.dO + q_row0 * DV;
  const float* statb = p.stats + (int64_t)bh * p.sq_pad * 2;
  const bf16_t* qtb = p.qt + (int64_t)bh * n_q_tiles * (BR * DQK);
  const bf16_t* dotb = p.dot + (int64_t)bh * n_q_tiles * (BR * DV);

  acc_t accK[C::N_DQT][NKT], accV[C::N_DVT][NKT];
#pragma unroll
  for (int t = 0; t < C::N_DQT; ++t)
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) accK[t][kt] = acc_t{};
#pragma unroll
  for (int t = 0; t < C::N_DVT; ++t)
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) accV[t][kt] = acc_t{};

  const int key_lane = k0 + w * KPW + lc;  // this lane's key in key tile 0 of the wave

  if (i_lo <= i_hi) {
    auto tile = [&](int i) -> char* { return smem + C::OFF_T + (C::NBUF == 2 ? (i & 1) : 0) * C::TILE_BYTES; };
    // ---- q tile i into its LDS buffer ----------------------------------------------------------
    auto load_tile = [&](int i) {
      char* t = tile(i);
      gather_frags<DQK>(Qb, i * BR, p.Sq, C::N_KQ, t + C::T_QA, w, lane);
      copy_frags(qtb + (int64_t)i * (BR * DQK), C::N_DQT * 2, t + C::T_QT, w, lane);
      gather_frags<DV>(dOb, i * BR, p.Sq, C::N_KV, t + C::T_OA, w, lane);
      copy_frags(dotb + (int64_t)i * (BR * DV), C::N_DVT * 2, t + C::T_OT, w, lane);
      if (w == 0)  // 64 floats: [lse2, delta] x 32 rows, already padded to sq_pad rows
        g2lds4(statb + (int64_t)i * BR * 2 + lane, t + C::T_ST);
    };
    load_tile(i_hi);
    // ---- K fragments into LDS (B operand of GEMM1 and/or GEMM4) -------------------------------
    if constexpr (C::KLDS) gather_frags<DQK>(Kb, k0, p.Skv, (BC / 32) * C::N_KQ, sK, w, lane);
    // ---- V (and K) slices into registers -------------------------------------------------------
    bf16x8 vreg[NKT][C::N_KV];
    bf16x8 kreg[C::KREG ? NKT : 1][C::KREG ? C::N_KQ : 1];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
      int key = key_lane + kt * 32;
      key = key < p.Skv ? key : p.Skv - 1;  // keys past the sequence are masked out of every product
      const bf16_t* vr = Vb + (int64_t)key * DV + g * 8;
#pragma unroll
      for (int t = 0; t < C::N_KV; ++t) vreg[kt][t] = *reinterpret_cast<const bf16x8*>(vr + t * 16);
      if constexpr (C::KREG) {
        const bf16_t* kr = Kb + (int64_t)key * DQK + g * 8;
#pragma unroll
        for (int t = 0; t < C::N_KQ; ++t) kreg[kt][t] = *reinterpret_cast<const bf16x8*>(kr + t * 16);
      }
    }

    for (int i = i_hi; i >= i_lo; --i) {
      const int q0 = i * BR;
      const char* T = tile(i);
      const float* sStat = reinterpret_cast<const float*>(T + C::T_ST);
      wait_vmem();
      __syncthreads();  // tile i landed everywhere; every wave is done with the previous tile
      if (C::NBUF == 2 && i > i_lo) load_tile(i - 1);

      if constexpr (!C::DET) {
        // GEMM4 of the previous q tile (dS in sST), deferred so its atomics overlap this tile
        if (i < i_hi) {
          gemm4_atomic<C>(sST, sK, p.dq_accum + (q_row0 + q0 + BR) * DQK, q0 + BR, mg.Lq, w, lane);
          __syncthreads();  // every wave is done reading sST
        }
      }

      // ---- per 32-key tile: GEMM1, GEMM2, softmax replay, dS -------------------------------------
      // (one key tile at a time keeps only one S/dP pair live, leaving registers for operand
      // prefetch; the Q and dO fragments are re-read from LDS for the second key tile)
      const bool edge = tile_needs_mask(mg, q0, BR, k0, BC);
      uint32_t pb[NKT][8], sb[NKT][8];
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        acc_t S = acc_t{}, dP = acc_t{};
#pragma unroll
        for (int t = 0; t < C::N_KQ; ++t) {
          const bf16x8 a = frag(T + C::T_QA, t, lane);
          if constexpr (C::KREG) {
            S = M::mma(a, kreg[kt][t], S);
          } else {
            S = M::mma(a, frag(sK, (w * NKT + kt) * C::N_KQ + t, lane), S);
          }
        }
#pragma unroll
        for (int t = 0; t < C::N_KV; ++t) dP = M::mma(frag(T + C::T_OA, t, lane), vreg[kt][t], dP);
        if (edge)
          softmax_ds<true>(S, dP, sStat, g, p.scale_log2, mg, q0 + g * 4, key_lane + kt * 32,
                           pb[kt], sb[kt]);
        else
          softmax_ds<false>(S, dP, sStat, g, p.scale_log2, mg, q0 + g * 4, key_lane + kt * 32,
                            pb[kt], sb[kt]);

        // dS in register order: block (w, kt, x) of 64 lanes x 8 bytes holds, for lane l,
        // dS^T[key = w*KPW + kt*32 + l%32][q = 4*(l/32) + 8*x + 0..3]
        if constexpr (C::DET) {
          bf16_t* wsb =
              p.ds_ws + (((int64_t)bh * p.n_kv_tiles + j) * n_q_tiles + i) * (BC * BR);
#pragma unroll
          for (int x = 0; x < 4; ++x)
            *reinterpret_cast<u32x2*>(wsb + (((w * NKT + kt) * 4 + x) * 64 + lane) * 4) =
                u32x2{sb[kt][2 * x], sb[kt][2 * x + 1]};
        } else {
#pragma unroll
          for (int x = 0; x < 4; ++x)
            *reinterpret_cast<u32x2*>(sST + (((w * NKT + kt) * 4 + x) * 64 + lane) * 8) =
                u32x2{sb[kt][2 * x], sb[kt][2 * x + 1]};
        }
      }

      // ---- GEMM3 (dV^T += dO^T P) and GEMM5 (dK^T += Q^T dS) ----------------------------------
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {  // 32 q rows = two 16-deep contraction steps
#pragma unroll
        for (int dt = 0; dt < C::N_DVT; ++dt) {
          const bf16x8 a = frag(T + C::T_OT, dt * 2 + tb, lane);
#pragma unroll
          for (int kt = 0; kt < NKT; ++kt) {
            const bf16x8 bP = __builtin_bit_cast(
                bf16x8, u32x4{pb[kt][4 * tb], pb[kt][4 * tb + 1], pb[kt][4 * tb + 2], pb[kt][4 * tb + 3]});
            accV[dt][kt] = M::mma(a, bP, accV[dt][kt]);
          }
        }
#pragma unroll
        for (int dt = 0; dt < C::N_DQT; ++dt) {
          const bf16x8 a = frag(T + C::T_QT, dt * 2 + tb, lane);
#pragma unroll
          for (int kt = 0; kt < NKT; ++kt) {
            const bf16x8 bS = __builtin_bit_cast(
                bf16x8, u32x4{sb[kt][4 * tb], sb[kt][4 * tb + 1], sb[kt][4 * tb + 2], sb[kt][4 * tb + 3]});
            accK[dt][kt] = M::mma(a, bS, accK[dt][kt]);
          }
        }
      }
      if constexpr (C::NBUF == 1) {
        __syncthreads();  // every wave is done with the single q-tile buffer
        if (i > i_lo) load_tile(i - 1);
      }
    }
    if constexpr (!C::DET) {
      __syncthreads();  // the last tile's dS is complete
      gemm4_atomic<C>(sST, sK, p.dq_accum + (q_row0 + i_lo * BR) * DQK, i_lo * BR, mg.Lq, w, lane);
    }
  }

  // ---- epilogue: dK (scaled) and dV, written once; keys past the sequence are zero -------------
  const int oh = (p.out_heads == p.Hq) ? h : kvh;
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt) {
    const int key = key_lane + kt * 32;
    if (key < p.Skv) {
      const int64_t orow = (int64_t)(b * p.out_heads + oh) * p.Skv + key;
      bf16_t* dkr = p.dk_out + orow * DQK;
      bf16_t* dvr = p.dv_out + orow * DV;
#pragma unroll
      for (int dt = 0; dt < C::N_DQT; ++dt)
#pragma unroll
        for (int r0 = 0; r0 < 16; r0 += 4) {
          const int d = dt * 32 + acc_row<32>(r0, g);
          *reinterpret_cast<u32x2*>(dkr + d) =
              u32x2{pack_bf16x2(accK[dt][kt][r0] * p.scale, accK[dt][kt][r0 + 1] * p.scale),
                    pack_bf16x2(accK[dt][kt][r0 + 2] * p.scale, accK[dt][kt][r0 + 3] * p.scale)};
        }
#pragma unroll
      for (int dt = 0; dt < C::N_DVT; ++dt)
#pragma unroll
        for (int r0 = 0; r0 < 16; r0 += 4) {
          const int d = dt * 32 + acc_row<32>(r0, g);
          *reinterpret_cast<u32x2*>(dvr + d) =
              u32x2{pack_bf16x2(accV[dt][kt][r0], accV[dt][kt][r0 + 1]),
                    pack_bf16x2(accV[dt][kt][r0 + 2], accV[dt][kt][r0 + 3])};
        }
    }
  }
}

}  // namespace sdpa
