// Deterministic dQ kernel of the two-kernel route ("SDPA Backward (SM120)", sections
// "Determinism" and "Deterministic vs. non-deterministic dQ"): dQ = scale * dS K.  Each 32-row q
// tile of one query head is owned by one wave, which accumulates in registers over an ascending
// walk of exactly the KV tiles the main kernel stored for that q tile, then stores bf16 once.  No
// atomics and a fixed order per q tile, so the result is bitwise reproducible.
//
// The pass streams the dS workspace once from HBM, so it is bound by how many bytes are in flight:
//   * a workgroup of NW waves owns NW consecutive q tiles of one head, so every 64-key chunk of K
//     (re-read from L2) serves 32 * NW query rows (NW = 8 at head dim <= 128: two waves per SIMD
//     hide each other's LDS latency; NW = 4 above, where the accumulators are twice as large);
//   * chunks are staged through LDS with LDS-DMA buffer loads, NSTAGE deep (3 or 4), so up to
//     NSTAGE - 1 chunks of dS (4 KiB per q tile) are in flight per workgroup while one is consumed.
// The workspace holds each stored (KV tile, q tile) block as 2 KiB dS quads per 32 keys (layout in
// bwd_main.h), so any 64 consecutive keys of a block are one contiguous 4 KiB piece.  dS and K (as
// swizzled GEMM1 fragments) are read as MFMA operands with the transpose instruction, which the
// quad rotation and the K swizzle keep free of bank conflicts.
#pragma once
#include "bwd_main.h"

namespace sdpa {

struct Dq2kParams {
  const bf16_t* ds_ws;        // (B*Hq, n_kv_tiles, n_q_tiles) blocks of BC x 32 bf16
  const bf16_t* k;            // (B, Hkv, Skv, Dqk)
  bf16_t* dq;                 // (B, Hq, Sq, Dqk)
  const int* seq_q_lens;
  const int* seq_kv_lens;
  int B, Hq, Hkv, Sq, Skv, group;
  int causal, window_left, window_right, bottom_right;
  int n_kv_tiles, n_q_tiles;
  float scale;
};

template <int DQK_, int BC_, int NW_>
struct Dq2kCfg {
  static constexpr int DQK = DQK_, BC = BC_, NW = NW_;
  static constexpr int BR = 32, NT = NW * 64, KC = 64;       // KC: keys per chunk
  static constexpr int QT = NW;                              // q tiles per workgroup, one per wave
  static constexpr int N_DT = DQK / 32;                      // 32-column d tiles per wave
  static constexpr int ST_BYTES = KC * BR * 2;               // 4 KiB of dS per q tile and chunk
  static constexpr int DS_BYTES = QT * ST_BYTES;
  static constexpr int K_FRAGS = (KC / 32) * (DQK / 16);     // K fragments of one chunk
  static constexpr int STAGE_BYTES = DS_BYTES + K_FRAGS * 1024;
  static constexpr int NSTAGE_FIT = (160 * 1024) / STAGE_BYTES;
  static constexpr int NSTAGE = NSTAGE_FIT < 4 ? NSTAGE_FIT : 4;
  static constexpr int LDS_BYTES = NSTAGE * STAGE_BYTES;
  // LDS-DMA instructions each wave issues per stage (the same for every stage and wave, so "all
  // but the newest k stages have landed" is a constant vmcnt)
  static constexpr int DS_PER_WAVE = DS_BYTES / 1024 / NW;
  static constexpr int K_PER_WAVE = K_FRAGS / NW;
  static constexpr int OPS_PER_STAGE = DS_PER_WAVE + K_PER_WAVE;
  static_assert(BC % KC == 0, "whole chunks per KV tile");
  static_assert((DS_BYTES / 1024) % NW == 0 && K_FRAGS % NW == 0, "even DMA split over waves");
  static_assert(NSTAGE >= 2 && LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert((NSTAGE - 2) * OPS_PER_STAGE < 64, "vmcnt range");
};

// s_waitcnt vmcnt(N) with expcnt / lgkmcnt left alone (gfx9 encoding: vmcnt bits [3:0] and [15:14])
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Wait until at most `ahead` stages of OPS LDS-DMA instructions, issued after the stage about to
// be consumed, are still in flight (ahead <= MAXA <= 2).
template <int OPS, int MAXA>
__device__ __forceinline__ void wait_stage(int ahead) {
  static_assert(MAXA <= 2, "at most two stages ahead");
  if constexpr (MAXA >= 2) {
    if (ahead >= 2) {
      wait_vmem_le<2 * OPS>();
      return;
    }
  }
  if constexpr (MAXA >= 1) {
    if (ahead >= 1) {
      wait_vmem_le<OPS>();
      return;
    }
  }
  wait_vmem_le<0>();
}

template <class C>
__global__ void __launch_bounds__(C::NT, 1) dq2k_kernel(Dq2kParams p) {
  using M = Mfma<32>;
  using acc_t = M::acc_t;
  constexpr int BR = C::BR, BC = C::BC, DQK = C::DQK, KC = C::KC, QT = C::QT;
  constexpr int CPT = BC / KC;  // chunks per KV tile
  constexpr int PIECES = C::ST_BYTES / 1024;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, lc = lane & 31;

  // Longest-first: under a causal mask the last q tiles see the most keys, so they go first.
  const int nbh = p.B * p.Hq;
  const int n_groups = (p.n_q_tiles + QT - 1) / QT;
  const int bh = blockIdx.x % nbh;
  const int grp = n_groups - 1 - (int)(blockIdx.x / nbh);
  const int h = bh % p.Hq, b = bh / p.Hq;
  const int kvh = h / p.group;
  const int i0 = grp * QT;

  MaskGeom mg;
  mg.Lq = p.seq_q_lens ? min(max(p.seq_q_lens[b], 0), p.Sq) : p.Sq;
  mg.Lkv = p.seq_kv_lens ? min(max(p.seq_kv_lens[b], 0), p.Skv) : p.Skv;
  mg.diag = p.bottom_right ? mg.Lkv - mg.Lq : 0;
  mg.causal = p.causal;
  mg.W = p.window_left;
  mg.R = p.window_right;

  // Chunk range [cf, ce) of each q tile of the group: the KV tiles whose stored band contains the
  // tile form one contiguous run (both ends of q_tile_range are non-decreasing in the KV tile
  // index); chunks that start past the keys hold only zeros and are skipped.
  const int c_keys = (p.Skv + KC - 1) / KC;
  int cf[QT], ce[QT];
  int c_lo = 0x7fffffff, c_hi = 0;
#pragma unroll
  for (int x = 0; x < QT; ++x) {
    const int i = i0 + x;
    int j_first = p.n_kv_tiles, j_last = -1;
    if (i < p.n_q_tiles) {
      for (int j = 0; j < p.n_kv_tiles; ++j) {
        int lo, hi;
        q_tile_range(mg, j * BC, BC, BR, &lo, &hi);
        if (lo <= i && i <= hi) {
          j_first = j < j_first ? j : j_first;
          j_last = j;
        }
      }
    }
    cf[x] = j_first * CPT;
    ce[x] = (j_last + 1) * CPT < c_keys ? (j_last + 1) * CPT : c_keys;
    if (cf[x] < ce[x]) {
      c_lo = cf[x] < c_lo ? cf[x] : c_lo;
      c_hi = ce[x] > c_hi ? ce[x] : c_hi;
    }
  }
  const int my_first = cf[w], my_end = ce[w];

  const bf16_t* wsh = p.ds_ws + (int64_t)bh * p.n_kv_tiles * p.n_q_tiles * (BC * BR);
  const bf16_t* Kb = p.k + (int64_t)(b * p.Hkv + kvh) * p.Skv * DQK;
  const rsrc_t rK = buf_rsrc(Kb, (int64_t)p.Skv * DQK * 2);

  // Stage of chunk c: the 4 KiB dS pieces of the group's q tiles, then the K fragments.  Every
  // wave issues the same number of DMA instructions for every stage: a piece of a q tile that does
  // not cover chunk c (or lies past the last q tile) is still read, from an allocated block of the
  // same head, and never consumed.
  auto load_stage = [&](int c, int s) {
    char* base = smem + s * C::STAGE_BYTES;
    const int j = c / CPT, part = c % CPT;
#pragma unroll
    for (int u = 0; u < C::DS_PER_WAVE; ++u) {
      const int f = w + u * C::NW;  // 1 KiB piece f of the stage's dS area
      const int x = f / PIECES;
      const int tile = (i0 + x) < p.n_q_tiles ? (i0 + x) : (p.n_q_tiles - 1);
      const bf16_t* blk = wsh + ((int64_t)j * p.n_q_tiles + tile) * (BC * BR) + part * (KC * BR);
      dma16(buf_rsrc(blk, C::ST_BYTES), (uint32_t)(f % PIECES) * 1024 + lane * 16,
            base + f * 1024);
    }
    gather_frags<DQK, C::NW, true>(rK, c * KC, p.Skv, C::K_FRAGS, base + C::DS_BYTES, w, lane);
  };

  const Gemm4Lanes tl(lane);
  acc_t acc[C::N_DT];
#pragma unroll
  for (int t = 0; t < C::N_DT; ++t) acc[t] = acc_t{};

  if (c_lo < c_hi) {
#pragma unroll
    for (int s = 0; s < C::NSTAGE - 1; ++s)
      if (c_lo + s < c_hi) load_stage(c_lo + s, s);
    // chunk c sits in stage (c - c_lo) % NSTAGE; unrolled by NSTAGE so every stage offset is a
    // constant and the compiler can tell the stage being read from the ones being filled
    for (int cb = c_lo; cb < c_hi; cb += C::NSTAGE) {
#pragma unroll
      for (int u = 0; u < C::NSTAGE; ++u) {
        const int c = cb + u;
        if (c >= c_hi) break;
        // stages this wave issued after chunk c: min(NSTAGE - 2, c_hi - 1 - c)
        const int ahead = (c_hi - 1 - c) < (C::NSTAGE - 2) ? (c_hi - 1 - c) : (C::NSTAGE - 2);
        wait_stage<C::OPS_PER_STAGE, C::NSTAGE - 2>(ahead);
        lds_barrier();  // chunk c landed for every wave; every wave is done with chunk c - 1
        if (c + C::NSTAGE - 1 < c_hi) load_stage(c + C::NSTAGE - 1, (u + C::NSTAGE - 1) % C::NSTAGE);
        if (my_first <= c && c < my_end) {
          const char* sST = smem + u * C::STAGE_BYTES + w * C::ST_BYTES;
          const char* sK = smem + u * C::STAGE_BYTES + C::DS_BYTES;
#pragma unroll
          for (int t = 0; t < KC / 16; ++t) {
            const bf16x8 a = tl.ds(sST, t);
#pragma unroll
            for (int dt = 0; dt < C::N_DT; ++dt)
              acc[dt] = M::mma(a, tl.template k<DQK>(sK, t, dt), acc[dt]);
          }
        }
      }
    }
  }

  // dQ = scale * acc; rows past the buffer are not stored, rows past len_q come out exactly zero
  if (i0 + w < p.n_q_tiles) {
    const int q0 = (i0 + w) * BR;
    bf16_t* dqb = p.dq + (int64_t)(b * p.Hq + h) * p.Sq * DQK;
#pragma unroll
    for (int dt = 0; dt < C::N_DT; ++dt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int q = q0 + acc_row<32>(r, g);
        if (q < p.Sq) dqb[(int64_t)q * DQK + dt * 32 + lc] = float_to_bf16(acc[dt][r] * p.scale);
      }
    }
  }
}

}  // namespace sdpa
