// Deterministic dQ kernel of the two-kernel route ("SDPA Backward (SM120)", sections
// "Determinism" and "Deterministic vs. non-deterministic dQ"): dQ = scale * dS K, one workgroup per
// 32-row q tile of one query head, accumulating in registers over an ascending walk of exactly the
// KV tiles the main kernel stored for that q tile, then a single bf16 store.  No atomics and a
// fixed order, so the result is bitwise reproducible.
//
// The workspace holds each stored (KV tile, q tile) block in the main kernel's register order
// (see bwd_main.h); any 64 consecutive keys of a block are one contiguous 4 KiB piece.  Chunks of
// 64 keys of dS and of K (gathered as the main kernel's K fragments) are copied straight into LDS
// (LDS-DMA buffer loads, double-buffered) and read as MFMA operands with the transpose instruction.
// Waves split the head dim in 32-column tiles.  The dS quads and the swizzled K fragments make the
// transpose reads bank-conflict-free (layouts in bwd_main.h).
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

template <int DQK_, int BC_>
struct Dq2kCfg {
  static constexpr int DQK = DQK_, BC = BC_;
  static constexpr int BR = 32, NW = 4, NT = 256, KC = 64;   // KC: keys per LDS chunk
  static constexpr int N_DT = DQK / 32;                      // 32-column d tiles
  static constexpr int PER_W = (N_DT + NW - 1) / NW;         // d tiles per wave (at most)
  static constexpr int ST_BYTES = KC * BR * 2;               // 4 KiB of dS
  static constexpr int K_BYTES = KC * DQK * 2;               // K fragments of 64 keys
  static constexpr int BUF_BYTES = ST_BYTES + K_BYTES;
  static constexpr int LDS_BYTES = 2 * BUF_BYTES;
  static_assert(BC % KC == 0, "whole chunks per KV tile");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

template <class C>
__global__ void __launch_bounds__(C::NT, 1) dq2k_kernel(Dq2kParams p) {
  using M = Mfma<32>;
  using acc_t = M::acc_t;
  constexpr int BR = C::BR, BC = C::BC, DQK = C::DQK, KC = C::KC;
  constexpr int CPT = BC / KC;  // chunks per KV tile
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, lc = lane & 31;

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
  // chunks in ascending key order; chunks that start past the keys hold only zeros and are skipped
  const int c_first = j_first * CPT;
  int c_end = (j_last + 1) * CPT;
  const int c_keys = (p.Skv + KC - 1) / KC;
  c_end = c_end < c_keys ? c_end : c_keys;

  const bf16_t* wsh = p.ds_ws + (int64_t)bh * p.n_kv_tiles * p.n_q_tiles * (BC * BR);
  const bf16_t* Kb = p.k + (int64_t)(b * p.Hkv + kvh) * p.Skv * DQK;
  const rsrc_t rK = buf_rsrc(Kb, (int64_t)p.Skv * DQK * 2);

  auto load_chunk = [&](int c, int buf) {
    char* base = smem + buf * C::BUF_BYTES;
    const int j = c / CPT, part = c % CPT;
    const bf16_t* blk = wsh + ((int64_t)j * p.n_q_tiles + i) * (BC * BR) + part * KC * BR;
    copy_frags<C::NW>(buf_rsrc(blk, C::ST_BYTES), 0, C::ST_BYTES / 1024, base, w, lane);
    gather_frags<DQK, C::NW, true>(rK, c * KC, p.Skv, (KC / 32) * (DQK / 16), base + C::ST_BYTES,
                                   w, lane);
  };

  const Gemm4Lanes tl(lane);

  acc_t acc[C::PER_W];
#pragma unroll
  for (int t = 0; t < C::PER_W; ++t) acc[t] = acc_t{};

  if (c_first < c_end) load_chunk(c_first, 0);
  for (int c = c_first; c < c_end; ++c) {
    const int buf = (c - c_first) & 1;
    wait_vmem();
    __syncthreads();  // chunk c landed; every wave is done with the other buffer
    if (c + 1 < c_end) load_chunk(c + 1, buf ^ 1);
    const char* sST = smem + buf * C::BUF_BYTES;
    const char* sK = sST + C::ST_BYTES;
#pragma unroll
    for (int t = 0; t < KC / 16; ++t) {
      const bf16x8 a = tl.ds(sST, t);
#pragma unroll
      for (int x = 0; x < C::PER_W; ++x) {
        const int dt = w + x * C::NW;
        if (dt < C::N_DT) {
          const bf16x8 bk = tl.template k<DQK>(sK, t, dt);
          acc[x] = M::mma(a, bk, acc[x]);
        }
      }
    }
  }

  // dQ = scale * acc; rows past the buffer are not stored, rows past len_q come out exactly zero
  bf16_t* dqb = p.dq + (int64_t)(b * p.Hq + h) * p.Sq * DQK;
#pragma unroll
  for (int x = 0; x < C::PER_W; ++x) {
    const int dt = w + x * C::NW;
    if (dt < C::N_DT) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int q = q0 + acc_row<32>(r, g);
        if (q < p.Sq) dqb[(int64_t)q * DQK + dt * 32 + lc] = float_to_bf16(acc[x][r] * p.scale);
      }
    }
  }
}

}  // namespace sdpa
