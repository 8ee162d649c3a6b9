// Ordered dQ reduction of the dQ-partial route ("SDPA Backward (SM120)", sections "Determinism" and
// "Deterministic vs. non-deterministic dQ": per-KV-tile dQ partials, then a reduction in a fixed
// KV order):
//     dQ[b, h, q, :] = io( scale * sum_{j ascending} partial[bh, j, q tile] )
// The main kernel stores one 32 x Dqk fp32 block per (KV tile j, q tile i) it visits (GEMM4's
// result, layout in bwd_main.h); this kernel sums, for each q tile, exactly those blocks in
// ascending j with one fp32 accumulator per element and rounds once.  No atomics and a fixed
// order, so the result is bitwise reproducible.
//
// It is a pure stream of the partials (bound by HBM): one workgroup per (q tile, batch, query
// head) of 2 Dqk threads, each summing four 16-byte vectors of every block (coalesced: vector
// tid + 2 Dqk x), four blocks of loads in flight ahead of the adds.  The sums go through LDS once
// to leave as row-major 16-byte vectors of the io type.  A block's layout is GEMM4's (bwd_main.h):
//   L16 (16 x 16 output blocks): vector v = 64 (h Dqk/16 + cb) + l holds rows 16h + 4(l/16) + 0..3,
//        column 16 cb + l % 16;
//   else (32 x 32 d tiles):      vector v = 256 dt + 64 x + l holds rows 8x + 4(l/32) + 0..3,
//        column 32 dt + l % 32.
#pragma once
#include "common.h"
#include "masks.h"

namespace sdpa {

struct DqReduceParams {
  const float* dqp_ws;  // (B*Hq, n_kv_tiles, n_q_tiles) blocks of 32 x Dqk fp32
  bf16_t* dq;           // (B, Hq, Sq, Dqk), element strides sdq
  Strides sdq;
  const int* seq_q_lens;
  const int* seq_kv_lens;
  int B, Hq, Sq, Skv;
  int causal, window_left, window_right, bottom_right;
  int n_kv_tiles, n_q_tiles;
  int bc;               // keys per KV tile of the main kernel
  int dqk_act;          // dQ head dim (<= DQK): the columns written
  float scale;
  // relay route: dqp_ws holds one finished sum per (head, q tile) (n_kv_tiles = 1), present when
  // the tile has a visitor; relay_ctl[8] must equal relay_items and relay_ctl[9] be 0, else every
  // dQ element is written as NaN
  const int* relay_ctl;
  int relay_items;
};

template <int DQK, bool F16, bool L16>
__global__ void __launch_bounds__(DQK * 2) dq_reduce_kernel(DqReduceParams p) {
  constexpr int NT = DQK * 2, BR = 32, U = 4;
  constexpr int ROWF = DQK + 4;  // padded LDS row (floats)
  __shared__ __attribute__((aligned(16))) float sT[BR * ROWF];
  const int tid = threadIdx.x;

  // q tiles in descending order (under a causal mask the last ones sum the most blocks);
  // consecutive workgroups are different heads
  const int nbh = p.B * p.Hq;
  const int bh = blockIdx.x % nbh;
  const int i = p.n_q_tiles - 1 - (int)(blockIdx.x / nbh);
  const int b = bh / p.Hq, h = bh % p.Hq;
  MaskGeom mg;
  mg.Lq = p.seq_q_lens ? min(max(p.seq_q_lens[b], 0), p.Sq) : p.Sq;
  mg.Lkv = p.seq_kv_lens ? min(max(p.seq_kv_lens[b], 0), p.Skv) : p.Skv;
  mg.diag = p.bottom_right ? mg.Lkv - mg.Lq : 0;
  mg.causal = p.causal;
  mg.W = p.window_left;
  mg.R = p.window_right;
  const int q0 = i * BR;

  // KV tiles the live rows of this q tile can see (the union of the rows' key ranges); each one
  // is summed when the main kernel's q-tile range for it contains i, which is exactly the set of
  // blocks it stored
  int jlo = 0, jhi = -1;
  if (q0 < mg.Lq && mg.Lkv > 0) {
    const int qlast = min(q0 + BR, mg.Lq) - 1;
    int klo = 0, khi = mg.Lkv - 1;
    if (mg.causal) khi = min(khi, qlast + mg.diag + mg.R);
    if (mg.W >= 0) klo = max(klo, q0 + mg.diag - mg.W);
    if (klo <= khi) {
      jlo = klo / p.bc;
      jhi = khi / p.bc;
    }
  }
  auto stored = [&](int j) {
    int lo, hi;
    q_tile_range(mg, j * p.bc, p.bc, BR, &lo, &hi);
    return lo <= i && i <= hi;
  };
  bool bad = false;
  if (p.relay_ctl) {
    // the relay's sum of this q tile, present when its first possible visitor saw it
    bad = p.relay_ctl[8] != p.relay_items || p.relay_ctl[9] != 0;
    const int jf = first_kv_tile(mg, i, BR, p.bc);
    const bool any = jlo <= jhi && stored(jf);
    jlo = 0;
    jhi = any ? 0 : -1;
  }

  const int64_t blk = (int64_t)BR * DQK / 4;  // float4s per block
  const floatx4* src = reinterpret_cast<const floatx4*>(p.dqp_ws) +
                       ((int64_t)bh * p.n_kv_tiles * p.n_q_tiles + i) * blk + tid;
  const int64_t jstride = (int64_t)p.n_q_tiles * blk;
  floatx4 s[4] = {floatx4{}, floatx4{}, floatx4{}, floatx4{}};
  for (int j0 = jlo; j0 <= jhi; j0 += U) {
    floatx4 v[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int jj = min(j0 + u, jhi);  // past the range: re-read the last block, unused
#pragma unroll
      for (int x = 0; x < 4; ++x) v[u][x] = __builtin_nontemporal_load(src + jj * jstride + NT * x);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (j0 + u <= jhi && (p.relay_ctl || stored(j0 + u))) {
#pragma unroll
        for (int x = 0; x < 4; ++x) s[x] += v[u][x];
      }
    }
  }

#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int vec = tid + NT * x, l = vec & 63;
    int row0, col;
    if constexpr (L16) {
      const int b16 = vec >> 6;
      row0 = 16 * (b16 / (DQK / 16)) + 4 * (l >> 4);
      col = 16 * (b16 % (DQK / 16)) + (l & 15);
    } else {
      row0 = 8 * ((vec >> 6) & 3) + 4 * (l >> 5);
      col = 32 * (vec >> 8) + (l & 31);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) sT[(row0 + e) * ROWF + col] = s[x][e] * p.scale;
  }
  __syncthreads();

  constexpr int V = DQK / 8;  // 8-element output vectors per row
  bf16_t* dqb = p.dq + b * p.sdq.b + h * p.sdq.h;
#pragma unroll
  for (int c = tid; c < BR * V; c += NT) {
    const int r = c / V, cv = c % V, q = q0 + r;
    if (q >= p.Sq || cv * 8 >= p.dqk_act) continue;
    u32x4 out = u32x4{0u, 0u, 0u, 0u};
    if (bad) {
      const uint32_t nan2 = Elem<F16>::pack2(__builtin_nanf(""), __builtin_nanf(""));
      out = u32x4{nan2, nan2, nan2, nan2};
    } else if (q < mg.Lq) {
      const floatx4 a = *reinterpret_cast<const floatx4*>(sT + r * ROWF + cv * 8);
      const floatx4 d = *reinterpret_cast<const floatx4*>(sT + r * ROWF + cv * 8 + 4);
      out = u32x4{Elem<F16>::pack2(a[0], a[1]), Elem<F16>::pack2(a[2], a[3]),
                  Elem<F16>::pack2(d[0], d[1]), Elem<F16>::pack2(d[2], d[3])};
    }
    *reinterpret_cast<u32x4*>(dqb + q * p.sdq.s + cv * 8) = out;
  }
}

}  // namespace sdpa
