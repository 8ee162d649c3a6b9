// Mask geometry shared by the host (workspace/route logic) and the kernels.
//
// "SDPA Backward (SM120)", sections "API Usage" and "Causal, sliding-window, and padding masks":
// a query row q and key k of batch entry b are visible together when
//     q < len_q,  k < len_kv,
//     causal  => k <= q + diag + R          (diag = 0 top-left, len_kv - len_q bottom-right)
//     W >= 0  => k >= q + diag - W          (left window, inclusive lower bound)
// Fully masked tiles are skipped through loop bounds; only tiles that straddle an edge evaluate
// the predicate per element.
#pragma once
#include <hip/hip_runtime.h>

namespace sdpa {

struct MaskGeom {
  int Lq, Lkv;      // actual lengths of this batch entry
  int diag;         // diagonal offset
  int causal;       // 0/1
  int W;            // left window, < 0 = none
  int R;            // right band widening of the causal diagonal
};

__host__ __device__ __forceinline__ bool mask_visible(const MaskGeom& m, int q, int k) {
  bool vis = (q < m.Lq) && (k < m.Lkv);
  if (m.causal) vis = vis && (k <= q + m.diag + m.R);
  if (m.W >= 0) vis = vis && (k >= q + m.diag - m.W);
  return vis;
}

// Inclusive range [*lo, *hi] of q tiles (BR rows each) that see at least one key of the kv tile
// starting at k0 (BC keys).  Empty when *lo > *hi.
__host__ __device__ __forceinline__ void q_tile_range(const MaskGeom& m, int k0, int BC, int BR,
                                                       int* lo, int* hi) {
  *lo = 0;
  *hi = -1;
  if (k0 >= m.Lkv || m.Lq <= 0) return;
  int kmax = (k0 + BC < m.Lkv ? k0 + BC : m.Lkv) - 1;
  int qlo = 0, qhi = m.Lq - 1;
  if (m.causal) {
    int t = k0 - m.diag - m.R;  // smallest q that sees key k0
    qlo = t > 0 ? t : 0;
  }
  if (m.W >= 0) {
    int t = kmax - m.diag + m.W;  // largest q that sees key kmax
    qhi = t < qhi ? t : qhi;
  }
  if (qlo > qhi) return;
  *lo = qlo / BR;
  *hi = qhi / BR;
}

// The first key tile (BC keys) that sees q tile i (BR rows), when any does: the key tiles that see
// a q tile are contiguous, and only a left window moves the first of them off tile 0
// ("SDPA Backward (SM120)", "Deterministic vs. non-deterministic dQ", the relay's turn offset).
__host__ __device__ __forceinline__ int first_kv_tile(const MaskGeom& m, int i, int BR, int BC) {
  if (m.W < 0) return 0;
  const int t = i * BR + m.diag - m.W;
  return t > 0 ? t / BC : 0;
}

// Does tile (q0 .. q0+BR-1) x (k0 .. k0+BC-1) contain any masked pair?
__host__ __device__ __forceinline__ bool tile_needs_mask(const MaskGeom& m, int q0, int BR, int k0,
                                                         int BC) {
  if (q0 + BR > m.Lq || k0 + BC > m.Lkv) return true;
  if (m.causal && (k0 + BC - 1 > q0 + m.diag + m.R)) return true;
  if (m.W >= 0 && (k0 < q0 + BR - 1 + m.diag - m.W)) return true;
  return false;
}

}  // namespace sdpa
