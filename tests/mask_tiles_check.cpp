// Host check of the tile-range helpers of attention_backward_sdpa_amd/csrc/masks.h against the
// element-wise mask rule ("SDPA Backward (SM120)", "Causal, sliding-window, and padding masks"),
// over a grid of mask geometries:
//   * q tile i lies in q_tile_range(key tile j) exactly when the tile pair holds a visible pair;
//   * the key tiles that see a q tile are contiguous and start at first_kv_tile (the relay's turn
//     of key tile j at q tile i is j - first_kv_tile(i));
//   * tile_needs_mask is set on every tile pair that holds a masked pair.
// Prints "ok <configurations checked>" or the first failure; exit status 0 only when all hold.
#include <cstdio>

#include "../attention_backward_sdpa_amd/csrc/masks.h"

using sdpa::MaskGeom;

int main() {
  const int BR = 32;
  long configs = 0;
  const int lens[] = {0, 1, 31, 32, 33, 100, 257, 300};
  const int windows[] = {-1, 0, 5, 40, 100};
  const int bcs[] = {128, 256};
  for (int Lq : lens)
    for (int Lkv : lens)
      for (int causal = 0; causal < 2; ++causal)
        for (int br = 0; br < 2; ++br)
          for (int W : windows)
            for (int R : {0, 3, 50})
              for (int BC : bcs) {
                if (!causal && (br || R)) continue;  // diag and R only matter under causal
                if (!causal && !br && W < 0 && R) continue;
                MaskGeom m;
                m.Lq = Lq;
                m.Lkv = Lkv;
                m.diag = br ? Lkv - Lq : 0;
                m.causal = causal;
                m.W = W;
                m.R = R;
                const int nq = (Lq + BR - 1) / BR + 1, nk = (Lkv + BC - 1) / BC + 1;
                for (int i = 0; i < nq; ++i) {
                  int first = -1, last = -1, count = 0;
                  for (int j = 0; j < nk; ++j) {
                    bool any = false, masked = false;
                    for (int q = i * BR; q < (i + 1) * BR; ++q)
                      for (int k = j * BC; k < (j + 1) * BC; ++k) {
                        const bool v = sdpa::mask_visible(m, q, k);
                        any = any || v;
                        masked = masked || !v;
                      }
                    int lo, hi;
                    sdpa::q_tile_range(m, j * BC, BC, BR, &lo, &hi);
                    const bool in = lo <= i && i <= hi;
                    if (in != any) {
                      printf("q_tile_range: Lq=%d Lkv=%d causal=%d br=%d W=%d R=%d BC=%d i=%d j=%d "
                             "in=%d any=%d\n", Lq, Lkv, causal, br, W, R, BC, i, j, in, any);
                      return 1;
                    }
                    if (masked && !sdpa::tile_needs_mask(m, i * BR, BR, j * BC, BC)) {
                      printf("tile_needs_mask: Lq=%d Lkv=%d causal=%d br=%d W=%d R=%d BC=%d i=%d "
                             "j=%d\n", Lq, Lkv, causal, br, W, R, BC, i, j);
                      return 1;
                    }
                    if (any) {
                      if (first < 0) first = j;
                      last = j;
                      ++count;
                    }
                  }
                  if (count > 0 && (last - first + 1 != count ||
                                    first != sdpa::first_kv_tile(m, i, BR, BC))) {
                    printf("visitors: Lq=%d Lkv=%d causal=%d br=%d W=%d R=%d BC=%d i=%d first=%d "
                           "last=%d count=%d first_kv_tile=%d\n", Lq, Lkv, causal, br, W, R, BC, i,
                           first, last, count, sdpa::first_kv_tile(m, i, BR, BC));
                    return 1;
                  }
                }
                ++configs;
              }
  // Dense sweep of the first-visitor rule (every left window 0..300, diagonal offsets of both
  // signs, both key tiles), with the visitor sets taken from q_tile_range, checked exact above.
  for (int BC : bcs)
    for (int W = 0; W <= 300; ++W)
      for (int diag = -70; diag <= 70; diag += 7)
        for (int causal = 0; causal < 2; ++causal) {
          MaskGeom m;
          m.Lq = 700;
          m.Lkv = 700 + diag;
          m.diag = diag;
          m.causal = causal;
          m.W = W;
          m.R = 0;
          const int nq = (m.Lq + BR - 1) / BR, nk = (m.Lkv + BC - 1) / BC;
          for (int i = 0; i < nq; ++i) {
            int first = -1, last = -1, count = 0;
            for (int j = 0; j < nk; ++j) {
              int lo, hi;
              sdpa::q_tile_range(m, j * BC, BC, BR, &lo, &hi);
              if (lo <= i && i <= hi) {
                if (first < 0) first = j;
                last = j;
                ++count;
              }
            }
            if (count > 0 && (last - first + 1 != count ||
                              first != sdpa::first_kv_tile(m, i, BR, BC))) {
              printf("visitors (sweep): W=%d diag=%d causal=%d BC=%d i=%d first=%d count=%d "
                     "first_kv_tile=%d\n", W, diag, causal, BC, i, first, count,
                     sdpa::first_kv_tile(m, i, BR, BC));
              return 1;
            }
          }
          ++configs;
        }
  printf("ok %ld\n", configs);
  return 0;
}
