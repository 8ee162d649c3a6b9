// dq2k with the keys of every chunk split over pairs of waves: dQ = scale * dS K, the ordered
// reduction of the deterministic two-kernel route ("SDPA Backward (SM120)", sections
// "Determinism" and "Deterministic vs. non-deterministic dQ"), for head dims up to 128.
//
// dq2k_kernel gives each of its 8 waves one q tile and the whole of every 64-key chunk.  Here the
// waves x and x + QT share q tile x of a group of QT: wave x + QT h contracts keys 32 h .. 32 h + 31
// of every chunk (MFMA steps 2 h, 2 h + 1) and streams only that half of the chunk's dS.  A wave
// then needs at most 128 registers, so a CU holds 16 waves, four per SIMD:
//   * QT = 4: 8 waves and about 64 KiB of LDS per workgroup, two workgroups per CU.  The grid has
//     twice as many workgroups as dq2k_kernel's, each half as long: finer units for the
//     longest-first order to balance on small grids;
//   * QT = 8: 16 waves per workgroup, one per CU, each K chunk in LDS serving 8 q tiles as in
//     dq2k_kernel.
//   * K is shared as in dq2k_kernel: every wave loads its share of each chunk's fragments KR
//     chunks early and writes it to one of two LDS buffers; one barrier per chunk.
//   * Each wave accumulates its half of the keys in registers, over the same ascending walk of its
//     tile's chunks.  At the end wave x + QT hands its sums to wave x through LDS, and wave x adds
//     them to its own (first half + second half, a fixed order) and stores the rows: the result is
//     bitwise reproducible, though not bitwise equal to dq2k_kernel's single running sum.
#pragma once
#include "dq2k.h"

namespace sdpa {

template <int DQK_, int BC_, bool F16_ = false, int QT_ = 4>
struct Dq2kHalfCfg {
  static constexpr int QT = QT_;                             // q tiles per workgroup
  static constexpr int DQK = DQK_, BC = BC_, NW = 2 * QT;
  static constexpr bool F16 = F16_;  // fp16 io and dS instead of bf16
  static constexpr int BR = 32, NT = NW * 64, KC = 64;       // KC: keys per chunk
  static constexpr int MIN_WG = QT == 4 ? 2 : 1;             // workgroups per CU
  static constexpr int N_DT = DQK / 32;                      // 32-column d tiles per wave
  static constexpr int STEPS = KC / 32;                      // MFMA key steps per wave and chunk
  static constexpr int DS_LOADS = KC * BR / 1024;            // 16-byte loads per lane and chunk
  static constexpr int DS_AREA = KC * BR;                    // bytes of a wave's half chunk
  static constexpr int K_FRAGS = (KC / 32) * (DQK / 16);     // K fragments of one chunk
  static constexpr int K_BYTES = K_FRAGS * 1024;
  static constexpr int K_PER_WAVE = K_FRAGS / NW;
  static constexpr int AHEAD = 2, KR = 2;                    // dS / K chunks held in registers
  static constexpr int UNROLL = lcm_c(lcm_c(AHEAD, KR), 2);  // ring slots and LDS buffer constant
  static constexpr int OFF_DS = 2 * K_BYTES;                 // per-wave dS transpose areas
  static constexpr int LOOP_BYTES = OFF_DS + NW * DS_AREA;
  static constexpr int SUM_BYTES = N_DT * 16 * 64 * 4;       // one wave's fp32 sums
  static constexpr int EPI_PITCH = DQK * 2 + 16;             // bytes per dQ row in the epilogue
  static_assert(BR * EPI_PITCH <= SUM_BYTES, "a tile's staged rows fit in its partner's sums area");
  static constexpr int END_BYTES = QT * SUM_BYTES;
  static constexpr int LDS_BYTES = LOOP_BYTES > END_BYTES ? LOOP_BYTES : END_BYTES;
  static_assert(DQK <= 128, "head dims up to 128");
  static_assert(BC % KC == 0, "whole chunks per KV tile");
  static_assert(K_FRAGS % NW == 0, "even K split over waves");
  static_assert(MIN_WG * LDS_BYTES <= 160 * 1024, "LDS budget");
};

template <class C>
__global__ void __launch_bounds__(C::NT, C::MIN_WG) dq2k_half_kernel(Dq2kParams p) {
  using M = Mfma32<C::F16>;
  using acc_t = typename M::acc_t;
  constexpr int BR = C::BR, BC = C::BC, DQK = C::DQK, KC = C::KC, QT = C::QT;
  constexpr int CPT = BC / KC;  // chunks per KV tile
  constexpr int AHEAD = C::AHEAD, KR = C::KR, U = C::UNROLL;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, lc = lane & 31;
  const int xt = w % QT, hk = w / QT;  // this wave's q tile of the group and half of the keys

  // Groups of QT q tiles, longest first; the query heads sharing a K on one XCD (as dq2k_kernel).
  const int nbh = p.B * p.Hq;
  const int n_groups = (p.n_q_tiles + QT - 1) / QT;
  const int slot = blockIdx.x % nbh;
  const int grp = n_groups - 1 - (int)(blockIdx.x / nbh);
  const int nbkv = p.B * p.Hkv;
  const int member = slot / nbkv, bk = slot % nbkv;
  const int b = bk / p.Hkv, kvh = bk % p.Hkv;
  const int h = kvh * p.group + member;
  const int bh = b * p.Hq + h;
  const int i0 = grp * QT;

  MaskGeom mg;
  mg.Lq = p.seq_q_lens ? min(max(p.seq_q_lens[b], 0), p.Sq) : p.Sq;
  mg.Lkv = p.seq_kv_lens ? min(max(p.seq_kv_lens[b], 0), p.Skv) : p.Skv;
  mg.diag = p.bottom_right ? mg.Lkv - mg.Lq : 0;
  mg.causal = p.causal;
  mg.W = p.window_left;
  mg.R = p.window_right;

  // chunk range [cf, ce) of each q tile of the group (one ballot per q tile over 64 KV tiles at
  // a time, as dq2k_kernel)
  const int c_keys = (p.Skv + KC - 1) / KC;
  int j_first[QT], j_last[QT];
#pragma unroll
  for (int x = 0; x < QT; ++x) {
    j_first[x] = p.n_kv_tiles;
    j_last[x] = -1;
  }
  for (int jb = 0; jb < p.n_kv_tiles; jb += 64) {
    const int j = jb + lane;
    int lo = 0, hi = -1;
    if (j < p.n_kv_tiles) q_tile_range(mg, j * BC, BC, BR, &lo, &hi);
#pragma unroll
    for (int x = 0; x < QT; ++x) {
      const int i = i0 + x;
      const uint64_t m = __ballot(i < p.n_q_tiles && lo <= i && i <= hi);
      if (m != 0) {
        const int f = jb + __ffsll((unsigned long long)m) - 1;
        const int l = jb + 63 - __clzll((long long)m);
        j_first[x] = f < j_first[x] ? f : j_first[x];
        j_last[x] = l;
      }
    }
  }
  int cf[QT], ce[QT];
  int c_lo = 0x7fffffff, c_hi = 0;
#pragma unroll
  for (int x = 0; x < QT; ++x) {
    cf[x] = j_first[x] * CPT;
    ce[x] = (j_last[x] + 1) * CPT < c_keys ? (j_last[x] + 1) * CPT : c_keys;
    if (cf[x] < ce[x]) {
      c_lo = cf[x] < c_lo ? cf[x] : c_lo;
      c_hi = ce[x] > c_hi ? ce[x] : c_hi;
    }
  }
  const int my_first = cf[xt], my_end = ce[xt];

  // this wave's q tile (clamped: a tile past the last one loads a valid block it never uses), and
  // its half of each chunk: the 2 KiB piece of 32 keys at offset 2048 hk of the chunk's 4 KiB
  const int my_tile = (i0 + xt) < p.n_q_tiles ? (i0 + xt) : (p.n_q_tiles - 1);
  const char* wsq = reinterpret_cast<const char*>(
                        p.ds_ws + ((int64_t)bh * p.n_kv_tiles * p.n_q_tiles + my_tile) * (BC * BR)) +
                    hk * 2048 + lane * 16;
  const bf16_t* Kb = p.k + b * p.sk.b + kvh * p.sk.h;
  // K columns at or past the tensor's head dim only reach dQ columns that are not stored: an
  // in-bounds, range-checked buffer over the head's rows (below 2^31 bytes) is all they need
  const __amdgpu_buffer_rsrc_t rK = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(Kb), (short)0, (int)(((int64_t)(p.Skv - 1) * p.sk.s + p.dqk_act) * 2),
      0x00020000);

  const Gemm4Lanes tl(lane);
  acc_t acc[C::N_DT];
#pragma unroll
  for (int t = 0; t < C::N_DT; ++t) acc[t] = acc_t{};

  const int n = c_hi - c_lo;  // chunks of the group (uniform over the workgroup)
  if (n > 0) {
    // chunk r (relative to c_lo; loads past the end re-read the last chunk)
    auto load_ds = [&](int r, u32x4 (&dst)[C::DS_LOADS]) {
      const int c = c_lo + (r < n ? r : n - 1);
      const char* src = wsq + ((int64_t)(c / CPT) * p.n_q_tiles * (BC * BR) + (c % CPT) * (KC * BR)) * 2;
#pragma unroll
      for (int s = 0; s < C::DS_LOADS; ++s)
        dst[s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + s * 1024));
    };
    auto load_k = [&](int r, u32x4 (&dst)[C::K_PER_WAVE]) {
      const int c = c_lo + (r < n ? r : n - 1);
#pragma unroll
      for (int u = 0; u < C::K_PER_WAVE; ++u)
        dst[u] = __builtin_amdgcn_raw_buffer_load_b128(
            rK, frag_src_elem<DQK, true>(w + u * C::NW, c * KC, p.Skv, lane, (int)p.sk.s) * 2, 0, 0);
    };
    auto store_k = [&](const u32x4 (&src)[C::K_PER_WAVE], int buf) {
#pragma unroll
      for (int u = 0; u < C::K_PER_WAVE; ++u)
        *reinterpret_cast<u32x4*>(smem + buf * C::K_BYTES + (w + u * C::NW) * 1024 + lane * 16) =
            src[u];
    };

    u32x4 dsr[AHEAD][C::DS_LOADS];
    char* sdS = smem + C::OFF_DS + w * C::DS_AREA;  // this wave's transpose area
    u32x4 kr[KR][C::K_PER_WAVE];
    load_k(0, kr[0]);
#pragma unroll
    for (int a = 0; a < AHEAD; ++a) load_ds(a, dsr[a]);
    store_k(kr[0], 0);
#pragma unroll
    for (int a = 1; a <= KR; ++a) load_k(a, kr[a % KR]);
    lds_barrier();  // K chunk 0 in buffer 0

    for (int rb = 0; rb < n; rb += U) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = rb + u;
        if (r >= n) break;
        const int c = c_lo + r;
        if (my_first <= c && c < my_end) {
          const char* sK = smem + (u & 1) * C::K_BYTES;
          // the half chunk's two 16-byte pieces: accumulator groups 0, 1 and 2, 3 of the writing
          // lane, back to the quad layout of one 32-key tile
#pragma unroll
          for (int s = 0; s < C::DS_LOADS; ++s) {
            const u32x4 v = dsr[u % AHEAD][s];
            *reinterpret_cast<u32x2*>(sdS + ds_store_off(lane, 2 * s)) = u32x2{v[0], v[1]};
            *reinterpret_cast<u32x2*>(sdS + ds_store_off(lane, 2 * s + 1)) = u32x2{v[2], v[3]};
          }
#pragma unroll
          for (int s = 0; s < C::STEPS; ++s) {
            const bf16x8 a = tl.ds(sdS, s);
#pragma unroll
            for (int dt = 0; dt < C::N_DT; ++dt)
              acc[dt] = M::mma(a, tl.template k<DQK>(sK, 2 * hk + s, dt), acc[dt]);
          }
        }
        load_ds(r + AHEAD, dsr[u % AHEAD]);
        // K of chunk r + 1 into the other buffer (every wave finished reading it before the last
        // barrier), then refill its register slot
        store_k(kr[(u + 1) % KR], (u + 1) & 1);
        load_k(r + 1 + KR, kr[(u + 1) % KR]);
        lds_barrier();
      }
    }
  }

  // The second half's sums to the first half's wave (the loop's last barrier has passed: every
  // wave is done with the K and dS areas), lane-major, 16 bytes per lane and accumulator quad.
  char* sums = smem + xt * C::SUM_BYTES;
  if (hk == 1) {
#pragma unroll
    for (int dt = 0; dt < C::N_DT; ++dt)
#pragma unroll
      for (int x = 0; x < 4; ++x)
        *reinterpret_cast<floatx4*>(sums + ((dt * 4 + x) * 64 + lane) * 16) =
            floatx4{acc[dt][4 * x], acc[dt][4 * x + 1], acc[dt][4 * x + 2], acc[dt][4 * x + 3]};
  }
  lds_barrier();
  if (hk == 1 || i0 + xt >= p.n_q_tiles) return;
#pragma unroll
  for (int dt = 0; dt < C::N_DT; ++dt)
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const floatx4 v = *reinterpret_cast<const floatx4*>(sums + ((dt * 4 + x) * 64 + lane) * 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[dt][4 * x + e] += v[e];
    }

  // dQ = scale * acc through this wave's own part of LDS (its partner's sums, all read above; a
  // wave's LDS accesses execute in order) as packed rows, as in dq2k_kernel: for accumulator rows
  // r, r + 1 an even lane packs row r's columns lc, lc + 1 and an odd lane row r + 1's columns
  // lc - 1, lc (DPP quad permutation 1, 0, 3, 2); read back row-major, every lane stores 16
  // contiguous bytes of a row.  Rows past the buffer and columns past the head dim are not stored.
  char* epi = sums;
  const bool odd = lc & 1;
#pragma unroll
  for (int dt = 0; dt < C::N_DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float x0 = acc[dt][r] * p.scale, x1 = acc[dt][r + 1] * p.scale;
      auto swap = [](float v) {
        return __builtin_bit_cast(
            float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
      };
      const uint32_t w_even = Elem<C::F16>::pack2(x0, swap(x0));  // row r: columns lc, lc + 1
      const uint32_t w_odd = Elem<C::F16>::pack2(swap(x1), x1);   // row r + 1: lc - 1, lc
      const int row = acc_row<32>(r, g) + (odd ? 1 : 0);
      *reinterpret_cast<uint32_t*>(epi + row * C::EPI_PITCH + (dt * 32 + (lc & ~1)) * 2) =
          odd ? w_odd : w_even;
    }
  constexpr int CPR = DQK / 8;  // 16-byte pieces per row
  constexpr int NX = BR * CPR / 64;
  const int q0 = (i0 + xt) * BR;
  bf16_t* dqb = p.dq + b * p.sdq.b + h * p.sdq.h;
  u32x4 v[NX];
#pragma unroll
  for (int x = 0; x < NX; ++x) {
    const int k = x * 64 + lane;
    v[x] = *reinterpret_cast<const u32x4*>(epi + (k / CPR) * C::EPI_PITCH + (k % CPR) * 16);
  }
#pragma unroll
  for (int x = 0; x < NX; ++x) {
    const int k = x * 64 + lane, row = k / CPR, ch = k % CPR;
    const int q = q0 + row;
    if (q < p.Sq && ch * 8 < p.dqk_act)
      *reinterpret_cast<u32x4*>(dqb + (int64_t)q * p.sdq.s + ch * 8) = v[x];
  }
}

}  // namespace sdpa
