// dq2k for head dim 256: dQ = scale * dS K, the ordered reduction of the
// deterministic two-kernel route ("SDPA Backward (SM120)", sections "Determinism" and
// "Deterministic vs. non-deterministic dQ"), with the head dim split over pairs of waves.
//
// In dq2k_kernel every wave owns one q tile and reads the whole K chunk (32 KiB at head dim 256)
// from LDS for it, so the transposed K reads of the 8 waves are most of the kernel's LDS traffic.
// Here the waves of a pair (2p, 2p + 1) share the q tiles 2p and 2p + 1 of the group, and wave
// 2p + h computes both tiles' dQ columns of half h of the head dim: each K operand read serves two
// q tiles, and a CU reads K once per chunk instead of eight times over, for a third less LDS
// traffic in all.
//   * dS: wave 2p + h still streams one q tile's blocks (tile 2p + h) into registers, AHEAD chunks
//     ahead, and writes chunk r + 1 as quads into a shared, double-buffered LDS area during chunk
//     r, so after the chunk's barrier both waves of the pair read both tiles' dS (transposed, as
//     in dq2k_kernel).  A tile outside its chunk range contributes zeros.
//   * K: as in dq2k_kernel, every wave loads its share of each chunk's swizzled fragments into
//     registers KR chunks early and writes it to one of two LDS buffers; one barrier per chunk.
//   * The walk over a q tile's key range is the same ascending order as dq2k_kernel's, so the
//     result is bitwise reproducible.
//   * Epilogue: each wave stages its two tiles' half rows in LDS, and after a barrier stores the
//     full rows of the tile it streamed.
// Measured on MI355X (non-causal S=8192, head dim 256): 319-320 -> 309 us.  The kernel is not bound
// by its LDS reads alone; at head dim 192 (the MLA workload) the split was 1-2 % slower.
#pragma once
#include "dq2k.h"

namespace sdpa {

template <int DQK_, int BC_, bool F16_ = false>
struct Dq2kSplitCfg {
  static constexpr int DQK = DQK_, BC = BC_, NW = 8;
  static constexpr bool F16 = F16_;  // fp16 io and dS instead of bf16
  static constexpr int BR = 32, NT = NW * 64, KC = 64;       // KC: keys per chunk
  static constexpr int QT = NW;                              // q tiles per workgroup
  static constexpr int N_DT = DQK / 32;                      // 32-column d tiles of a row
  static constexpr int N_DTH = N_DT / 2;                     // d tiles of one wave (half the row)
  static constexpr int STEPS = KC / 16;                      // MFMA key steps per chunk
  static constexpr int DS_LOADS = KC * BR * 2 / 1024;        // 16-byte loads per lane and chunk
  static constexpr int DS_TILE = KC * BR * 2;                // dS bytes of one q tile and chunk
  static constexpr int K_FRAGS = (KC / 32) * (DQK / 16);     // K fragments of one chunk
  static constexpr int K_BYTES = K_FRAGS * 1024;
  static constexpr int K_PER_WAVE = K_FRAGS / NW;
  static constexpr int AHEAD = 2, KR = 2;                    // dS / K chunks held in registers
  static constexpr int UNROLL = lcm_c(lcm_c(AHEAD, KR), 2);  // ring slots and LDS buffer constant
  static constexpr int OFF_DS = 2 * K_BYTES;                 // two dS buffers of QT tiles each
  static constexpr int DS_BUF = QT * DS_TILE;
  static constexpr int EPI_PITCH = DQK * 2 + 16;             // bytes per dQ row in the epilogue
  static constexpr int EPI_BYTES = QT * BR * EPI_PITCH;
  static constexpr int LOOP_BYTES = OFF_DS + 2 * DS_BUF;
  static constexpr int LDS_BYTES = LOOP_BYTES > EPI_BYTES ? LOOP_BYTES : EPI_BYTES;
  static_assert(N_DT % 2 == 0, "the head dim splits into two halves of 32-column tiles");
  static_assert(BC % KC == 0, "whole chunks per KV tile");
  static_assert(K_FRAGS % NW == 0, "even K split over waves");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

template <class C>
__global__ void __launch_bounds__(C::NT, 1) dq2k_split_kernel(Dq2kParams p) {
  using M = Mfma32<C::F16>;
  using acc_t = typename M::acc_t;
  constexpr int BR = C::BR, BC = C::BC, DQK = C::DQK, KC = C::KC, QT = C::QT;
  constexpr int CPT = BC / KC;  // chunks per KV tile
  constexpr int AHEAD = C::AHEAD, KR = C::KR, U = C::UNROLL, NH = C::N_DTH;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, lc = lane & 31;
  const int pr = w >> 1, hd = w & 1;  // wave pair (q tiles 2 pr, 2 pr + 1) and half of the head dim
  const int tl = 2 * pr + hd;         // the q tile whose dS this wave streams and whose dQ it stores

  // Group and chunk ranges exactly as dq2k_kernel: longest-first groups of QT q tiles, the query
  // heads sharing a K on one XCD, one ballot per q tile over 64 KV tiles at a time.
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
  // chunk ranges of the pair's two tiles and of the streamed tile
  const int pf0 = cf[2 * pr], pe0 = ce[2 * pr], pf1 = cf[2 * pr + 1], pe1 = ce[2 * pr + 1];
  const int lf = cf[tl], le = ce[tl];

  // the streamed tile's dS blocks (clamped: a tile past the last q tile loads a valid block whose
  // chunks are all outside its range)
  const int my_tile = (i0 + tl) < p.n_q_tiles ? (i0 + tl) : (p.n_q_tiles - 1);
  const char* wsq = reinterpret_cast<const char*>(
                        p.ds_ws + ((int64_t)bh * p.n_kv_tiles * p.n_q_tiles + my_tile) * (BC * BR)) +
                    lane * 16;
  const bf16_t* Kb = p.k + b * p.sk.b + kvh * p.sk.h;
  // K columns at or past the tensor's head dim only reach dQ columns that are not stored: an
  // in-bounds, range-checked buffer over the head's rows (below 2^31 bytes) is all they need
  const __amdgpu_buffer_rsrc_t rK = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(Kb), (short)0, (int)(((int64_t)(p.Skv - 1) * p.sk.s + p.dqk_act) * 2),
      0x00020000);

  const Gemm4Lanes gl(lane);
  acc_t acc[2][NH];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int j = 0; j < NH; ++j) acc[t][j] = acc_t{};

  const int n = c_hi - c_lo;  // chunks of the group (uniform over the workgroup)
  if (n > 0) {
    // chunk r of the streamed tile (relative to c_lo; loads past the end re-read the last chunk)
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
    // chunk x of the streamed tile into dS buffer buf as quads (piece s = 32-key tile s / 2,
    // accumulator groups 2 (s % 2) and 2 (s % 2) + 1 of the writing lane); zeros where the chunk
    // lies outside the tile's range (the workspace block there was never written)
    auto write_ds = [&](int x, const u32x4 (&src)[C::DS_LOADS], int buf) {
      const int c = c_lo + x;
      const bool act = lf <= c && c < le;
      char* d0 = smem + C::OFF_DS + buf * C::DS_BUF + tl * C::DS_TILE;
#pragma unroll
      for (int s = 0; s < C::DS_LOADS; ++s) {
        const u32x4 v = act ? src[s] : u32x4{};
        char* d = d0 + (s >> 1) * 2048;
        *reinterpret_cast<u32x2*>(d + ds_store_off(lane, 2 * (s & 1))) = u32x2{v[0], v[1]};
        *reinterpret_cast<u32x2*>(d + ds_store_off(lane, 2 * (s & 1) + 1)) = u32x2{v[2], v[3]};
      }
    };

    u32x4 dsr[AHEAD][C::DS_LOADS];  // slot x % AHEAD holds chunk x
    u32x4 kr[KR][C::K_PER_WAVE];
    load_k(0, kr[0]);
#pragma unroll
    for (int a = 0; a < AHEAD; ++a) load_ds(a, dsr[a]);
    store_k(kr[0], 0);
#pragma unroll
    for (int a = 1; a <= KR; ++a) load_k(a, kr[a % KR]);
    write_ds(0, dsr[0], 0);
    load_ds(AHEAD, dsr[0]);
    lds_barrier();  // K and dS of chunk 0 in buffer 0

    for (int rb = 0; rb < n; rb += U) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = rb + u;
        if (r >= n) break;
        const int c = c_lo + r;
        if ((pf0 <= c && c < pe0) || (pf1 <= c && c < pe1)) {
          const char* sK = smem + (u & 1) * C::K_BYTES;
          const char* sD = smem + C::OFF_DS + (u & 1) * C::DS_BUF + 2 * pr * C::DS_TILE;
#pragma unroll
          for (int s = 0; s < C::STEPS; ++s) {
            const bf16x8 a0 = gl.ds(sD, s), a1 = gl.ds(sD + C::DS_TILE, s);
#pragma unroll
            for (int j = 0; j < NH; ++j) {
              const bf16x8 kb = gl.template k<DQK>(sK, s, hd * NH + j);  // one read, two tiles
              acc[0][j] = M::mma(a0, kb, acc[0][j]);
              acc[1][j] = M::mma(a1, kb, acc[1][j]);
            }
          }
        }
        // chunk r + 1 into the other buffers (every wave finished reading them before the last
        // barrier), then refill the register slots
        write_ds(r + 1, dsr[(u + 1) % AHEAD], (u + 1) & 1);
        load_ds(r + 1 + AHEAD, dsr[(u + 1) % AHEAD]);
        store_k(kr[(u + 1) % KR], (u + 1) & 1);
        load_k(r + 1 + KR, kr[(u + 1) % KR]);
        lds_barrier();
      }
    }
  }

  // dQ = scale * acc through LDS (the loop's last barrier has passed: every wave is done with the
  // K and dS buffers).  Each wave stages its half rows of both tiles of its pair with the lane-pair
  // DPP packing of dq2k_kernel; after the barrier it reads back and stores the full rows of its
  // streamed tile, 16 contiguous bytes per lane.  Rows past the buffer and columns past the head
  // dim are not stored.
  {
    const bool odd = lc & 1;
    auto swap = [](float v) {
      return __builtin_bit_cast(
          float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
    };
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      char* epi = smem + (2 * pr + t) * (BR * C::EPI_PITCH);
#pragma unroll
      for (int j = 0; j < NH; ++j)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float x0 = acc[t][j][r] * p.scale, x1 = acc[t][j][r + 1] * p.scale;
          const uint32_t w_even = Elem<C::F16>::pack2(x0, swap(x0));  // row r: columns lc, lc + 1
          const uint32_t w_odd = Elem<C::F16>::pack2(swap(x1), x1);   // row r + 1: lc - 1, lc
          const int row = acc_row<32>(r, g) + (odd ? 1 : 0);
          *reinterpret_cast<uint32_t*>(epi + row * C::EPI_PITCH + ((hd * NH + j) * 32 + (lc & ~1)) * 2) =
              odd ? w_odd : w_even;
        }
    }
  }
  lds_barrier();  // both halves of every tile's rows staged
  if (i0 + tl < p.n_q_tiles) {
    const char* epi = smem + tl * (BR * C::EPI_PITCH);
    constexpr int CPR = DQK / 8;  // 16-byte pieces per row
    constexpr int NX = BR * CPR / 64;
    const int q0 = (i0 + tl) * BR;
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
}

}  // namespace sdpa
