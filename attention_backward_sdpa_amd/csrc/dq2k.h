// Deterministic dQ kernel of the two-kernel route ("SDPA Backward (SM120)", sections
// "Determinism" and "Deterministic vs. non-deterministic dQ"): dQ = scale * dS K.  Each 32-row q
// tile of one query head is owned by one wave, which accumulates in registers over an ascending
// walk of exactly the KV tiles the main kernel stored for that q tile, then stores bf16 once.  No
// atomics and a fixed order per q tile, so the result is bitwise reproducible.
//
// The pass streams the dS workspace once from HBM, so it is bound by how many bytes are in flight:
//   * each wave loads its own q tile's dS straight into registers (the workspace holds each stored
//     (KV tile, q tile) block as 2 KiB per 32 keys, the writing lane's two quad pairs as 16-byte
//     pieces, layout in bwd_main.h, so 64 consecutive keys are one contiguous 4 KiB piece, four
//     16-byte non-temporal loads per lane), AHEAD chunks ahead of its MFMAs: 8 waves x AHEAD x
//     4 KiB in flight per workgroup, with no shared LDS space or barrier spent on dS.  Just before
//     use the wave writes the chunk to its own 4 KiB LDS area as quads (ds_store_off) and reads it
//     back transposed (ds_read_b64_tr_b16) as the A operand; the quad rotation keeps both
//     conflict-free;
//   * K is the only shared operand.  A workgroup of 8 waves owns 8 consecutive q tiles of one head,
//     so every 64-key chunk of K (as swizzled GEMM1 fragments, re-read from L2) serves 256 query
//     rows.  Each wave loads its share of a chunk into registers KR chunks early and writes it to
//     one of two LDS buffers at the end of the previous chunk; one barrier per chunk.  K is read
//     as the B operand with the transpose instruction, conflict-free under the swizzle;
//   * every load is an ordinary load, so the compiler's own vmcnt waits are exact.  Loads past the
//     group's last chunk re-read that chunk (L2 hits) so the pipeline has no conditional loads.
#pragma once
#include "bwd_main.h"

namespace sdpa {

struct Dq2kParams {
  const bf16_t* ds_ws;        // (B*Hq, n_kv_tiles, n_q_tiles) blocks of BC x 32 bf16
  const bf16_t* k;            // (B, Hkv, Skv, Dqk), element strides sk
  bf16_t* dq;                 // (B, Hq, Sq, Dqk), element strides sdq
  Strides sk, sdq;
  const int* seq_q_lens;
  const int* seq_kv_lens;
  int B, Hq, Hkv, Sq, Skv, group;
  int causal, window_left, window_right, bottom_right;
  int n_kv_tiles, n_q_tiles;
  int dqk_act;                // K / dQ head dim (<= DQK): dQ columns past it are not written, so
                              // the K columns past it are read unmasked (in bounds)
  float scale;
};

constexpr int gcd_c(int a, int b) { return b == 0 ? a : gcd_c(b, a % b); }
constexpr int lcm_c(int a, int b) { return a / gcd_c(a, b) * b; }

template <int DQK_, int BC_, bool F16_ = false>
struct Dq2kCfg {
  static constexpr int DQK = DQK_, BC = BC_, NW = 8;
  static constexpr bool F16 = F16_;  // fp16 io and dS instead of bf16
  static constexpr int BR = 32, NT = NW * 64, KC = 64;       // KC: keys per chunk
  static constexpr int QT = NW;                              // q tiles per workgroup, one per wave
  static constexpr int N_DT = DQK / 32;                      // 32-column d tiles per wave
  static constexpr int STEPS = KC / 16;                      // MFMA key steps per chunk
  static constexpr int DS_LOADS = KC * BR * 2 / 1024;        // 16-byte loads per lane and chunk
  static constexpr int K_FRAGS = (KC / 32) * (DQK / 16);     // K fragments of one chunk
  static constexpr int K_BYTES = K_FRAGS * 1024;
  static constexpr int K_PER_WAVE = K_FRAGS / NW;
  // chunks of dS in flight per wave, and of K held in registers (fewer at head dim 256, where the
  // 128 accumulator registers leave less room).  Measured: two chunks of dS above head dim 128 and
  // three at or below it beat deeper rings (the registers they free go to a denser schedule; a
  // single 32 KiB chunk per CU in flight already reaches the stream's rate)
  static constexpr int AHEAD = DQK > 128 ? 2 : 3;
  static constexpr int KR = DQK > 192 ? 2 : 3;
  static constexpr int UNROLL = lcm_c(lcm_c(AHEAD, KR), 2);  // ring slots and LDS buffer constant
  static constexpr int OFF_DS = 2 * K_BYTES;                 // per-wave dS transpose areas
  static constexpr int EPI_PITCH = DQK * 2 + 16;             // bytes per dQ row in the epilogue
  static constexpr int EPI_BYTES = NW * BR * EPI_PITCH;
  static constexpr int LDS_BYTES =
      OFF_DS + NW * KC * BR * 2 > EPI_BYTES ? OFF_DS + NW * KC * BR * 2 : EPI_BYTES;
  static_assert(BC % KC == 0, "whole chunks per KV tile");
  static_assert(K_FRAGS % NW == 0, "even K split over waves");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

template <class C>
__global__ void __launch_bounds__(C::NT, 1) dq2k_kernel(Dq2kParams p) {
  using M = Mfma32<C::F16>;
  using acc_t = typename M::acc_t;
  constexpr int BR = C::BR, BC = C::BC, DQK = C::DQK, KC = C::KC, QT = C::QT;
  constexpr int CPT = BC / KC;  // chunks per KV tile
  constexpr int AHEAD = C::AHEAD, KR = C::KR, U = C::UNROLL;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, lc = lane & 31;

  // Longest-first: under a causal mask the last q tiles see the most keys, so they go first.
  const int nbh = p.B * p.Hq;
  const int n_groups = (p.n_q_tiles + QT - 1) / QT;
  // Consecutive workgroups take the (batch, KV head) pairs first and the group's query heads
  // second (slot = member * B*Hkv + b*Hkv + kvh), so with B*Hkv a multiple of the 8 XCDs the query
  // heads sharing a K land on one XCD (workgroup n runs on XCD n % 8) and its K reads hit that L2.
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

  // Chunk range [cf, ce) of each q tile of the group: the KV tiles whose stored band contains the
  // tile form one contiguous run (both ends of q_tile_range are non-decreasing in the KV tile
  // index); chunks that start past the keys hold only zeros and are skipped.  The lanes evaluate
  // 64 KV tiles at a time and a ballot per q tile picks the run's ends (a per-tile scalar loop
  // would cost every wave thousands of scalar instructions on the CU's shared scalar unit).
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
  const int my_first = cf[w], my_end = ce[w];

  // this wave's q tile (clamped: a wave past the last q tile loads a valid block it never uses)
  const int my_tile = (i0 + w) < p.n_q_tiles ? (i0 + w) : (p.n_q_tiles - 1);
  const char* wsq = reinterpret_cast<const char*>(
                        p.ds_ws + ((int64_t)bh * p.n_kv_tiles * p.n_q_tiles + my_tile) * (BC * BR)) +
                    lane * 16;
  const bf16_t* Kb = p.k + b * p.sk.b + kvh * p.sk.h;
  // K columns at or past the tensor's head dim only reach dQ columns that are not stored, so they
  // need no zeroing, only in-bounds reads: a range-checked buffer over the head's rows (the host
  // keeps the span below 2^31 bytes) returns zeros past the last row's last column
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
    // (the rings hold raw 32-bit words: kept as bf16 vectors across the loop, the compiler splits
    // them into 16-bit halves, which waits for every outstanding load)
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
    char* sdS = smem + C::OFF_DS + w * (KC * BR * 2);  // this wave's transpose area
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
          // piece s = 32-key tile s / 2, accumulator groups 2 (s % 2) and 2 (s % 2) + 1 of the
          // writing lane: back to the quad layout
#pragma unroll
          for (int s = 0; s < C::DS_LOADS; ++s) {
            const u32x4 v = dsr[u % AHEAD][s];
            char* t = sdS + (s >> 1) * 2048;
            *reinterpret_cast<u32x2*>(t + ds_store_off(lane, 2 * (s & 1))) = u32x2{v[0], v[1]};
            *reinterpret_cast<u32x2*>(t + ds_store_off(lane, 2 * (s & 1) + 1)) = u32x2{v[2], v[3]};
          }
#pragma unroll
          for (int s = 0; s < C::STEPS; ++s) {
            const bf16x8 a = tl.ds(sdS, s);
#pragma unroll
            for (int dt = 0; dt < C::N_DT; ++dt) acc[dt] = M::mma(a, tl.template k<DQK>(sK, s, dt), acc[dt]);
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

  // dQ = scale * acc, through LDS as packed rows (the loop's last barrier has passed: every wave
  // is done with the K and dS areas).  A lane holds one column of 16 rows, so for accumulator rows
  // r, r + 1 (adjacent rows) an even lane packs row r's columns lc, lc + 1 and an odd lane row
  // r + 1's columns lc - 1, lc, swapping the missing value with its neighbour (DPP quad
  // permutation 1, 0, 3, 2); read back row-major, every lane stores 16 contiguous bytes of a row.
  // Rows past len_q come out exactly zero; rows past the buffer and columns past the head dim are
  // not stored.
  if (i0 + w < p.n_q_tiles) {
    char* epi = smem + w * (BR * C::EPI_PITCH);
    const bool odd = lc & 1;
#pragma unroll
    for (int dt = 0; dt < C::N_DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        // both neighbours' values move (the select then picks between two finished words, not
        // between accumulator elements, which the compiler would turn into a variable index)
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
    const int q0 = (i0 + w) * BR;
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
