// Fused five-GEMM attention-backward main kernel for gfx950.
//
// "SDPA Backward (SM120)", section "Main-kernel pipeline: KV-stationary, five chained GEMMs": each
// workgroup holds one key/value tile for one query head (the K and V rows of KV head
// q_head / group), reads it a single time, then visits the q tiles that can see it, last first.
// Per q tile:
//     GEMM1  S  = Q K^T                       P  = exp2(S * scale * log2e - LSE * log2e)
//     GEMM2  dP = dO V^T                      dS = P * (dP - delta)
//     GEMM3  dV += P^T dO      (bf16 P)
//     GEMM5  dK += dS^T Q      (bf16 dS)
//     GEMM4  dQ  = dS K  -> fp32 atomic add into dq_accum
// dK/dV stay in registers for the whole pass and are written once (dK scaled by the softmax
// scale).  The deterministic routes ("Deterministic vs. non-deterministic dQ": per-KV-tile
// partials, then an ordered reduction) replace the atomics by plain stores, either
//   * of the unscaled bf16 dS tile (GEMM4 moves to the dq2k kernel, which reduces in ascending KV
//     order), or
//   * of GEMM4's fp32 result, one 32 x Dqk dQ partial per (KV tile, q tile), which the dq_reduce
//     kernel sums in ascending KV order,
// or keep GEMM4 and pass one running fp32 sum per (query head, q tile) from KV tile to KV tile in
// ascending order ("Deterministic vs. non-deterministic dQ", ordered-reduction relay; see the
// relay notes below).
//
// MI355X mapping (differs from the pages' SM120 warp-specialised design):
//   * NW waves of 64 lanes; wave w owns KPW = 32 keys, so the key tile is BC = 32 * NW.  At head
//     dims up to 192 there are 8 waves, two per SIMD, each within 256 registers: the hardware then
//     overlaps one wave's softmax VALU work and LDS latency with the other wave's MFMAs, and the
//     256-key tile halves the dQ atomics and the Q/dO re-reads per key.  At head dim 256, 4 waves
//     with 512 registers each hold the larger dK/dV accumulators; so do the kernels whose extra
//     per-element state does not fit 256 registers (a bias held in registers, the relay's bias
//     and QAT variants).
//   * S and dP are computed with q as the MFMA row index and keys as the column index
//     (v_mfma_f32_32x32x16_bf16), so each wave's P and dS accumulators are already the B operand of
//     GEMM3/GEMM5 (contraction over q) and its dK^T/dV^T partials complete inside the wave.
//   * LDS holds every shared operand as ready-made MFMA fragments (1 KiB each, lane-major, the 16-byte
//     chunks of each 256-byte row XOR-swizzled), so every GEMM1/GEMM2 operand read is one
//     bank-conflict-free ds_read_b128 at a per-lane base plus an immediate offset, and the same
//     fragments read transposed (ds_read_b64_tr_b16, also conflict-free) give the contraction-over-q
//     operands of GEMM3/GEMM5 and the contraction-over-keys operand K of GEMM4:
//       - Q and dO tiles (32 q rows), gathered straight from Q / dO with 16-byte LDS-DMA loads;
//         read as A operands of GEMM1 / GEMM2 and, transposed, as Q^T / dO^T for GEMM5 / GEMM3;
//       - the key tile K as B operands of GEMM1 (registers instead in the 4-wave kernels at head
//         dims 192 and 256) and, transposed, of GEMM4.
//     The q-tile buffers are double-buffered and filled one tile ahead of the compute.
//   * The wave's V slice is held in registers as the B operand of GEMM2.
//   * dS-panel route: each lane stores its bf16 dS values straight from registers, 16 contiguous
//     bytes per lane (1 KiB per instruction, non-temporal); no LDS round trip.
//   * fp32-atomic and dQ-partial routes: dS is written to LDS in the same register order and
//     GEMM4 reads it (and K) with ds_read_b64_tr_b16.  GEMM4 of q tile i runs at the start of the
//     next iteration so its atomics (or partial stores) drain while that iteration computes.
//   * The preprocess kernel supplies LSE * log2(e) per row (+inf for rows without keys), so the
//     replay is one FMA and one v_exp_f32 per element.
//   * Head dim 32 (8 waves, no bias, not the relay): the two waves of each SIMD (w and w + 4) run
//     half a q tile apart (staggered groups, see the q-tile loop), so that their softmax replays do
//     not coincide.
#pragma once
#include "common.h"
#include "masks.h"
#include "nvfp4.h"

namespace sdpa {

struct MainParams {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  const bf16_t* dO;
  Strides sq, sk, sv, sdo;  // element strides of q, k, v, dO
  Strides sdk, sdv;         // of dk, dv (used when dK/dV are written directly, not as partials)
  const float* stats;       // (B*Hq, sq_pad, 2): [LSE*log2e or +inf, delta] per q row
  float* dq_accum;          // (B, Hq, Sq, Dqk) fp32, non-deterministic route
  float* dqp_ws;            // (B*Hq, n_kv_tiles, sq_pad/32) blocks of 32 x Dqk fp32 dQ partials
  bf16_t* ds_ws;            // (B*Hq, n_kv_tiles, sq_pad/32) blocks of BC x 32 bf16 dS
  bf16_t* dk_out;           // dK: (B, Hkv, Skv, Dqk), or partials (B, Hq, n_split, Skv, Dqk)
  bf16_t* dv_out;           // dV: likewise with Dv
  const int* seq_q_lens;    // (B,) or null
  const int* seq_kv_lens;   // (B,) or null
  int dqk_act, dv_act;      // the tensors' head dims (<= the kernel's DQK / DV; columns past
                            // them read as zero and are not written)
  int B, Hq, Hkv, Sq, Skv, group;
  int partials;             // 1: write per-(query head, part) partials for the reduction
  int n_split;              // parts the q-tile range of a key tile is split into
  int causal, window_left, window_right, bottom_right;
  int n_kv_tiles;
  int sq_pad, skv_pad;      // statistics / dS workspace extents
  float scale;              // softmax scale
  float scale_log2;         // scale * log2(e)
  // additive bias ("API Usage" bias_tensor): (Bb, Hq, Sq, Skv) contiguous, Bb = 1 or B
  const void* bias;         // io-type or fp32 elements
  void* dbias;              // (Bb, Hq, Sq, Skv) dBias = dS (fp32, or the io type with dbias_io), or null
  int64_t bias_bstride;     // elements between batch entries of bias / dbias (0 for Bb = 1)
  int bias_f32;             // bias elements are fp32 (else the io type)
  int dbias_atomic;         // dBias accumulates over batch entries (Bb = 1, B > 1): fp32 atomics
  int dbias_io;             // dBias elements of the io type, each written once (not with dbias_atomic)
  // ordered relay (DQ_RELAY)
  float* relay_acc;         // (B*Hq, sq_pad/32) blocks of 32 x Dqk fp32: the running dQ sums
  int* relay_turn;          // (B*Hq, sq_pad/32): KV tiles that have added into each sum (zeroed)
  int* relay_ctl;           // [0, 8) per-XCD item tickets, [8] items done, [9] waits abandoned
  int relay_queues;         // XCDs of the device (1..8): one item queue each
};

// How the main kernel emits dQ.
enum DqMode {
  DQ_ATOMIC = 0,   // GEMM4 in the kernel, fp32 atomic adds into dq_accum
  DQ_DS = 1,       // no GEMM4: bf16 dS tiles to the workspace (dq2k reduces)
  DQ_PARTIAL = 2,  // GEMM4 in the kernel, fp32 partial tiles to the workspace (dq_reduce sums)
  DQ_RELAY = 3,    // GEMM4 in the kernel, added in ascending KV order into one fp32 sum per q tile
};

template <int DQK_, int DV_, int KPW_, int NW_, int MODE_, bool F16_ = false, int BIAS_ = 0,
          bool PAD_ = false, bool QAT_ = false>
struct MainCfg {
  static constexpr int DQK = DQK_, DV = DV_, KPW = KPW_, NW = NW_;
  static constexpr int MODE = MODE_;
  // the tensors' head dims are below DQK / DV (MainParams::dqk_act, dv_act): operand columns past
  // them read as zero, result columns past them are not stored.  Without it the code is that of
  // exact head dims.
  static constexpr bool PAD = PAD_;
  // NVFP4 attention QAT ("NVFP4 Attention QAT Backward", "Overview"): the inputs are already
  // fake-quantised; GEMM3 takes the fake-quantised P (dV = fake(P)^T dO) while dS, and so dQ and
  // dK, use the unquantised P.  MHA, head dim 128, bf16; the fp32 P goes through a wave-private
  // LDS area for the group scales (8 waves, or 4 on the relay route).
  static constexpr bool QAT = QAT_;
  static_assert(!QAT_ || (DQK_ == 128 && DV_ == 128 && !F16_ && BIAS_ == 0),
                "the QAT variant is bf16, head dim 128, no bias");
  // 0: no bias; 1: additive bias in the replayed scores; 2: bias and its gradient dBias = dS
  static constexpr int BIAS = BIAS_;
  static constexpr bool DS_OUT = MODE == DQ_DS;  // dS leaves the kernel, GEMM4 does not run here
  static constexpr bool G4 = !DS_OUT;            // GEMM4 runs here (dS staged in LDS)
  static constexpr bool F16 = F16_;  // fp16 io (and fp16 P / dS operands) instead of bf16
  static constexpr int NT = NW * 64, MT = 32, BR = 32, FRAG = 1024;
  static constexpr int BC = NW * KPW;
  static constexpr int NKT = KPW / 32;         // 32-key MFMA tiles per wave
  static constexpr bool KREG = DQK >= 192 && NW == 4;  // GEMM1's K operand from registers
  static constexpr bool KLDS = !KREG || G4;  // K fragments in LDS (GEMM1 and/or GEMM4)
  // LDS operand reads kept in flight ahead of the MFMAs (fewer where the 256-register budget of
  // the two-waves-per-SIMD layout is nearly full with the head-dim-192 accumulators)
  static constexpr int AHEAD = (NW == 8 && DQK > 128) ? 2 : 6;
  using M = Mfma32<F16>;
  static constexpr int N_DQT = DQK / MT, N_DVT = DV / MT;
  // GEMM4 on 16 x 16 output blocks (v_mfma_f32_16x16x32) where the 32-column d tiles would leave
  // whole SIMDs without GEMM4 work (fewer tiles than SIMDs: head dim 64): DQK / 8 blocks, NB4 per
  // wave.  Where every SIMD gets a tile (head dims 128, 192) the 32 x 32 tiles stay: measured on
  // MI355X, spreading GEMM4 over all waves there was slower (the causal GQA S=4096 D=128 main
  // kernel 350 -> 385 us on the dQ-partial route, head dim 192 724 -> 809 us on the atomic
  // route), because the waves without a tile start the next q tile early and so offset the two
  // waves of each SIMD between their softmax and MFMA phases.
  // Head dim 32 has only DQK / 8 = 4 blocks: waves 0-3 take one each, the others none.
  static constexpr int G4_BLOCKS = DQK / 8;
  static constexpr bool G4_16 =
      G4 && N_DQT < 4 && (G4_BLOCKS % NW == 0 || NW % G4_BLOCKS == 0);
  static constexpr int NB4 = G4_BLOCKS >= NW ? G4_BLOCKS / NW : 1;
  static constexpr int N_KQ = DQK / 16, N_KV = DV / 16;
  // q-tile buffer: [Q A-frags | dO A-frags | stats], fragments swizzled (see gather_frags)
  static constexpr int T_QA = 0;
  static constexpr int T_OA = T_QA + N_KQ * FRAG;
  static constexpr int T_ST = T_OA + N_KV * FRAG;
  // 8 waves with a bias: the tile's BR x BC bias elements (io type) travel with the q tile into
  // LDS (LDS-DMA, row-major); the 4-wave layout prefetches each lane's 16 elements into registers
  static constexpr bool BIAS_LDS = BIAS_ > 0 && NW_ == 8;
  static constexpr int T_BIAS = T_ST + 2 * BR * 4;
  static constexpr int TILE_BYTES = T_BIAS + (BIAS_LDS ? BR * BC * 2 : 0);
  static constexpr int SK_BYTES = KLDS ? BC * DQK * 2 : 0;
  static constexpr int SST_BYTES = G4 ? BC * BR * 2 : 0;
  // relay: the running sum of the next q tile, staged one iteration ahead (each wave stages the
  // parts of the block its GEMM4 adds to)
  static constexpr int RS_BYTES = MODE == DQ_RELAY ? BR * DQK * 4 : 0;
  // QAT: one 4 KiB fp32 P tile and 256 bytes of group scales per wave
  static constexpr int QS_WAVE = 4096 + 256;
  static constexpr int QS_BYTES = QAT_ ? NW * QS_WAVE : 0;
  static constexpr int NBUF2 =
      (SK_BYTES + 2 * TILE_BYTES + SST_BYTES + RS_BYTES + QS_BYTES <= 160 * 1024) ? 2 : 1;
  // Staggered wave groups (8 waves, no bias, no QAT, not the relay): waves 0-3 and 4-7, which
  // share the four SIMDs pairwise, run half a q tile apart, so that one wave's softmax replay
  // (VALU) overlaps the other wave's MFMAs (see the q-tile loop).  Needs a third q-tile buffer.
  // Measured on MI355X against the single-group loop (same box, causal GQA S=4096): head dim 32
  // main kernel 178 -> 160 us (dQ partials) and 181 -> 170 us (fp32 atomics); head dim 64 2-8 %
  // slower, head dim 128 neutral (dQ partials) to 3 % slower (dS panels).  Head dim 32 only.
  static constexpr bool PP = NW == 8 && DQK_ == 32 && MODE != DQ_RELAY && BIAS_ == 0 && !QAT_ &&
                             SK_BYTES + 3 * TILE_BYTES + 2 * SST_BYTES <= 160 * 1024;
  static constexpr int NBUF = PP ? 3 : NBUF2;
  // dS staging for GEMM4, double-buffered by q-tile parity where LDS allows: GEMM4 of the previous
  // q tile then needs no barrier of its own and overlaps the other waves' work
  static constexpr int NSST =
      PP ? 2
         : ((G4 && SK_BYTES + NBUF2 * TILE_BYTES + 2 * SST_BYTES + RS_BYTES + QS_BYTES <= 160 * 1024)
                ? 2
                : 1);
  // staggered groups: waves 4-7 hold GEMM4 blocks too (head dim 64: 16 x 16 blocks on all waves)
  static constexpr bool G4_B = G4 && (G4_16 ? G4_BLOCKS > NW / 2 : N_DQT > NW / 2);
  static constexpr int OFF_K = 0;
  static constexpr int OFF_T = OFF_K + SK_BYTES;
  static constexpr int OFF_ST = OFF_T + NBUF * TILE_BYTES;
  static constexpr int OFF_RS = OFF_ST + NSST * SST_BYTES;
  static constexpr int OFF_QS = OFF_RS + RS_BYTES;
  // epilogue: each wave's dK, then dV, tile (32 keys) staged as rows of EPI_PITCH bytes
  static constexpr int EPI_PITCH = (DQK > DV ? DQK : DV) * 2 + 16;
  static constexpr int EPI_BYTES = NW * 32 * EPI_PITCH;
  static constexpr int LDS_BYTES =
      OFF_QS + QS_BYTES > EPI_BYTES ? OFF_QS + QS_BYTES : EPI_BYTES;
  static_assert(KPW == 32, "one 32-key MFMA tile per wave (the q-tile loop body assumes it)");
  static_assert(NW == 4 || NW == 8, "one or two waves per SIMD");
  static_assert(DQK % 32 == 0 && DV % 32 == 0, "head dims must be multiples of 32");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// The q-tile, K and dS operands go straight from global memory into LDS with the buffer form of
// the LDS-DMA load (buffer_load ... lds): each lane supplies a byte offset into a raw buffer
// resource, the data lands at the wave-uniform LDS base (M0) + 16 (or 4) bytes * lane.  The loads
// are issued from inline assembly, so the compiler neither sees them as pending LDS writes (which
// would make it wait for every one of them before any LDS read or workgroup barrier) nor counts
// them: every consumer waits for them explicitly with vmcnt before a barrier.  M0 is written only
// here (no other instruction in these kernels reads it).  The LDS base is wave-uniform by
// construction; readfirstlane states that to the compiler so it lands in a scalar register.
typedef u32x4 rsrc_t;

// Raw buffer descriptor over `bytes` bytes at `base` (stride 0, 32-bit data format); reads past
// the end return zero.  The host keeps every buffer below 2^31 bytes.
__device__ __forceinline__ rsrc_t buf_rsrc(const void* base, int64_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return rsrc_t{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, (uint32_t)bytes, 0x00020000u};
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma4(rsrc_t r, uint32_t off, void* lds_wave_base) {
  const uint32_t l = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds_wave_base);
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(off), "s"(r), "s"(l)
               : "memory", "m0");
}
__device__ __forceinline__ void dma16(rsrc_t r, uint32_t off, void* lds_wave_base) {
  const uint32_t l = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds_wave_base);
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(off), "s"(r), "s"(l)
               : "memory", "m0");
}
// The same at device scope (sc1): the load is coherent with the device-scope stores of other CUs
// and XCDs (the relay's running sums)
__device__ __forceinline__ void dma16_dev(rsrc_t r, uint32_t off, void* lds_wave_base) {
  const uint32_t l = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds_wave_base);
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen sc1 lds"
               :
               : "v"(off), "s"(r), "s"(l)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima)
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Gather `nfrag` MFMA fragments of a row-major (rows_valid, D) bf16 matrix (buffer `src`) into
// LDS, one 16-byte load per fragment and wave: fragment (rt, t) of rows row0 + 32*rt .. +31 holds,
// for 16-byte chunk n, row 32*rt + n % 32 and columns 16*t + 8*(n / 32) .. +7 (so lane l of a
// linear read gets the B/A operand layout of v_mfma_f32_32x32x16_bf16).  Fragment f = rt*(D/16) + t
// lands at lds + f * 1 KiB.  With SWZ the chunks of each 256-byte row r of fragment f are stored
// at position (n % 16) ^ (4 * kswz(r, f)) (see kswz): the LDS-DMA destination is fixed per lane,
// so the permutation is applied to the source rows.  Rows at or past rows_valid re-read row
// rows_valid - 1 (finite data that every product masks out).  Fragments are spread over the NW
// waves.
//
// kswz spreads the 4 rows of a 32-key group that one ds_read_b64_tr_b16 of GEMM4 touches (two
// 256-byte rows of two adjacent fragments) over disjoint bank quarters, which makes those
// transpose reads conflict-free; a linear 16-lane row read stays a permutation of one row.
__device__ __forceinline__ constexpr int kswz(int row, int frag) { return (row >> 1) + 2 * (frag & 1); }

// Element offset (in the source, rows rs elements apart) of the 16 bytes this lane contributes to
// fragment f, and the first column of those 16 bytes.
template <int D, bool SWZ>
__device__ __forceinline__ int frag_src_col(int f, int lane) {
  int n = lane;
  if constexpr (SWZ) n = (lane & 48) | ((lane & 15) ^ (4 * kswz(lane >> 4, f)));
  return 16 * (f % (D / 16)) + 8 * (n >> 5);
}

template <int D, bool SWZ>
__device__ __forceinline__ int frag_src_elem(int f, int row0, int rows_valid, int lane, int rs) {
  const int rt = f / (D / 16);
  int n = lane;
  if constexpr (SWZ) n = (lane & 48) | ((lane & 15) ^ (4 * kswz(lane >> 4, f)));
  int row = row0 + 32 * rt + (n & 31);
  row = row < rows_valid ? row : rows_valid - 1;
  return row * rs + frag_src_col<D, SWZ>(f, lane);
}

// A byte offset past every buffer's range (the host keeps ranges below 2^31): the load returns
// zeros.  Used for the 16-byte chunks at or past the tensor's head dim (D is a multiple of 8),
// which pad the operands to the kernel's head dim.
constexpr uint32_t kOutOfRange = 0x80000000u;

template <int D, int NW, bool SWZ = false>
__device__ __forceinline__ void gather_frags(rsrc_t src, int row0, int rows_valid, int rs,
                                             int nfrag, char* lds, int w, int lane,
                                             int d_act = D) {
  for (int f = w; f < nfrag; f += NW)
    dma16(src,
          frag_src_col<D, SWZ>(f, lane) < d_act
              ? (uint32_t)frag_src_elem<D, SWZ>(f, row0, rows_valid, lane, rs) * 2
              : kOutOfRange,
          lds + f * 1024);
}

// Byte offset of this lane's 16-byte chunk in a linear read of swizzled fragment f (f's parity
// is all that matters).
__device__ __forceinline__ int swz_chunk(int lane, int f) {
  return (lane >> 4) * 256 + ((lane & 15) ^ (4 * kswz(lane >> 4, f))) * 16;
}

// dS of one 32-key MFMA tile (keys of one wave and key tile) is kept as 2 KiB of 8-byte quads:
// quad (key, qg) holds dS[q = 4 qg .. 4 qg + 3][key] (bf16) at byte 256 qg + 8 ((key + 4 qg) & 31).
// The rotation makes both the writer (32 keys of one qg per half-wave) and the GEMM4 transpose
// reads (4 keys x 8 qg per half-wave) touch 32 distinct bank pairs.  Offset of the quad that lane
// l stores for accumulator group x (q = 4 (l / 32) + 8 x + 0..3, key = l % 32):
__device__ __forceinline__ int ds_store_off(int lane, int x) {
  const int g = lane >> 5;
  return 512 * x + 256 * g + (((lane & 31) + 4 * g + 8 * x) & 31) * 8;
}

// Per-lane offsets of the GEMM4 (dQ = dS K) transpose reads: dS as the A operand (rows q,
// contraction over keys) and K as the B operand (contraction over keys, columns d).  MFMA step t
// covers keys 16 t .. 16 t + 15 of the key tile; each operand is two ds_read_b64_tr_b16 of 4 keys.
// Within a 16-lane block, addressing lane r = 4 jj + cc points at key 4-row jj, 4-column group cc.
struct Gemm4Lanes {
  int a[4];  // dS: key offsets 0, 4, 16, 20 within the 32-key tile
  int b[2];  // K: key offsets 0 and 4 within the 16-key step
  __device__ __forceinline__ explicit Gemm4Lanes(int lane) {
    const int jj = (lane & 15) >> 2, cc = lane & 3, g = lane >> 5, hi = (lane >> 4) & 1;
    const int qg = 4 * hi + cc;  // q = 4 qg .. +3 (output lanes 16 hi + 0..15 of the block)
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int key = 16 * (x >> 1) + 4 * (x & 1) + 8 * g + jj;
      a[x] = 256 * qg + ((key + 4 * qg) & 31) * 8;
    }
    // K fragment 2 dt + hi, chunk n = 32 (cc >> 1) + 16 (t & 1) + 8 g + 4 sec + jj, 8-byte half cc & 1
#pragma unroll
    for (int sec = 0; sec < 2; ++sec)
      b[sec] = hi * 1024 + (cc >> 1) * 512 +
               ((8 * g + 4 * sec + jj) ^ (4 * kswz(2 * (cc >> 1), hi))) * 16 + 8 * (cc & 1);
  }
  __device__ __forceinline__ bf16x8 ds(const char* sST, int t) const {
    const int base = (t >> 1) * 2048;
    return concat(lds_read_tr(sST, base + a[2 * (t & 1)]), lds_read_tr(sST, base + a[2 * (t & 1) + 1]));
  }
  template <int DQK>
  __device__ __forceinline__ bf16x8 k(const char* sK, int t, int dt) const {
    const int base = ((t >> 1) * (DQK / 16) + 2 * dt) * 1024 + (t & 1) * 256;
    return concat(lds_read_tr(sK, base + b[0]), lds_read_tr(sK, base + b[1]));
  }
};

// The lane index as a value the compiler cannot see through: offsets derived from it are then
// recomputed where they are used instead of being hoisted out of the q-tile loop, where at head
// dims 192 and up they would be spilled and reloaded (each reload waits for every outstanding
// vector memory access of the wave).
__device__ __forceinline__ int opaque_lane(int lane) {
  asm volatile("" : "+v"(lane));
  return lane;
}

// Scheduling hint for a block of NMFMA MFMAs fed by NREAD LDS reads: issue AHEAD reads first, then
// alternate one MFMA with the reads that keep the queue AHEAD deep, so LDS latency hides behind
// the matrix core instead of stalling each MFMA on an lgkmcnt(0).
template <int NREAD, int NMFMA, int AHEAD>
__device__ __forceinline__ void schedule_reads_ahead() {
  constexpr int first = NREAD < AHEAD ? NREAD : AHEAD;
  constexpr int rest = NREAD - first;
  constexpr int per = (rest + NMFMA - 1) / NMFMA;  // reads interleaved after each MFMA
  __builtin_amdgcn_sched_group_barrier(0x100, first, 0);
#pragma unroll
  for (int m = 0; m < NMFMA; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (per > 0) __builtin_amdgcn_sched_group_barrier(0x100, per, 0);
  }
}

// The rows of an edge tile that see one key, as offsets from the lane's first row q_lane: the
// visibility rule of masks.h solved for q (causal: q >= k - diag - R; window: q <= k - diag + W;
// q < len_q; none when k >= len_kv), so the per-element test is two compares.
struct KeyRows {
  int lo = 0, hi = 0;
  KeyRows() = default;
  __device__ __forceinline__ KeyRows(const MaskGeom& mg, int q_lane, int key) {
    int a = 0, z = mg.Lq - 1;
    if (key >= mg.Lkv) z = -1;
    if (mg.causal) a = max(a, key - mg.diag - mg.R);
    if (mg.W >= 0) z = min(z, key - mg.diag + mg.W);
    lo = a - q_lane;
    hi = z - q_lane;
  }
};

// Softmax replay and dS for one 32-key MFMA tile of this lane's key column, accumulator groups
// X0 and X0 + 1 (the q rows of contraction step X0 / 2 of GEMM3/GEMM5):
// P = exp2(S * scale * log2e - LSE * log2e), dS = P * (dP - delta); both are packed to io-type
// pairs in accumulator order (pb/sb[v/2] holds registers v, v+1).  No masking here: on edge tiles
// mask_pairs clears the invisible pairs afterwards.
template <bool F16, int X0, int BIAS = 0, bool QAT = false>
__device__ __forceinline__ void softmax_ds(const floatx16& S, const floatx16& dP,
                                           const float* sStat, int g, float scale_log2,
                                           uint32_t (&pb)[8], uint32_t (&sb)[8],
                                           const float* bl = nullptr, float* dsf = nullptr,
                                           float* pf = nullptr) {
#pragma unroll
  for (int x = X0; x < X0 + 2; ++x) {
    // rows of accumulator registers 4x..4x+3 of this lane: g*4 + 8x + 0..3
    const floatx4 a = *reinterpret_cast<const floatx4*>(sStat + 2 * (g * 4 + 8 * x));
    const floatx4 c = *reinterpret_cast<const floatx4*>(sStat + 2 * (g * 4 + 8 * x) + 4);
    const float l4[4] = {a[0], a[2], c[0], c[2]};
    const float d4[4] = {a[1], a[3], c[1], c[3]};
    float pv[4], dv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // with a bias: exponent + bias * log2(e) (bl holds the lane's bias * log2 e per register)
      const float off = BIAS ? bl[4 * x + e] - l4[e] : -l4[e];
      pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[4 * x + e], scale_log2, off));
      dv[e] = pv[e] * (dP[4 * x + e] - d4[e]);
      if constexpr (BIAS == 2) dsf[4 * x + e] = dv[e];
      if constexpr (QAT) pf[4 * x + e] = pv[e];  // fp32 P for the fake quantisation
    }
    pb[2 * x] = Elem<F16>::pack2(pv[0], pv[1]);
    pb[2 * x + 1] = Elem<F16>::pack2(pv[2], pv[3]);
    sb[2 * x] = Elem<F16>::pack2(dv[0], dv[1]);
    sb[2 * x + 1] = Elem<F16>::pack2(dv[2], dv[3]);
  }
}

// Visible rows of this lane's key among its accumulator rows, as a 32-bit mask over the row
// offset c = 8 x + e from the lane's first row (KeyRows gives the visible offsets [lo, hi]).
__device__ __forceinline__ uint32_t visible_rows(const KeyRows& vis) {
  const int lo = vis.lo > 0 ? vis.lo : 0;
  const int hi = vis.hi < 31 ? vis.hi : 31;
  if (lo > hi) return 0u;
  return ((2u << hi) - 1u) & ~((1u << lo) - 1u);
}

// Edge tiles: clear the packed P / dS of invisible pairs in accumulator groups X0, X0 + 1 (their
// unmasked replay may be anything, even inf or NaN; the result is exactly 0).
template <int X0>
__device__ __forceinline__ void mask_pairs(uint32_t m, uint32_t (&pb)[8], uint32_t (&sb)[8]) {
#pragma unroll
  for (int x = X0; x < X0 + 2; ++x) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = 8 * x + 2 * h;  // rows c, c + 1 in the two halves of the word
      const uint32_t keep = (((m >> c) & 1u) * 0x0000FFFFu) | (((m >> (c + 1)) & 1u) * 0xFFFF0000u);
      pb[2 * x + h] &= keep;
      sb[2 * x + h] &= keep;
    }
  }
}

template <int V>
struct IntTag {
  static constexpr int value = V;
};

// Per-lane offsets of the GEMM3 / GEMM5 A operands, dO^T and Q^T (rows d, contraction over the
// tile's 32 q rows), read with ds_read_b64_tr_b16 straight from the swizzled A fragments of GEMM1 /
// GEMM2.  MFMA step tb covers q 16 tb .. +15 in the order in which the accumulator layout delivers P
// and dS as B operands: k slot 8 g + 4 sec + m holds q = 16 tb + 8 sec + 4 g + m.  Addressing lane
// r = 4 jj + cc of a 16-lane block points at q row 16 tb + 8 sec + 4 g + jj, columns 4 cc .. +3 of
// fragment 2 dt + (lane / 16) % 2.
struct TrALanes {
  int o[2];  // sec = 0, 1
  __device__ __forceinline__ explicit TrALanes(int lane) {
    const int jj = (lane & 15) >> 2, cc = lane & 3, g = lane >> 5, hi = (lane >> 4) & 1;
#pragma unroll
    for (int sec = 0; sec < 2; ++sec)
      o[sec] = hi * 1024 + (cc >> 1) * 512 +
               ((8 * sec + 4 * g + jj) ^ (4 * kswz(2 * (cc >> 1), hi))) * 16 + 8 * (cc & 1);
  }
  __device__ __forceinline__ bf16x8 read(const char* frags, int dt, int tb) const {
    const int base = dt * 2048 + tb * 256;
    return concat(lds_read_tr(frags, base + o[0]), lds_read_tr(frags, base + o[1]));
  }
};

// dS staging layout of the 16x16 GEMM4 (same 2 KiB per 32-key wave tile as the quads above, with
// its own rotation): quad (key, qg) at byte 256 qg + 8 ((key + rot16(qg)) & 31).  The writer (32
// keys of one qg per half-wave) and the GEMM4 transpose reads (keys 8G + 4 sec + 0..3 of lane
// groups G = 0, 1 or 2, 3, four consecutive qg per half-wave) both touch every bank pair once.
__device__ __forceinline__ constexpr int rot16(int qg) { return 4 * (qg & 1) + 16 * ((qg >> 1) & 1); }
__device__ __forceinline__ int ds_store_off16(int lane, int x) {
  const int qg = 2 * x + (lane >> 5);
  return 256 * qg + (((lane & 31) + rot16(qg)) & 31) * 8;
}

// Per-lane offsets of the 16x16 GEMM4 transpose reads of wave w.  Its blocks all lie in row half
// h = w % 2 and have 16-column blocks cb of one parity c = (w / 2) % 2 (NW / 2 is even).  MFMA
// step s covers the keys of wave tile s (32 keys); lane group G = lane / 16 holds k slots
// 8G .. 8G + 7 = keys 8G + 0..7 of the step, as two ds_read_b64_tr_b16 of 4 keys (sec 0, 1).
// Within a 16-lane block, addressing lane r = 4 jj + cc points at key 8G + 4 sec + jj and
//   dS: q group qg = 4h + cc (rows 4 qg .. +3 of the quad), output lane i = q row 16h + i;
//   K:  row (G / 2) + 2 (cc / 2) of the fragment, chunk 8 (G % 2) + 4 sec + jj (swizzled as
//       gather_frags stores it), 8-byte half cc % 2: d columns 4 cc .. +3 of the 16-column block.
struct Gemm4Lanes16 {
  int a[2], b[2];
  __device__ __forceinline__ Gemm4Lanes16(int lane, int w) {
    const int G = lane >> 4, jj = (lane & 15) >> 2, cc = lane & 3;
    const int h = w & 1, c = (w >> 1) & 1;
    const int qg = 4 * h + cc;
#pragma unroll
    for (int sec = 0; sec < 2; ++sec) {
      const int key = 8 * G + 4 * sec + jj;
      a[sec] = 256 * qg + 8 * ((key + rot16(qg)) & 31);
      b[sec] = ((G >> 1) + 2 * (cc >> 1)) * 256 +
               ((8 * (G & 1) + 4 * sec + jj) ^ (4 * kswz(2 * (cc >> 1), c))) * 16 + 8 * (cc & 1);
    }
  }
  __device__ __forceinline__ bf16x8 ds(const char* sST, int s) const {
    return concat(lds_read_tr(sST, s * 2048 + a[0]), lds_read_tr(sST, s * 2048 + a[1]));
  }
  template <int DQK>
  __device__ __forceinline__ bf16x8 k(const char* sK, int s, int cb) const {
    const int base = (s * (DQK / 16) + cb) * 1024;
    return concat(lds_read_tr(sK, base + b[0]), lds_read_tr(sK, base + b[1]));
  }
};

// ---- ordered relay ("Deterministic vs. non-deterministic dQ", ordered-reduction relay) ----------
// The KV tiles that see q tile i of a query head add their GEMM4 results into one fp32 running sum
// of that (head, q tile), in ascending KV order; turn[head, i] counts the KV tiles that have added.
// The visitors of a q tile are contiguous in KV index (both ends of a key tile's q-tile range grow
// with the key tile), so key tile j's turn at q tile i is j - jfirst(i), jfirst(i) being the first
// visitor, which stores its result without reading.  The sum of a (head, q tile) block uses the
// dQ-partial block layout of GEMM4 (below).  On MI355X:
//   * forward progress: a workgroup does not work on the item of its blockIdx but takes the next
//     ticket of its XCD's queue once it runs, and an item only ever waits for items earlier in the
//     same queue.  The earliest unfinished item is therefore held by a running workgroup that waits
//     for nothing unfinished, whatever order the workgroups are dispatched in.
//   * coherence: sums and turns are written and read with device-scope (sc1) accesses only, which
//     miss the CU's L1 and are coherent across the device; the turn is published once every wave's
//     stores of the sum have completed.  No cache-wide writeback or invalidation is needed.  (XCD
//     x's queue holds the query heads bh with bh % queues == x, as the blockIdx order of the other
//     routes does, so a head's K/V and Q/dO stay in one L2.)
//   * the successor stages the sum into LDS with LDS-DMA loads one q tile ahead (after waiting for
//     its turn), together with the next tile's operands, and adds it in GEMM4.
//   * a wait longer than kRelaySpinLimit polls is abandoned and counted in ctl[9]; once that has
//     happened the other waits end at once, so every launch finishes (the dQ conversion then
//     writes NaN).
constexpr int kRelaySpinLimit = 1 << 18;
constexpr int kHwregXccId = 20 | (0 << 6) | (3 << 11);  // hwreg(HW_REG_XCC_ID, 0, 4)
constexpr int kSc1 = 16;  // cache-policy operand of the buffer builtins: sc1 (device scope)

// Wave-uniform wait until *turn >= want.
__device__ __forceinline__ void relay_wait(int* turn, int want, int* ctl, int lane) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(turn, (short)0, 4, 0x00020000);
  for (int n = 0;; ++n) {
    const int v = __builtin_amdgcn_readfirstlane((int)__builtin_amdgcn_raw_buffer_load_b32(r, 0, 0, kSc1));
    if (v >= want) return;
    if ((n & 63) == 63 &&
        (n >= kRelaySpinLimit ||
         __hip_atomic_load(ctl + 9, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0)) {
      if (n >= kRelaySpinLimit && lane == 0)
        __hip_atomic_fetch_add(ctl + 9, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// Publish a turn (one lane), device scope.
__device__ __forceinline__ void relay_publish(int* turn, int value) {
  __builtin_amdgcn_raw_buffer_store_b32(
      value, __builtin_amdgcn_make_buffer_rsrc(turn, (short)0, 4, 0x00020000), 0, 0, kSc1);
}

// Store 16 bytes of a running sum (a block of `bytes` at base), device scope.
__device__ __forceinline__ void relay_store16(float* base, int bytes, int byte_off, floatx4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(
      __builtin_bit_cast(u32x4, v), __builtin_amdgcn_make_buffer_rsrc(base, (short)0, bytes, 0x00020000),
      byte_off, 0, kSc1);
}

// GEMM4 for one q tile on 16 x 16 blocks (C::G4_16): wave w computes blocks w + NW m, m < NB4,
// block b = (row half b % 2, 16-column block b / 2).  Emission as in gemm4 below, with the
// partial block's layout: block (h, cb) is 1 KiB at float offset 256 (h (Dqk / 16) + cb), lane l's
// four floats (rows 16h + 4 (l / 16) + 0..3, column 16 cb + l % 16) the 16 bytes at 4 l.
template <class C>
__device__ __forceinline__ void gemm4_16(const char* sST, const char* sK, float* dst, int q0,
                                         int Lq, int w, int lane, const char* rs = nullptr,
                                         bool add = false) {
  using M16 = Mfma16<C::F16>;
  constexpr int DQK = C::DQK, NB = C::NB4, NW = C::NW;
  if (w >= C::G4_BLOCKS) return;  // head dim 32: waves past the 4 blocks have none
  const Gemm4Lanes16 tl(C::DQK >= 192 ? opaque_lane(lane) : lane, w);
  floatx4 acc[NB];
#pragma unroll
  for (int m = 0; m < NB; ++m) acc[m] = floatx4{};
#pragma unroll
  for (int s = 0; s < C::BC / 32; ++s) {
    const bf16x8 a = tl.ds(sST, s);
#pragma unroll
    for (int m = 0; m < NB; ++m) acc[m] = M16::mma(a, tl.template k<DQK>(sK, s, (w + NW * m) >> 1), acc[m]);
  }
  const int h = w & 1, G = lane >> 4, col_l = lane & 15;
#pragma unroll
  for (int m = 0; m < NB; ++m) {
    const int cb = (w + NW * m) >> 1;
    if constexpr (C::MODE == DQ_PARTIAL) {
      __builtin_nontemporal_store(acc[m], reinterpret_cast<floatx4*>(dst + (h * (DQK / 16) + cb) * 256) + lane);
    } else if constexpr (C::MODE == DQ_RELAY) {
      // the running sum (staged in LDS at the block's offset) plus this key tile's block
      const int off = (h * (DQK / 16) + cb) * 256;
      floatx4 v = acc[m];
      if (add) v += reinterpret_cast<const floatx4*>(rs)[off / 4 + lane];
      relay_store16(dst, C::BR * DQK * 4, (off + 4 * lane) * 4, v);
    } else {
      float* col0 = dst + 16 * cb + col_l;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * h + 4 * G + r;
        if (q0 + row < Lq)
          __hip_atomic_fetch_add(col0 + row * DQK, acc[m][r], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

// GEMM4 for one q tile: dQ (32 q x Dqk) = dS K over the tile's keys.  dS sits in sST in register
// order (block (w,kt,x) of 64 lanes x 4 q, see the writer) and K in sK as B fragments of GEMM1;
// both are read with the transpose instruction.  Wave w handles the 32-column d tiles w, w + NW,
// ... (with 8 waves and Dqk = 128 only waves 0-3 have a tile; each shares its SIMD with a wave
// that has none).  The result leaves the kernel as
//   * DQ_ATOMIC: fp32 atomic adds into the dq_accum rows starting at `dst` (row q0); rows at or
//     past Lq are skipped;
//   * DQ_PARTIAL: plain non-temporal stores of the tile's partial block at `dst`: d tile dt is
//     4 KiB at float offset 1024 dt, lane l's accumulator registers 4x .. 4x + 3 (rows
//     8x + 4(l / 32) + 0..3, column 32 dt + l % 32) being the 16 bytes at float offset
//     256 x + 4 l, so every store instruction writes 1 KiB contiguously.  Rows past Lq hold the
//     products of their cleared dS (zeros); the reduction does not use them;
//   * DQ_RELAY: the same block layout, as the running sum of the (head, q tile): the block plus
//     the sum staged in LDS at `rs` (when `add`), stored at device scope.
template <class C>
__device__ __forceinline__ void gemm4(const char* sST, const char* sK, float* dst, int q0, int Lq,
                                      int w, int lane, const char* rs = nullptr, bool add = false) {
  using M = typename C::M;
  using acc_t = typename M::acc_t;
  constexpr int DQK = C::DQK;
  // head dims 192 and up: lane offsets recomputed here (see opaque_lane); below, the registers
  // to hold them are there
  const int ol = C::DQK >= 192 ? opaque_lane(lane) : lane;
  const int g = ol >> 5, lc = ol & 31;
  const Gemm4Lanes tl(ol);
  const bool full = q0 + C::BR <= Lq;
  for (int dt = w; dt < C::N_DQT; dt += C::NW) {
    acc_t acc = acc_t{};
#pragma unroll
    for (int t = 0; t < C::BC / 16; ++t) acc = M::mma(tl.ds(sST, t), tl.template k<DQK>(sK, t, dt), acc);
    if constexpr (C::MODE == DQ_PARTIAL) {
      floatx4* blk = reinterpret_cast<floatx4*>(dst + dt * 1024) + lane;
#pragma unroll
      for (int x = 0; x < 4; ++x)
        __builtin_nontemporal_store(floatx4{acc[4 * x], acc[4 * x + 1], acc[4 * x + 2], acc[4 * x + 3]},
                                    blk + 64 * x);
    } else if constexpr (C::MODE == DQ_RELAY) {
      // the running sum (staged in LDS in the block layout) plus this key tile's block
      const floatx4* stg = reinterpret_cast<const floatx4*>(rs) + dt * 256 + lane;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        floatx4 v = floatx4{acc[4 * x], acc[4 * x + 1], acc[4 * x + 2], acc[4 * x + 3]};
        if (add) v += stg[64 * x];
        relay_store16(dst, C::BR * DQK * 4, (dt * 1024 + 256 * x + 4 * lane) * 4, v);
      }
    } else {
      // register r holds row 4g + rc(r), rc(r) = 8 (r / 4) + r % 4: the lane-dependent part goes
      // into the base pointer, the rest is a constant per register (no per-row addresses to keep)
      float* base = dst + dt * 32 + lc + (4 * g) * DQK;
      if (full) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          __hip_atomic_fetch_add(base + ((r / 4) * 8 + r % 4) * DQK, acc[r], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
      } else {
        const int live = Lq - q0 - 4 * g;  // registers whose rc is below this are rows < Lq
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rc = (r / 4) * 8 + r % 4;
          if (rc < live)
            __hip_atomic_fetch_add(base + rc * DQK, acc[r], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
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
  // dS staging buffer of q tile i
  auto sST = [&](int i) -> char* {
    return smem + C::OFF_ST + (C::NSST == 2 ? (i & 1) : 0) * C::SST_BYTES;
  };

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform per wave
  const int g = lane >> 5, lc = lane & 31;

  // Longest-first order: all heads of key tile 0 (part 0, then the other parts of its q-tile
  // range) first: causal tiles near the start see the most q tiles.  Consecutive blocks are
  // different heads, so the 8 XCDs split the heads.
  const int nbh = p.B * p.Hq;
  int item = blockIdx.x;
  if constexpr (C::MODE == DQ_RELAY) {
    // the relay takes the next item of this XCD's queue instead (same order within a queue; see
    // the relay notes): queue x holds the heads bh = x, x + queues, ... of every key tile
    __shared__ int s_item;
    if (tid == 0) {
      const int nq = p.relay_queues;
      const int x = (int)((unsigned)__builtin_amdgcn_s_getreg(kHwregXccId) % (unsigned)nq);
      const int t = __hip_atomic_fetch_add(p.relay_ctl + x, 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
      const int nbh_x = (nbh - x + nq - 1) / nq;
      s_item = t < p.n_kv_tiles * p.n_split * nbh_x ? (t / nbh_x) * nbh + x + nq * (t % nbh_x) : -1;
    }
    __syncthreads();
    item = __builtin_amdgcn_readfirstlane(s_item);
    if (item < 0) return;  // more workgroups than items on this XCD
  }
  const int bh = item % nbh;
  const int js = item / nbh;
  const int j = js / p.n_split, part = js % p.n_split;
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
  if (p.n_split > 1 && i_lo <= i_hi) {  // this workgroup's part of the range (part 0 on top)
    const int per = (i_hi - i_lo + p.n_split) / p.n_split;
    i_hi -= part * per;
    i_lo = i_hi - per + 1 > i_lo ? i_hi - per + 1 : i_lo;
  }

  const int n_q_tiles = p.sq_pad / BR;
  const int64_t q_row0 = (int64_t)(b * p.Hq + h) * p.Sq;  // row of the contiguous dq_accum
  // where GEMM4's result for q tile i goes: the tile's first dq_accum row (atomic route) or its
  // partial block (bh, j, i) of 32 x Dqk floats
  auto dq_dst = [&](int i) -> float* {
    if constexpr (C::MODE == DQ_PARTIAL)
      return p.dqp_ws + (((int64_t)bh * p.n_kv_tiles + j) * n_q_tiles + i) * (BR * DQK);
    else if constexpr (C::MODE == DQ_RELAY)
      return p.relay_acc + ((int64_t)bh * n_q_tiles + i) * (BR * DQK);
    else
      return p.dq_accum + (q_row0 + (int64_t)i * BR) * DQK;
  };
  // relay: this key tile's turn at q tile i, and the turn counter
  auto relay_rank = [&](int i) { return j - first_kv_tile(mg, i, BR, BC); };
  auto relay_turn = [&](int i) { return p.relay_turn + (int64_t)bh * n_q_tiles + i; };
  const bf16_t* Kb = p.k + b * p.sk.b + kvh * p.sk.h;
  const bf16_t* Vb = p.v + b * p.sv.b + kvh * p.sv.h;
  const bf16_t* Qb = p.q + b * p.sq.b + h * p.sq.h;
  const bf16_t* dOb = p.dO + b * p.sdo.b + h * p.sdo.h;
  const float* statb = p.stats + (int64_t)bh * p.sq_pad * 2;
  // one head's rows (the host keeps each span below 2^31 bytes)
  const int dqk_act = C::PAD ? p.dqk_act : DQK, dv_act = C::PAD ? p.dv_act : DV;
  const rsrc_t rQ = buf_rsrc(Qb, ((int64_t)(p.Sq - 1) * p.sq.s + dqk_act) * 2);
  const rsrc_t rdO = buf_rsrc(dOb, ((int64_t)(p.Sq - 1) * p.sdo.s + dv_act) * 2);
  const rsrc_t rStat = buf_rsrc(statb, (int64_t)p.sq_pad * 2 * 4);
  // the head's bias for the LDS-staged layout: io-type elements, the host keeps the span below
  // 2^31 bytes and Skv a multiple of 8 (16-byte chunks within a row)
  const rsrc_t rBias = buf_rsrc(
      C::BIAS_LDS ? reinterpret_cast<const bf16_t*>(p.bias) + (int64_t)b * p.bias_bstride +
                        (int64_t)h * p.Sq * p.Skv
                  : nullptr,
      C::BIAS_LDS ? (int64_t)p.Sq * p.Skv * 2 : 0);

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
  const int kofs[2] = {swz_chunk(lane, 0), swz_chunk(lane, 1)};  // fragment reads, by parity
  const TrALanes tra(lane);

  if (i_lo <= i_hi) {
    auto tile = [&](int i) -> char* {
      const int buf = C::NBUF == 3 ? i % 3 : C::NBUF == 2 ? (i & 1) : 0;
      return smem + C::OFF_T + buf * C::TILE_BYTES;
    };
    // ---- q tile i into its LDS buffer ----------------------------------------------------------
    auto load_tile = [&](int i) {
      char* t = tile(i);
      gather_frags<DQK, C::NW, true>(rQ, i * BR, p.Sq, (int)p.sq.s, C::N_KQ, t + C::T_QA, w, lane,
                                     dqk_act);
      gather_frags<DV, C::NW, true>(rdO, i * BR, p.Sq, (int)p.sdo.s, C::N_KV, t + C::T_OA, w, lane,
                                    dv_act);
      if (w == 0)  // 64 floats: [lse2, delta] x 32 rows, already padded to sq_pad rows
        dma4(rStat, (uint32_t)(i * BR * 2 + lane) * 4, t + C::T_ST);
      if constexpr (C::BIAS_LDS) {
        // bias rows i * BR .. + BR - 1, keys k0 .. k0 + BC - 1: 16-byte chunk c = 64 m + lane
        // holds row c / (BC / 8), keys 8 (c % (BC / 8)) .. + 7 (rows past Sq read zeros; keys past
        // Skv read the next row's values, which the masking clears)
#pragma unroll
        for (int m = w; m < C::BR * C::BC * 2 / 1024; m += C::NW) {
          const int c = m * 64 + lane, row = c / (BC / 8), col = (c % (BC / 8)) * 8;
          dma16(rBias, ((uint32_t)(i * BR + row) * (uint32_t)p.Skv + (uint32_t)(k0 + col)) * 2u,
                t + C::T_BIAS + m * 1024);
        }
      }
    };
    load_tile(i_hi);
    // ---- K fragments into LDS (B operand of GEMM1 and/or GEMM4) -------------------------------
    if constexpr (C::KLDS)
      gather_frags<DQK, C::NW, true>(buf_rsrc(Kb, ((int64_t)(p.Skv - 1) * p.sk.s + dqk_act) * 2),
                                     k0, p.Skv, (int)p.sk.s, (BC / 32) * C::N_KQ, sK, w, lane,
                                     dqk_act);
    // ---- V (and K) slices into registers -------------------------------------------------------
    bf16x8 vreg[NKT][C::N_KV];
    bf16x8 kreg[C::KREG ? NKT : 1][C::KREG ? C::N_KQ : 1];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
      int key = key_lane + kt * 32;
      key = key < p.Skv ? key : p.Skv - 1;  // keys past the sequence are masked out of every product
      // columns at or past the tensor's head dim are zero (read from column 0, then cleared)
      const bf16_t* vr = Vb + (int64_t)key * p.sv.s;
#pragma unroll
      for (int t = 0; t < C::N_KV; ++t) {
        const int col = g * 8 + t * 16;
        const bf16x8 x = *reinterpret_cast<const bf16x8*>(vr + (col < dv_act ? col : 0));
        vreg[kt][t] = col < dv_act ? x : bf16x8{};
      }
      if constexpr (C::KREG) {
        const bf16_t* kr = Kb + (int64_t)key * p.sk.s;
#pragma unroll
        for (int t = 0; t < C::N_KQ; ++t) {
          const int col = g * 8 + t * 16;
          const bf16x8 x = *reinterpret_cast<const bf16x8*>(kr + (col < dqk_act ? col : 0));
          kreg[kt][t] = col < dqk_act ? x : bf16x8{};
        }
      }
    }

    // dS-panel route: the previous q tile's packed dS, stored at the start of the next iteration
    // (after that iteration's tile loads), so the wait for those loads one iteration later
    // finds the stores long done instead of stalling on stores issued just before it
    uint32_t sb_prev[8];
    auto store_ds = [&](int i_t) {
      // dS of the wave's 32 keys to the workspace: 2 KiB per 32 keys, lane l's quads of
      // accumulator groups 2h and 2h + 1 as 16 contiguous bytes at 1024 h + 16 l (one coalesced
      // 1 KiB store per h; the dQ kernel rebuilds the quad layout below in LDS).  Streaming
      // stores (read once, by the dQ kernel): written past the last-level cache while this kernel
      // computes, rather than evicted dirty during the dQ kernel's reads.
      char* wsb = reinterpret_cast<char*>(
          p.ds_ws + (((int64_t)bh * p.n_kv_tiles + j) * n_q_tiles + i_t) * (BC * BR));
#pragma unroll
      for (int h = 0; h < 2; ++h)
        __builtin_nontemporal_store(
            u32x4{sb_prev[4 * h], sb_prev[4 * h + 1], sb_prev[4 * h + 2], sb_prev[4 * h + 3]},
            reinterpret_cast<u32x4*>(wsb + w * 2048 + h * 1024 + lane * 16));
    };

    // Additive bias: the lane's 16 bias elements of a q tile (accumulator rows, its key) as raw
    // 32-bit words (an fp32 value or a zero-extended 16-bit one), loaded one q tile ahead and not
    // touched until that tile's replay, so the loads complete under the previous tile's work.
    // dBias: the previous tile's masked fp32 dS, stored (or, for a batch-1 bias summed over the
    // batch, added with fp32 atomics) after the next tile's loads are issued.
    constexpr int NBV = C::BIAS && !C::BIAS_LDS ? 16 : 1;  // register-prefetched bias words
    constexpr int NBL = C::BIAS ? 16 : 1;                     // the replay's bias * log2(e)
    uint32_t bcur[NBV], bnext[NBV];
    float dsf[C::BIAS == 2 ? 16 : 1];
    float pf[C::QAT ? 16 : 1];
    const int64_t bias_bh = (int64_t)b * p.bias_bstride + (int64_t)h * p.Sq * p.Skv;
    const int bias_key = min(key_lane, p.Skv - 1);
    auto load_bias = [&](int i_t, uint32_t (&dst)[NBV]) {
      if constexpr (C::BIAS && !C::BIAS_LDS) {
        int64_t x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r)
          x[r] = bias_bh + (int64_t)min(i_t * BR + acc_row<32>(r, g), p.Sq - 1) * p.Skv + bias_key;
        if (p.bias_f32) {
#pragma unroll
          for (int r = 0; r < 16; ++r) dst[r] = reinterpret_cast<const uint32_t*>(p.bias)[x[r]];
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) dst[r] = reinterpret_cast<const bf16_t*>(p.bias)[x[r]];
        }
      }
    };
    // the bias of the raw words (or of the LDS-staged tile T), times log2(e), for the replay's
    // exponent
    auto bias_log2 = [&](const uint32_t (&raw)[NBV], const char* T, float (&dst)[NBL]) {
      if constexpr (C::BIAS_LDS) {
        const char* row0 = T + C::T_BIAS + (w * KPW + lc) * 2;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          dst[r] = Elem<C::F16>::lo(*reinterpret_cast<const uint16_t*>(row0 + acc_row<32>(r, g) * (BC * 2))) *
                   kLog2e;
      } else if constexpr (C::BIAS) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          dst[r] = (p.bias_f32 ? __uint_as_float(raw[r]) : Elem<C::F16>::lo(raw[r])) * kLog2e;
      }
    };
    auto store_dbias = [&](int i_t) {
      if constexpr (C::BIAS == 2) {
        const int row0 = i_t * BR;
        if (p.dbias_io) {
          // an io-type output whose elements are each written once: rounded here, once
          bf16_t* base = reinterpret_cast<bf16_t*>(p.dbias) + bias_bh + key_lane;
          if (row0 + BR <= p.Sq && k0 + BC <= p.Skv) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
              base[(int64_t)(row0 + acc_row<32>(r, g)) * p.Skv] = Elem<C::F16>::one(dsf[r]);
          } else if (key_lane < p.Skv) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int row = row0 + acc_row<32>(r, g);
              if (row < p.Sq) base[(int64_t)row * p.Skv] = Elem<C::F16>::one(dsf[r]);
            }
          }
          return;
        }
        float* base = reinterpret_cast<float*>(p.dbias) + bias_bh + key_lane;
        if (row0 + BR <= p.Sq && k0 + BC <= p.Skv && !p.dbias_atomic) {
#pragma unroll
          for (int r = 0; r < 16; ++r) base[(int64_t)(row0 + acc_row<32>(r, g)) * p.Skv] = dsf[r];
        } else if (key_lane < p.Skv) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = row0 + acc_row<32>(r, g);
            if (row < p.Sq) {
              if (p.dbias_atomic)
                __hip_atomic_fetch_add(base + (int64_t)row * p.Skv, dsf[r], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
              else
                base[(int64_t)row * p.Skv] = dsf[r];
            }
          }
        }
      }
    };
    load_bias(i_hi, bcur);

    // relay: the LDS copy of a running sum, and the staging of this wave's parts of it (the
    // 1 KiB chunks its GEMM4 adds to: 32 x 32 d tiles dt = w, w + NW, ..., or the 16 x 16 blocks
    // of gemm4_16), after waiting for this key tile's turn
    const char* rs = smem + C::OFF_RS;
    auto relay_stage = [&](int i_t) {
      if constexpr (C::MODE == DQ_RELAY) {
        const int rk = relay_rank(i_t);
        const bool has_part = C::G4_16 ? w < C::G4_BLOCKS : w < C::N_DQT;
        if (rk > 0 && has_part) {
          relay_wait(relay_turn(i_t), rk, p.relay_ctl, lane);
          const rsrc_t src = buf_rsrc(dq_dst(i_t), BR * DQK * 4);
          char* dstl = smem + C::OFF_RS;
          if constexpr (C::G4_16) {
#pragma unroll
            for (int m = 0; m < C::NB4; ++m) {
              const int off = ((w & 1) * (DQK / 16) + ((w + C::NW * m) >> 1)) * 1024;
              dma16_dev(src, off + lane * 16, dstl + off);
            }
          } else {
            for (int dt = w; dt < C::N_DQT; dt += C::NW)
#pragma unroll
              for (int x = 0; x < 4; ++x) {
                const int off = dt * 4096 + x * 1024;
                dma16_dev(src, off + lane * 16, dstl + off);
              }
          }
        }
      }
    };

    if constexpr (C::PP) {
      // ---- staggered wave groups ----------------------------------------------------------------
      // Waves w and w + 4 share a SIMD.  Between two barriers, group A (waves 0-3) runs q tile i
      // whole: GEMM1/GEMM2, the replay, GEMM3/GEMM5, then GEMM4 of tile i + 1; group B (waves 4-7)
      // runs GEMM3/GEMM5 of tile i + 1 (its P / dS kept in registers across the barrier), then
      // GEMM1/GEMM2 and the replay of tile i.  Each wave's replay then falls where the other wave
      // of its SIMD issues MFMAs (A's after its GEMM1/GEMM2, B's beside A's GEMM3/GEMM5/GEMM4)
      // instead of both replays leaving the matrix core idle at once.  Tiles i + 1, i and i - 1
      // are live together (three q-tile buffers); group B issues the tile loads and is the only
      // group that waits for them, so group A never waits on its atomics / stores.  GEMM4 of tile
      // i + 1 reads a dS staging buffer whose both halves were complete at the last barrier.
      const bool grpB = w >= C::NW / 2;  // wave-uniform
      // q tile i by group B: fragments wb, wb + 4, ... of Q and of dO (the gather_frags layout),
      // with the lane's row in the tile and its column offsets fixed for the whole loop (the four
      // fragments of a wave share the fragment parity, hence the swizzled row)
      constexpr int GB = C::NW / 2;
      constexpr int NFQ = (C::N_KQ + GB - 1) / GB, NFO = (C::N_KV + GB - 1) / GB;
      const int wb = w - GB;
      const int ln = (lane & 48) | ((lane & 15) ^ (4 * kswz(lane >> 4, wb)));
      const int row_l = ln & 31;
      auto load_tile_b = [&](int i) {
        char* t = tile(i);
        const int row = min(i * BR + row_l, p.Sq - 1);
        const uint32_t oq = (uint32_t)row * (uint32_t)p.sq.s, oo = (uint32_t)row * (uint32_t)p.sdo.s;
#pragma unroll
        for (int r = 0; r < NFQ; ++r) {
          const int f = wb + GB * r;
          const int col = 16 * f + 8 * (ln >> 5);  // one 32-row tile: fragment f is column block f
          if (f < C::N_KQ)
            dma16(rQ, (!C::PAD || col < dqk_act) ? (oq + col) * 2 : kOutOfRange, t + C::T_QA + f * 1024);
        }
#pragma unroll
        for (int r = 0; r < NFO; ++r) {
          const int f = wb + GB * r;
          const int col = 16 * f + 8 * (ln >> 5);
          if (f < C::N_KV)
            dma16(rdO, (!C::PAD || col < dv_act) ? (oo + col) * 2 : kOutOfRange, t + C::T_OA + f * 1024);
        }
        if (wb == 0) dma4(rStat, (uint32_t)(i * BR * 2 + lane) * 4, t + C::T_ST);
      };
      auto store_ds_regs = [&](const uint32_t (&s)[8], int i_t) {  // as store_ds
        char* wsb = reinterpret_cast<char*>(
            p.ds_ws + (((int64_t)bh * p.n_kv_tiles + j) * n_q_tiles + i_t) * (BC * BR));
#pragma unroll
        for (int h = 0; h < 2; ++h)
          __builtin_nontemporal_store(u32x4{s[4 * h], s[4 * h + 1], s[4 * h + 2], s[4 * h + 3]},
                                      reinterpret_cast<u32x4*>(wsb + w * 2048 + h * 1024 + lane * 16));
      };
      // GEMM1 / GEMM2 and the replay of q tile i for the wave's 32 keys: P / dS packed into pb /
      // sb, invisible pairs cleared on edge tiles, dS staged in LDS for GEMM4
      auto m1s = [&](int i, uint32_t (&pb)[8], uint32_t (&sb)[8]) __attribute__((always_inline)) {
        const int q0 = i * BR;
        const char* T = tile(i);
        const float* sStat = reinterpret_cast<const float*>(T + C::T_ST);
        acc_t S = acc_t{}, dP = acc_t{};
#pragma unroll
        for (int t = 0; t < (C::N_KQ > C::N_KV ? C::N_KQ : C::N_KV); ++t) {
          if (t < C::N_KQ)
            S = M::mma(lds_read_b128(T + C::T_QA, t * 1024 + kofs[t & 1]),
                       lds_read_b128(sK, (w * C::N_KQ + t) * 1024 + kofs[t & 1]), S);
          if (t < C::N_KV)
            dP = M::mma(lds_read_b128(T + C::T_OA, t * 1024 + kofs[t & 1]), vreg[0][t], dP);
        }
        schedule_reads_ahead<2 * C::N_KQ + C::N_KV, C::N_KQ + C::N_KV, C::AHEAD>();
        softmax_ds<C::F16, 0>(S, dP, sStat, g, p.scale_log2, pb, sb);
        softmax_ds<C::F16, 2>(S, dP, sStat, g, p.scale_log2, pb, sb);
        if (tile_needs_mask(mg, q0, BR, k0, BC)) {
          const uint32_t vis_m = visible_rows(KeyRows(mg, q0 + g * 4, key_lane));
          mask_pairs<0>(vis_m, pb, sb);
          mask_pairs<2>(vis_m, pb, sb);
        }
        if constexpr (C::G4) {
#pragma unroll
          for (int x = 0; x < 4; ++x)
            *reinterpret_cast<u32x2*>(sST(i) + w * 2048 +
                                      (C::G4_16 ? ds_store_off16(lane, x) : ds_store_off(lane, x))) =
                u32x2{sb[2 * x], sb[2 * x + 1]};
        }
      };
      // GEMM3 (dV^T += dO^T P) and GEMM5 (dK^T += Q^T dS) of q tile i
      auto m2 = [&](int i, const uint32_t (&pb)[8], const uint32_t (&sb)[8]) __attribute__((always_inline)) {
        const char* T = tile(i);
        auto step = [&](auto tb_tag) __attribute__((always_inline)) {
          constexpr int tb = decltype(tb_tag)::value;
#pragma unroll
          for (int dt = 0; dt < C::N_DVT; ++dt)
            accV[dt][0] = M::mma(tra.read(T + C::T_OA, dt, tb),
                                 __builtin_bit_cast(bf16x8, u32x4{pb[4 * tb], pb[4 * tb + 1],
                                                                  pb[4 * tb + 2], pb[4 * tb + 3]}),
                                 accV[dt][0]);
#pragma unroll
          for (int dt = 0; dt < C::N_DQT; ++dt)
            accK[dt][0] = M::mma(tra.read(T + C::T_QA, dt, tb),
                                 __builtin_bit_cast(bf16x8, u32x4{sb[4 * tb], sb[4 * tb + 1],
                                                                  sb[4 * tb + 2], sb[4 * tb + 3]}),
                                 accK[dt][0]);
        };
        __builtin_amdgcn_s_setprio(2);
        step(IntTag<0>{});
        step(IntTag<1>{});
        schedule_reads_ahead<4 * (C::N_DVT + C::N_DQT), 2 * (C::N_DVT + C::N_DQT), C::AHEAD>();
        __builtin_amdgcn_s_setprio(0);
      };
      auto g4 = [&](int i) __attribute__((always_inline)) {
        if constexpr (C::G4_16)
          gemm4_16<C>(sST(i), sK, dq_dst(i), i * BR, mg.Lq, w, lane);
        else
          gemm4<C>(sST(i), sK, dq_dst(i), i * BR, mg.Lq, w, lane);
      };

      wait_vmem();  // tile i_hi, K and V
      lds_barrier();
      // one loop per group (each keeps only its own values live); both pass the same barriers
      if (grpB) {
        uint32_t pb[8], sb[8];  // P / dS of the tile whose GEMM3/GEMM5 comes next
        for (int i = i_hi; i >= i_lo; --i) {
          if (i > i_lo) load_tile_b(i - 1);  // into tile i + 2's buffer (done with at the barrier)
          if (i < i_hi) {
            if constexpr (C::DS_OUT) store_ds_regs(sb, i + 1);
            if constexpr (C::G4_B) g4(i + 1);
            m2(i + 1, pb, sb);
          }
          m1s(i, pb, sb);
          wait_vmem();    // tile i - 1 (and this group's dS stores / GEMM4 emission)
          lds_barrier();  // tile i - 1 landed; dS of tile i complete in LDS
        }
        if constexpr (C::DS_OUT) store_ds_regs(sb, i_lo);
        m2(i_lo, pb, sb);
        if constexpr (C::G4_B) g4(i_lo);
      } else {
        for (int i = i_hi; i >= i_lo; --i) {
          uint32_t pb[8], sb[8];
          m1s(i, pb, sb);
          if constexpr (C::DS_OUT) store_ds_regs(sb, i);
          m2(i, pb, sb);
          if constexpr (C::G4) {
            if (i < i_hi) g4(i + 1);
          }
          lds_barrier();
        }
        if constexpr (C::G4) g4(i_lo);
      }
    } else {
      for (int i = i_hi; i >= i_lo; --i) {
        const int q0 = i * BR;
        const char* T = tile(i);
        const float* sStat = reinterpret_cast<const float*>(T + C::T_ST);
        wait_vmem();      // this wave's loads of tile i (and its older atomics / stores) are done
        lds_barrier();    // tile i landed everywhere; every wave is done with the previous tile
        if constexpr (C::MODE == DQ_RELAY) {
          // every wave's sums of q tile i + 2 (stored in the previous iteration) are complete
          if (tid == 0 && i + 2 <= i_hi) relay_publish(relay_turn(i + 2), relay_rank(i + 2) + 1);
        }
        if (C::NBUF == 2 && i > i_lo) load_tile(i - 1);
        if constexpr (C::DS_OUT) {
          if (i < i_hi) store_ds(i + 1);
        }
        if constexpr (C::BIAS && !C::BIAS_LDS) {
          if (i < i_hi) store_dbias(i + 1);
          if (i > i_lo) load_bias(i - 1, bnext);
        }

        if constexpr (C::G4) {
          // GEMM4 of the previous q tile (dS in sST), deferred so its atomics / partial stores
          // overlap this tile
          if (i < i_hi) {
            const bool add = C::MODE == DQ_RELAY && relay_rank(i + 1) > 0;
            if constexpr (C::G4_16)
              gemm4_16<C>(sST(i + 1), sK, dq_dst(i + 1), q0 + BR, mg.Lq, w, lane, rs, add);
            else
              gemm4<C>(sST(i + 1), sK, dq_dst(i + 1), q0 + BR, mg.Lq, w, lane, rs, add);
            // single buffer: every wave is done reading it before this tile's dS overwrites it
            // (the atomics / stores keep draining)
            if constexpr (C::NSST == 1) lds_barrier();
          }
          // relay: once the key tile before this one has added into q tile i's sum, stage that sum
          // (this wave's parts of it) for GEMM4 of tile i in the next iteration
          if constexpr (C::MODE == DQ_RELAY) relay_stage(i);
        }

        // ---- the wave's 32 keys: GEMM1, GEMM2, softmax replay, dS, GEMM3, GEMM5 --------------------
        const bool edge = tile_needs_mask(mg, q0, BR, k0, BC);
        acc_t S = acc_t{}, dP = acc_t{};
        // GEMM1 and GEMM2 are independent chains: alternate them so neither waits on the other's
        // accumulator, and keep the operand reads a few MFMAs ahead of their use
#pragma unroll
        for (int t = 0; t < (C::N_KQ > C::N_KV ? C::N_KQ : C::N_KV); ++t) {
          if (t < C::N_KQ) {
            const bf16x8 a = lds_read_b128(T + C::T_QA, t * 1024 + kofs[t & 1]);
            if constexpr (C::KREG) {
              S = M::mma(a, kreg[0][t], S);
            } else {
              S = M::mma(a, lds_read_b128(sK, (w * C::N_KQ + t) * 1024 + kofs[t & 1]), S);
            }
          }
          if (t < C::N_KV)
            dP = M::mma(lds_read_b128(T + C::T_OA, t * 1024 + kofs[t & 1]), vreg[0][t], dP);
        }
        schedule_reads_ahead<(C::KREG ? 1 : 2) * C::N_KQ + C::N_KV, C::N_KQ + C::N_KV, C::AHEAD>();

        // GEMM3 (dV^T += dO^T P) and GEMM5 (dK^T += Q^T dS), contraction step tb over q rows
        // 16 tb .. 16 tb + 15, whose P / dS come from accumulator groups 2 tb and 2 tb + 1
        // (the step index is a type so the P / dS register indices are constants)
        uint32_t pb[8], sb[8];
        auto gemm35_step = [&](auto tb_tag) __attribute__((always_inline)) {
          constexpr int tb = decltype(tb_tag)::value;
#pragma unroll
          for (int dt = 0; dt < C::N_DVT; ++dt)
            accV[dt][0] = M::mma(tra.read(T + C::T_OA, dt, tb),
                                 __builtin_bit_cast(bf16x8, u32x4{pb[4 * tb], pb[4 * tb + 1],
                                                                  pb[4 * tb + 2], pb[4 * tb + 3]}),
                                 accV[dt][0]);
#pragma unroll
          for (int dt = 0; dt < C::N_DQT; ++dt)
            accK[dt][0] = M::mma(tra.read(T + C::T_QA, dt, tb),
                                 __builtin_bit_cast(bf16x8, u32x4{sb[4 * tb], sb[4 * tb + 1],
                                                                  sb[4 * tb + 2], sb[4 * tb + 3]}),
                                 accK[dt][0]);
        };
        // Softmax replay of all 32 rows, unmasked and branch-free; edge tiles then clear their
        // invisible pairs in the packed words (keeping the masking out of the block the MFMA
        // accumulators flow through avoids register copies at the join).
        float bl[NBL];
        bias_log2(bcur, T, bl);
        softmax_ds<C::F16, 0, C::BIAS, C::QAT>(S, dP, sStat, g, p.scale_log2, pb, sb, bl, dsf, pf);
        softmax_ds<C::F16, 2, C::BIAS, C::QAT>(S, dP, sStat, g, p.scale_log2, pb, sb, bl, dsf, pf);
        if (edge) {
          const uint32_t vis_m = visible_rows(KeyRows(mg, q0 + g * 4, key_lane));
          mask_pairs<0>(vis_m, pb, sb);
          mask_pairs<2>(vis_m, pb, sb);
          if constexpr (C::BIAS == 2) {
            // register 4x + e holds row offset 8x + e from the lane's first row
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (!((vis_m >> (8 * (r / 4) + (r % 4))) & 1u)) dsf[r] = 0.f;
          }
          if constexpr (C::QAT) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (!((vis_m >> (8 * (r / 4) + (r % 4))) & 1u)) pf[r] = 0.f;
          }
        }
        // 8 waves: dBias of this tile leaves at once (the 4-wave layout defers it past the next
        // tile's loads; here the registers to hold it are not there)
        if constexpr (C::BIAS == 2 && C::BIAS_LDS) store_dbias(i);
        // QAT: GEMM3's P operand is the fake-quantised masked P (groups of 16 keys of a row)
        if constexpr (C::QAT) nvfp4_p_pack_lds(pf, pb, smem + C::OFF_QS + w * C::QS_WAVE, lane);
        if constexpr (C::BIAS) {
#pragma unroll
          for (int r = 0; r < NBV; ++r) bcur[r] = bnext[r];
        }
        if constexpr (C::DS_OUT) {
#pragma unroll
          for (int x = 0; x < 8; ++x) sb_prev[x] = sb[x];
        } else {
          // dS of the wave's 32 keys to LDS as 2 KiB of quads (see ds_store_off / ds_store_off16)
#pragma unroll
          for (int x = 0; x < 4; ++x)
            *reinterpret_cast<u32x2*>(sST(i) + w * 2048 +
                                      (C::G4_16 ? ds_store_off16(lane, x) : ds_store_off(lane, x))) =
                u32x2{sb[2 * x], sb[2 * x + 1]};
        }
        // (raised wave priority: this MFMA-only phase issues ahead of the other wave's softmax)
        __builtin_amdgcn_s_setprio(2);
        gemm35_step(IntTag<0>{});
        gemm35_step(IntTag<1>{});
        schedule_reads_ahead<4 * (C::N_DVT + C::N_DQT), 2 * (C::N_DVT + C::N_DQT), C::AHEAD>();
        __builtin_amdgcn_s_setprio(0);
        if constexpr (C::NBUF == 1) {
          lds_barrier();  // every wave is done with the single q-tile buffer
          if (i > i_lo) load_tile(i - 1);
        }
      }
      if constexpr (C::DS_OUT) store_ds(i_lo);
      if constexpr (!C::BIAS_LDS) store_dbias(i_lo);
      if constexpr (C::G4) {
        if constexpr (C::MODE == DQ_RELAY) wait_vmem();  // the staged sum of q tile i_lo
        lds_barrier();  // the last tile's dS is complete
        const bool add = C::MODE == DQ_RELAY && relay_rank(i_lo) > 0;
        if constexpr (C::G4_16)
          gemm4_16<C>(sST(i_lo), sK, dq_dst(i_lo), i_lo * BR, mg.Lq, w, lane, rs, add);
        else
          gemm4<C>(sST(i_lo), sK, dq_dst(i_lo), i_lo * BR, mg.Lq, w, lane, rs, add);
      }
      if constexpr (C::MODE == DQ_RELAY) {
        wait_vmem();  // this wave's sums of q tiles i_lo + 1 and i_lo are stored
        lds_barrier();
        if (tid == 0) {
          if (i_lo + 1 <= i_hi) relay_publish(relay_turn(i_lo + 1), relay_rank(i_lo + 1) + 1);
          relay_publish(relay_turn(i_lo), relay_rank(i_lo) + 1);
        }
      }
    }  // staggered groups / one group
  }
  if constexpr (C::MODE == DQ_RELAY) {
    if (tid == 0)
      __hip_atomic_fetch_add(p.relay_ctl + 8, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- epilogue: dK (scaled) and dV, written once; keys past the sequence are zero -------------
  // A lane holds one key's column of accumulators (4 consecutive head-dim values per group), so
  // a direct store would scatter every instruction over 32 key rows.  Each wave instead stages its
  // 32-key tile in LDS as rows (8-byte writes) and reads it back row-major, so each lane stores 16
  // contiguous bytes and each store instruction covers whole rows.  dK first, then dV in the same
  // rows (this wave's own LDS: its accesses stay in order).
  static_assert(NKT == 1, "one 32-key tile per wave");
  lds_barrier();  // every wave is done with the loop's LDS (no LDS-DMA is in flight after it)
  {
    char* ep = smem + w * 32 * C::EPI_PITCH;
    const int64_t oslot = p.partials ? (int64_t)bh * p.n_split + part : (int64_t)b * p.Hkv + kvh;
    const int key0 = key_lane - lc;  // the wave's first key
    auto out_tile = [&](const acc_t (*acc)[NKT], auto n_dt_tag, float scale, bf16_t* out_base,
                        const Strides& st, int d_kernel, int d_act) {
      constexpr int NDT = decltype(n_dt_tag)::value;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r0 = 0; r0 < 16; r0 += 4)
          *reinterpret_cast<u32x2*>(ep + lc * C::EPI_PITCH + (dt * 32 + acc_row<32>(r0, g)) * 2) =
              u32x2{Elem<C::F16>::pack2(acc[dt][0][r0] * scale, acc[dt][0][r0 + 1] * scale),
                    Elem<C::F16>::pack2(acc[dt][0][r0 + 2] * scale, acc[dt][0][r0 + 3] * scale)};
      constexpr int CPR = NDT * 32 * 2 / 16;  // 16-byte pieces per key row
      constexpr int NX = 32 * CPR / 64;
      u32x4 v[NX];
#pragma unroll
      for (int x = 0; x < NX; ++x) {
        const int k = x * 64 + lane;
        v[x] = *reinterpret_cast<const u32x4*>(ep + (k / CPR) * C::EPI_PITCH + (k % CPR) * 16);
      }
#pragma unroll
      for (int x = 0; x < NX; ++x) {
        const int k = x * 64 + lane, row = k / CPR, ch = k % CPR;
        const int key = key0 + row;
        if (key >= p.Skv) continue;
        if (C::PAD && !p.partials && ch * 8 >= d_act) continue;  // past the tensor's head dim
        // partials: contiguous per (query head, part); final dK/dV: the caller's layout
        bf16_t* dst = p.partials ? out_base + (oslot * p.Skv + key) * d_kernel
                                 : out_base + b * st.b + kvh * st.h + key * st.s;
        *reinterpret_cast<u32x4*>(dst + ch * 8) = v[x];
      }
    };
    out_tile(accK, IntTag<C::N_DQT>{}, p.scale, p.dk_out, p.sdk, DQK, dqk_act);
    out_tile(accV, IntTag<C::N_DVT>{}, 1.0f, p.dv_out, p.sdv, DV, dv_act);
  }
}

}  // namespace sdpa
