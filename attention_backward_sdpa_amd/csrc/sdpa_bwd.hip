// Host side of the attention-backward library: argument validation, workspace carving, route
// choice and kernel launches on the caller's stream.  Implements include/sdpa_bwd.h.
//
// Chain ("SDPA Backward (SM120)", section "The kernel chain"):
//   preprocess -> main -> [GQA reduce] -> dQ convert           (fp32-atomic dQ route)
//   preprocess -> main(dS out) -> [GQA reduce] -> dq2k         (deterministic, dS panels)
//   preprocess -> main(dQ partials) -> [GQA reduce] -> dq_reduce  (deterministic, dQ partials)
// The pages overlap consecutive launches with programmatic dependent launch; CDNA has no such
// feature, so the launches are simply ordered on the stream.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/sdpa_bwd.h"
#include "dq2k.h"
#include "dq2k_half.h"
#include "dq2k_split.h"
#include "dq_reduce.h"
#include "main_launch.h"
#include "small_kernels.h"

using namespace sdpa;

namespace {

constexpr int64_t kAlign = 256;
inline int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Tile geometry per supported (Dqk, Dv): waves per workgroup NW, keys per wave KPW = 32, key
// tile BC = NW * KPW, q tile BR = 32.  Kernel head dims up to 192 run 8 waves (two per SIMD, 256
// registers each, 256-key tiles); head dim 256 runs 4 waves with 512 registers for the bigger
// dK/dV accumulators (128-key tiles).
struct Geometry {
  int nw, kpw, bc, br;
};

// The kernel head dims that serve a call's (Dqk, Dv) ("Support surface": head dims that are
// multiples of 8 up to 256 compute on the next supported size, reading zeros past the actual
// extent): the smallest supported pair covering both.  Dv <= Dqk.
bool kernel_dims(int Dqk, int Dv, int* kq, int* kv) {
  if (Dqk < 8 || Dv < 8 || Dqk > 256 || Dv > Dqk || (Dqk & 7) || (Dv & 7)) return false;
  static const int pairs[5][2] = {{32, 32}, {64, 64}, {128, 128}, {192, 128}, {256, 256}};
  for (const auto& pr : pairs)
    if (Dqk <= pr[0] && Dv <= pr[1]) {
      *kq = pr[0];
      *kv = pr[1];
      return true;
    }
  return false;
}

// `narrow`: the 4-wave layout (512 registers per wave) at every head dim, for the extras that
// need it (see plan): a bias held in registers a q tile ahead, the relay's bias and QAT kernels.
bool geometry_for(int Dqk, int Dv, Geometry* g, bool narrow = false) {
  if (Dqk == 32 && Dv == 32) *g = {8, 32, 256, 32};
  else if (Dqk == 64 && Dv == 64) *g = {8, 32, 256, 32};
  else if (Dqk == 128 && Dv == 128) *g = {8, 32, 256, 32};
  else if (Dqk == 192 && Dv == 128) *g = {8, 32, 256, 32};
  else if (Dqk == 256 && Dv == 256) *g = {4, 32, 128, 32};
  else return false;
  if (narrow) *g = {4, 32, 128, 32};
  return true;
}

// The additive bias of one call ("API Usage" bias_tensor): (bias_batch, Hq, Sq, Skv) contiguous.
struct BiasArgs {
  const void* bias = nullptr;
  float* dbias = nullptr;
  int dtype = SDPA_BWD_BF16;  // SDPA_BWD_BF16 / SDPA_BWD_FP16 (the io type) or SDPA_BWD_FP32
  int batch = 1;              // 1 or B
  bool dbias_io = false;      // dbias holds io-type elements (see run(): written directly, or
                              // accumulated in fp32 and converted by dbias_cvt)
};

// Number of parts the q-tile range of every key tile is split into (each part a workgroup of its
// own, writing dK/dV partials that the reduction sums in a fixed order).  A grid of fewer than
// two workgroups per CU leaves CUs idle, and under a causal mask the key tiles near the start see
// many more q tiles than the rest; splitting the ranges evens the per-workgroup work.  Parts keep
// at least 8 q tiles.
constexpr int kNumCUs = 256;

int q_split(int B, int Hq, int Sq, int Skv, const Geometry& g) {
  const int64_t grid = (int64_t)((Skv + g.bc - 1) / g.bc) * B * Hq;
  const int n_q_tiles = (Sq + g.br - 1) / g.br;
  int split = 1;
  while (split < 4 && grid * split < 2 * kNumCUs && n_q_tiles / (2 * split) >= 8) split *= 2;
  return split;
}

// dQ routes.  The `deterministic` argument: 0 fp32 atomics, 1 deterministic (the fp32 dQ partials
// where they are a smaller workspace stream per (KV tile, q row) than the BC bf16 dS values, else
// the dS panels: at equal bytes, head dim 128, the dS-panel chain measured faster on MI355X; and
// the ordered relay when that route's buffer, quadratic in the sequence lengths, would exceed
// kQuadraticCap), 2 dS panels + dq2k, 3 fp32 dQ partials + dq_reduce, 4 the ordered relay (one
// running fp32 sum per q tile, passed from key tile to key tile in ascending order).
enum Route { R_ATOMIC = 0, R_DS = 1, R_DQP = 2, R_RELAY = 3, R_INVALID = -1 };

// "Determinism": shapes whose dS buffer does not fit fall back to the relay, whose workspace is
// linear in the sequence lengths.  The bound is a fixed 4 GiB (under 1.5 % of an MI355X's HBM), so
// the choice depends on the call's arguments only, never on the device or on free memory.
constexpr int64_t kQuadraticCap = int64_t{1} << 32;

// Bytes of the route's per-(KV tile, q tile) buffer (0 for the atomic and relay routes).
int64_t quadratic_bytes(Route r, int B, int Hq, int Sq, int Skv, int Dqk, const Geometry& g) {
  const int64_t sq_pad = align_up(Sq, g.br), skv_pad = align_up(Skv, g.bc);
  if (r == R_DS) return (int64_t)B * Hq * skv_pad * sq_pad * 2;
  if (r == R_DQP) return (int64_t)B * Hq * (skv_pad / g.bc) * sq_pad * Dqk * 4;
  return 0;
}

Route route_for(int deterministic, int Dqk, const Geometry& g, int B, int Hq, int Sq, int Skv) {
  switch (deterministic) {
    case 0: return R_ATOMIC;
    case 1: {
      const Route r = (int64_t)Dqk * 4 < (int64_t)g.bc * 2 ? R_DQP : R_DS;
      return quadratic_bytes(r, B, Hq, Sq, Skv, Dqk, g) > kQuadraticCap ? R_RELAY : r;
    }
    case 2: return R_DS;
    case 3: return R_DQP;
    case 4: return R_RELAY;
    default: return R_INVALID;
  }
}

// A bias of the io type whose rows split into 16-byte chunks runs the 8-wave layout (256-key
// tiles, the bias tile staged in LDS with its q tile) at kernel head dims up to 128; any other bias,
// and every bias on the relay route (whose 8-wave bias kernel does not fit in 256 registers), the
// 4-wave layout.  The chunks need Skv a multiple of 8 and a 16-byte-aligned tensor, and one head's
// bias is addressed through 32-bit buffer offsets.
bool bias_in_lds(const void* bias, int bias_dtype, int io_dtype, int kq, int Sq, int Skv) {
  return bias != nullptr && bias_dtype == io_dtype && Skv % 8 == 0 &&
         ((uintptr_t)bias & 15) == 0 && (int64_t)Sq * Skv * 2 < (int64_t{1} << 31) && kq <= 128;
}

// Layout classes of a call: no per-element extra; an extra that rides on the 8-wave layout except
// on the relay route (a bias staged in LDS, the NVFP4 QAT variant: their 8-wave relay kernels do
// not fit in 256 registers); an extra that needs the 4-wave layout (any other bias).
enum Extra { X_NONE = 0, X_WIDE = 1, X_NARROW = 2 };

// The main kernel's geometry and the dQ route of a call with kernel head dims (kq, kv).
bool plan(int kq, int kv, int deterministic, int B, int Hq, int Sq, int Skv, Extra x,
          Geometry* geo, Route* route) {
  if (!geometry_for(kq, kv, geo, x == X_NARROW)) return false;
  *route = route_for(deterministic, kq, *geo, B, Hq, Sq, Skv);
  if (x == X_WIDE && *route == R_RELAY) {
    geometry_for(kq, kv, geo, true);
    *route = route_for(deterministic, kq, *geo, B, Hq, Sq, Skv);
  }
  return true;
}

Extra bias_extra(const void* bias, int bias_dtype, int io_dtype, int kq, int Sq, int Skv) {
  if (bias == nullptr) return X_NONE;
  return bias_in_lds(bias, bias_dtype, io_dtype, kq, Sq, Skv) ? X_WIDE : X_NARROW;
}

// Item queues of the relay: one per XCD of the current device (1..8), queried once per device.
int relay_queues() {
  static std::atomic<int> cached[64];  // 0 until queried
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 1;
  if (dev < 64) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 1;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || n < 1) n = 1;
  n = n > 8 ? 8 : n;
  if (dev < 64) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

struct Carve {
  int64_t stats = 0, dq_accum = -1, ds = -1, dqp = -1, dk_ws = -1, dv_ws = -1, total = 0;
  int64_t dbias_f32 = -1;
  int64_t relay_turn = -1, relay_ctl = -1;
  int64_t sq_pad = 0, skv_pad = 0;
};

// dbias_elems: elements of an fp32 dBias accumulator (an io-type dBias summed over the batch),
// else 0.
Carve carve(int B, int Hq, int Hkv, int Sq, int Skv, int Dqk, int Dv, Route route,
            const Geometry& g, int64_t dbias_elems = 0) {
  Carve c;
  int64_t off = 0;
  c.sq_pad = align_up(Sq, g.br);
  c.skv_pad = align_up(Skv, g.bc);
  c.stats = off;  // [LSE * log2e, delta] per padded q row
  off = align_up(off + (int64_t)B * Hq * c.sq_pad * 2 * 4, kAlign);
  if (route == R_ATOMIC) {
    c.dq_accum = off;
    off = align_up(off + (int64_t)B * Hq * Sq * Dqk * 4, kAlign);
  } else if (route == R_DS) {
    c.ds = off;
    off = align_up(off + (int64_t)B * Hq * c.skv_pad * c.sq_pad * 2, kAlign);
  } else if (route == R_RELAY) {  // one 32 x Dqk fp32 running sum per (b, h, q tile)
    c.dqp = off;
    off = align_up(off + (int64_t)B * Hq * c.sq_pad * Dqk * 4, kAlign);
    c.relay_turn = off;  // one turn counter per (b, h, q tile)
    off = align_up(off + (int64_t)B * Hq * (c.sq_pad / g.br) * 4, kAlign);
    c.relay_ctl = off;   // 16 control words
    off = align_up(off + 16 * 4, kAlign);
  } else {  // one 32 x Dqk fp32 block per (b, h, KV tile, q tile)
    c.dqp = off;
    off = align_up(off + (int64_t)B * Hq * (c.skv_pad / g.bc) * c.sq_pad * Dqk * 4, kAlign);
  }
  const int split = q_split(B, Hq, Sq, Skv, g);
  if (Hq != Hkv || split > 1) {  // per-(query head, part) dK/dV partials
    c.dk_ws = off;
    off = align_up(off + (int64_t)B * Hq * split * Skv * Dqk * 2, kAlign);
    c.dv_ws = off;
    off = align_up(off + (int64_t)B * Hq * split * Skv * Dv * 2, kAlign);
  }
  if (dbias_elems > 0) {
    c.dbias_f32 = off;
    off = align_up(off + dbias_elems * 4, kAlign);
  }
  c.total = off;
  return c;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Element strides of the eight (B, H, S, D) tensors, head dim contiguous.
enum { T_Q, T_K, T_V, T_O, T_DO, T_DQ, T_DK, T_DV, N_TENSORS };
struct Layouts {
  Strides t[N_TENSORS];
};

Layouts contiguous_layouts(int Hq, int Hkv, int Sq, int Skv, int Dqk, int Dv) {
  auto bhsd = [](int H, int S, int D) {
    return Strides{(int64_t)H * S * D, (int64_t)S * D, (int64_t)D};
  };
  Layouts L;
  L.t[T_Q] = L.t[T_DQ] = bhsd(Hq, Sq, Dqk);
  L.t[T_O] = L.t[T_DO] = bhsd(Hq, Sq, Dv);
  L.t[T_K] = L.t[T_DK] = bhsd(Hkv, Skv, Dqk);
  L.t[T_V] = L.t[T_DV] = bhsd(Hkv, Skv, Dv);
  return L;
}

// Every row 16-byte aligned (with a 16-byte-aligned base), rows of one head at least a row
// apart, and one head's span addressable through 32-bit buffer offsets.
int check_layouts(const Layouts& L, int Sq, int Skv, int Dqk, int Dv) {
  const int S[N_TENSORS] = {Sq, Skv, Skv, Sq, Sq, Sq, Skv, Skv};
  const int D[N_TENSORS] = {Dqk, Dqk, Dv, Dv, Dv, Dqk, Dqk, Dv};
  for (int x = 0; x < N_TENSORS; ++x) {
    const Strides& st = L.t[x];
    if (st.b < 0 || st.h < 0 || st.s < D[x]) return SDPA_BWD_INVALID_ARG;
    if ((st.b | st.h | st.s) & 7) return SDPA_BWD_UNSUPPORTED;
    if (S[x] > 0 && ((int64_t)(S[x] - 1) * st.s + D[x]) * 2 >= ((int64_t)1 << 31))
      return SDPA_BWD_UNSUPPORTED;
  }
  return SDPA_BWD_OK;
}

int validate(const void* q, const void* k, const void* v, const void* o, const void* dO,
             const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq,
             int Skv, int Dqk, int Dv, int window_left, int window_right, Geometry* geo,
             bool narrow = false) {
  if (B < 0 || Hq < 0 || Hkv < 0 || Sq < 0 || Skv < 0) return SDPA_BWD_INVALID_ARG;
  if (Hkv == 0 || Hq == 0 || Hq % Hkv != 0) return SDPA_BWD_INVALID_ARG;
  if (window_left < -1 || window_right < 0) return SDPA_BWD_INVALID_ARG;
  int kq, kv;
  if (!kernel_dims(Dqk, Dv, &kq, &kv) || !geometry_for(kq, kv, geo, narrow))
    return SDPA_BWD_UNSUPPORTED;
  // the kernels address one head's rows (and its padded tiles) through 32-bit buffer offsets
  const int64_t s_max = (Sq > Skv ? Sq : Skv) + geo->bc;
  if (s_max * (kq > kv ? kq : kv) * 2 >= ((int64_t)1 << 31)) return SDPA_BWD_UNSUPPORTED;
  // a tensor with no elements may be NULL
  const bool has_q = (int64_t)B * Sq > 0, has_k = (int64_t)B * Skv > 0;
  if (has_q && (!q || !o || !dO || !lse || !dq)) return SDPA_BWD_INVALID_ARG;
  if (has_k && (!k || !v || !dk || !dv)) return SDPA_BWD_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dO) ||
      ((uintptr_t)lse & 3) != 0 || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return SDPA_BWD_UNSUPPORTED;
  return SDPA_BWD_OK;
}

template <class C>
hipError_t launch_dq2k(const Dq2kParams& dp, int grid, hipStream_t s) {
  const hipError_t e = lds_limit_once<C>(dq2k_kernel<C>, C::LDS_BYTES);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dq2k_kernel<C>, dim3(grid), dim3(C::NT), C::LDS_BYTES, s, dp);
  return hipGetLastError();
}

// The main kernel of the route for kernel head dim Dqk (instantiated in main_d<Dqk>.hip).
// bias: 0 none, 1 bias, 2 bias and dBias; `bc` is the key tile plan chose (it selects the layout).
hipError_t run_main(int Dqk, const MainParams& mp, Route route, bool f16, int bias, int grid,
                    int bc, hipStream_t s, bool qat = false) {
  const DqMode mode = route == R_DS    ? DQ_DS
                      : route == R_DQP ? DQ_PARTIAL
                      : route == R_RELAY ? DQ_RELAY
                                         : DQ_ATOMIC;
  if (Dqk == 32) return launch_main_dqk<32>(mp, mode, f16, bias, grid, bc, s, qat);
  if (Dqk == 64) return launch_main_dqk<64>(mp, mode, f16, bias, grid, bc, s, qat);
  if (Dqk == 128) return launch_main_dqk<128>(mp, mode, f16, bias, grid, bc, s, qat);
  if (Dqk == 192) return launch_main_dqk<192>(mp, mode, f16, bias, grid, bc, s, qat);
  return launch_main_dqk<256>(mp, mode, f16, bias, grid, bc, s, qat);
}

// the reduction reads the partial blocks in the layout of the main kernel that wrote them (the
// 8- and 4-wave layouts of a head dim write the same one)
template <int DQK, int DV, int NW>
constexpr bool partial_l16() { return MainCfg<DQK, DV, 32, NW, DQ_PARTIAL>::G4_16; }
static_assert(partial_l16<32, 32, 8>() == partial_l16<32, 32, 4>() &&
                  partial_l16<64, 64, 8>() == partial_l16<64, 64, 4>() &&
                  partial_l16<128, 128, 8>() == partial_l16<128, 128, 4>() &&
                  partial_l16<192, 128, 8>() == partial_l16<192, 128, 4>(),
              "one partial-block layout per head dim");

template <bool F16>
hipError_t launch_dq_reduce_t(const DqReduceParams& rp, int Dqk, int grid, hipStream_t s) {
  if (Dqk == 32)
    hipLaunchKernelGGL((dq_reduce_kernel<32, F16, partial_l16<32, 32, 8>()>), dim3(grid), dim3(64), 0, s, rp);
  else if (Dqk == 64)
    hipLaunchKernelGGL((dq_reduce_kernel<64, F16, partial_l16<64, 64, 8>()>), dim3(grid), dim3(128), 0, s, rp);
  else if (Dqk == 128)
    hipLaunchKernelGGL((dq_reduce_kernel<128, F16, partial_l16<128, 128, 8>()>), dim3(grid), dim3(256), 0, s, rp);
  else if (Dqk == 192)
    hipLaunchKernelGGL((dq_reduce_kernel<192, F16, partial_l16<192, 128, 8>()>), dim3(grid), dim3(384), 0, s, rp);
  else
    hipLaunchKernelGGL((dq_reduce_kernel<256, F16, partial_l16<256, 256, 4>()>), dim3(grid), dim3(512), 0, s, rp);
  return hipGetLastError();
}

template <int DQK, int BC, bool F16>
hipError_t dispatch_dq2k(const Dq2kParams& dp, int bc, hipStream_t s) {
  using C = Dq2kCfg<DQK, BC, F16>;
  if (BC != bc) return hipErrorInvalidValue;  // must read the dS blocks the main kernel wrote
  // one workgroup per group of C::QT consecutive q tiles of one (batch, query head)
  const int64_t grid = (int64_t)((dp.n_q_tiles + C::QT - 1) / C::QT) * dp.B * dp.Hq;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  return launch_dq2k<C>(dp, (int)grid, s);
}

// head dim 256: the head dim split over wave pairs (dq2k_split.h).  Measured against dq2k_kernel
// (same box, two passes): non-causal S=8192 D=256 319-320 -> 309 us; on the MLA workload's head
// dim 192 it was 1-2 % slower, which keeps dq2k_kernel there.
template <int DQK, int BC, bool F16>
hipError_t dispatch_dq2k_split(const Dq2kParams& dp, int bc, hipStream_t s) {
  using C = Dq2kSplitCfg<DQK, BC, F16>;
  if (BC != bc) return hipErrorInvalidValue;  // must read the dS blocks the main kernel wrote
  const int64_t grid = (int64_t)((dp.n_q_tiles + C::QT - 1) / C::QT) * dp.B * dp.Hq;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  const hipError_t e = lds_limit_once<C>(dq2k_split_kernel<C>, C::LDS_BYTES);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dq2k_split_kernel<C>, dim3((unsigned)grid), dim3(C::NT), C::LDS_BYTES, s, dp);
  return hipGetLastError();
}

// Head dims 64 and 128: the keys of every chunk split over wave pairs (dq2k_half.h).  Measured
// against dq2k_kernel (one q tile per wave, 8 per workgroup; same box, two passes each):
//   * 4 q tiles per workgroup (8 waves, two workgroups per CU): head dim 64 on causal GQA S=4096
//     128 -> 112-115 us; head dim 128 under a mask that makes the groups' lengths differ, where a
//     grid of 8-q-tile groups has fewer than two workgroups per CU (causal MHA B2 H16 S=2048:
//     60-62 -> 56-57 us); on the larger head-dim-128 grids slower (causal GQA S=4096 139-141 ->
//     160 us), twice the K traffic per q tile;
//   * 8 q tiles per workgroup (16 waves, one workgroup per CU; K shared as in dq2k_kernel): head
//     dim 128 otherwise, causal GQA S=4096 130-131 -> 124-126 us, non-causal MHA B1 H16 S=4096
//     (256 groups of equal length) 131 -> 105-106 us, fp16 133 -> 127-129 us.
// Head dim 192 keeps dq2k_kernel (the 16-wave layout's LDS and registers do not fit there).
bool dq2k_fine_groups(const Dq2kParams& dp) {
  const bool uneven = dp.causal || dp.window_left >= 0 || dp.seq_q_lens || dp.seq_kv_lens;
  return uneven && (int64_t)((dp.n_q_tiles + 7) / 8) * dp.B * dp.Hq < 2 * kNumCUs;
}

template <int DQK, int BC, bool F16, int QT>
hipError_t dispatch_dq2k_half(const Dq2kParams& dp, int bc, hipStream_t s) {
  using C = Dq2kHalfCfg<DQK, BC, F16, QT>;
  if (BC != bc) return hipErrorInvalidValue;  // must read the dS blocks the main kernel wrote
  const int64_t grid = (int64_t)((dp.n_q_tiles + C::QT - 1) / C::QT) * dp.B * dp.Hq;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  const hipError_t e = lds_limit_once<C>(dq2k_half_kernel<C>, C::LDS_BYTES);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dq2k_half_kernel<C>, dim3((unsigned)grid), dim3(C::NT), C::LDS_BYTES, s, dp);
  return hipGetLastError();
}

template <int BC, bool F16>
hipError_t dispatch_dq2k_half_128(const Dq2kParams& dp, int bc, hipStream_t s) {
  return dq2k_fine_groups(dp) ? dispatch_dq2k_half<128, BC, F16, 4>(dp, bc, s)
                              : dispatch_dq2k_half<128, BC, F16, 8>(dp, bc, s);
}

template <bool F16>
hipError_t run_dq2k_t(int Dqk, const Dq2kParams& dp, int bc, hipStream_t s) {
  if (bc == 256) {
    if (Dqk == 64) return dispatch_dq2k_half<64, 256, F16, 4>(dp, bc, s);
    if (Dqk == 128) return dispatch_dq2k_half_128<256, F16>(dp, bc, s);
    if (Dqk == 192) return dispatch_dq2k<192, 256, F16>(dp, bc, s);
    return hipErrorInvalidValue;
  }
  // 128-key tiles: head dim 256, and every head dim under a bias held in registers
  if (Dqk == 64) return dispatch_dq2k_half<64, 128, F16, 4>(dp, bc, s);
  if (Dqk == 128) return dispatch_dq2k_half_128<128, F16>(dp, bc, s);
  if (Dqk == 192) return dispatch_dq2k<192, 128, F16>(dp, bc, s);
  return dispatch_dq2k_split<256, 128, F16>(dp, bc, s);
}

hipError_t run_dq2k(int Dqk, bool f16, const Dq2kParams& dp, int bc, hipStream_t s) {
  return f16 ? run_dq2k_t<true>(Dqk, dp, bc, s) : run_dq2k_t<false>(Dqk, dp, bc, s);
}

template <bool F16>
hipError_t launch_convert_t(const ConvertParams& cp, int Dqk, int grid, hipStream_t s) {
  if (Dqk == 32) hipLaunchKernelGGL((dq_convert_kernel<32, F16>), dim3(grid), dim3(256), 0, s, cp);
  else if (Dqk == 64) hipLaunchKernelGGL((dq_convert_kernel<64, F16>), dim3(grid), dim3(256), 0, s, cp);
  else if (Dqk == 128) hipLaunchKernelGGL((dq_convert_kernel<128, F16>), dim3(grid), dim3(256), 0, s, cp);
  else if (Dqk == 192) hipLaunchKernelGGL((dq_convert_kernel<192, F16>), dim3(grid), dim3(256), 0, s, cp);
  else hipLaunchKernelGGL((dq_convert_kernel<256, F16>), dim3(grid), dim3(256), 0, s, cp);
  return hipGetLastError();
}

hipError_t launch_convert(const ConvertParams& cp, int Dqk, bool f16, int grid, hipStream_t s) {
  return f16 ? launch_convert_t<true>(cp, Dqk, grid, s) : launch_convert_t<false>(cp, Dqk, grid, s);
}

hipError_t launch_dq_reduce(const DqReduceParams& rp, int Dqk, bool f16, int grid, hipStream_t s) {
  return f16 ? launch_dq_reduce_t<true>(rp, Dqk, grid, s) : launch_dq_reduce_t<false>(rp, Dqk, grid, s);
}

template <bool F16>
void launch_preprocess_t(const PreParams& pp, int Dv, dim3 grid, hipStream_t s) {
  const dim3 block(256);
  if (Dv == 32) hipLaunchKernelGGL((preprocess_kernel<32, F16>), grid, block, 0, s, pp);
  else if (Dv == 64) hipLaunchKernelGGL((preprocess_kernel<64, F16>), grid, block, 0, s, pp);
  else if (Dv == 128) hipLaunchKernelGGL((preprocess_kernel<128, F16>), grid, block, 0, s, pp);
  else hipLaunchKernelGGL((preprocess_kernel<256, F16>), grid, block, 0, s, pp);
}

hipError_t launch_preprocess(const PreParams& pp, int Dv, bool f16, int64_t tiles, hipStream_t s) {
  if (tiles == 0) return hipSuccess;
  if (tiles > 0x7fffffff) return hipErrorInvalidValue;
  if (f16) launch_preprocess_t<true>(pp, Dv, dim3((unsigned)tiles), s);
  else launch_preprocess_t<false>(pp, Dv, dim3((unsigned)tiles), s);
  return hipGetLastError();
}

hipError_t zero_rows(void* p, const Strides& st, int B, int H, int S, int D, hipStream_t s) {
  const int64_t nbh = (int64_t)B * H;
  if (nbh == 0 || S == 0) return hipSuccess;
  int64_t bx = ((int64_t)S * D / 8 + 255) / 256;
  bx = bx > 1024 ? 1024 : bx;
  const int by = nbh > 65535 ? 65535 : (int)nbh;
  hipLaunchKernelGGL(zero_rows_kernel, dim3((unsigned)bx, by), dim3(256), 0, s, (bf16_t*)p, st, H,
                     S, D, (int)nbh);
  return hipGetLastError();
}

// dbias_cvt over n elements (src null: zeros); the vector form when n is a multiple of 8 and dst
// is 16-byte aligned.
hipError_t launch_dbias_cvt(const float* src, void* dst, int64_t n, bool f16, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int vec = (n % 8 == 0 && ((uintptr_t)dst & 15) == 0) ? 1 : 0;
  int64_t grid = ((vec ? n / 8 : n) + 255) / 256;
  grid = grid > 16384 ? 16384 : grid;
  if (f16)
    hipLaunchKernelGGL(dbias_cvt_kernel<true>, dim3((unsigned)grid), dim3(256), 0, s, src,
                       (bf16_t*)dst, n, vec);
  else
    hipLaunchKernelGGL(dbias_cvt_kernel<false>, dim3((unsigned)grid), dim3(256), 0, s, src,
                       (bf16_t*)dst, n, vec);
  return hipGetLastError();
}

int run(const void* q, const void* k, const void* v, const void* o, const void* dO,
        const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq, int Skv,
        int Dqk, int Dv, float scale, int causal, int window_left, int deterministic,
        const int* seq_q_lens, const int* seq_kv_lens, int bottom_right, int window_right,
        const sdpa_bwd_layout* layouts, int dtype, const float* sink, float* dsink,
        const BiasArgs& ba, void* workspace, size_t workspace_bytes, bool check_ws,
        hipStream_t stream, void* const* events, bool qat = false) {
  Geometry geo;
  const bool has_bias = ba.bias != nullptr;
  // checked here with the 4-wave geometry when an extra may need it; plan() below picks the
  // layout, and the spans are checked again with its key tile
  int st = validate(q, k, v, o, dO, lse, dq, dk, dv, B, Hq, Hkv, Sq, Skv, Dqk, Dv, window_left,
                    window_right, &geo, has_bias || qat);
  if (st != SDPA_BWD_OK) return st;
  int KDqk, KDv;  // the kernel's head dims (>= the tensors' Dqk, Dv)
  kernel_dims(Dqk, Dv, &KDqk, &KDv);
  if (dtype != SDPA_BWD_BF16 && dtype != SDPA_BWD_FP16) return SDPA_BWD_UNSUPPORTED;
  if (ba.dbias && !has_bias) return SDPA_BWD_INVALID_ARG;
  if (has_bias) {
    if (ba.batch != 1 && ba.batch != B) return SDPA_BWD_INVALID_ARG;
    if (ba.dtype != dtype && ba.dtype != SDPA_BWD_FP32) return SDPA_BWD_UNSUPPORTED;
    if (((uintptr_t)ba.bias & (ba.dtype == SDPA_BWD_FP32 ? 3 : 1)) ||
        ((uintptr_t)ba.dbias & (ba.dbias_io ? 1 : 3)))
      return SDPA_BWD_UNSUPPORTED;
  }
  if (dsink && (!sink || ((uintptr_t)sink & 3) || ((uintptr_t)dsink & 3))) return SDPA_BWD_INVALID_ARG;
  const bool f16 = dtype == SDPA_BWD_FP16;
  Layouts L = contiguous_layouts(Hq, Hkv, Sq, Skv, Dqk, Dv);
  if (layouts)
    for (int x = 0; x < N_TENSORS; ++x)
      L.t[x] = Strides{layouts[x].batch, layouts[x].head, layouts[x].seq};
  st = check_layouts(L, Sq, Skv, Dqk, Dv);
  if (st != SDPA_BWD_OK) return st;
  Route route = R_INVALID;
  plan(KDqk, KDv, deterministic, B, Hq, Sq, Skv,
       qat ? X_WIDE : bias_extra(ba.bias, ba.dtype, dtype, KDqk, Sq, Skv), &geo, &route);
  if (route == R_INVALID) return SDPA_BWD_INVALID_ARG;
  // the chosen key tile may be larger than validate() assumed: one head's rows (and its padded
  // tiles) stay addressable through 32-bit buffer offsets
  if (((int64_t)(Sq > Skv ? Sq : Skv) + geo.bc) * (KDqk > KDv ? KDqk : KDv) * 2 >= ((int64_t)1 << 31))
    return SDPA_BWD_UNSUPPORTED;
  // dBias of a batch-1 bias sums over the batch with fp32 atomics: not reproducible ("Support
  // surface", bias), so the deterministic routes need a per-batch bias then
  const bool dbias_atomic = ba.dbias && ba.batch == 1 && B > 1;
  if (dbias_atomic && route != R_ATOMIC) return SDPA_BWD_UNSUPPORTED;
  // an io-type dBias: the main kernel writes each element once, rounded once, unless it sums over
  // the batch; then it accumulates in an fp32 workspace copy that dbias_cvt rounds afterwards
  // (the same single rounding of the same fp32 value either way)
  const bool dbias_acc = ba.dbias && ba.dbias_io && dbias_atomic;
  const bool dbias_direct_io = ba.dbias && ba.dbias_io && !dbias_atomic;
  // empty problems need no workspace (sdpa_bwd_workspace_size returns 0 for them)
  const bool empty = B == 0 || Sq == 0 || Skv == 0;
  const int64_t dbias_elems = (int64_t)ba.batch * Hq * Sq * Skv;
  const Carve c = empty ? Carve{}
                        : carve(B, Hq, Hkv, Sq, Skv, KDqk, KDv, route, geo,
                                dbias_acc ? dbias_elems : 0);
  if (c.total > 0 && workspace == nullptr) return SDPA_BWD_INVALID_ARG;
  if (check_ws && (uint64_t)c.total > (uint64_t)workspace_bytes) return SDPA_BWD_WORKSPACE_TOO_SMALL;
  if (c.total > 0 && ((uintptr_t)workspace % kAlign) != 0) return SDPA_BWD_UNSUPPORTED;
  if (!(scale > 0.f) || !isfinite(scale)) scale = 1.0f / sqrtf((float)Dqk);
  auto rec = [&](int n) {
    if (events && events[n]) (void)hipEventRecord((hipEvent_t)events[n], stream);
  };

  hipError_t e = hipSuccess;
  // dsink over the preprocess's delta (no rows when the problem is empty: zeros)
  auto launch_dsink = [&](const float* stats, int sq_pad, bool none) -> hipError_t {
    if (!dsink) return hipSuccess;
    DsinkParams dp{};
    dp.sink = sink;
    dp.lse = lse;
    dp.stats = stats;
    dp.dsink = dsink;
    dp.seq_q_lens = seq_q_lens;
    dp.B = none ? 0 : B;
    dp.Hq = Hq;
    dp.Sq = Sq;
    dp.sq_pad = sq_pad;
    hipLaunchKernelGGL(dsink_kernel, dim3(Hq), dim3(256), 0, stream, dp);
    return hipGetLastError();
  };
  rec(0);
  if (empty) {
    // nothing attends: every gradient that exists is zero
    e = zero_rows(dq, L.t[T_DQ], B, Hq, Sq, Dqk, stream);
    if (e == hipSuccess) e = zero_rows(dk, L.t[T_DK], B, Hkv, Skv, Dqk, stream);
    if (e == hipSuccess) e = zero_rows(dv, L.t[T_DV], B, Hkv, Skv, Dv, stream);
    if (e == hipSuccess) e = launch_dsink(nullptr, 0, true);
    if (e == hipSuccess && ba.dbias && ba.dbias_io && dbias_elems > 0) {
      // nothing attends: dBias is zero
      e = launch_dbias_cvt(nullptr, ba.dbias, dbias_elems, f16, stream);
    } else if (e == hipSuccess && ba.dbias && (int64_t)ba.batch * Sq * Skv > 0) {
      // nothing attends: dBias is zero
      DbiasFillParams fp{ba.dbias, nullptr, nullptr, Hq, Sq, Skv, geo.bc, geo.br, 0, -1, 0, 0, 1, 0};
      hipLaunchKernelGGL(dbias_fill_kernel, dim3((unsigned)((int64_t)ba.batch * Hq * ((Sq + 31) / 32))),
                         dim3(256), 0, stream, fp);
      e = hipGetLastError();
    }
    for (int n = 1; n < 5; ++n) rec(n);
    return e == hipSuccess ? SDPA_BWD_OK : SDPA_BWD_LAUNCH_FAILED;
  }

  char* ws = (char*)workspace;
  float* stats = (float*)(ws + c.stats);
  float* dq_accum = route == R_ATOMIC ? (float*)(ws + c.dq_accum) : nullptr;
  const int split = q_split(B, Hq, Sq, Skv, geo);
  const bool partials = Hq != Hkv || split > 1;  // dK/dV go through the reduction

  PreParams pp{};
  pp.o = (const bf16_t*)o;
  pp.dO = (const bf16_t*)dO;
  pp.so = L.t[T_O];
  pp.sdo = L.t[T_DO];
  pp.lse = lse;
  pp.stats = stats;
  pp.dq_accum = dq_accum;
  pp.seq_q_lens = seq_q_lens;
  pp.Hq = Hq;
  pp.Sq = Sq;
  pp.sq_pad = (int)c.sq_pad;
  pp.Dqk = KDqk;
  pp.dv_act = Dv;
  pp.zero_rows = route == R_ATOMIC ? 1 : 0;
  pp.relay_turn = route == R_RELAY ? (int*)(ws + c.relay_turn) : nullptr;
  pp.relay_ctl = route == R_RELAY ? (int*)(ws + c.relay_ctl) : nullptr;
  e = launch_preprocess(pp, KDv, f16, (int64_t)B * Hq * (c.sq_pad / geo.br), stream);
  if (e == hipSuccess) e = launch_dsink(stats, (int)c.sq_pad, false);
  // the dBias the main kernel writes: the caller's output (fp32 or, written directly, the io
  // type), or the fp32 workspace accumulator of a batch-summed io-type output
  void* dbias_main = dbias_acc ? (void*)(ws + c.dbias_f32) : ba.dbias;
  if (e == hipSuccess && ba.dbias) {
    // zero the dBias blocks the main kernel does not write (all of them when it accumulates)
    DbiasFillParams fp{};
    fp.dbias = dbias_main;
    fp.io = dbias_direct_io ? 1 : 0;
    fp.seq_q_lens = seq_q_lens;
    fp.seq_kv_lens = seq_kv_lens;
    fp.Hq = Hq;
    fp.Sq = Sq;
    fp.Skv = Skv;
    fp.bc = geo.bc;
    fp.br = geo.br;
    fp.causal = causal ? 1 : 0;
    fp.window_left = window_left;
    fp.window_right = causal ? window_right : 0;
    fp.bottom_right = bottom_right ? 1 : 0;
    fp.all = dbias_atomic ? 1 : 0;
    const int64_t fgrid = (int64_t)ba.batch * Hq * ((Sq + geo.br - 1) / geo.br);
    if (fgrid > 0x7fffffff) return SDPA_BWD_UNSUPPORTED;
    hipLaunchKernelGGL(dbias_fill_kernel, dim3((unsigned)fgrid), dim3(256), 0, stream, fp);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return SDPA_BWD_LAUNCH_FAILED;
  rec(1);

  MainParams mp{};
  mp.q = (const bf16_t*)q;
  mp.k = (const bf16_t*)k;
  mp.v = (const bf16_t*)v;
  mp.dO = (const bf16_t*)dO;
  mp.sq = L.t[T_Q];
  mp.sk = L.t[T_K];
  mp.sv = L.t[T_V];
  mp.sdo = L.t[T_DO];
  mp.sdk = L.t[T_DK];
  mp.sdv = L.t[T_DV];
  mp.stats = stats;
  mp.dq_accum = dq_accum;
  mp.ds_ws = route == R_DS ? (bf16_t*)(ws + c.ds) : nullptr;
  mp.dqp_ws = route == R_DQP ? (float*)(ws + c.dqp) : nullptr;
  mp.relay_acc = route == R_RELAY ? (float*)(ws + c.dqp) : nullptr;
  mp.relay_turn = pp.relay_turn;
  mp.relay_ctl = pp.relay_ctl;
  mp.relay_queues = 1;
  mp.dk_out = partials ? (bf16_t*)(ws + c.dk_ws) : (bf16_t*)dk;
  mp.dv_out = partials ? (bf16_t*)(ws + c.dv_ws) : (bf16_t*)dv;
  mp.seq_q_lens = seq_q_lens;
  mp.seq_kv_lens = seq_kv_lens;
  mp.dqk_act = Dqk;
  mp.dv_act = Dv;
  mp.B = B;
  mp.Hq = Hq;
  mp.Hkv = Hkv;
  mp.Sq = Sq;
  mp.Skv = Skv;
  mp.group = Hq / Hkv;
  mp.partials = partials ? 1 : 0;
  mp.n_split = split;
  mp.causal = causal ? 1 : 0;
  mp.window_left = window_left;
  mp.window_right = causal ? window_right : 0;
  mp.bottom_right = bottom_right ? 1 : 0;
  mp.n_kv_tiles = (Skv + geo.bc - 1) / geo.bc;
  mp.sq_pad = (int)c.sq_pad;
  mp.skv_pad = (int)c.skv_pad;
  mp.scale = scale;
  mp.scale_log2 = scale * kLog2e;
  mp.bias = ba.bias;
  mp.dbias = dbias_main;
  mp.bias_bstride = ba.batch == 1 ? 0 : (int64_t)Hq * Sq * Skv;
  mp.bias_f32 = ba.dtype == SDPA_BWD_FP32 ? 1 : 0;
  mp.dbias_atomic = dbias_atomic ? 1 : 0;
  mp.dbias_io = dbias_direct_io ? 1 : 0;
  int64_t main_grid = (int64_t)mp.n_kv_tiles * split * B * Hq;
  const int64_t relay_items = main_grid;
  if (route == R_RELAY) {
    // one item queue per XCD; every XCD gets as many workgroups as its longest queue (workgroups
    // are spread over the XCDs round-robin; those without an item exit at once)
    const int nq = relay_queues();
    mp.relay_queues = nq;
    main_grid = (int64_t)nq * mp.n_kv_tiles * split * (((int64_t)B * Hq + nq - 1) / nq);
  }
  if (main_grid > 0x7fffffff) return SDPA_BWD_UNSUPPORTED;
  e = run_main(KDqk, mp, route, f16, has_bias ? (ba.dbias ? 2 : 1) : 0, (int)main_grid, geo.bc,
               stream, qat);
  if (e != hipSuccess) return SDPA_BWD_LAUNCH_FAILED;
  if (dbias_acc) {
    e = launch_dbias_cvt((const float*)dbias_main, ba.dbias, dbias_elems, f16, stream);
    if (e != hipSuccess) return SDPA_BWD_LAUNCH_FAILED;
  }
  rec(2);

  if (partials) {
    ReduceParams rp{};
    rp.dk_ws = mp.dk_out;
    rp.dv_ws = mp.dv_out;
    rp.dk = (bf16_t*)dk;
    rp.dv = (bf16_t*)dv;
    rp.sdk = L.t[T_DK];
    rp.sdv = L.t[T_DV];
    rp.n_kvh = B * Hkv;
    rp.Hkv = Hkv;
    rp.Skv = Skv;
    rp.Dqk = KDqk;
    rp.Dv = KDv;
    rp.dqk_act = Dqk;
    rp.dv_act = Dv;
    rp.group = (Hq / Hkv) * split;  // slots (query head of the group, part), in that order
    const int64_t per_head = (int64_t)Skv * (KDqk + KDv) / 8;
    int64_t bx = (per_head + 255) / 256;
    bx = bx > 4096 ? 4096 : bx;
    const int by = rp.n_kvh > 65535 ? 65535 : rp.n_kvh;
    if (f16)
      hipLaunchKernelGGL(gqa_reduce_kernel<true>, dim3((unsigned)bx, by), dim3(256), 0, stream, rp);
    else
      hipLaunchKernelGGL(gqa_reduce_kernel<false>, dim3((unsigned)bx, by), dim3(256), 0, stream, rp);
    if (hipGetLastError() != hipSuccess) return SDPA_BWD_LAUNCH_FAILED;
  }
  rec(3);

  if (route == R_ATOMIC) {
    ConvertParams cp{};
    cp.acc = dq_accum;
    cp.dq = (bf16_t*)dq;
    cp.sdq = L.t[T_DQ];
    cp.seq_q_lens = seq_q_lens;
    cp.Hq = Hq;
    cp.Sq = Sq;
    cp.dqk_act = Dqk;
    cp.scale = scale;
    const int64_t cgrid = (int64_t)B * Hq * ((Sq + 31) / 32);
    if (cgrid > 0x7fffffff) return SDPA_BWD_UNSUPPORTED;
    e = launch_convert(cp, KDqk, f16, (int)cgrid, stream);
    if (e != hipSuccess) return SDPA_BWD_LAUNCH_FAILED;
  } else if (route == R_DQP || route == R_RELAY) {
    DqReduceParams rp{};
    rp.dqp_ws = route == R_RELAY ? mp.relay_acc : mp.dqp_ws;
    rp.dq = (bf16_t*)dq;
    rp.sdq = L.t[T_DQ];
    rp.seq_q_lens = seq_q_lens;
    rp.seq_kv_lens = seq_kv_lens;
    rp.B = B;
    rp.Hq = Hq;
    rp.Sq = Sq;
    rp.Skv = Skv;
    rp.causal = mp.causal;
    rp.window_left = window_left;
    rp.window_right = mp.window_right;
    rp.bottom_right = mp.bottom_right;
    rp.n_kv_tiles = route == R_RELAY ? 1 : mp.n_kv_tiles;
    rp.n_q_tiles = (int)(c.sq_pad / geo.br);
    rp.bc = geo.bc;
    rp.dqk_act = Dqk;
    rp.scale = scale;
    rp.relay_ctl = route == R_RELAY ? mp.relay_ctl : nullptr;
    rp.relay_items = (int)relay_items;
    const int64_t rgrid = (int64_t)B * Hq * rp.n_q_tiles;
    if (rgrid > 0x7fffffff) return SDPA_BWD_UNSUPPORTED;
    e = launch_dq_reduce(rp, KDqk, f16, (int)rgrid, stream);
    if (e != hipSuccess) return SDPA_BWD_LAUNCH_FAILED;
  } else {
    Dq2kParams dp{};
    dp.ds_ws = mp.ds_ws;
    dp.k = (const bf16_t*)k;
    dp.dq = (bf16_t*)dq;
    dp.sk = L.t[T_K];
    dp.sdq = L.t[T_DQ];
    dp.seq_q_lens = seq_q_lens;
    dp.seq_kv_lens = seq_kv_lens;
    dp.B = B;
    dp.Hq = Hq;
    dp.Hkv = Hkv;
    dp.Sq = Sq;
    dp.Skv = Skv;
    dp.group = Hq / Hkv;
    dp.causal = mp.causal;
    dp.window_left = window_left;
    dp.window_right = mp.window_right;
    dp.bottom_right = mp.bottom_right;
    dp.n_kv_tiles = mp.n_kv_tiles;
    dp.n_q_tiles = (int)(c.sq_pad / geo.br);
    dp.dqk_act = Dqk;
    dp.scale = scale;
    // head dim 32 runs dq2k's 64-wide kernel: K's extra columns reach only unstored dQ columns
    e = run_dq2k(KDqk == 32 ? 64 : KDqk, f16, dp, geo.bc, stream);
    if (e != hipSuccess) return SDPA_BWD_LAUNCH_FAILED;
  }
  rec(4);
  return SDPA_BWD_OK;
}

}  // namespace

// NVFP4 QAT: the fake-quantised copies of Q, K and V at the start of the workspace.
int64_t qat_hat_bytes(int B, int H, int Sq, int Skv) {
  return align_up((int64_t)B * H * Sq * 128 * 2, kAlign) +
         2 * align_up((int64_t)B * H * Skv * 128 * 2, kAlign);
}

hipError_t launch_fake_quant(const void* x, void* y, int64_t elems, hipStream_t s) {
  const int64_t groups = elems / 16;
  if (groups == 0) return hipSuccess;
  int64_t grid = (groups + 255) / 256;
  grid = grid > 8192 ? 8192 : grid;
  hipLaunchKernelGGL(nvfp4_fake_quant_kernel, dim3((unsigned)grid), dim3(256), 0, s,
                     (const bf16_t*)x, (bf16_t*)y, groups);
  return hipGetLastError();
}

// ---- allocation-free entry point ---------------------------------------------------------------
// sdpa_bwd_noalloc carves its workspace from this file-scope device array instead of a caller's
// buffer.  Each device the library runs on holds its own copy, at its own address, until the
// process ends.  In host code `scratch` is only the runtime's handle of the symbol: its device
// address is looked up once per device (scratch_on_current_device) and only that address is
// passed to the kernels.
static __device__ __align__(256) char scratch[SDPA_BWD_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// The device address of `scratch` on the current device, looked up on the first call made with
// that device current and kept; NULL when the lookup fails.
void* scratch_on_current_device() {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    addr[dev] = p;
  }
  return addr[dev];
}

// The route as the header's SDPA_BWD_DQ_* value (-1 for R_INVALID).
int route_code(Route r) {
  switch (r) {
    case R_ATOMIC: return SDPA_BWD_DQ_ATOMIC;
    case R_DS: return SDPA_BWD_DQ_DS_PANELS;
    case R_DQP: return SDPA_BWD_DQ_PARTIALS;
    case R_RELAY: return SDPA_BWD_DQ_RELAY;
    default: return -1;
  }
}

extern "C" {

size_t sdpa_bwd_workspace_size(int B, int Hq, int Hkv, int Sq, int Skv, int Dqk, int Dv,
                               int causal, int window_left, int deterministic, int has_seqlens) {
  (void)causal;
  (void)window_left;
  (void)has_seqlens;
  Geometry geo;
  int kq, kv;
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Sq < 0 || Skv < 0 || Hq % Hkv != 0) return 0;
  if (!kernel_dims(Dqk, Dv, &kq, &kv) || !geometry_for(kq, kv, &geo)) return 0;
  if (B == 0 || Sq == 0 || Skv == 0) return 0;
  const Route route = route_for(deterministic, kq, geo, B, Hq, Sq, Skv);
  if (route == R_INVALID) return 0;
  return (size_t)carve(B, Hq, Hkv, Sq, Skv, kq, kv, route, geo).total;
}

int sdpa_bwd_dq_route(int B, int Hq, int Hkv, int Sq, int Skv, int Dqk, int Dv,
                      int deterministic) {
  Geometry geo;
  int kq, kv;
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Sq < 0 || Skv < 0 || Hq % Hkv != 0) return -1;
  if (!kernel_dims(Dqk, Dv, &kq, &kv) || !geometry_for(kq, kv, &geo)) return -1;
  return route_code(route_for(deterministic, kq, geo, B, Hq, Sq, Skv));
}

size_t sdpa_bwd_nvfp4_qat_workspace_size(int B, int H, int Sq, int Skv, int D, int causal,
                                         int deterministic) {
  if (B < 0 || H <= 0 || Sq < 0 || Skv < 0 || D != 128 || (causal && Sq != Skv)) return 0;
  if (B == 0 || Sq == 0 || Skv == 0) return 0;
  Geometry geo;
  Route route = R_INVALID;
  plan(128, 128, deterministic, B, H, Sq, Skv, X_WIDE, &geo, &route);
  if (route == R_INVALID) return 0;
  return (size_t)(qat_hat_bytes(B, H, Sq, Skv) + carve(B, H, H, Sq, Skv, 128, 128, route, geo).total);
}

int sdpa_bwd_nvfp4_qat(const void* q, const void* k, const void* v, const void* o_hp,
                       const void* dO, const float* lse, void* dq, void* dk, void* dv, int B,
                       int H, int Sq, int Skv, int D, float scale, int causal, int deterministic,
                       void* workspace, size_t workspace_bytes, void* stream,
                       void* const* events) {
  if (B < 0 || H <= 0 || Sq < 0 || Skv < 0) return SDPA_BWD_INVALID_ARG;
  if (D != 128 || (causal && Sq != Skv)) return SDPA_BWD_UNSUPPORTED;
  // everything run() checks, on the caller's tensors, before the quantisation launches
  Geometry geo;
  int st = validate(q, k, v, o_hp, dO, lse, dq, dk, dv, B, H, H, Sq, Skv, D, D, -1, 0, &geo, true);
  if (st != SDPA_BWD_OK) return st;
  if (route_for(deterministic, 128, geo, B, H, Sq, Skv) == R_INVALID) return SDPA_BWD_INVALID_ARG;
  const hipStream_t s = (hipStream_t)stream;
  if (B == 0 || Sq == 0 || Skv == 0)  // nothing to quantise; the chain writes the zeros
    return run(q, k, v, o_hp, dO, lse, dq, dk, dv, B, H, H, Sq, Skv, D, D, scale, causal, -1,
               deterministic, nullptr, nullptr, 0, 0, nullptr, SDPA_BWD_BF16, nullptr, nullptr,
               BiasArgs{}, workspace, workspace_bytes, true, s, events, true);
  const size_t need = sdpa_bwd_nvfp4_qat_workspace_size(B, H, Sq, Skv, D, causal, deterministic);
  if (workspace == nullptr) return SDPA_BWD_INVALID_ARG;
  if (workspace_bytes < need) return SDPA_BWD_WORKSPACE_TOO_SMALL;
  if (((uintptr_t)workspace % kAlign) != 0) return SDPA_BWD_UNSUPPORTED;
  char* ws = (char*)workspace;
  const int64_t nq = (int64_t)B * H * Sq * 128, nk = (int64_t)B * H * Skv * 128;
  char* qh = ws;
  char* kh = qh + align_up(nq * 2, kAlign);
  char* vh = kh + align_up(nk * 2, kAlign);
  const int64_t hat = qat_hat_bytes(B, H, Sq, Skv);
  hipError_t e = launch_fake_quant(q, qh, nq, s);
  if (e == hipSuccess) e = launch_fake_quant(k, kh, nk, s);
  if (e == hipSuccess) e = launch_fake_quant(v, vh, nk, s);
  if (e != hipSuccess) return SDPA_BWD_LAUNCH_FAILED;
  return run(qh, kh, vh, o_hp, dO, lse, dq, dk, dv, B, H, H, Sq, Skv, D, D, scale, causal, -1,
             deterministic, nullptr, nullptr, 0, 0, nullptr, SDPA_BWD_BF16, nullptr, nullptr,
             BiasArgs{}, ws + hat, workspace_bytes - (size_t)hat, true, s, events, true);
}

int sdpa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
             const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq,
             int Skv, int Dqk, int Dv, float scale, int causal, int window_left,
             int deterministic, void* workspace, void* stream) {
  return run(q, k, v, o, dO, lse, dq, dk, dv, B, Hq, Hkv, Sq, Skv, Dqk, Dv, scale, causal,
             window_left, deterministic, nullptr, nullptr, 0, 0, nullptr, SDPA_BWD_BF16, nullptr,
             nullptr, BiasArgs{}, workspace, 0, false, (hipStream_t)stream, nullptr);
}

int sdpa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dO,
                const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq,
                int Skv, int Dqk, int Dv, float scale, int causal, int window_left,
                int deterministic, const int* seq_q_lens, const int* seq_kv_lens,
                int causal_bottom_right, int window_right, void* workspace,
                size_t workspace_bytes, void* stream) {
  return run(q, k, v, o, dO, lse, dq, dk, dv, B, Hq, Hkv, Sq, Skv, Dqk, Dv, scale, causal,
             window_left, deterministic, seq_q_lens, seq_kv_lens, causal_bottom_right,
             window_right, nullptr, SDPA_BWD_BF16, nullptr, nullptr, BiasArgs{}, workspace,
             workspace_bytes, true, (hipStream_t)stream, nullptr);
}

int sdpa_bwd_ex_events(const void* q, const void* k, const void* v, const void* o,
                       const void* dO, const float* lse, void* dq, void* dk, void* dv, int B,
                       int Hq, int Hkv, int Sq, int Skv, int Dqk, int Dv, float scale, int causal,
                       int window_left, int deterministic, const int* seq_q_lens,
                       const int* seq_kv_lens, int causal_bottom_right, int window_right,
                       void* workspace, size_t workspace_bytes, void* stream,
                       void* const* events) {
  return run(q, k, v, o, dO, lse, dq, dk, dv, B, Hq, Hkv, Sq, Skv, Dqk, Dv, scale, causal,
             window_left, deterministic, seq_q_lens, seq_kv_lens, causal_bottom_right,
             window_right, nullptr, SDPA_BWD_BF16, nullptr, nullptr, BiasArgs{}, workspace,
             workspace_bytes, true, (hipStream_t)stream, events);
}

int sdpa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dO,
                     const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv,
                     int Sq, int Skv, int Dqk, int Dv, float scale, int causal, int window_left,
                     int deterministic, const int* seq_q_lens, const int* seq_kv_lens,
                     int causal_bottom_right, int window_right, void* stream) {
  // host-side size check first: a problem larger than the scratch is declined before any GPU call
  const size_t need = sdpa_bwd_workspace_size(B, Hq, Hkv, Sq, Skv, Dqk, Dv, causal, window_left,
                                              deterministic, seq_q_lens != nullptr);
  if (need > (size_t)SDPA_BWD_NOALLOC_SCRATCH_BYTES) return SDPA_BWD_SCRATCH_TOO_SMALL;
  // need == 0: arguments run() rejects, or an empty problem, which uses no workspace
  void* ws = nullptr;
  if (need > 0) {
    ws = scratch_on_current_device();
    if (ws == nullptr) return SDPA_BWD_LAUNCH_FAILED;
  }
  return run(q, k, v, o, dO, lse, dq, dk, dv, B, Hq, Hkv, Sq, Skv, Dqk, Dv, scale, causal,
             window_left, deterministic, seq_q_lens, seq_kv_lens, causal_bottom_right,
             window_right, nullptr, SDPA_BWD_BF16, nullptr, nullptr, BiasArgs{}, ws,
             ws ? (size_t)SDPA_BWD_NOALLOC_SCRATCH_BYTES : 0, true, (hipStream_t)stream, nullptr);
}

int sdpa_bwd_flex(const void* q, const void* k, const void* v, const void* o, const void* dO,
                  const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq,
                  int Skv, int Dqk, int Dv, float scale, int causal, int window_left,
                  int deterministic, const int* seq_q_lens, const int* seq_kv_lens,
                  int causal_bottom_right, int window_right, const sdpa_bwd_layout* layouts,
                  int dtype, void* workspace, size_t workspace_bytes, void* stream,
                  void* const* events) {
  return run(q, k, v, o, dO, lse, dq, dk, dv, B, Hq, Hkv, Sq, Skv, Dqk, Dv, scale, causal,
             window_left, deterministic, seq_q_lens, seq_kv_lens, causal_bottom_right,
             window_right, layouts, dtype, nullptr, nullptr, BiasArgs{}, workspace, workspace_bytes,
             true, (hipStream_t)stream, events);
}

int sdpa_bwd_run(const sdpa_bwd_args* a) {
  if (!a) return SDPA_BWD_INVALID_ARG;
  BiasArgs ba;
  ba.bias = a->bias;
  ba.dbias = a->dbias;
  ba.dtype = a->bias_dtype;
  ba.batch = a->bias_batch;
  ba.dbias_io = a->dbias_io != 0;
  return run(a->q, a->k, a->v, a->o, a->dO, a->lse, a->dq, a->dk, a->dv, a->B, a->Hq, a->Hkv,
             a->Sq, a->Skv, a->Dqk, a->Dv, a->scale, a->causal, a->window_left, a->deterministic,
             a->seq_q_lens, a->seq_kv_lens, a->causal_bottom_right, a->window_right, a->layouts,
             a->dtype, a->sink, a->dsink, ba, a->workspace, a->workspace_bytes, true,
             (hipStream_t)a->stream, a->events);
}

size_t sdpa_bwd_run_workspace_size(const sdpa_bwd_args* a) {
  if (!a) return 0;
  Geometry geo;
  if (a->B < 0 || a->Hq <= 0 || a->Hkv <= 0 || a->Sq < 0 || a->Skv < 0 || a->Hq % a->Hkv != 0)
    return 0;
  int kq, kv;
  Route route = R_INVALID;
  if (!kernel_dims(a->Dqk, a->Dv, &kq, &kv) ||
      !plan(kq, kv, a->deterministic, a->B, a->Hq, a->Sq, a->Skv,
            bias_extra(a->bias, a->bias_dtype, a->dtype, kq, a->Sq, a->Skv), &geo, &route))
    return 0;
  if (a->B == 0 || a->Sq == 0 || a->Skv == 0) return 0;
  if (route == R_INVALID) return 0;
  // the fp32 accumulator of an io-type dBias summed over the batch (see run())
  const int64_t dbias_elems = a->dbias && a->bias && a->dbias_io && a->bias_batch == 1 && a->B > 1
                                  ? (int64_t)a->Hq * a->Sq * a->Skv
                                  : 0;
  return (size_t)carve(a->B, a->Hq, a->Hkv, a->Sq, a->Skv, kq, kv, route, geo, dbias_elems).total;
}

int sdpa_bwd_run_dq_route(const sdpa_bwd_args* a) {
  if (!a) return -1;
  Geometry geo;
  if (a->B < 0 || a->Hq <= 0 || a->Hkv <= 0 || a->Sq < 0 || a->Skv < 0 || a->Hq % a->Hkv != 0)
    return -1;
  int kq, kv;
  Route route = R_INVALID;
  if (!kernel_dims(a->Dqk, a->Dv, &kq, &kv) ||
      !plan(kq, kv, a->deterministic, a->B, a->Hq, a->Sq, a->Skv,
            bias_extra(a->bias, a->bias_dtype, a->dtype, kq, a->Sq, a->Skv), &geo, &route))
    return -1;
  return route_code(route);
}

int sdpa_bwd_preprocess(const void* o, const void* dO, const float* lse, float* stats,
                        float* dq_accum, const int* seq_q_lens, int B, int Hq, int Sq, int Dv,
                        int Dqk, void* stream) {
  if (B < 0 || Hq < 0 || Sq < 0) return SDPA_BWD_INVALID_ARG;
  int kq, kv;
  if (!kernel_dims(Dqk, Dv, &kq, &kv)) return SDPA_BWD_UNSUPPORTED;
  if (!o || !dO || !lse || !stats) return SDPA_BWD_INVALID_ARG;
  if (!aligned16(o) || !aligned16(dO) || !aligned16(stats) || (dq_accum && !aligned16(dq_accum)) ||
      ((uintptr_t)lse & 3) != 0)
    return SDPA_BWD_UNSUPPORTED;
  PreParams pp{};  // every field set below; the relay counters stay NULL
  pp.o = (const bf16_t*)o;
  pp.dO = (const bf16_t*)dO;
  pp.so = pp.sdo = Strides{(int64_t)Hq * Sq * Dv, (int64_t)Sq * Dv, (int64_t)Dv};  // contiguous BHSD
  pp.lse = lse;
  pp.stats = stats;
  pp.dq_accum = dq_accum;
  pp.seq_q_lens = seq_q_lens;
  pp.relay_turn = nullptr;
  pp.relay_ctl = nullptr;
  pp.sq_pad = (int)align_up(Sq, 32);
  pp.Hq = Hq;
  pp.Sq = Sq;
  pp.Dqk = Dqk;     // the caller's dq_accum rows are Dqk floats
  pp.dv_act = Dv;
  pp.zero_rows = dq_accum ? 1 : 0;
  const int64_t tiles = (int64_t)B * Hq * (pp.sq_pad / 32);
  return launch_preprocess(pp, kv, false, tiles, (hipStream_t)stream) == hipSuccess
             ? SDPA_BWD_OK
             : SDPA_BWD_LAUNCH_FAILED;
}

const char* sdpa_bwd_status_string(int status) {
  switch (status) {
    case SDPA_BWD_OK: return "ok";
    case SDPA_BWD_INVALID_ARG: return "invalid argument";
    case SDPA_BWD_UNSUPPORTED: return "unsupported configuration";
    case SDPA_BWD_WORKSPACE_TOO_SMALL: return "workspace too small";
    case SDPA_BWD_LAUNCH_FAILED: return "kernel launch failed";
    case SDPA_BWD_SCRATCH_TOO_SMALL:
      return "problem needs more workspace than the static scratch of sdpa_bwd_noalloc";
    default: return "unknown status";
  }
}

}  // extern "C"
