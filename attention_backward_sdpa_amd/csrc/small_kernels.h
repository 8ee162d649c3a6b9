// Bandwidth-bound kernels of the attention-backward chain ("SDPA Backward (SM120)", section
// "The kernel chain"): the row-dot preprocess (delta = rowsum(O * dO), fused with zeroing the fp32
// dQ accumulator), the dQ convert (fp32 accumulator -> bf16, times the softmax scale), the
// fixed-order GQA dK/dV group reduction ("GQA/MQA group reduction") and the sink-gradient reduce.
#pragma once
#include "common.h"
#include "masks.h"
#include "nvfp4.h"

namespace sdpa {

// ---- preprocess ---------------------------------------------------------------------------------
// One workgroup per 32-row q tile of one (batch, query head):
//   * stats[row] = [LSE * log2(e), delta] with delta = rowsum(O * dO) in fp32.  Rows at or past the
//     batch entry's query length, rows past the buffer and rows whose LSE is -inf (no visible key
//     in the forward) get [+inf, 0], so the main kernel replays P = 0 for them without a NaN.
//     The row's Dv/8 lanes reduce with butterfly shuffles in a fixed order (deterministic).
//   * when zero_rows is set, the tile's rows of the fp32 dQ accumulator below the batch entry's
//     query length are cleared (the main kernel adds into no other row, and the convert kernel
//     writes the rest of dQ as zeros without reading them).  O and dO are read only for those rows.
struct PreParams {
  const bf16_t* o;
  const bf16_t* dO;
  Strides so, sdo;           // element strides of o and dO
  const float* lse;
  float* stats;              // (B*Hq, sq_pad, 2)
  float* dq_accum;           // (B*Hq, Sq, Dqk) or null
  const int* seq_q_lens;
  int Hq, Sq, sq_pad, Dqk;   // Dqk: the dq_accum row length (the kernel's head dim)
  int dv_act;                // O / dO head dim (<= DV); the row dot covers these columns
  int zero_rows;
  int* relay_turn;           // (B*Hq, sq_pad/32) turn counters of the relay route, zeroed, or null
  int* relay_ctl;            // the relay's 16 control words, zeroed by workgroup 0, or null
};

template <int DV, bool F16>
__global__ void __launch_bounds__(256) preprocess_kernel(PreParams p) {
  constexpr int BR = 32;
  constexpr int LPR = DV / 8;              // lanes per row for the row dot
  constexpr int RPP = 256 / LPR;           // rows per pass
  const int tid = threadIdx.x;
  const int nt = p.sq_pad / BR;
  const int64_t bh = blockIdx.x / nt;
  const int i = blockIdx.x % nt;
  const int q0 = i * BR;
  const int b = (int)(bh / p.Hq), h = (int)(bh % p.Hq);
  const bf16_t* ob = p.o + b * p.so.b + h * p.so.h;
  const bf16_t* dob = p.dO + b * p.sdo.b + h * p.sdo.h;
  const int Lq = p.seq_q_lens ? min(max(p.seq_q_lens[b], 0), p.Sq) : p.Sq;
  if (p.relay_turn && tid == 0) p.relay_turn[blockIdx.x] = 0;
  if (p.relay_ctl && blockIdx.x == 0 && tid < 16) p.relay_ctl[tid] = 0;

  // every pass's loads go out before the first row dot
  constexpr int NP = (BR + RPP - 1) / RPP;
  const int sub = tid % LPR;
  u32x4 av[NP], cv[NP];
  float lv[NP];
#pragma unroll
  for (int pi = 0; pi < NP; ++pi) {
    const int r = pi * RPP + tid / LPR, s = q0 + r;
    av[pi] = cv[pi] = u32x4{0u, 0u, 0u, 0u};
    lv[pi] = -INFINITY;
    if (r < BR && s < Lq) {
      if (sub == 0) lv[pi] = p.lse[bh * p.Sq + s];
      if (sub * 8 < p.dv_act) {
        av[pi] = *reinterpret_cast<const u32x4*>(ob + s * p.so.s + sub * 8);
        cv[pi] = *reinterpret_cast<const u32x4*>(dob + s * p.sdo.s + sub * 8);
      }
    }
  }
#pragma unroll
  for (int pi = 0; pi < NP; ++pi) {
    const int r = pi * RPP + tid / LPR, s = q0 + r;
    if (r >= BR) break;  // head dim 32: one pass covers 64 rows, the tile has 32
    const bool live = s < Lq;
    const int64_t row = bh * p.Sq + s;
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc += Elem<F16>::lo(av[pi][e]) * Elem<F16>::lo(cv[pi][e]);
      acc += Elem<F16>::hi(av[pi][e]) * Elem<F16>::hi(cv[pi][e]);
    }
#pragma unroll
    for (int off = LPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, LPR);
    if (sub == 0) {
      const float l = lv[pi];
      const bool none = !(l > -INFINITY);  // -inf (or NaN) LSE: the row saw no key
      reinterpret_cast<float2*>(p.stats)[bh * p.sq_pad + s] =
          make_float2(none ? INFINITY : l * kLog2e, (live && !none) ? acc : 0.f);
    }
    if (p.zero_rows && live) {
      float4* dst = reinterpret_cast<float4*>(p.dq_accum + row * p.Dqk);
      for (int x = sub; x < p.Dqk / 4; x += LPR) dst[x] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
}

// ---- dQ convert ---------------------------------------------------------------------------------
// dQ = bf16(scale * dq_accum) for the rows below the batch entry's query length; the other rows
// (never added into, and not cleared by the preprocess) are written as zeros without reading the
// accumulator.  One workgroup per 32-row q tile of one (batch, query head); 8 elements per thread
// and step (two 16-byte loads, one 16-byte store).
struct ConvertParams {
  const float* acc;          // (B*Hq, Sq, Dqk), contiguous
  bf16_t* dq;                // (B, Hq, Sq, Dqk), element strides sdq
  Strides sdq;
  const int* seq_q_lens;
  int Hq, Sq;
  int dqk_act;               // dQ head dim (<= DQK, the accumulator's row length)
  float scale;
};

template <int DQK, bool F16>
__global__ void __launch_bounds__(256) dq_convert_kernel(ConvertParams p) {
  constexpr int V = DQK / 8;  // 8-element vectors per row
  const int nt = (p.Sq + 31) / 32;
  const int64_t bh = blockIdx.x / nt;
  const int q0 = (int)(blockIdx.x % nt) * 32;
  const int b = (int)(bh / p.Hq), h = (int)(bh % p.Hq);
  const int Lq = p.seq_q_lens ? min(max(p.seq_q_lens[b], 0), p.Sq) : p.Sq;
  bf16_t* dqb = p.dq + b * p.sdq.b + h * p.sdq.h;
  // every load of the thread goes out before the first conversion
  constexpr int NIT = (32 * V + 255) / 256;
  floatx4 a[NIT], d[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int v = threadIdx.x + it * 256, s = q0 + v / V, c = v % V;
    a[it] = d[it] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (v < 32 * V && s < Lq && c * 8 < p.dqk_act) {
      const int64_t x = (bh * p.Sq + s) * V + c;
      a[it] = reinterpret_cast<const floatx4*>(p.acc)[2 * x];
      d[it] = reinterpret_cast<const floatx4*>(p.acc)[2 * x + 1];
    }
  }
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int v = threadIdx.x + it * 256, s = q0 + v / V, c = v % V;
    if (v >= 32 * V || s >= p.Sq || c * 8 >= p.dqk_act) continue;
    const float k = p.scale;
    const u32x4 out = u32x4{Elem<F16>::pack2(a[it][0] * k, a[it][1] * k),
                            Elem<F16>::pack2(a[it][2] * k, a[it][3] * k),
                            Elem<F16>::pack2(d[it][0] * k, d[it][1] * k),
                            Elem<F16>::pack2(d[it][2] * k, d[it][3] * k)};
    *reinterpret_cast<u32x4*>(dqb + s * p.sdq.s + c * 8) = out;
  }
}

// ---- GQA reduce ---------------------------------------------------------------------------------
// out[b, kvh, s, :] = bf16( sum_{g = 0 .. group-1} ws[b, kvh*group + g, s, :] ), summed in fp32
// in ascending g.  The partials are contiguous per slot; the outputs follow the caller's layout.
// grid.y walks the KV heads (b * Hkv + kvh), grid.x one 16-byte output vector per thread over
// the head's dK vectors and then its dV vectors.
struct ReduceParams {
  const bf16_t* dk_ws;
  const bf16_t* dv_ws;
  bf16_t* dk;
  bf16_t* dv;
  Strides sdk, sdv;
  int n_kvh, Hkv;            // B * Hkv, Hkv
  int Skv, Dqk, Dv;          // the partials' row lengths (the kernel's head dims)
  int dqk_act, dv_act;       // dK / dV head dims (<= Dqk / Dv): the columns written
  int group;                 // partial slots per KV head, summed in this order
};

template <bool F16>
__global__ void __launch_bounds__(256) gqa_reduce_kernel(ReduceParams p) {
  const int k8 = p.Dqk / 8, v8 = p.Dv / 8;
  const int nk = p.Skv * k8, nv = p.Skv * v8;  // vectors per head (the host keeps these < 2^28)
  for (int kvhead = blockIdx.y; kvhead < p.n_kvh; kvhead += gridDim.y) {
    const int b = kvhead / p.Hkv, kvh = kvhead % p.Hkv;
    for (int x = blockIdx.x * 256 + threadIdx.x; x < nk + nv; x += gridDim.x * 256) {
      const bool isk = x < nk;
      const int y = isk ? x : x - nk;
      const int per = isk ? nk : nv, d8 = isk ? k8 : v8;
      const int key = y / d8, c = y - key * d8;
      if (c * 8 >= (isk ? p.dqk_act : p.dv_act)) continue;
      const u32x4* src = reinterpret_cast<const u32x4*>(isk ? p.dk_ws : p.dv_ws) +
                         (int64_t)kvhead * p.group * per + y;
      // the slots' loads go out four at a time, then add in ascending slot order
      float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int g0 = 0; g0 < p.group; g0 += 4) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (g0 + u < p.group) v[u] = src[(int64_t)(g0 + u) * per];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (g0 + u >= p.group) break;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            s[2 * e] += Elem<F16>::lo(v[u][e]);
            s[2 * e + 1] += Elem<F16>::hi(v[u][e]);
          }
        }
      }
      const Strides& st = isk ? p.sdk : p.sdv;
      bf16_t* dst = (isk ? p.dk : p.dv) + b * st.b + kvh * st.h + key * st.s + c * 8;
      *reinterpret_cast<u32x4*>(dst) =
          u32x4{Elem<F16>::pack2(s[0], s[1]), Elem<F16>::pack2(s[2], s[3]),
                Elem<F16>::pack2(s[4], s[5]), Elem<F16>::pack2(s[6], s[7])};
    }
  }
}

// ---- dsink ----------------------------------------------------------------------------------------
// "The kernel chain" (dsink) and "Support surface" (sink tokens): the gradient of a per-query-head
// sink logit, dsink[h] = -sum_{b, q} exp(sink[h] - LSE[b,h,q]) * delta[b,h,q], over the rows below
// the batch entry's query length whose LSE is finite (delta as the preprocess stored it).  One
// workgroup per query head; each thread sums the rows tid, tid + 256, ... in fp64, then a fixed
// tree adds the 256 partial sums: the same order on every run, so the result is bitwise
// reproducible.  Empty problems (B * Sq = 0) write 0.
struct DsinkParams {
  const float* sink;    // (Hq,)
  const float* lse;     // (B, Hq, Sq)
  const float* stats;   // (B*Hq, sq_pad, 2) from the preprocess, or null when B * Sq = 0
  float* dsink;         // (Hq,)
  const int* seq_q_lens;
  int B, Hq, Sq, sq_pad;
};

__global__ void __launch_bounds__(256) dsink_kernel(DsinkParams p) {
  __shared__ double part[256];
  const int h = blockIdx.x, tid = threadIdx.x;
  const double sk = (double)p.sink[h];
  double acc = 0.0;
  const int64_t rows = (int64_t)p.B * p.Sq;
  for (int64_t x = tid; x < rows; x += 256) {
    const int b = (int)(x / p.Sq), q = (int)(x % p.Sq);
    const int Lq = p.seq_q_lens ? min(max(p.seq_q_lens[b], 0), p.Sq) : p.Sq;
    if (q >= Lq) continue;
    const int64_t bh = (int64_t)b * p.Hq + h;
    const float l = p.lse[bh * p.Sq + q];
    if (!(l > -INFINITY)) continue;  // no key and no sink in the forward (or NaN): nothing
    const float delta = p.stats[(bh * p.sq_pad + q) * 2 + 1];
    acc += exp(sk - (double)l) * (double)delta;
  }
  part[tid] = acc;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off) part[tid] += part[tid + off];
    __syncthreads();
  }
  if (tid == 0) p.dsink[h] = (float)(0.0 - part[0]);
}

// ---- dBias fill -----------------------------------------------------------------------------------
// dBias (Bb, Hq, Sq, Skv), fp32 or the io type: the main kernel writes every element of the (q tile, key tile)
// blocks it visits (masked pairs as 0); this kernel zeroes the elements of every other block, or
// of every block when the main kernel accumulates dBias over the batch with atomics.  One
// workgroup per (bias batch entry, query head, q tile); threads stride over the columns of the
// tile's rows, a column's key tile deciding whether it is written here.
struct DbiasFillParams {
  void* dbias;              // fp32 elements, or 16-bit io-type elements with `io`
  const int* seq_q_lens;
  const int* seq_kv_lens;
  int Hq, Sq, Skv;
  int bc, br;               // key tile and q tile of the main kernel
  int causal, window_left, window_right, bottom_right;
  int all;                  // zero every element
  int io;                   // 16-bit io-type elements (zero is all bits clear for bf16 and fp16)
};

__global__ void __launch_bounds__(256) dbias_fill_kernel(DbiasFillParams p) {
  const int nqt = (p.Sq + p.br - 1) / p.br;
  const int64_t bh = blockIdx.x / nqt;
  const int i = (int)(blockIdx.x % nqt);
  const int b = (int)(bh / p.Hq);  // the bias batch entry is the batch entry when Bb = B
  MaskGeom mg;
  mg.Lq = p.seq_q_lens ? min(max(p.seq_q_lens[b], 0), p.Sq) : p.Sq;
  mg.Lkv = p.seq_kv_lens ? min(max(p.seq_kv_lens[b], 0), p.Skv) : p.Skv;
  mg.diag = p.bottom_right ? mg.Lkv - mg.Lq : 0;
  mg.causal = p.causal;
  mg.W = p.window_left;
  mg.R = p.window_right;
  const int64_t first = (bh * p.Sq + (int64_t)i * p.br) * p.Skv;
  const int rows = min(p.br, p.Sq - i * p.br);
  for (int c = threadIdx.x; c < p.Skv; c += 256) {
    bool visited = false;
    if (!p.all) {
      int lo, hi;
      q_tile_range(mg, (c / p.bc) * p.bc, p.bc, p.br, &lo, &hi);
      visited = lo <= i && i <= hi;
    }
    if (visited) continue;
    if (p.io) {
      bf16_t* base = reinterpret_cast<bf16_t*>(p.dbias) + first;
      for (int r = 0; r < rows; ++r) base[(int64_t)r * p.Skv + c] = 0;
    } else {
      float* base = reinterpret_cast<float*>(p.dbias) + first;
      for (int r = 0; r < rows; ++r) base[(int64_t)r * p.Skv + c] = 0.f;
    }
  }
}

// ---- dbias_cvt ---------------------------------------------------------------------------------
// "The kernel chain" (dbias_cvt) and "Support surface" (bias): an io-type dBias output is the
// fp32 dBias (accumulated in the workspace by the main kernel and the fill above) rounded once
// to the io type.  Flat over the (Bb, Hq, Sq, Skv) elements; `vec`: 8 elements per thread and step
// (two 16-byte loads, one 16-byte store; n a multiple of 8 and dst 16-byte aligned), else one.
// With src = null every element is written as 0 (problems where nothing attends).
template <bool F16>
__global__ void __launch_bounds__(256) dbias_cvt_kernel(const float* src, bf16_t* dst, int64_t n,
                                                        int vec) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  if (vec) {
    for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < n / 8; x += stride) {
      u32x4 out = u32x4{0u, 0u, 0u, 0u};
      if (src) {
        const floatx4 a = reinterpret_cast<const floatx4*>(src)[2 * x];
        const floatx4 b = reinterpret_cast<const floatx4*>(src)[2 * x + 1];
        out = u32x4{Elem<F16>::pack2(a[0], a[1]), Elem<F16>::pack2(a[2], a[3]),
                    Elem<F16>::pack2(b[0], b[1]), Elem<F16>::pack2(b[2], b[3])};
      }
      reinterpret_cast<u32x4*>(dst)[x] = out;
    }
  } else {
    for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < n; x += stride)
      dst[x] = Elem<F16>::one(src ? src[x] : 0.f);
  }
}

// ---- strided zero fill (gradients of shapes where nothing attends) ------------------------------
// out[b, h, s, :] = 0 for a (B, H, S, D) bf16 tensor with element strides st; one thread per
// 16-byte vector, grid.y over (b, h).
__global__ void __launch_bounds__(256) zero_rows_kernel(bf16_t* out, Strides st, int H, int S,
                                                        int D, int nbh) {
  const int d8 = D / 8;
  for (int bhi = blockIdx.y; bhi < nbh; bhi += gridDim.y) {
    bf16_t* base = out + (bhi / H) * st.b + (bhi % H) * st.h;
    for (int x = blockIdx.x * 256 + threadIdx.x; x < S * d8; x += gridDim.x * 256) {
      const int s = x / d8, c = x - s * d8;
      *reinterpret_cast<u32x4*>(base + s * st.s + c * 8) = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

// ---- NVFP4 QAT input quantisation ---------------------------------------------------------------
// Fake-quantise a contiguous bf16 tensor in groups of 16 consecutive elements: one thread per
// group (two 16-byte loads and stores), grid-stride over n_groups.
__global__ void __launch_bounds__(256) nvfp4_fake_quant_kernel(const bf16_t* x, bf16_t* y,
                                                               int64_t n_groups) {
  for (int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x; gi < n_groups;
       gi += (int64_t)gridDim.x * 256) {
    const u32x4* src = reinterpret_cast<const u32x4*>(x + gi * 16);
    const u32x4 w0 = src[0], w1 = src[1];
    float v[16];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = __uint_as_float(w0[e] << 16);
      v[2 * e + 1] = __uint_as_float(w0[e] & 0xffff0000u);
      v[8 + 2 * e] = __uint_as_float(w1[e] << 16);
      v[8 + 2 * e + 1] = __uint_as_float(w1[e] & 0xffff0000u);
    }
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) amax = fmaxf(amax, __builtin_fabsf(v[e]));
    const float scale = nvfp4_scale(amax);
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = scale > 0.f ? nvfp4_value(v[e], scale) : 0.f;
    u32x4* dst = reinterpret_cast<u32x4*>(y + gi * 16);
    dst[0] = u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                   pack_bf16x2(v[6], v[7])};
    dst[1] = u32x4{pack_bf16x2(v[8], v[9]), pack_bf16x2(v[10], v[11]), pack_bf16x2(v[12], v[13]),
                   pack_bf16x2(v[14], v[15])};
  }
}

}  // namespace sdpa
