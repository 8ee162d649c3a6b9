// Bandwidth-bound kernels of the attention-backward chain ("SDPA Backward (SM120)", section
// "The kernel chain"): the row-dot preprocess (delta = rowsum(O * dO), fused with zeroing the fp32
// dQ accumulator), the dQ convert (fp32 accumulator -> bf16, times the softmax scale) and the
// fixed-order GQA dK/dV group reduction ("GQA/MQA group reduction").
#pragma once
#include "common.h"

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
  const float* lse;
  float* stats;              // (B*Hq, sq_pad, 2)
  float* dq_accum;           // (B*Hq, Sq, Dqk) or null
  const int* seq_q_lens;
  int Hq, Sq, sq_pad, Dqk;
  int zero_rows;
};

template <int DV>
__global__ void __launch_bounds__(256) preprocess_kernel(PreParams p) {
  constexpr int BR = 32;
  constexpr int LPR = DV / 8;              // lanes per row for the row dot
  constexpr int RPP = 256 / LPR;           // rows per pass
  const int tid = threadIdx.x;
  const int nt = p.sq_pad / BR;
  const int64_t bh = blockIdx.x / nt;
  const int i = blockIdx.x % nt;
  const int q0 = i * BR;
  const int b = (int)(bh / p.Hq);
  const int Lq = p.seq_q_lens ? min(max(p.seq_q_lens[b], 0), p.Sq) : p.Sq;

  for (int r0 = 0; r0 < BR; r0 += RPP) {
    const int r = r0 + tid / LPR, sub = tid % LPR, s = q0 + r;
    const bool live = s < Lq;
    const int64_t row = bh * p.Sq + s;
    float acc = 0.f;
    if (live) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(p.o + row * DV + sub * 8);
      const u32x4 c = *reinterpret_cast<const u32x4*>(p.dO + row * DV + sub * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc += __uint_as_float(a[e] << 16) * __uint_as_float(c[e] << 16);
        acc += __uint_as_float(a[e] & 0xffff0000u) * __uint_as_float(c[e] & 0xffff0000u);
      }
    }
#pragma unroll
    for (int off = LPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, LPR);
    if (sub == 0) {
      const float l = live ? p.lse[row] : -INFINITY;
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
  const float* acc;          // (B*Hq, Sq, Dqk)
  bf16_t* dq;                // (B*Hq, Sq, Dqk)
  const int* seq_q_lens;
  int Hq, Sq;
  float scale;
};

template <int DQK>
__global__ void __launch_bounds__(256) dq_convert_kernel(ConvertParams p) {
  constexpr int V = DQK / 8;  // 8-element vectors per row
  const int nt = (p.Sq + 31) / 32;
  const int64_t bh = blockIdx.x / nt;
  const int q0 = (int)(blockIdx.x % nt) * 32;
  const int b = (int)(bh / p.Hq);
  const int Lq = p.seq_q_lens ? min(max(p.seq_q_lens[b], 0), p.Sq) : p.Sq;
  for (int v = threadIdx.x; v < 32 * V; v += 256) {
    const int s = q0 + v / V;
    if (s >= p.Sq) break;
    const int64_t x = (bh * p.Sq + s) * V + v % V;
    u32x4 out = u32x4{0u, 0u, 0u, 0u};
    if (s < Lq) {
      const floatx4 a = reinterpret_cast<const floatx4*>(p.acc)[2 * x];
      const floatx4 c = reinterpret_cast<const floatx4*>(p.acc)[2 * x + 1];
      const float k = p.scale;
      out = u32x4{pack_bf16x2(a[0] * k, a[1] * k), pack_bf16x2(a[2] * k, a[3] * k),
                  pack_bf16x2(c[0] * k, c[1] * k), pack_bf16x2(c[2] * k, c[3] * k)};
    }
    reinterpret_cast<u32x4*>(p.dq)[x] = out;
  }
}

// ---- GQA reduce ---------------------------------------------------------------------------------
// out[b, kvh, s, :] = bf16( sum_{g = 0 .. group-1} ws[b, kvh*group + g, s, :] ), summed in fp32
// in ascending g.  One thread per 16-byte output vector; dK and dV handled by one launch
// (vectors [0, nk8) are dK, [nk8, nk8 + nv8) are dV).
struct ReduceParams {
  const bf16_t* dk_ws;
  const bf16_t* dv_ws;
  bf16_t* dk;
  bf16_t* dv;
  int64_t nk8, nv8;          // output 8-element vectors of dK and dV
  int64_t head_k8, head_v8;  // 8-element vectors per head (Skv * D / 8)
  int group;
};

__global__ void __launch_bounds__(256) gqa_reduce_kernel(ReduceParams p) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < p.nk8 + p.nv8; x += stride) {
    const bool isk = x < p.nk8;
    const int64_t y = isk ? x : x - p.nk8;
    const int64_t per = isk ? p.head_k8 : p.head_v8;
    const int64_t kvhead = y / per, within = y % per;  // kvhead = b * Hkv + kvh
    const u32x4* src = reinterpret_cast<const u32x4*>(isk ? p.dk_ws : p.dv_ws) +
                       (kvhead * p.group) * per + within;
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int gi = 0; gi < p.group; ++gi) {
      const u32x4 v = src[(int64_t)gi * per];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s[2 * e] += __uint_as_float(v[e] << 16);
        s[2 * e + 1] += __uint_as_float(v[e] & 0xffff0000u);
      }
    }
    reinterpret_cast<u32x4*>(isk ? p.dk : p.dv)[y] =
        u32x4{pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3]), pack_bf16x2(s[4], s[5]),
              pack_bf16x2(s[6], s[7])};
  }
}

}  // namespace sdpa
