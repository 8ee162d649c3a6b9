// NVFP4 fake quantisation for the attention-QAT backward ("NVFP4 Attention QAT Backward",
// "Overview"): every group of 16 consecutive values is mapped to E2M1 values (0, 0.5, 1, 1.5, 2,
// 3, 4, 6 and their negatives) times one E4M3 scale, then dequantised:
//     scale = E4M3(amax / 6),   x^ = E2M1(x / scale) * scale   (0 where amax = 0)
// Both roundings are to nearest even; the divisions are correctly rounded fp32 divisions, so an
// x / scale that lands exactly on an E2M1 midpoint keeps the tie.  The scale saturates at 448
// (the largest finite E4M3 value), the E2M1 value at 6.  x^ has at most 6 significant bits and is
// exact in bf16.
#pragma once
#include "common.h"

namespace sdpa {

// E4M3 (4 exponent bits, bias 7, 3 mantissa bits, subnormal step 2^-9) nearest-even rounding of a
// non-negative fp32 value, saturating at 448.
__device__ __forceinline__ float e4m3_rne(float a) {
  if (!(a > 0.f)) return 0.f;
  if (a < 0.015625f) return __builtin_rintf(a * 512.f) * (1.f / 512.f);  // below 2^-6
  uint32_t u = __float_as_uint(a);
  u += 0x7FFFFu + ((u >> 20) & 1u);  // round away the 20 low mantissa bits, ties to even
  u &= 0xFFF00000u;
  const float r = __uint_as_float(u);
  return r < 448.f ? r : 448.f;
}

// E2M1 nearest-even rounding of a non-negative value (steps 0.5 below 2, 1 below 4, 2 above; the
// even integers of each step are the even codes), saturating at 6.
__device__ __forceinline__ float e2m1_rne(float y) {
  float r;
  if (y < 2.f) r = __builtin_rintf(y * 2.f) * 0.5f;
  else if (y < 4.f) r = __builtin_rintf(y);
  else r = __builtin_rintf(y * 0.5f) * 2.f;
  return r < 6.f ? r : 6.f;
}

// The dequantised value of x in a group with this scale (scale > 0).
__device__ __forceinline__ float nvfp4_value(float x, float scale) {
  return __builtin_copysignf(e2m1_rne(__builtin_fabsf(x) / scale), x) * scale;
}

__device__ __forceinline__ float nvfp4_scale(float amax) { return e4m3_rne(amax / 6.f); }

// The probability operand of GEMM3 (dV += fake(P)^T dO) from the fp32 P of one wave's 32 keys
// (lane l holds key l % 32 and 16 accumulator rows), computed through a wave-private LDS area `qs`
// of 4096 + 256 bytes so that each group's scale is computed once rather than in all 16 of its
// lanes: the wave's 32 x 32 fp32 P tile is written row major, lane L reduces row L / 2, key group
// L % 2 (its four 16-byte chunks read in a rotated order, which keeps every read instruction free
// of bank conflicts) and stores that group's scale; each lane then reads the scales of its 16
// rows.  Only this wave touches `qs`, and a wave's LDS instructions execute in order, so no
// barrier is needed.  Returns the packed bf16 words in the order of the plain P words.
__device__ __forceinline__ void nvfp4_p_pack_lds(const float (&pf)[16], uint32_t (&pb)[8],
                                                 char* qs, int lane) {
  const int g = lane >> 5, lc = lane & 31;
  float* tile = reinterpret_cast<float*>(qs);            // [32 rows][32 keys]
  float* sc = reinterpret_cast<float*>(qs + 4096);       // [2 groups][32 rows]
#pragma unroll
  for (int r = 0; r < 16; ++r) tile[acc_row<32>(r, g) * 32 + lc] = pf[r];
  asm volatile("" ::: "memory");
  {
    const int row = lane >> 1, grp = lane & 1;
    const floatx4* src = reinterpret_cast<const floatx4*>(tile + row * 32 + grp * 16);
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const floatx4 v = src[(c + row) & 3];
      amax = fmaxf(fmaxf(amax, fmaxf(v[0], v[1])), fmaxf(v[2], v[3]));
    }
    sc[grp * 32 + row] = nvfp4_scale(amax);
  }
  asm volatile("" ::: "memory");
  float scale[16];
  const floatx4* scr = reinterpret_cast<const floatx4*>(sc + (lc >> 4) * 32 + g * 4);
#pragma unroll
  for (int x = 0; x < 4; ++x) {  // registers 4x .. 4x+3: rows 8x + 4g + 0..3
    const floatx4 v = scr[2 * x];
    scale[4 * x] = v[0];
    scale[4 * x + 1] = v[1];
    scale[4 * x + 2] = v[2];
    scale[4 * x + 3] = v[3];
  }
  float pq[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) pq[r] = scale[r] > 0.f ? nvfp4_value(pf[r], scale[r]) : 0.f;
#pragma unroll
  for (int x = 0; x < 8; ++x) pb[x] = pack_bf16x2(pq[2 * x], pq[2 * x + 1]);
}

}  // namespace sdpa
