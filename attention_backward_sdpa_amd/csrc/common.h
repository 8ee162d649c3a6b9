// Shared device helpers for the gfx950 (CDNA4) attention-backward kernels: bf16 storage,
// MFMA fragment types and the lane layouts of the two bf16 matrix-core instructions used.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa {

typedef uint16_t bf16_t;  // bfloat16 bit pattern in memory
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2 __attribute__((ext_vector_type(2)));

// Element strides of one logical (B, H, S, D) tensor whose head dim is contiguous ("dense_flex"
// layouts of "SDPA Backward (SM120)", section "API Usage": any dense layout, addressed in place).
struct Strides {
  int64_t b, h, s;
};

constexpr float kLog2e = 1.4426950408889634f;

// Round-to-nearest-even float -> bf16 using the hardware convert (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16_t float_to_bf16(float x) {
  __bf16 h = (__bf16)x;
  return __builtin_bit_cast(bf16_t, h);
}

// The io element type ("Support surface": FP16 / BF16), 16-bit patterns in memory (bf16_t holds
// either).  Float -> element converts round to nearest even (v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32).
template <bool F16>
struct Elem {
  __device__ __forceinline__ static uint32_t pack2(float lo, float hi) {
    if constexpr (F16) {
      const half2 v = {(_Float16)lo, (_Float16)hi};
      return __builtin_bit_cast(uint32_t, v);
    } else {
      return pack_bf16x2(lo, hi);
    }
  }
  __device__ __forceinline__ static bf16_t one(float x) {
    if constexpr (F16) {
      return __builtin_bit_cast(bf16_t, (_Float16)x);
    } else {
      return float_to_bf16(x);
    }
  }
  // the element in bits 0..15 / 16..31 of a word
  __device__ __forceinline__ static float lo(uint32_t w) {
    if constexpr (F16) {
      return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
    } else {
      return __uint_as_float(w << 16);
    }
  }
  __device__ __forceinline__ static float hi(uint32_t w) {
    if constexpr (F16) {
      return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
    } else {
      return __uint_as_float(w & 0xffff0000u);
    }
  }
};

// ---------------------------------------------------------------------------------------------
// MFMA tiles.  MT = 32 selects v_mfma_f32_32x32x16_bf16, MT = 16 selects v_mfma_f32_16x16x32_bf16.
// Lane layouts (verified on the device):
//   A operand (bf16x8): lane l holds row (l % MT), k slots (l / MT) * 8 + 0..7
//   B operand (bf16x8): lane l holds col (l % MT), k slots (l / MT) * 8 + 0..7
//   C/D (MT*MT/64 floats): lane l holds col (l % MT); register r holds
//        row = (r / 4) * (4 * NG) + (l / MT) * 4 + (r % 4),   NG = 64 / MT
// Only a consistent k numbering between A and B matters for the product, which is what lets an
// accumulator tile be fed back as an operand whose contraction index is the accumulator's row.
template <int MT>
struct Mfma;

template <>
struct Mfma<32> {
  static constexpr int NG = 2;           // lane groups
  static constexpr int KT = 16;          // contraction length per instruction
  static constexpr int NACC = 16;        // accumulator floats per lane
  typedef floatx16 acc_t;
  __device__ __forceinline__ static acc_t mma(bf16x8 a, bf16x8 b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Mfma<16> {
  static constexpr int NG = 4;
  static constexpr int KT = 32;
  static constexpr int NACC = 4;
  typedef floatx4 acc_t;
  __device__ __forceinline__ static acc_t mma(bf16x8 a, bf16x8 b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

// 32x32x16 MFMA on bf16 or fp16 operands (v_mfma_f32_32x32x16_bf16 / _f16, same lane layouts);
// operands travel as 128-bit bf16x8 containers of 16-bit patterns either way.
template <bool F16>
struct Mfma32 : Mfma<32> {
  __device__ __forceinline__ static acc_t mma(bf16x8 a, bf16x8 b, acc_t c) {
    if constexpr (F16) {
      return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, a),
                                                    __builtin_bit_cast(half8, b), c, 0, 0, 0);
    } else {
      return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
  }
};

// 16x16x32 MFMA on bf16 or fp16 operands (v_mfma_f32_16x16x32_bf16 / _f16, same lane layouts).
template <bool F16>
struct Mfma16 : Mfma<16> {
  __device__ __forceinline__ static acc_t mma(bf16x8 a, bf16x8 b, acc_t c) {
    if constexpr (F16) {
      return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a),
                                                    __builtin_bit_cast(half8, b), c, 0, 0, 0);
    } else {
      return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
  }
};

// Row (within the tile) of accumulator register r for lane group g.
template <int MT>
__device__ __forceinline__ constexpr int acc_row(int r, int g) {
  return (r / 4) * (4 * (64 / MT)) + g * 4 + (r % 4);
}

// Workgroup barrier that orders LDS only: this wave's LDS accesses complete first (lgkmcnt(0)),
// while its global loads, stores and atomics keep draining (unlike __syncthreads, whose fence also
// waits for every outstanding global access).  Data brought in by LDS-DMA loads must be waited for
// explicitly (vmcnt) before it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ bf16x8 lds_read_b128(const char* base, int off) {
  return *reinterpret_cast<const bf16x8*>(base + off);
}

// ds_read_b64_tr_b16: within each block of 16 lanes, lane i returns column i of the 4 x 16 block
// whose row (r / 4), columns 4*(r % 4) .. +3 are addressed by lane r of the block.
__device__ __forceinline__ bf16x4 lds_read_tr(const char* base, int off) {
  shortx4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) shortx4*)(base + off));
  return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ bf16x8 concat(bf16x4 a, bf16x4 b) {
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

}  // namespace sdpa
