// Device-side helpers for the gfx950 kernels: vector types, MFMA wrappers, BF16 packing
// and typed loads of the [*, H, 128] inputs.
//
// MFMA lane layouts used throughout (64-wide wave, lane L, row/col r = L % 16, group
// grp = L / 16):
//   v_mfma_f32_16x16x32_bf16: A lane holds A[r][k(grp, e)], e = 0..7; B lane holds
//                             B[k(grp, e)][r]; C lane holds C[4 grp + j][r], j = 0..3.
//   v_mfma_f32_16x16x16_bf16: the same with 4 k values per lane (k(grp, j)).
// Only the C mapping and the row/column = L % 16 rule matter for correctness; the k
// assignment is whatever the hardware uses, identically for A and B, because every
// operand pair below is built from the same (grp, e) index.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16(i16x4 a, i16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Round-to-nearest-even FP32 -> BF16 (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ i16x4 pack4(f32x4 x) {
  bf16x4 b = __builtin_convertvector(x, bf16x4);
  return __builtin_bit_cast(i16x4, b);
}

__device__ __forceinline__ bf16x8 pack8(f32x4 lo, f32x4 hi) {
  bf16x4 a = __builtin_convertvector(lo, bf16x4);
  bf16x4 b = __builtin_convertvector(hi, bf16x4);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ float bf16_bits_to_float(unsigned short u) {
  return __uint_as_float(static_cast<unsigned int>(u) << 16);
}

__device__ __forceinline__ unsigned short float_to_bf16_bits(float x) {
  __bf16 b = static_cast<__bf16>(x);
  return __builtin_bit_cast(unsigned short, b);
}

// Load 8 consecutive elements starting at element index `idx` (16-byte aligned for
// BF16, 32-byte aligned for FP32) and widen to float.
template <bool BF16>
__device__ __forceinline__ void load8(const void* base, int64_t idx, float* out) {
  if constexpr (BF16) {
    u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const unsigned short*>(base) + idx);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + idx);
    f32x4 a = p[0], b = p[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[i] = a[i];
      out[4 + i] = b[i];
    }
  }
}

template <bool BF16>
__device__ __forceinline__ float load1(const void* base, int64_t idx) {
  if constexpr (BF16) {
    return bf16_bits_to_float(static_cast<const unsigned short*>(base)[idx]);
  } else {
    return static_cast<const float*>(base)[idx];
  }
}

// Load 4 consecutive elements (8-byte aligned BF16 / 16-byte aligned FP32) as float.
template <bool BF16>
__device__ __forceinline__ f32x4 load4(const void* base, int64_t idx) {
  if constexpr (BF16) {
    u32x2 w = *reinterpret_cast<const u32x2*>(static_cast<const unsigned short*>(base) + idx);
    f32x4 r;
    r[0] = __uint_as_float(w[0] << 16);
    r[1] = __uint_as_float(w[0] & 0xffff0000u);
    r[2] = __uint_as_float(w[1] << 16);
    r[3] = __uint_as_float(w[1] & 0xffff0000u);
    return r;
  } else {
    return *reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + idx);
  }
}

// Store 4 consecutive elements, rounding to BF16 when asked.
template <bool BF16>
__device__ __forceinline__ void store4(void* base, int64_t idx, f32x4 x) {
  if constexpr (BF16) {
    *reinterpret_cast<i16x4*>(static_cast<unsigned short*>(base) + idx) = pack4(x);
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(base) + idx) = x;
  }
}

// The logistic function with the hardware reciprocal (v_rcp_f32, about 1 ulp) rather than
// an IEEE division (a dozen instructions): the in-kernel gate evaluates it for every
// channel of every token.
__device__ __forceinline__ float sigmoidf_(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

}  // namespace kda
