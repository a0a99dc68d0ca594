// Device-side helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Bitplane storage: per 16-row tile and 128-group a 2 KiB block.  Planes 2c
// and 2c + 1 form pair c at bytes 512 c .. 512 c + 511; within a pair row r
// takes 32 bytes at 32 r, and its quarter q (elements 32 q .. 32 q + 31 of
// the group) is 4 bytes of plane 2c followed by 4 bytes of plane 2c + 1, so
// one 8-byte load fetches both planes of a lane's 32-weight slice.  Bit i of
// a quarter's plane word is element 32 q + i.
constexpr int kBpBlock = 2048;
constexpr int kBpPair = 512;
__host__ __device__ constexpr int bp_byte(int p, int r, int j) {  // plane p, row r, byte j < 16
  return kBpPair * (p >> 1) + 32 * r + 8 * (j >> 2) + 4 * (p & 1) + (j & 3);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// fp16 bits -> fp32 (exact, subnormals included: v_cvt_f32_f16).
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// fp64 -> fp16 bits, round to nearest even, from the full 53-bit significand
// (a single rounding of the double value).
__device__ __forceinline__ uint32_t f64_to_f16_rne(double v) {
  uint64_t b = (uint64_t)__double_as_longlong(v);
  uint32_t sign = (uint32_t)(b >> 48) & 0x8000u;
  int ex = (int)((b >> 52) & 0x7FF);
  uint64_t man = b & ((1ull << 52) - 1);
  if (ex == 0x7FF) return sign | (man ? 0x7E00u : 0x7C00u);
  if (ex == 0) return sign;  // fp64 subnormals are far below fp16's range
  int e = ex - 1023;
  if (e > 15) return sign | 0x7C00u;
  if (e < -25) return sign;  // below half the smallest fp16 subnormal
  uint64_t full = man | (1ull << 52);
  int shift = (e >= -14) ? 42 : 42 + (-14 - e);  // <= 53
  uint64_t q = full >> shift;
  uint64_t rem = full & ((1ull << shift) - 1);
  uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (q & 1))) ++q;
  if (e >= -14) {
    int e16 = e + 15;
    if (q == (1ull << 11)) {
      q >>= 1;
      ++e16;
    }
    if (e16 >= 31) return sign | 0x7C00u;
    return sign | ((uint32_t)e16 << 10) | ((uint32_t)q & 0x3FFu);
  }
  return sign | (uint32_t)q;  // subnormal (q == 1024 encodes the min normal)
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// silu(g) = g / (1 + e^-g) with the hardware exp2 and reciprocal (about
// 2 ulp in fp32; the product is rounded to bf16 right after).  e^-g
// overflows to +inf for g < -88, giving g * 0 = -0.
__device__ __forceinline__ float silu_f32(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

// Bit-width of grouped pair p (flat index t*k + rank) of expert e under a
// bits mode: 1 per-pair array, 2 per-expert array, 3 rank rule (rank 1 ->
// 8 bits, ranks 2-4 -> 4, ranks 5-8 -> 2), otherwise 8.  Values clamp to
// [1, 8].
__device__ __forceinline__ int pair_bit_width(int p, int e, int k, int mode,
                                              const uint8_t* bits) {
  switch (mode) {
    case 1: return min(max((int)bits[p], 1), 8);
    case 2: return min(max((int)bits[e], 1), 8);
    case 3: {
      const int j = p % k;
      return j == 0 ? 8 : (j < 4 ? 4 : 2);
    }
    default: return 8;
  }
}

}  // namespace moe
