// Device-side helpers shared by the libkvq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBlockTokens = 16;
constexpr int kMetaBytes = 8;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bits_f(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t f_bits(float f) { return __float_as_uint(f); }

// bf16 <-> fp32 (bf16 is the upper half of an fp32).
__device__ __forceinline__ float bf16lo_to_f(uint32_t w) { return bits_f(w << 16); }
__device__ __forceinline__ float bf16hi_to_f(uint32_t w) { return bits_f(w & 0xffff0000u); }

// fp32 -> bf16 bits, round half to even (finite inputs).
__device__ __forceinline__ uint32_t f_to_bf16_rne(float f) {
  uint32_t u = f_bits(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Butterfly partner exchange inside a group of lanes (xor < 64).
__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }

// v_perm_b32: byte i of the result is selected by byte i of sel from the
// eight bytes {lo: b0..b3, hi: b4..b7}; selector 0x0c gives 0x00.
__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// (a & mask) | bias in one v_and_or_b32.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t bias) {
  return (a & mask) | bias;
}

// Packed fp16 add of a constant pair (v_pk_add_f16).
__device__ __forceinline__ uint32_t pk_add_h(uint32_t a, uint32_t c) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  h2 x = __builtin_bit_cast(h2, a);
  h2 y = __builtin_bit_cast(h2, c);
  return __builtin_bit_cast(uint32_t, x + y);
}

__device__ __forceinline__ uint32_t half_bits(_Float16 h) { return __builtin_bit_cast(uint16_t, h); }

// Wave-wide reductions (64 lanes) returning the result in every lane.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, shfl_xor(v, m));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += shfl_xor(v, m);
  return v;
}

}  // namespace kvq
