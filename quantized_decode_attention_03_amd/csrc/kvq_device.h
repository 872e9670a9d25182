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

// Loads of the paged cache's bytes, each read once per decode call, carry the
// non-temporal hint (streamed through the caches; KVQ_TUNE_NT=0 drops it). On
// MI355X it raises a plain 1 GiB read from 6.1 to 6.75 TB/s and the decode
// kernel's own load pattern to 6.4 TB/s (measured with kvq_measure_read_*).
#ifndef KVQ_TUNE_NT
#define KVQ_TUNE_NT 1
#endif
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 ld_cache_u4(const void* p) {
  if constexpr (KVQ_TUNE_NT) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
  } else {
    return *reinterpret_cast<const uint4*>(p);
  }
}
__device__ __forceinline__ uint2 ld_cache_u2(const void* p) {
  if constexpr (KVQ_TUNE_NT) {
    const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
    return make_uint2(v[0], v[1]);
  } else {
    return *reinterpret_cast<const uint2*>(p);
  }
}
__device__ __forceinline__ uint32_t ld_cache_u1(const void* p) {
  if constexpr (KVQ_TUNE_NT) return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
  else return *reinterpret_cast<const uint32_t*>(p);
}
__device__ __forceinline__ float2 ld_cache_f2(const void* p) {
  if constexpr (KVQ_TUNE_NT) {
    const f32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x2_t*>(p));
    return make_float2(v[0], v[1]);
  } else {
    return *reinterpret_cast<const float2*>(p);
  }
}

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

// float16 metadata: widening, and rounding down / up to a float16 value (the
// conversion rounds half to even; a result on the wrong side of x steps to
// the neighbouring float16, -0 and +0 stepping to the smallest subnormals).
__device__ __forceinline__ float f16_to_f(uint32_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
}
__device__ __forceinline__ uint32_t f16_down(float x) {
  const uint32_t h = half_bits(static_cast<_Float16>(x));
  if (!(f16_to_f(h) > x)) return h;
  return (h & 0x7fffu) == 0 ? 0x8001u : ((h & 0x8000u) ? h + 1 : h - 1);
}
__device__ __forceinline__ uint32_t f16_up(float x) {
  const uint32_t h = half_bits(static_cast<_Float16>(x));
  if (!(f16_to_f(h) < x)) return h;
  return (h & 0x7fffu) == 0 ? 0x0001u : ((h & 0x8000u) ? h - 1 : h + 1);
}

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

namespace kvq {

// ---------------------------------------------------------------------------
// DPP wave reductions (gfx9 row_shr / row_bcast patterns): the result lands in
// lane 63 and is read into a scalar. Each step is one VALU op with a DPP
// source, with no LDS round trip.
// ---------------------------------------------------------------------------
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

template <int CTRL, int ROWMASK>
__device__ __forceinline__ float dpp_or(float old, float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old), __builtin_bit_cast(int, v),
                                                               CTRL, ROWMASK, 0xf, false));
}

// old == src for max: lanes with no DPP source keep their own value, which lets
// the compiler fold each step into one v_max_f32 with a DPP operand.
__device__ __forceinline__ float wave_max_scalar(float x) {
  x = fmaxf(x, dpp_or<kDppRowShr1, 0xf>(x, x));
  x = fmaxf(x, dpp_or<kDppRowShr2, 0xf>(x, x));
  x = fmaxf(x, dpp_or<kDppRowShr4, 0xf>(x, x));
  x = fmaxf(x, dpp_or<kDppRowShr8, 0xf>(x, x));
  x = fmaxf(x, dpp_or<kDppRowBcast15, 0xa>(x, x));
  x = fmaxf(x, dpp_or<kDppRowBcast31, 0xc>(x, x));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

template <int CTRL, int ROWMASK>
__device__ __forceinline__ float dpp_zero(float v) {  // lanes with no source read 0
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWMASK, 0xf, true));
}

// Sums over the wave of four per-lane values at once: two exchanges (lanes
// l ^ 32, then l ^ 16) fold them into one register (rows of 16 lanes: value 0,
// 2, 1, 3, each summed over four lanes), a row reduction finishes, and each
// row's last lane holds its value's sum. (Plain lane shuffles: of the two
// results of the half-swap builtins, this compiler can return the first for
// both.)
__device__ __forceinline__ void wave_sum4(const float (&x)[4], float (&out)[4]) {
  const int lane = static_cast<int>(threadIdx.x) & 63;
  const bool h32 = (lane & 32) != 0, h16 = (lane & 16) != 0;
  const float a = (h32 ? x[1] : x[0]) + __shfl_xor(h32 ? x[0] : x[1], 32, 64);  // lanes <32: x0, else x1
  const float b = (h32 ? x[3] : x[2]) + __shfl_xor(h32 ? x[2] : x[3], 32, 64);  // lanes <32: x2, else x3
  float r = (h16 ? b : a) + __shfl_xor(h16 ? a : b, 16, 64);                     // rows: x0, x2, x1, x3
  r += dpp_zero<kDppRowShr1, 0xf>(r);
  r += dpp_zero<kDppRowShr2, 0xf>(r);
  r += dpp_zero<kDppRowShr4, 0xf>(r);
  r += dpp_zero<kDppRowShr8, 0xf>(r);
  const int ri = __builtin_bit_cast(int, r);
  out[0] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ri, 15));
  out[2] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ri, 31));
  out[1] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ri, 47));
  out[3] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ri, 63));
}

__device__ __forceinline__ float wave_sum_scalar(float x) {
  x += dpp_zero<kDppRowShr1, 0xf>(x);
  x += dpp_zero<kDppRowShr2, 0xf>(x);
  x += dpp_zero<kDppRowShr4, 0xf>(x);
  x += dpp_zero<kDppRowShr8, 0xf>(x);
  x += dpp_zero<kDppRowBcast15, 0xa>(x);
  x += dpp_zero<kDppRowBcast31, 0xc>(x);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

// The value of lane lane ^ X (X = 1, 2, 4 or 8: a partner in the same row of
// 16 lanes) by DPP: quad permutations for 1 and 2, a rotation of the row by 8
// for 8, and for 4 a shift up or down by 4 picked by the lane's bit 2.
constexpr int kDppQuadXor1 = 0xB1, kDppQuadXor2 = 0x4E, kDppRowShl4 = 0x104,
              kDppRowRor8 = 0x128;
template <int X>
__device__ __forceinline__ float xor_lanes16(float v, int lane) {
  const int i = __builtin_bit_cast(int, v);
  if constexpr (X == 1) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, i, kDppQuadXor1, 0xf, 0xf, false));
  } else if constexpr (X == 2) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, i, kDppQuadXor2, 0xf, 0xf, false));
  } else if constexpr (X == 4) {
    const int up = __builtin_amdgcn_update_dpp(0, i, kDppRowShl4, 0xf, 0xf, false);  // lane + 4
    const int dn = __builtin_amdgcn_update_dpp(0, i, kDppRowShr4, 0xf, 0xf, false);  // lane - 4
    return __builtin_bit_cast(float, (lane & 4) ? dn : up);
  } else {
    static_assert(X == 8, "partners inside a row of 16 lanes");
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, i, kDppRowRor8, 0xf, 0xf, false));
  }
}

// A constant materialised in a VGPR: lets v_and_or_b32 / v_perm_b32 take it
// as their vector operand (gfx9 VOP3 encodings take no literal constants and
// at most one scalar operand).
__device__ __forceinline__ uint32_t vconst(uint32_t c) {
  uint32_t r;
  asm("v_mov_b32 %0, %1" : "=v"(r) : "i"(c));
  return r;
}

}  // namespace kvq
