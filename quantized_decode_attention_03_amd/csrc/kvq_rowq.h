// One head row's quantize-on-append, LPR = 4 or 8 lanes per row, shared by the
// append kernel (4) and the merge kernel's fused append of one token.
//
// What is computed follows the SAW-INT4 summary page (gist.science/ar/paper/
// 2604.19157), sections 2 and 3: rotate the row with the block-diagonal
// Hadamard matrix, then quantize it token-wise, asymmetric, to b bits (fp32
// minimum and scale (max - min) / (2^b - 1), codes rounded half to even), or
// round it to bf16 for 16-bit rows. Lane m of the row's lane group holds the
// contiguous channels [m*CPR, (m+1)*CPR), CPR = D/LPR.
//
// The Walsh-Hadamard butterflies of stride < CPR run in registers, the
// strides CPR and 2*CPR between the lanes of a quad through DPP quad
// permutations, and 4*CPR (8 lanes per row) by an xor-4 lane shuffle. They
// run in fp64: the +-1 sums of bf16 or fp32 inputs are
// exact there, so scaling by 1/sqrt(n) and rounding to fp32 reproduces the
// rotation's value (an exact matrix product, one rounding). Every multiply
// and add rounds on its own (no fused multiply-add), as the stored codes and
// the dequantized values are defined.
#pragma once

#include "kvq_device.h"

namespace kvq {

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const int lo = __builtin_amdgcn_mov_dpp(static_cast<int>(u), CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_mov_dpp(static_cast<int>(u >> 32), CTRL, 0xf, 0xf, false);
  return __builtin_bit_cast(double, (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) |
                                        static_cast<uint32_t>(lo));
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

template <int CPR, int MAXST>
__device__ __forceinline__ void butterflies_in_lane(double (&x)[CPR]) {
#pragma unroll
  for (int st = 1; st < MAXST; st <<= 1) {
#pragma unroll
    for (int j = 0; j < CPR; ++j) {
      if (!(j & st)) {
        const double u = x[j], v = x[j | st];
        x[j] = u + v;
        x[j | st] = u - v;
      }
    }
  }
}

// Unnormalised transform over blocks of n channels of the row; m is the lane's
// index in the row's lane group.
template <int CPR, int LPR = 4>
__device__ __forceinline__ void fwht_row_f64(double (&x)[CPR], int m, int n) {
  // blocks at least a lane wide (the common case) take every in-lane stride
  if (n >= CPR) {
    butterflies_in_lane<CPR, CPR>(x);
  } else {
#pragma unroll
    for (int st = 1; st < CPR; st <<= 1) {
      if (st < n) {
#pragma unroll
        for (int j = 0; j < CPR; ++j) {
          if (!(j & st)) {
            const double u = x[j], v = x[j | st];
            x[j] = u + v;
            x[j | st] = u - v;
          }
        }
      }
    }
  }
  // lower lane of a pair keeps x + y, upper keeps y - x: fma(+-1, x, y) rounds
  // once, exactly like the add or subtract
  if (CPR < n) {
    const double sgn = (m & 1) ? -1.0 : 1.0;
#pragma unroll
    for (int j = 0; j < CPR; ++j) x[j] = fma(sgn, x[j], dpp_f64<kDppQuadXor1>(x[j]));
  }
  if (2 * CPR < n) {
    const double sgn = (m & 2) ? -1.0 : 1.0;
#pragma unroll
    for (int j = 0; j < CPR; ++j) x[j] = fma(sgn, x[j], dpp_f64<kDppQuadXor2>(x[j]));
  }
  if constexpr (LPR == 8) {
    if (4 * CPR < n) {
      const double sgn = (m & 4) ? -1.0 : 1.0;
#pragma unroll
      for (int j = 0; j < CPR; ++j) x[j] = fma(sgn, x[j], __shfl_xor(x[j], 4, 64));
    }
  }
}

// The lane's CPR values of the rotated row: x (fp32 inputs) in, x' out.
template <int CPR, int LPR = 4>
__device__ __forceinline__ void rotate_row(float (&x)[CPR], int m, int n, double rs_n) {
  double xd[CPR];
#pragma unroll
  for (int j = 0; j < CPR; ++j) xd[j] = static_cast<double>(x[j]);
  fwht_row_f64<CPR, LPR>(xd, m, n);
#pragma unroll
  for (int j = 0; j < CPR; ++j) x[j] = static_cast<float>(xd[j] * rs_n);
}

// Codes of 8 consecutive values (already scaled to code units u) packed
// little-endian: BITS=4 -> one word, 2 -> 16 bits, 8 -> two words, 3 -> 24 bits.
// v_cvt_pk_u8_f32 rounds half to even and saturates to [0, 255]; u lies in
// [0, 2^b - 1 + 2^-22 (2^b - 1)], so every code is already in range.
template <int BITS>
__device__ __forceinline__ uint64_t pack8(const float* u) {
  if constexpr (BITS == 8) {
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      w0 = __builtin_amdgcn_cvt_pk_u8_f32(u[j], j, w0);
      w1 = __builtin_amdgcn_cvt_pk_u8_f32(u[4 + j], j, w1);
    }
    return w0 | (static_cast<uint64_t>(w1) << 32);
  } else if constexpr (BITS == 4 || BITS == 2) {
    uint32_t ev = 0, od = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ev = __builtin_amdgcn_cvt_pk_u8_f32(u[2 * j], j, ev);
      od = __builtin_amdgcn_cvt_pk_u8_f32(u[2 * j + 1], j, od);
    }
    if constexpr (BITS == 4) return ev | (od << 4);
    const uint32_t t = ev | (od << 2);              // byte k: c[2k] | c[2k+1] << 2
    const uint32_t v = (t | (t >> 4)) & 0x00ff00ffu; // byte 0: c0..c3, byte 2: c4..c7
    return (v & 0xffu) | ((v >> 8) & 0xff00u);
  } else {  // BITS == 3
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) w |= static_cast<uint32_t>(__builtin_rintf(u[j])) << (3 * j);
    return w;
  }
}

// A quantized row as the quad holds it: the row's {s, mn} (fp32, or the
// float16 pair of float16 metadata in meta_h) and the lane's packed codes.
template <int CPR>
struct RowQ {
  float s, mn;
  uint32_t meta_h;       // float16 metadata: s in the low half, mn in the high half
  uint64_t g[CPR / 8];   // packed codes of 8 channels each
  float u[CPR];          // the values in code units (x' - mn) / s, before rounding
};

// Quantize the rotated row x' (BITS < 16): row minimum and maximum over the
// row's lanes, then s, 1/s and the codes. With float16 metadata the minimum is
// rounded down and the scale up to float16, so the pair still bounds the row,
// and the codes are taken against the rounded pair.
template <int BITS, int CPR, int LPR = 4>
__device__ __forceinline__ void quantize_row(const float (&x)[CPR], bool meta16, RowQ<CPR>& q) {
#pragma clang fp contract(off)
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int j = 1; j < CPR; ++j) { mn = fminf(mn, x[j]); mx = fmaxf(mx, x[j]); }
  mn = fminf(mn, dpp_f32<kDppQuadXor1>(mn));
  mx = fmaxf(mx, dpp_f32<kDppQuadXor1>(mx));
  mn = fminf(mn, dpp_f32<kDppQuadXor2>(mn));
  mx = fmaxf(mx, dpp_f32<kDppQuadXor2>(mx));
  if constexpr (LPR == 8) {
    mn = fminf(mn, __shfl_xor(mn, 4, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 4, 64));
  }
  const float qmax = static_cast<float>((1 << BITS) - 1);
  float s = 0.f, inv = 0.f;
  uint32_t meta_h = 0;
  if (meta16) {
    const uint32_t mnh = f16_down(mn);
    mn = f16_to_f(mnh);
    const float rng = mx - mn;
    uint32_t sh = 0;
    if (rng > 0.f) {
      sh = f16_up(rng / qmax);
      s = f16_to_f(sh);
      inv = 1.f / s;
    }
    meta_h = sh | (mnh << 16);
  } else {
    const float rng = mx - mn;
    if (rng > 0.f) {
      s = rng / qmax;  // IEEE division (correctly rounded)
      inv = qmax / rng;
    }
  }
#pragma unroll
  for (int j = 0; j < CPR; ++j) q.u[j] = (x[j] - mn) * inv;
#pragma unroll
  for (int k = 0; k < CPR / 8; ++k) q.g[k] = pack8<BITS>(q.u + 8 * k);
  q.s = s;
  q.mn = mn;
  q.meta_h = meta_h;
}

// Store the lane's codes at dst (the row's codes start at dst - m*CPR*BITS/8;
// CPR 16 or 32) and, from the row's first lane, the row's metadata at meta
// (the slot's entry of the page's metadata array).
template <int BITS, int CPR>
__device__ __forceinline__ void store_row(const RowQ<CPR>& q, uint8_t* dst, uint8_t* meta, int m, bool meta16) {
  const uint64_t* g = q.g;
  if constexpr (BITS == 4) {
    if constexpr (CPR == 32)
      *reinterpret_cast<uint4*>(dst) = make_uint4(static_cast<uint32_t>(g[0]), static_cast<uint32_t>(g[1]),
                                                  static_cast<uint32_t>(g[2]), static_cast<uint32_t>(g[3]));
    else
      *reinterpret_cast<uint2*>(dst) = make_uint2(static_cast<uint32_t>(g[0]), static_cast<uint32_t>(g[1]));
  } else if constexpr (BITS == 2) {
    if constexpr (CPR == 32)
      *reinterpret_cast<uint2*>(dst) = make_uint2(static_cast<uint32_t>(g[0] | (g[1] << 16)),
                                                  static_cast<uint32_t>(g[2] | (g[3] << 16)));
    else
      *reinterpret_cast<uint32_t*>(dst) = static_cast<uint32_t>(g[0] | (g[1] << 16));
  } else if constexpr (BITS == 8) {
#pragma unroll
    for (int k = 0; k < CPR / 16; ++k)
      reinterpret_cast<uint4*>(dst)[k] =
          make_uint4(static_cast<uint32_t>(g[2 * k]), static_cast<uint32_t>(g[2 * k] >> 32),
                     static_cast<uint32_t>(g[2 * k + 1]), static_cast<uint32_t>(g[2 * k + 1] >> 32));
  } else {  // BITS == 3: 24 bits per group of 8
    if constexpr (CPR == 32) {  // 12 bytes at a 4-byte aligned offset
      uint32_t* w = reinterpret_cast<uint32_t*>(dst);
      w[0] = static_cast<uint32_t>(g[0] | (g[1] << 24));
      w[1] = static_cast<uint32_t>((g[1] >> 8) | (g[2] << 16));
      w[2] = static_cast<uint32_t>((g[2] >> 16) | (g[3] << 8));
    } else {  // 6 bytes at a 2-byte aligned offset
      uint16_t* w = reinterpret_cast<uint16_t*>(dst);
      w[0] = static_cast<uint16_t>(g[0]);
      w[1] = static_cast<uint16_t>((g[0] >> 16) | (g[1] << 8));
      w[2] = static_cast<uint16_t>(g[1] >> 8);
    }
  }
  if (m == 0) {
    if (meta16) *reinterpret_cast<uint32_t*>(meta) = q.meta_h;
    else *reinterpret_cast<float2*>(meta) = make_float2(q.s, q.mn);
  }
}

// A 16-bit row: the lane's CPR rotated values rounded half to even to bf16.
template <int CPR>
__device__ __forceinline__ void store_row_bf16(const float (&x)[CPR], uint8_t* dst) {
#pragma unroll
  for (int k = 0; k < CPR / 8; ++k) {
    uint4 w;
    w.x = f_to_bf16_rne(x[8 * k + 0]) | (f_to_bf16_rne(x[8 * k + 1]) << 16);
    w.y = f_to_bf16_rne(x[8 * k + 2]) | (f_to_bf16_rne(x[8 * k + 3]) << 16);
    w.z = f_to_bf16_rne(x[8 * k + 4]) | (f_to_bf16_rne(x[8 * k + 5]) << 16);
    w.w = f_to_bf16_rne(x[8 * k + 6]) | (f_to_bf16_rne(x[8 * k + 7]) << 16);
    reinterpret_cast<uint4*>(dst)[k] = w;
  }
}

}  // namespace kvq
