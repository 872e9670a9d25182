// Fused quantized decode attention over the paged INT-b KV cache.
//
// What is computed: o = softmax(q K^T / sqrt(d)) V for one query per q-head,
// over the dequantized cache. The cache stores rotated rows (x' = R x, R the
// block-diagonal Hadamard matrix), so the query is rotated once (q' = R q),
// scores are taken against the stored keys directly, and the output is
// un-rotated once per head (o = R^T o'), as the SAW-INT4 summary page
// (gist.science/ar/paper/2604.19157), section 3, describes: rotation and
// quantization are folded into reading the cache, with no separate pass.
// Tokens may sit in any order and in several precision segments
// (LogQuant summary page, 2503.19950, Methodology section 4: A.V = A_P.V_P).
//
// Work decomposition (split-K / flash-decoding): one wave per (sequence, KV
// head, split of pages). A split walks its pages four at a time (64 tokens):
//  * QK on the matrix cores. 2-, 4- and 8-bit keys: v_mfma_i32_16x16x64_i8
//    with A = the G query rows of this KV head, each as three signed-byte
//    digits of a 24-bit fixed-point number (rows 4h..4h+2), and B = the
//    page's key codes as bytes (a mask and a shift per four codes); the int32
//    sums are exact. 3-bit keys, bf16 keys and keys per channel:
//    v_mfma_f32_16x16x32_f16 with A = hi and lo fp16 halves of q' (rows 0-3
//    and 4-7, so the product carries ~22 bits of q) and B = exact fp16 numbers
//    1024 + sigma*c made by one v_and_or_b32 per pair, the constant removed
//    afterwards.
//  * The four pages' score tiles are packed into one dense set of four
//    registers (lane = token, register = query head) with
//    v_permlane16_swap / v_permlane32_swap.
//  * Online softmax in log2 units on that dense layout; the weights
//    w = p * scale are split into fp16 hi/lo halves and transposed through
//    LDS into the A operand of the PV product.
//  * PV on the matrix cores: v_mfma_f32_16x16x32_f16, A = weights (hi rows
//    0..G-1, lo rows 4..4+G-1), B = value codes as exact fp16 numbers
//    1024 + sigma*c (one v_and_or_b32 per pair), centred exactly by one
//    packed fp16 add, 32 tokens per instruction. (Leaving the offset in and
//    removing it with a second MFMA against a constant costs the same time and
//    loses precision: the matrix core rounds sums carrying 1024 * sum(w).) The
//    min term sum_t p_t (mn_t + 2^(b-1) s_t) is accumulated per head on the
//    vector ALU and added at the end.
// Each split writes (running max, sum of p, o') to the workspace; a second
// kernel merges the splits of all segments and applies R^T.
#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_rowq.h"

#include <algorithm>
#include <cmath>

namespace kvq {

namespace {


__device__ __forceinline__ float4_t mfma_f16(u32x4_t a, u32x4_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ float4_t mfma_bf16(u32x4_t a, u32x4_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
// 16x16 tile, 64 products per element: A and B 16 signed bytes a lane, exact int32 sums
__device__ __forceinline__ i32x4_t mfma_i8(u32x4_t a, u32x4_t b, i32x4_t c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4_t, a), __builtin_bit_cast(i32x4_t, b), c,
                                               0, 0, 0);
}
template <bool BF16>
__device__ __forceinline__ float4_t mfma(u32x4_t a, u32x4_t b, float4_t c) {
  if constexpr (BF16) return mfma_bf16(a, b, c);
  else return mfma_f16(a, b, c);
}

template <int S>
__device__ __forceinline__ uint32_t shl_signed(uint32_t w) {
  if constexpr (S >= 0) return w << S;
  else return w >> (-S);
}

// ---------------------------------------------------------------------------
// Key formats. A lane (token t = lane % 16, quarter g4 = lane / 16) holds the
// quarter [g4*D/4, (g4+1)*D/4) of token t's stored row; chunk c of the QK
// product takes 8 of those channels as the lane's 8 K-slots. channel(c, e) is
// the channel (relative to the quarter) in K-slot e of chunk c; sigma is the
// power of two each code is scaled by inside its fp16 number 1024 + sigma*c.
// base is the constant part of the B value (1024, or -kCentre*sigma for a
// centred format), whose product with the query is removed per head.
// ---------------------------------------------------------------------------
template <int KB, int D> struct KFmt;

template <int D> struct KFmt<4, D> {
  static constexpr int kWords = D / 32;  // quarter = D/8 bytes
  static constexpr bool bf16 = false;
  // Centred: one packed add turns 1024 + sigma*c into sigma*(c - 8), so the
  // products carry no 1024 offset (at sigma 1 that offset would be about 136x
  // the signal and the matrix core's fp32 sums would lose ~7 bits to it).
  static constexpr float kCentre = 8.f;
  // nibbles 0 and 2 sit at bits 0-3 of their half (sigma 1), nibbles 1 and 3 at
  // bits 4-7 (sigma 16); both reach their place with at most one shift
  __device__ static float sigma(int /*c*/, int e) { return (e & 2) ? 16.f : 1.f; }
  __device__ static float base(int c, int e) { return -kCentre * sigma(c, e); }
  __device__ static int channel(int c, int e) {
    constexpr int rel[8] = {0, 4, 1, 5, 2, 6, 3, 7};
    return 8 * c + rel[e];
  }
  __device__ static u32x4_t unpack(const uint32_t (&w)[kWords], int c, uint32_t bias) {
    const uint32_t x = w[c], x8 = x >> 8;
    constexpr uint32_t c1 = 0xe408e408u, c16 = 0xe480e480u;  // fp16 pairs -(1024 + 8), -(1024 + 128)
    u32x4_t r;
    r[0] = pk_add_h(and_or(x, 0x000f000fu, bias), c1);
    r[1] = pk_add_h(and_or(x, 0x00f000f0u, bias), c16);
    r[2] = pk_add_h(and_or(x8, 0x000f000fu, bias), c1);
    r[3] = pk_add_h(and_or(x8, 0x00f000f0u, bias), c16);
    return r;
  }
};

template <int D> struct KFmt<2, D> {
  static constexpr int kWords = D / 64;  // quarter = D/16 bytes
  static constexpr bool bf16 = false;
  __device__ static float sigma(int, int) { return 256.f; }
  static constexpr float kCentre = 0.f;
  __device__ static float base(int, int) { return 1024.f; }
  __device__ static int channel(int c, int e) {
    const int m = c >> 1, k = 4 * (c & 1) + (e >> 1);
    return 16 * m + ((e & 1) ? 8 : 0) + k;
  }
  template <int K>
  __device__ static uint32_t pair(uint32_t x, uint32_t b) { return and_or(shl_signed<8 - 2 * K>(x), 0x03000300u, b); }
  __device__ static u32x4_t unpack(const uint32_t (&w)[kWords], int c, uint32_t b) {
    const uint32_t x = w[c >> 1];
    u32x4_t r;
    if (c & 1) { r[0] = pair<4>(x, b); r[1] = pair<5>(x, b); r[2] = pair<6>(x, b); r[3] = pair<7>(x, b); }
    else       { r[0] = pair<0>(x, b); r[1] = pair<1>(x, b); r[2] = pair<2>(x, b); r[3] = pair<3>(x, b); }
    return r;
  }
};

template <int D> struct KFmt<8, D> {
  static constexpr int kWords = D / 16;  // quarter = D/4 bytes
  static constexpr bool bf16 = false;
  __device__ static float sigma(int, int) { return 1.f; }
  static constexpr float kCentre = 0.f;
  __device__ static float base(int, int) { return 1024.f; }
  __device__ static int channel(int c, int e) {
    constexpr int rel[8] = {0, 2, 1, 3, 4, 6, 5, 7};
    return 8 * c + rel[e];
  }
  __device__ static u32x4_t unpack(const uint32_t (&w)[kWords], int c, uint32_t b) {
    const uint32_t x0 = w[2 * c], x1 = w[2 * c + 1];
    u32x4_t r;
    r[0] = and_or(x0, 0x00ff00ffu, b);
    r[1] = and_or(x0 >> 8, 0x00ff00ffu, b);
    r[2] = and_or(x1, 0x00ff00ffu, b);
    r[3] = and_or(x1 >> 8, 0x00ff00ffu, b);
    return r;
  }
};

template <int D> struct KFmt<3, D> {
  static constexpr int kWords = (3 * D / 32 + 3) / 4;  // quarter = 3D/32 bytes (12 or 6)
  static constexpr bool bf16 = false;
  static constexpr float kCentre = 0.f;
  // Chunk c holds code pairs 4c..4c+3 of the quarter's bit stream. A pair
  // (k, k + 5) lies 15 bits apart: one shift of the stream puts code k at bits
  // 7-9 of the low half (sigma 128) and code k + 5 at bits 6-8 of the high half
  // (sigma 64), and one and-or makes both fp16 values 1024 + sigma*c. Pairs
  // 0..kFast-1 are such pairs, in blocks of ten codes; the rest (codes 30, 31
  // at head_dim 128; 11, 12 and 13, 14 at 64) take each code apart (sigma 128).
  static constexpr int kFast = D == 128 ? 15 : 6;
  __device__ static constexpr bool fast(int p) { return p < kFast; }
  __device__ static constexpr int code_of(int p, int j) {
    return fast(p) ? 10 * (p / 5) + p % 5 + 5 * j : (D == 128 ? 30 + j : 11 + 2 * (p - 6) + j);
  }
  __device__ static float sigma(int c, int e) { return fast(4 * c + e / 2) && (e & 1) ? 64.f : 128.f; }
  __device__ static float base(int, int) { return 1024.f; }
  __device__ static int channel(int c, int e) { return code_of(4 * c + e / 2, e & 1); }
  template <int K>
  __device__ static uint32_t code(const uint32_t (&w)[kWords]) {
    constexpr int bit = 3 * K, i = bit / 32, sh = bit % 32;
    if constexpr (sh <= 29) return (w[i] >> sh) & 7u;
    else return ((w[i] >> sh) | (w[i + 1] << (32 - sh))) & 7u;
  }
  template <int P>
  __device__ static uint32_t pair(const uint32_t (&w)[kWords], uint32_t b) {
    if constexpr (fast(P)) {
      constexpr int s = 3 * code_of(P, 0) - 7;  // stream bit that lands at bit 0
      uint32_t x;
      if constexpr (s < 0) {
        x = w[0] << (-s);
      } else {
        constexpr int i = s / 32, sh = s % 32;
        const uint32_t hi = i + 1 < kWords ? w[i + 1 < kWords ? i + 1 : i] : 0u;
        x = sh ? __builtin_amdgcn_alignbit(hi, w[i], sh) : w[i];
      }
      return and_or(x, 0x01c00380u, b);
    } else {
      return (((code<code_of(P, 1)>(w) << 16) | code<code_of(P, 0)>(w)) << 7) | b;
    }
  }
  template <int C>
  __device__ static u32x4_t unpack_c(const uint32_t (&w)[kWords], uint32_t b) {
    return u32x4_t{pair<4 * C>(w, b), pair<4 * C + 1>(w, b), pair<4 * C + 2>(w, b), pair<4 * C + 3>(w, b)};
  }
  __device__ static u32x4_t unpack(const uint32_t (&w)[kWords], int c, uint32_t b) {
    if constexpr (D == 128) {
      switch (c) {
        case 0: return unpack_c<0>(w, b);
        case 1: return unpack_c<1>(w, b);
        case 2: return unpack_c<2>(w, b);
        default: return unpack_c<3>(w, b);
      }
    } else {
      return c == 0 ? unpack_c<0>(w, b) : unpack_c<1>(w, b);
    }
  }
};

template <int D> struct KFmt<16, D> {
  static constexpr int kWords = D / 8;  // quarter = D/2 bytes of bf16
  static constexpr bool bf16 = true;
  __device__ static float sigma(int, int) { return 1.f; }
  static constexpr float kCentre = 0.f;
  __device__ static float base(int, int) { return 0.f; }
  __device__ static int channel(int c, int e) { return 8 * c + e; }
  __device__ static u32x4_t unpack(const uint32_t (&w)[kWords], int c, uint32_t) {
    u32x4_t r;
    r[0] = w[4 * c]; r[1] = w[4 * c + 1]; r[2] = w[4 * c + 2]; r[3] = w[4 * c + 3];
    return r;
  }
};

// Integer scores for 2-, 4- and 8-bit keys: the codes become bytes (one mask,
// and a shift for all but the first field of a word) and meet the query, held
// as three signed-byte digits of a 24-bit fixed-point number, in the int8
// matrix core, whose int32 sums are exact. Against the fp16 path this halves
// the QK matrix instructions (64 channels per step) and the unpacking, and
// needs no centring: no large offset enters a rounded sum. The score is then
// s * sum(q~ c) + mn * sum(q~), as for the other formats without centring
// (8-bit codes, above the signed byte range, enter as c - 128: kOff = 128).
// channel(s, p) is the channel (relative to the lane's quarter) in byte p of
// step s; A and B take the same order, which the sums do not depend on.
#ifndef KVQ_TUNE_KI8
#define KVQ_TUNE_KI8 1
#endif
template <int KB, int D>
struct KI8 {
  static constexpr bool on = KVQ_TUNE_KI8 && (KB == 2 || KB == 4 || KB == 8);
  static constexpr int kSteps = D / 64;  // 16 channels of the quarter per step
  static constexpr float kOff = KB == 8 ? 128.f : 0.f;
  __device__ static constexpr int channel(int s, int p) {
    const int d = p >> 2, q = p & 3;
    if constexpr (KB == 2) return 16 * s + 4 * q + d;                     // word s, field 4q + d
    else if constexpr (KB == 4) return 8 * (2 * s + (d >> 1)) + 2 * q + (d & 1);  // word 2s + d/2, nibble 2q + d%2
    else return 16 * s + 4 * d + q;                                       // word 4s + d, byte q
  }
  __device__ static u32x4_t bytes(const uint32_t (&w)[KFmt<KB, D>::kWords], int s) {
    u32x4_t r;
    if constexpr (KB == 2) {
      const uint32_t x = w[s];
      r[0] = x & 0x03030303u;
      r[1] = (x >> 2) & 0x03030303u;
      r[2] = (x >> 4) & 0x03030303u;
      r[3] = (x >> 6) & 0x03030303u;
    } else if constexpr (KB == 4) {
      r[0] = w[2 * s] & 0x0f0f0f0fu;
      r[1] = (w[2 * s] >> 4) & 0x0f0f0f0fu;
      r[2] = w[2 * s + 1] & 0x0f0f0f0fu;
      r[3] = (w[2 * s + 1] >> 4) & 0x0f0f0f0fu;
    } else {
#pragma unroll
      for (int d = 0; d < 4; ++d) r[d] = w[4 * s + d] ^ 0x80808080u;
    }
    return r;
  }
};

// Load the lane's quarter row of key codes (kWords dwords).
template <int KB, int D>
__device__ __forceinline__ void load_kquarter(const uint8_t* p, uint32_t (&w)[KFmt<KB, D>::kWords]) {
  constexpr int kW = KFmt<KB, D>::kWords;
  if constexpr (KB == 3 && D == 64) {  // 6 bytes, 2-byte aligned
    const uint16_t* s = reinterpret_cast<const uint16_t*>(p);
    w[0] = s[0] | (static_cast<uint32_t>(s[1]) << 16);
    w[1] = s[2];
  } else if constexpr (kW == 1) {
    w[0] = ld_cache_u1(p);
  } else if constexpr (kW == 2) {
    const uint2 v = ld_cache_u2(p);
    w[0] = v.x; w[1] = v.y;
  } else if constexpr (kW == 3) {
    w[0] = ld_cache_u1(p); w[1] = ld_cache_u1(p + 4); w[2] = ld_cache_u1(p + 8);
  } else {
#pragma unroll
    for (int j = 0; j < kW; j += 4) {
      const uint4 v = ld_cache_u4(p + 4 * j);
      w[j] = v.x; w[j + 1] = v.y; w[j + 2] = v.z; w[j + 3] = v.w;
    }
  }
}

// ---------------------------------------------------------------------------
// Value formats. A lane (column n = lane % 16, token group g4 = lane / 16)
// owns the channels [n*D/16, (n+1)*D/16) of 8 tokens; chunk c of the PV
// product is output channel n*D/16 + c. Each fp16 pair holds two tokens'
// centred codes sigma_c * (code - 2^(b-1)), exact.
// ---------------------------------------------------------------------------
template <int VB, int D> struct VFmt;

// Bytes each lane reads from one token row, and where.
template <int VB, int D>
__device__ __forceinline__ int v_lane_offset(int n) {
  constexpr int bits_per_lane = VB * D / 16;
  if constexpr (VB == 3) return (bits_per_lane * n) / 8;  // byte holding the first bit (an unaligned dword load)
  else if constexpr (bits_per_lane >= 32) return n * bits_per_lane / 8;
  else return ((bits_per_lane * n) / 32) * 4;  // sub-dword ranges: load the containing dword
}

template <int VB, int D> struct VRaw {
  static constexpr int bits_per_lane = VB * D / 16;
  static constexpr int kWords = bits_per_lane >= 32 ? bits_per_lane / 32 : 1;
};

template <int VB, int D>
__device__ __forceinline__ void load_vtoken(const uint8_t* p, uint32_t* w) {
  constexpr int kW = VRaw<VB, D>::kWords;
  if constexpr (VB == 3) {
    // 24 (or 12) bits from a byte offset: one dword load at that byte (the
    // target reads unaligned dwords from global memory); the dword's last
    // byte belongs to the next lane or row, still inside the area
    __builtin_memcpy(&w[0], p, 4);
  } else if constexpr (kW == 1) {
    w[0] = ld_cache_u1(p);
  } else if constexpr (kW == 2) {
    const uint2 v = ld_cache_u2(p);
    w[0] = v.x; w[1] = v.y;
  } else {
    const uint4 v = ld_cache_u4(p);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  }
}

// Per token pair (t0 in the low fp16, t1 in the high fp16), value of chunk c.
template <int VB, int D> struct VFmt {
  static constexpr int kW = VRaw<VB, D>::kWords;
  static constexpr bool bf16 = VB == 16;
  static constexpr int kChunks = D / 16;
  // Bring the lane's field of each token into the low 16 bits (per half) of a
  // combined word, or for 3-bit into a 24-bit aligned value per token.
  __device__ static float sigma(int c) {
    if constexpr (VB == 4) return (c & 1) ? 16.f : 1.f;
    else if constexpr (VB == 2) return D == 128 ? static_cast<float>(1 << (2 * (c < 5 ? c : c - 5)))
                                                 : static_cast<float>(1 << (2 * c));
    else if constexpr (VB == 3) return 128.f;
    else return 1.f;
  }
  // Centring: one packed fp16 add of -(1024 + 2^(b-1) sigma_c) per pair turns
  // 1024 + sigma_c c into the exact centred value sigma_c (c - 2^(b-1)), so
  // the accumulator carries sigma_c * sum_t w_t (c_t - 2^(b-1)) and no offset.
  // Chunks with equal sigma share one constant (a class).
  __device__ static constexpr int cls(int c) {
    return VB == 4 ? (c & 1) : VB == 2 ? (D == 128 ? (c < 5 ? c : c - 5) : c) : 0;
  }
  static constexpr uint32_t center_bits(int k) {  // fp16 pair of -(1024 + 2^(b-1) sigma)
    const int sg = VB == 4 ? (k ? 16 : 1) : VB == 2 ? (1 << (2 * k)) : VB == 3 ? 128 : 1;
    const uint32_t h = 0xe400u | static_cast<uint32_t>((1 << (VB - 1)) * sg);
    return h | (h << 16);
  }
};

// Produce the B operand (4 dwords = 8 tokens) of value chunk c for one lane.
// raw[e][*] are the 8 tokens' words; n is the lane's column.
template <int VB, int D>
__device__ __forceinline__ u32x4_t v_operand(const uint32_t (&raw)[8][VRaw<VB, D>::kWords], int n, int c,
                                             uint32_t bias) {
  u32x4_t r;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const uint32_t* a = raw[2 * v];
    const uint32_t* b = raw[2 * v + 1];
    uint32_t out;
    if constexpr (VB == 4) {
      // channels [n*D/16, ...): D=128: the whole dword n; D=64: half (n & 1) of dword n/2
      uint32_t sel;
      if constexpr (D == 128) sel = c < 4 ? 0x05040100u : 0x07060302u;
      else sel = (n & 1) ? 0x07060302u : 0x05040100u;
      uint32_t x = perm_b32(b[0], a[0], sel);
      const int cc = D == 128 ? (c & 3) : c;
      if (cc >= 2) x >>= 8;
      const uint32_t mask = (cc & 1) ? 0x00f000f0u : 0x000f000fu;
      out = and_or(x, mask, bias);
      out = pk_add_h(out, VFmt<VB, D>::center_bits(VFmt<VB, D>::cls(c)));
    } else if constexpr (VB == 2) {
      uint32_t x;
      int cc;
      if constexpr (D == 128) {
        x = perm_b32(b[0], a[0], (n & 1) ? 0x07060302u : 0x05040100u);
        cc = c;
        if (c >= 5) { x >>= 10; cc = c - 5; }
      } else {
        const uint32_t k = n & 3;
        x = perm_b32(b[0], a[0], 0x0c000c00u | ((4 + k) << 16) | k);
        cc = c;
      }
      out = and_or(x, 0x00030003u << (2 * cc), bias);
      out = pk_add_h(out, VFmt<VB, D>::center_bits(VFmt<VB, D>::cls(c)));
    } else if constexpr (VB == 8) {
      const int word = D == 128 ? (c >> 2) : 0;
      const uint32_t k = c & 3;
      const uint32_t x = perm_b32(b[word], a[word], 0x0c000c00u | ((4 + k) << 16) | k);
      out = x | bias;
      out = pk_add_h(out, VFmt<VB, D>::center_bits(0));
    } else if constexpr (VB == 3) {
      // Both tokens' fields in one word (token a in bits 0-15, token b in
      // 16-31, the same code at the same offset; a byte permute, shared by the
      // chunks): one shift then puts code c at bits 7-9 of each half and one
      // and-or makes the fp16 pair. Head_dim 128: codes 0-4 from bytes 0-1,
      // codes 5-7 from bytes 1-2 (code 5 at bit 7).
      constexpr int bpl = 3 * D / 16;  // 24 or 12 bits per lane
      uint32_t y;
      int sft;
      if constexpr (D == 128) {
        if (c < 5) {
          y = perm_b32(b[0], a[0], 0x05040100u);
          sft = 3 * c - 7;
        } else {
          y = perm_b32(b[0], a[0], 0x06050201u);
          sft = 3 * (c - 5);
        }
      } else {
        const uint32_t sh = (bpl * n) & 7;  // the lane's first bit within the loaded byte
        y = perm_b32(b[0] >> sh, a[0] >> sh, 0x05040100u);
        sft = 3 * c - 7;
      }
      out = and_or(sft < 0 ? y << (-sft) : y >> sft, 0x03800380u, bias);
      out = pk_add_h(out, VFmt<VB, D>::center_bits(0));
    } else {  // bf16 values: channel n*D/16 + c is half (c & 1) of word c/2
      const int word = c >> 1;
      out = perm_b32(b[word], a[word], (c & 1) ? 0x07060302u : 0x05040100u);
    }
    r[v] = out;
  }
  return r;
}

template <int D>
__device__ __forceinline__ int v_channel(int n, int c) { return n * (D / 16) + c; }

// ---------------------------------------------------------------------------
// The partial kernel.
// ---------------------------------------------------------------------------

// Raw data of one group (four pages) for one lane, loaded before it is used so
// the next group's loads are in flight while the current group is computed.
template <int KB, int VB, int D>
struct GroupRaw {
  uint32_t k[4][KFmt<KB, D>::kWords];         // key quarter rows, one per page
  uint32_t v[2][8][VRaw<VB, D>::kWords];       // value words, 8 tokens per page pair
  float ks, kmn, vs, vmn;                      // metadata of this lane's token
  float4 kcm[4];                               // per-channel keys: {s, mn} of this lane's two channels, per page
  bool valid;                                  // this lane's token is a cached token
  uint32_t vmask;                              // bit 8*pp2+e: value token e of pair pp2 is cached
  int gid;                                     // group index in the unit (>= unit groups: none)
};

// Running max of the scores may grow by up to this much (log2 units) before the
// accumulators are rescaled, so weights stay below 2^4 between rescales.
constexpr float kRescaleSlack = 4.f;

// Every load is issued unconditionally (pages past the split or unmapped read
// block 0 and are masked afterwards), so the number of loads in flight is
// static and the wait before a group's compute leaves the next group's loads
// outstanding. Each load instruction reads one page, so its base address is
// wave-uniform and the per-lane part is a loop-invariant offset.
constexpr int kXcds = 8;  // accelerator dies of the chip; workgroups go round-robin over them
#ifndef KVQ_TUNE_STATIC_EIGHTHS
#define KVQ_TUNE_STATIC_EIGHTHS 5
#endif
// Share of a unit's groups dealt out in fixed order before the shared tail
// (measured with non-temporal cache loads at the 32k Llama-shaped decode, one
// box: 5/8 110.0 us, 4/8 and 6/8 110.4-110.8, 3/8 111.8, 2/8 113.0, 0 115.6).
constexpr int kStaticEighths = KVQ_TUNE_STATIC_EIGHTHS;

template <int KB, int VB, int D, bool M16, bool KC>
__device__ __forceinline__ void load_group(const DecodeSeg& a, const uint8_t* pool, const int32_t (&blks)[4],
                                           int grp, int p1, int seq_len, int skip, int64_t koff, int64_t voff,
                                           int lane, int kc0, int kc1, GroupRaw<KB, VB, D>& g) {
  constexpr int RBK = D * KB / 8, RBV = D * VB / 8, QBYTES = RBK / 4;
  const int tslot = lane & 15, g4 = lane >> 4;
  int64_t boff[4];
  uint32_t pv = 0;  // bit pp: page grp + pp is mapped
  // (32-bit compare: table entries are int32; a negative entry wraps above any bound)
  const uint32_t nblk = a.pool_blocks > 0x7fffffff ? 0x80000000u : static_cast<uint32_t>(a.pool_blocks);
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) {
    const int page = grp + pp;
    const int32_t blk = blks[pp];
    const bool ok = page < p1 && static_cast<uint32_t>(blk) < nblk;
    pv |= static_cast<uint32_t>(ok) << pp;
    boff[pp] = ok ? blk * a.block_bytes : 0;
  }
  const int kl = tslot * RBK + g4 * QBYTES;  // lane offsets (loop invariant)
  const int vl = g4 * RBV + v_lane_offset<VB, D>(tslot);
  constexpr int MB = M16 ? 4 : kMetaBytes;  // metadata bytes per row
  const int ml = tslot * MB;
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) load_kquarter<KB, D>(pool + boff[pp] + koff + kl, g.k[pp]);
  // token layout: lane = (page g4, slot tslot); each page's metadata by its 16 lanes
  const int tpos = (grp + g4) * kBlockTokens + tslot;
  g.valid = ((pv >> g4) & 1u) && tpos < seq_len && tpos != skip;
  // (all lanes active: a load under a divergent branch would make the compiler
  // wait for every outstanding load, including the prefetch)
  const int64_t my_boff = (g4 & 2) ? ((g4 & 1) ? boff[3] : boff[2]) : ((g4 & 1) ? boff[1] : boff[0]);
  const uint8_t* mbase = pool + my_boff + ml;
  g.ks = 1.f; g.kmn = 0.f; g.vs = 1.f; g.vmn = 0.f;
  if constexpr (KB != 16) {
    if constexpr (KC) {
      // per-channel keys: each page's {s, mn} pairs of the lane's two fragment
      // channels (byte offsets kc0, kc1 in the page's channel metadata)
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        const uint8_t* km = pool + boff[pp] + koff + kBlockTokens * RBK;
        const float2 m0 = ld_cache_f2(km + kc0);
        const float2 m1 = ld_cache_f2(km + kc1);
        g.kcm[pp] = make_float4(m0.x, m0.y, m1.x, m1.y);
      }
    } else if constexpr (M16) {
      const uint32_t mk = ld_cache_u1(mbase + koff + kBlockTokens * RBK);
      g.ks = f16_to_f(mk & 0xffffu); g.kmn = f16_to_f(mk >> 16);
    } else {
      const float2 mk = ld_cache_f2(mbase + koff + kBlockTokens * RBK);
      g.ks = mk.x; g.kmn = mk.y;
    }
  }
  if constexpr (VB != 16) {
    if constexpr (M16) {
      const uint32_t mv = ld_cache_u1(mbase + voff + kBlockTokens * RBV);
      g.vs = f16_to_f(mv & 0xffffu); g.vmn = f16_to_f(mv >> 16);
    } else {
      const float2 mv = ld_cache_f2(mbase + voff + kBlockTokens * RBV);
      g.vs = mv.x; g.vmn = mv.y;
    }
  }
  // value layout: lane = (column n = tslot, K-slot group g4); K-slot e of a page
  // pair is slot 4*(e & 3) + g4 of page 2*pp2 + (e >> 2). One load instruction
  // (fixed e) then reads four consecutive token rows, whole cache lines that no
  // other load of the group touches.
  g.vmask = 0;
#pragma unroll
  for (int pp2 = 0; pp2 < 2; ++pp2) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int pg = 2 * pp2 + (e >> 2);
      load_vtoken<VB, D>(pool + boff[pg] + voff + 4 * (e & 3) * RBV + vl, g.v[pp2][e]);
      const int vpos = (grp + pg) * kBlockTokens + 4 * (e & 3) + g4;
      const bool ok = ((pv >> pg) & 1u) && vpos < seq_len && vpos != skip;
      g.vmask |= static_cast<uint32_t>(ok) << (8 * pp2 + e);
    }
  }
}

// Group buffers in flight while one is computed (prefetch depth) and waves
// per SIMD each instance is compiled for.
#ifndef KVQ_TUNE_DEPTH
#define KVQ_TUNE_DEPTH 2
#endif
#ifndef KVQ_TUNE_WAVES128
#define KVQ_TUNE_WAVES128 2
#endif
#ifndef KVQ_TUNE_QF_REGS
#define KVQ_TUNE_QF_REGS 1
#endif
template <int KB, int VB, int D>
struct PrefetchDepth {
  static constexpr int value = KVQ_TUNE_DEPTH;
};

// The wide formats (8- and 16-bit keys, bf16 values, and the 8-bit values
// beside 3- or 4-bit keys at head_dim 128; 16-bit keys beside 3- or 16-bit
// values and 8-bit keys beside bf16 values at head_dim 64) need more than half
// the register file: one wave per SIMD. The choice is checked by compiling
// every instance and requiring zero spills.
template <int KB, int VB, int D>
struct PartialWaves {
  static constexpr bool wide =
      D == 128 ? (VB == 16 || KB == 16 || KB == 8 || ((KB == 4 || KB == 3) && VB == 8))
               : ((KB == 16 && (VB == 3 || VB == 16)) || (KB == 8 && VB == 16));
  static constexpr int value = wide ? 1 : (D == 128 ? KVQ_TUNE_WAVES128 : 2);
};

template <int KB, int VB, int D>
struct SplitState {
  float4_t acc[D / 16];  // PV accumulators (rows: hi heads 0..3 | lo heads 0..3 | zero)
  float m_run[4];        // reference max per query head (log2 units)
  float l_part[4];       // per-lane partial sum of p
  float mn_part[4];      // per-lane partial sum of p * (mn + 2^(b-1) s)
};

// Per-channel keys: the lane's share of building each page's query fragments.
// A key is s_i c_i + mn_i with a pair per channel and page, so the QK A operand
// is q~ scaled per channel, rebuilt per page: lane (quarter g4, w = lane % 16)
// owns word w % 4 of chunk w / 4, i.e. two channels of its quarter, for all
// four query rows, and its share of the page constant sum_i q~_i (mn_i - s_i
// base_i / sigma_i).
struct KcLane {
  float qk[4][2];  // q~ of the four query rows at the two channels (0 for rows >= group)
  float isig[2];   // 1 / sigma of the channels' fp16 code values
  float bsig[2];   // base / sigma: the constant part of a code value, in code units
  int word;        // u32 index of the word in the hi fragment area (row 0); -1: no word (head_dim 64)
};

template <int KB, int VB, int D, bool KC>
__device__ __forceinline__ void compute_group(GroupRaw<KB, VB, D>& g, const u32x4_t (&qf)[D / 32],
                                              const u32x4_t (&qi)[D / 64], float inv_ql, const float (&biasq)[4], const float (&q2)[4], float inv_qsc, int G,
                                              int lane, uint32_t bias, uint16_t (*wt)[4][64],
                                              const uint16_t* wzero, SplitState<KB, VB, D>& st,
                                              const KcLane& kl, uint4 (*qa)[64]) {
  using KF = KFmt<KB, D>;
  using VF = VFmt<VB, D>;
  constexpr int NCK = D / 32, NCV = D / 16;
  constexpr bool KMETA = KB != 16, VMETA = VB != 16;
  constexpr float NEG_INF = -__builtin_huge_valf();
  const int row = lane & 15, g4 = lane >> 4;

  // QK: one 16x16 tile per page, columns = tokens (fp16 path: rows 0-3 = hi
  // parts of the query heads, rows 4-7 = lo parts; each chunk's query fragment
  // feeds all four pages).
  constexpr bool QI8 = KI8<KB, D>::on && !KC;
  float4_t cq[4];
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) cq[pp] = float4_t{0.f, 0.f, 0.f, 0.f};
  float zs[4];  // (QI8) per page: sum q~ c of head g4 at token row of the page
  if constexpr (QI8) {
    // one integer tile per page: rows 4h + j = digit j of head h, so lane
    // group g4 holds head g4's three digit sums for token `row` of the page
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      i32x4_t acc = i32x4_t{0, 0, 0, 0};
#pragma unroll
      for (int st = 0; st < D / 64; ++st) acc = mfma_i8(qi[st], KI8<KB, D>::bytes(g.k[pp], st), acc);
      zs[pp] = fmaf(static_cast<float>(acc[0]), 65536.f * inv_ql,
                    fmaf(static_cast<float>(acc[1]), 256.f * inv_ql, static_cast<float>(acc[2]) * inv_ql));
    }
  } else if constexpr (KC) {
    // Per page: A = q~ s / sigma at a power-of-two page scale (fp16 hi in rows
    // 0-3 and lo in rows 4-7 of the LDS fragment area), B = the codes as in the row
    // layout; score = sum / scale + the page constant of each query row.
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      const float4 m = g.kcm[pp];
      const float f0 = m.x * kl.isig[0], f1 = m.z * kl.isig[1];
      const float n0 = fmaf(-m.x, kl.bsig[0], m.y), n1 = fmaf(-m.z, kl.bsig[1], m.w);
      float x[4][2], cp[4], amax = 0.f;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        x[h][0] = kl.qk[h][0] * f0;
        x[h][1] = kl.qk[h][1] * f1;
        amax = fmaxf(amax, fmaxf(fabsf(x[h][0]), fabsf(x[h][1])));
        cp[h] = fmaf(kl.qk[h][0], n0, kl.qk[h][1] * n1);
      }
      amax = wave_max_scalar(amax);
      float psc = 1.f;
      if (amax > 0.f) {
        int ex;
        frexpf(amax, &ex);
        psc = ldexpf(1.f, 10 - ex);
      }
      if (kl.word >= 0) {
        uint32_t* qw = reinterpret_cast<uint32_t*>(&qa[0][0]);
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const float y0 = x[h][0] * psc, y1 = x[h][1] * psc;
          const _Float16 h0 = static_cast<_Float16>(y0), h1 = static_cast<_Float16>(y1);
          const _Float16 l0 = static_cast<_Float16>(y0 - static_cast<float>(h0));
          const _Float16 l1 = static_cast<_Float16>(y1 - static_cast<float>(h1));
          qw[kl.word + 4 * h] = half_bits(h0) | (half_bits(h1) << 16);        // row h: hi
          qw[kl.word + 4 * h + 16] = half_bits(l0) | (half_bits(l1) << 16);   // row 4 + h: lo
        }
      }
      float cst[4];
      wave_sum4(cp, cst);
      __syncthreads();  // the fragment words are written before they are read
      const float ipsc = 1.f / psc;
#pragma unroll
      for (int c = 0; c < NCK; ++c) {
        const uint4 vq = qa[c][lane];
        cq[pp] = mfma<KF::bf16>(u32x4_t{vq.x, vq.y, vq.z, vq.w}, KF::unpack(g.k[pp], c, bias), cq[pp]);
      }
      // (the hi rows, lanes 0-15, take the constant once; the lo rows are added below)
#pragma unroll
      for (int i = 0; i < 4; ++i) cq[pp][i] = lane < 16 ? fmaf(cq[pp][i], ipsc, cst[i]) : cq[pp][i] * ipsc;
      __syncthreads();  // and read before the next page writes them
    }
  } else {
#pragma unroll
    for (int c = 0; c < NCK; ++c)
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) cq[pp] = mfma<KF::bf16>(qf[c], KF::unpack(g.k[pp], c, bias), cq[pp]);
  }
  // Pack the four tiles (hi sums in lanes 0-15, lo sums in 16-31) into lane =
  // token of the group, register i = head i: pages 0 and 2 (1 and 3) share a
  // register, lanes 0-31 and 32-63; hi + lo with lane l ^ 16; then lanes 16-31
  // take page 1 and lanes 32-47 page 2.
  float z[4];
  if constexpr (QI8) {
    // (lane group = head, register = page) to (lane group = page, register =
    // head): a transpose of 16-lane blocks in two swap stages
    const auto t02 = __builtin_amdgcn_permlane32_swap(f_bits(zs[0]), f_bits(zs[2]), false, false);
    const auto t13 = __builtin_amdgcn_permlane32_swap(f_bits(zs[1]), f_bits(zs[3]), false, false);
    const auto u01 = __builtin_amdgcn_permlane16_swap(t02[0], t13[0], false, false);
    const auto u23 = __builtin_amdgcn_permlane16_swap(t02[1], t13[1], false, false);
    const float sc[4] = {bits_f(u01[0]), bits_f(u01[1]), bits_f(u23[0]), bits_f(u23[1])};
    const float kmid = fmaf(KI8<KB, D>::kOff, g.ks, g.kmn);
#pragma unroll
    for (int i = 0; i < 4; ++i) z[i] = (g.valid && i < G) ? fmaf(g.ks, sc[i], kmid * q2[i]) : NEG_INF;
  } else {
    const float ks_q = g.ks * inv_qsc;
    // centred codes: s*sum q(c - m) + (mn + m*s)*sum q, the centre term per token
    const float kmid = KF::kCentre != 0.f ? fmaf(KF::kCentre, g.ks, g.kmn) : g.kmn;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const auto x02 = __builtin_amdgcn_permlane32_swap(f_bits(cq[0][i]), f_bits(cq[2][i]), false, false);
      const auto x13 = __builtin_amdgcn_permlane32_swap(f_bits(cq[1][i]), f_bits(cq[3][i]), false, false);
      float y02 = bits_f(x02[0]), y13 = bits_f(x13[0]);
      y02 += __shfl_xor(y02, 16, 64);
      y13 += __shfl_xor(y13, 16, 64);
      const auto r = __builtin_amdgcn_permlane16_swap(f_bits(y02), f_bits(y13), false, false);
      const float sc = bits_f(r[0]);
      float zi;
      if constexpr (KC) zi = sc;
      else if constexpr (KMETA && KF::kCentre != 0.f) zi = fmaf(ks_q, sc, kmid * q2[i]);
      else if constexpr (KMETA) zi = fmaf(ks_q, sc, fmaf(-ks_q, biasq[i], g.kmn * q2[i]));
      else zi = sc;
      z[i] = (g.valid && i < G) ? zi : NEG_INF;
    }
  }

  // online softmax (log2 units): the reference max is raised (and the
  // accumulators rescaled) only when a score exceeds it by more than the slack
  bool over = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) over = over || z[i] > st.m_run[i] + kRescaleSlack;
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(over) != 0, 0)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // (heads i >= G have z = -inf: never raised)
      const float gm = wave_max_scalar(z[i]);
      if (gm > st.m_run[i] + kRescaleSlack) {
        const float alpha = __builtin_amdgcn_exp2f(st.m_run[i] - gm);
#pragma unroll
        for (int c = 0; c < NCV; ++c) st.acc[c][i] *= alpha;
        st.l_part[i] *= alpha;
        st.mn_part[i] *= alpha;
        st.m_run[i] = gm;
      }
    }
  }
  // This lane's token (page lane / 16, slot s = lane % 16) is K-slot (s / 4) of
  // lane group s % 4 in the PV step: its weight goes to row position
  // 16 * page + 4 * (s % 4) + s / 4, so each lane group reads its K-slots
  // contiguously.
  const int wpos = (lane & 0x30) | ((lane & 3) << 2) | ((lane >> 2) & 3);
  const float vs_eff = VMETA ? (g.valid ? g.vs : 0.f) : 1.f;
  const float vmid_eff = VMETA ? (g.valid ? g.vmn + static_cast<float>(1 << (VB - 1)) * g.vs : 0.f) : 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {  // all four rows, branch-free: heads i >= G get p = 0
    const float p = __builtin_amdgcn_exp2f(z[i] - st.m_run[i]);  // masked: exp2(-inf) = 0
    st.l_part[i] += p;
    float w = p;
    if constexpr (VMETA) {
      w = p * vs_eff;
      st.mn_part[i] = fmaf(p, vmid_eff, st.mn_part[i]);
    }
    uint32_t hb, lb;
    if constexpr (VF::bf16) {
      hb = f_to_bf16_rne(w);
      lb = f_to_bf16_rne(w - bf16lo_to_f(hb));
    } else {
      const _Float16 hh = static_cast<_Float16>(w);
      hb = half_bits(hh);
      lb = half_bits(static_cast<_Float16>(w - static_cast<float>(hh)));
    }
    wt[0][i][wpos] = static_cast<uint16_t>(hb);
    wt[1][i][wpos] = static_cast<uint16_t>(lb);
  }
  __syncthreads();

  // PV: two 32-token steps; K-slot e of lane group g4 is token 4*(e & 3) + g4 of
  // the step's page e >> 2
#pragma unroll
  for (int pp2 = 0; pp2 < 2; ++pp2) {
    const uint16_t* asrc;
    int step = 16;
    if (row < 4 && row < G) asrc = &wt[0][row][32 * pp2 + 4 * g4];
    else if (row >= 4 && row < 4 + G) asrc = &wt[1][row - 4][32 * pp2 + 4 * g4];
    else { asrc = wzero; step = 0; }
    const uint2 a0 = *reinterpret_cast<const uint2*>(asrc);
    const uint2 a1 = *reinterpret_cast<const uint2*>(asrc + step);
    const u32x4_t aw = u32x4_t{a0.x, a0.y, a1.x, a1.y};
    if constexpr (VB == 16) {
      if ((g.vmask >> (8 * pp2) & 0xffu) != 0xffu) {  // a masked token in this pair: clear its words
        auto& vv = g.v[pp2];
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
          for (int j = 0; j < VRaw<VB, D>::kWords; ++j)
            vv[e][j] = (g.vmask >> (8 * pp2 + e) & 1u) ? vv[e][j] : 0u;
      }
    }
#pragma unroll
    for (int c = 0; c < NCV; ++c) {
      const u32x4_t bv = v_operand<VB, D>(g.v[pp2], row, c, bias);
      st.acc[c] = mfma<VF::bf16>(aw, bv, st.acc[c]);
    }
  }
  __syncthreads();
}

// The wave's LDS: the rotated queries, the QK A fragments and the PV weight
// staging. They depend on head_dim only, so one allocation serves every format
// of a multi-format launch.
template <int D>
struct PartialLds {
  float qs[4][D];
  uint4 qa[D / 32][64];  // QK A fragments in lane order: rows 0-3 the fp16 hi parts of q~, rows 4-7 the lo parts
  __attribute__((aligned(16))) uint16_t wt[2][4][64];
  __attribute__((aligned(16))) uint16_t wzero[8];
};

// KFmt::channel at run-time indices, by compile-time selects (no table in
// memory); used once per wave.
template <int KB, int D>
__device__ __forceinline__ int kf_channel_rt(int c, int e) {
  int r = 0;
#pragma unroll
  for (int cc = 0; cc < D / 32; ++cc)
#pragma unroll
    for (int ee = 0; ee < 8; ++ee) r = (cc == c && ee == e) ? KFmt<KB, D>::channel(cc, ee) : r;
  return r;
}

// One split of one (sequence, KV head) unit in format (KB, VB): the body of the
// partial kernels, inlined into each of them. KC: keys quantized per channel
// over each page (the per-channel layout), values per token.
// One stage of the query rotation's butterflies: channels j and j + ST (bit ST
// of j clear) become u + v and u - v. A lane's value k is channel
// (lane % 16) * QPL + k of query row lane / 16, so strides below QPL pair
// values of one lane and the others pair lanes lane and lane ^ (ST / QPL),
// inside a row of 16 lanes (DPP moves, no LDS).
template <int ST, int QPL>
__device__ __forceinline__ void q_butterfly(float (&qv)[QPL], int lane) {
  if constexpr (ST < QPL) {
#pragma unroll
    for (int k = 0; k < QPL; ++k) {
      if (k & ST) continue;
      const float u = qv[k], v = qv[k + ST];
      qv[k] = u + v;
      qv[k + ST] = u - v;
    }
  } else {
    constexpr int X = ST / QPL;
    const bool upper = (lane & X) != 0;
#pragma unroll
    for (int k = 0; k < QPL; ++k) {
      const float p = xor_lanes16<X>(qv[k], lane);
      qv[k] = upper ? p - qv[k] : qv[k] + p;
    }
  }
}

template <int KB, int VB, int D, bool M16, bool KC = false>
__device__ __forceinline__ void partial_split(const DecodeArgs& a, int si, int L, const int32_t* __restrict__ table,
                                              uint32_t* __restrict__ steal, float qscale, PartialLds<D>& lds) {
  using KF = KFmt<KB, D>;
  using VF = VFmt<VB, D>;
  constexpr int NCK = D / 32;               // QK chunks (32 channels each)
  constexpr int NCV = D / 16;               // PV chunks (16 output channels each)
  constexpr float NEG_INF = -__builtin_huge_valf();

  auto& qs = lds.qs;
  auto& qa = lds.qa;
  auto& wt = lds.wt;
  auto& wzero = lds.wzero;

  const int lane = threadIdx.x;
  const DecodeSeg& sg = a.seg[si];
  // One-dimensional grid of U units x W splits per segment (W a multiple of
  // the XCD count, each segment's range starting at a multiple of 8).
  // Workgroup L of the segment runs on XCD x = L % 8 as that XCD's m-th
  // workgroup of it, m = L / 8, and serves unit m % U as its split
  // x + 8 * (m / U). So every unit has waves on all eight XCDs and from early
  // and late in each XCD's dispatch order (of two waves on a SIMD the first
  // dispatched is issued first); sharing the tail then evens the units out.
  const int U = sg.n_heads * a.batch;
  const int m = L / kXcds;
  const int unit = m % U;
  const int split = L % kXcds + kXcds * (m / U);
  const int hidx = unit % sg.n_heads;
  const int b = unit / sg.n_heads;
  const int he = sg.head_base + hidx;
  const int h = a.heads[he];
  const int G = a.group;
  const int hq = a.hkv * G;
  const int64_t koff = a.k_off[he], voff = a.v_off[he];
  const int seq_len = sg.seq_lens[b];
  // the slot a fused append fills in this call: masked here (its old bytes
  // are read), attended to by the merge kernel from the new values
  const int skip = sg.skip_pos ? sg.skip_pos[b] : -1;
  const int pages = min((seq_len + kBlockTokens - 1) / kBlockTokens, sg.table_stride);
  const int slot = sg.slot_base + split;

  // Work sharing inside the unit (sequence b, KV head h), whose W waves each
  // write one partial. The unit's page groups (four pages each) are divided
  // into W/8 contiguous ranges, one per sharing group of eight waves: wave
  // split = x + 8r (x its XCD, r its dispatch round) joins group (r - x) mod
  // (W/8), so a group mixes all eight XCDs and early and late waves. In its
  // group's range of NG groups a wave first takes the SG groups
  // [i*SG, (i+1)*SG) (together kStaticEighths/8 of the range, in order; i = x), then groups of
  // the shared tail [8*SG, NG), one at a time, from the group's counter in the
  // workspace. Wave speeds differ by tens of percent (the older of two waves
  // on a SIMD is issued first; some dies run slower); fast waves take more of
  // the tail, so a group's waves finish within about a page group of each
  // other. Eight waves per counter keep the atomics on one address few. Each
  // wave's fetches end with one that finds the tail used up; the wave whose
  // fetch is the eighth such clears the counter (of the two words kept per
  // group the second is unused). Without
  // sharing (deterministic order) wave i takes [i*SG, (i+1)*SG) with
  // SG = ceil(NG / 8) and there is no tail.
  const int W = sg.n_splits;
  const int S = W / kXcds;
  const int wx = split % kXcds, wr = split / kXcds;
  const int sgrp = ((wr - wx) % S + S) % S;
  const int NGU = (pages + 3) / 4;
  // (32-bit products below 2^31, the common case, avoid the 64-bit division sequence)
  const bool narrow = NGU < (1 << 20) && S <= 1024;
  const int g_lo = narrow ? static_cast<int>(static_cast<uint32_t>(NGU * sgrp) / static_cast<uint32_t>(S))
                          : static_cast<int>((static_cast<int64_t>(NGU) * sgrp) / S);
  const int g_hi = narrow ? static_cast<int>(static_cast<uint32_t>(NGU * (sgrp + 1)) / static_cast<uint32_t>(S))
                          : static_cast<int>((static_cast<int64_t>(NGU) * (sgrp + 1)) / S);
  const int NG = g_hi - g_lo;
  const int SG = a.share_tail ? (NG * kStaticEighths / 8) / kXcds : (NG + kXcds - 1) / kXcds;
  const int pool0 = min(SG * kXcds, NG);
  const uint32_t pool_groups = static_cast<uint32_t>(NG - pool0);
  uint32_t* const ctr = steal + 2 * ((static_cast<int64_t>(b) * a.hkv + h) * S + sgrp);
  const uint8_t* pool = sg.pool;
  const int32_t* trow = table + static_cast<int64_t>(b) * sg.table_stride;
  constexpr int QPL = 4 * D / 64;  // query values per lane: QPL contiguous channels of one query row
  // per-channel keys: the lane's fragment word (chunk kc_c, word kc_v of quarter
  // lane / 16) and the byte offsets of its two channels' metadata in a page
  const int kc_c = (lane & 15) >> 2, kc_v = lane & 3;
  int kc_ch0 = 0, kc_ch1 = 0;
  if constexpr (KC) {
    const int cw = kc_c < NCK ? kc_c : 0;
    kc_ch0 = (lane >> 4) * (D / 4) + kf_channel_rt<KB, D>(cw, 2 * kc_v);
    kc_ch1 = (lane >> 4) * (D / 4) + kf_channel_rt<KB, D>(cw, 2 * kc_v + 1);
  }
  const int kc0 = kc_ch0 * kMetaBytes, kc1 = kc_ch1 * kMetaBytes;
  constexpr int DEPTH = PrefetchDepth<KB, VB, D>::value;
  constexpr int NB = DEPTH + 1;  // group buffers
  GroupRaw<KB, VB, D> gbuf[NB];
  // The wave's groups in order ("positions"): its static groups, then tail
  // groups. Position q is resolved (its group known and its four block-table
  // entries requested) one position before its pages are loaded, and the tail
  // fetch that names it is issued one position before that, so neither the
  // counter nor the table is waited for when the loads go out. Everything is
  // a vector-memory access issued in program order, so each wait leaves the
  // later loads outstanding: per load_next, the table entries of this position
  // are read from registers, then the tail fetch, the table entries of the
  // next position and the pages of this position go out.
  int rpos = 0;                          // next position to resolve
  uint32_t inflight = 0;                 // lane 0: the outstanding tail fetch
  bool exhausted = pool_groups == 0;     // the tail is used up: no further fetches
  int next_gid = NG;                     // group of the resolved position (>= NG: none)
  int32_t next_tab = 0;                  // lane t0 + i: table entry of the resolved position's page i
  int tab_lane = 0;                      // t0: 0, or 4 when the entries came with the previous position's
  bool tab_pre = false;                  // lanes 4-7 of next_tab hold the next position's entries
  auto fetch = [&]() {
    uint32_t v = 0;
    if (lane == 0) v = atomicAdd(ctr, 1u);
    inflight = v;
  };
  auto resolve = [&]() {
    int gid = NG;
    if (rpos < SG) {
      gid = min(wx * SG + rpos, NG);
    } else if (!exhausted) {
      const uint32_t idx = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(inflight)));
      if (idx < pool_groups) {
        gid = pool0 + static_cast<int>(idx);
      } else {
        exhausted = true;
        // Each of the group's eight waves makes exactly one fetch past the
        // tail, and none after it; the one that gets the last of these
        // indices is the counter's last user and clears it for the next call.
        if (lane == 0 && idx == pool_groups + static_cast<uint32_t>(kXcds - 1)) atomicExch(ctr, 0u);
      }
    }
    // the position after this one is a tail position: fetch its group now
    if (rpos + 1 >= SG && !exhausted) fetch();
    ++rpos;
    next_gid = __builtin_amdgcn_readfirstlane(gid);  // wave-uniform: page addresses stay scalar
    if (tab_pre) {  // requested with the previous position (lanes 4-7)
      tab_lane = 4;
      tab_pre = false;
    } else {
      // Lanes 0-3: this position's four entries; lanes 4-7: the next
      // position's when it is a static one, so that of the two positions
      // loaded back to back at the start only the first waits for the table.
      // (unconditional, clamped into the sequence's row like the page loads)
      const int g = ((lane & 4) != 0 && rpos < SG) ? min(wx * SG + rpos, NG) : min(next_gid, NG);
      const int page = 4 * (g_lo + g) + (lane & 3);
      next_tab = trow[max(min(page, pages - 1), 0)];
      tab_lane = 0;
      tab_pre = rpos < SG;
    }
  };
  if (SG == 0 && !exhausted) fetch();
  resolve();
  // The first positions' block-table entries are requested first; the query
  // loads follow them, so the first page loads wait only for the table (the
  // loads complete in order), and preparing the query overlaps those pages.
  // Lane l reads channels [c0, c0 + QPL) of query row l / 16 (rows past the
  // group repeat the last row and are zeroed after the rotation): QPL
  // elements as two loads of QPL * 2 bytes, the second at the same address for
  // bf16, so the instructions are the same whatever the type.
  __builtin_amdgcn_sched_barrier(0);
  uint32_t qw[QPL];
  {
    const int r = min(lane >> 4, G - 1);
    const int c0 = (lane & 15) * QPL;
    const int64_t qrow = static_cast<int64_t>(b) * hq + h * G + r;
    const uint8_t* qp = static_cast<const uint8_t*>(a.q) + (qrow * D + c0) * (a.q_bf16 ? 2 : 4);
    const int second = a.q_bf16 ? 0 : QPL * 2;
    if constexpr (QPL == 8) {
      const uint4 w0 = *reinterpret_cast<const uint4*>(qp);
      const uint4 w1 = *reinterpret_cast<const uint4*>(qp + second);
      qw[0] = w0.x; qw[1] = w0.y; qw[2] = w0.z; qw[3] = w0.w;
      qw[4] = w1.x; qw[5] = w1.y; qw[6] = w1.z; qw[7] = w1.w;
    } else {
      const uint2 w0 = *reinterpret_cast<const uint2*>(qp);
      const uint2 w1 = *reinterpret_cast<const uint2*>(qp + second);
      qw[0] = w0.x; qw[1] = w0.y; qw[2] = w1.x; qw[3] = w1.y;
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  auto load_next = [&](GroupRaw<KB, VB, D>& g) {
    const int gid = next_gid;
    int32_t blks[4];
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) blks[pp] = __builtin_amdgcn_readlane(next_tab, tab_lane + pp);
    resolve();
    g.gid = gid;
    load_group<KB, VB, D, M16, KC>(sg, pool, blks, 4 * (g_lo + gid), pages, seq_len, skip, koff, voff, lane, kc0,
                                     kc1, g);
  };
#pragma unroll
  for (int j = 0; j < DEPTH; ++j) load_next(gbuf[j]);
  __builtin_amdgcn_sched_barrier(0);

  // ---- q' = R q for the G query heads of this KV head (butterflies in registers,
  // strides 1, 2, ... below the Hadamard block) ----
  float qv[QPL];
#pragma unroll
  for (int k = 0; k < QPL; ++k) {
    const uint32_t hb = (k & 1) ? (qw[k / 2] & 0xffff0000u) : (qw[k / 2] << 16);
    qv[k] = bits_f(a.q_bf16 ? hb : qw[k]);
  }
  {
    const int n = a.had_block;
    if (n > 1) q_butterfly<1>(qv, lane);
    if (n > 2) q_butterfly<2>(qv, lane);
    if (n > 4) q_butterfly<4>(qv, lane);
    if (n > 8) q_butterfly<8>(qv, lane);
    if (n > 16) q_butterfly<16>(qv, lane);
    if (n > 32) q_butterfly<32>(qv, lane);
    if constexpr (D > 64) {
      if (n > 64) q_butterfly<64>(qv, lane);
    }
  }
  {
    const int r = lane >> 4;
    float4* dst = reinterpret_cast<float4*>(&qs[r][(lane & 15) * QPL]);
#pragma unroll
    for (int j = 0; j < QPL / 4; ++j)
      dst[j] = r < G ? make_float4(qv[4 * j], qv[4 * j + 1], qv[4 * j + 2], qv[4 * j + 3]) : make_float4(0.f, 0.f, 0.f, 0.f);
    // q~ = q' * qscale of this unit's query heads, for the short bf16 segment
    // the merge kernel attends to itself (one wave per unit writes it)
    if (sg.write_q && split == 0 && r < G) {
      float4* qd = reinterpret_cast<float4*>(a.qrot + ((static_cast<int64_t>(b) * hq + h * G + r) * D + (lane & 15) * QPL));
#pragma unroll
      for (int j = 0; j < QPL / 4; ++j)
        qd[j] = make_float4(qv[4 * j] * qscale, qv[4 * j + 1] * qscale, qv[4 * j + 2] * qscale, qv[4 * j + 3] * qscale);
    }
  }
  if (lane < 8) wzero[lane] = 0;
  __syncthreads();

  const int row = lane & 15;
  const int g4 = lane >> 4;
  float biasq[4], q2[4];
  float inv_qsc = 1.f;
  constexpr bool QI8 = KI8<KB, D>::on && !KC;
  constexpr int KS = D / 64;
  u32x4_t qi[KS];   // integer QK A operands (QI8)
  float inv_ql = 0.f;  // (QI8) 1 / fixed-point scale of query head g4, whose sums this lane's tile rows hold
  if constexpr (QI8) {
    // ---- QK A operands, integer: row r = lane % 16 holds digit r % 4 (the
    // 2^16, 2^8 and 1 digits; the fourth row zero) of query head r / 4, at the
    // channels of quarter g4 in KI8 order. x = rint(q~ * 2^(22 - e)), e the
    // exponent of the head's largest |q~|, so |x| < 2^22 and
    // x = d0 * 2^16 + d1 * 2^8 + d2 with each digit a signed byte. ----
    const int qh = row >> 2, dig = row & 3;
    const float f = qh < G ? qscale : 0.f;
    // The head's largest |q~| and sum_j q~_j: the four digit rows of a head
    // (lanes 4*qh .. 4*qh+3, a DPP quad) each take D/16 of the quarter's
    // channels, then the quad and the four quarters (lanes row, row+16,
    // row+32, row+48) are combined.
    constexpr int CD = D / 16;
    float amax = 0.f;
    double q2l = 0.0;  // sum_j q~_hj, this lane's share
#pragma unroll
    for (int j = 0; j < CD; ++j) {
      const float qt = qs[qh][g4 * (D / 4) + dig * CD + j] * f;
      amax = fmaxf(amax, fabsf(qt));
      q2l += static_cast<double>(qt);
    }
    amax = fmaxf(amax, dpp_f32<kDppQuadXor1>(amax));
    amax = fmaxf(amax, dpp_f32<kDppQuadXor2>(amax));
    q2l += dpp_f64<kDppQuadXor1>(q2l);
    q2l += dpp_f64<kDppQuadXor2>(q2l);
    amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
    q2l += __shfl_xor(q2l, 16, 64);
    q2l += __shfl_xor(q2l, 32, 64);
    float qsc = 1.f;
    if (amax > 0.f) {
      int ex;
      frexpf(amax, &ex);
      qsc = ldexpf(1.f, 22 - ex);
    }
    // Digits: with y = x + 0x808080, byte k of y is digit k + 128 (balanced
    // base-256 digits, no carries since |x| <= 2^22), so this row's signed
    // digit is byte 2 - dig of y with its top bit flipped. v_perm gathers that
    // byte of four values into one word; the fourth row of a head stays zero.
    const uint32_t bsel = static_cast<uint32_t>(2 - dig);
    const uint32_t sel_lo = dig == 3 ? 0x0c0c0c0cu : (0x0c0c0000u | ((4u + bsel) << 8) | bsel);
    const uint32_t sel_hi = dig == 3 ? 0x0c0c0c0cu : (((4u + bsel) << 24) | (bsel << 16) | 0x0c0cu);
    const uint32_t flip = dig == 3 ? 0u : 0x80808080u;
#pragma unroll
    for (int st = 0; st < KS; ++st)
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        uint32_t y[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float qt = qs[qh][g4 * (D / 4) + KI8<KB, D>::channel(st, 4 * d + q)] * f;
          y[q] = static_cast<uint32_t>(static_cast<int>(rintf(qt * qsc))) + 0x808080u;
        }
        qi[st][d] = (perm_b32(y[1], y[0], sel_lo) | perm_b32(y[3], y[2], sel_hi)) ^ flip;
      }
    // head g4's scale from lane 4 * g4 (row 4 g4: head g4)
    inv_ql = 1.f / __shfl(qsc, 4 * g4, 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      biasq[i] = 0.f;
      q2[i] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, static_cast<float>(q2l)), 4 * i));
    }
  } else {
    // ---- QK A operands: row r = lane % 16, K-slots of quarter g4. Rows 0-3 hold
    // the hi fp16 parts of query heads 0-3, rows 4-7 the lo parts, so one MFMA
    // per chunk and page gives both sums (lanes 0-15 and 16-31 of the tile) ----
    const int qrow = row & 3;                   // the query head of this row
    const bool qact = row < 8 && qrow < G;
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < NCK; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // (read for every lane and scaled by zero in inactive rows: a read under
        // a condition becomes a branch and a wait per value)
        const float r = qs[qrow][g4 * (D / 4) + KF::channel(c, e)];
        const float v = r * (qact ? qscale / KF::sigma(c, e) : 0.f);
        amax = fmaxf(amax, fabsf(v));
      }
    amax = wave_max_scalar(amax);
    // Power-of-two scale keeping the fp16 halves away from subnormals.
    float qsc = 1.f;
    if (!KF::bf16 && amax > 0.f) {
      int ex;
      frexpf(amax, &ex);
      qsc = ldexpf(1.f, 10 - ex);
    }
    double q1 = 0.0;  // this lane's share of sum A * (base + centre*sigma): the offset to remove
    double q2l = 0.0; // and of sum_j q~_j (the min term)
#pragma unroll
    for (int c = 0; c < NCK; ++c) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        uint32_t hp = 0, lp = 0;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int e = 2 * v + half;
          const float qt = qs[qrow][g4 * (D / 4) + KF::channel(c, e)] * (qact ? qscale : 0.f);
          const float x = qt / KF::sigma(c, e) * qsc;
          uint32_t hb, lb;
          float hv, lv;
          if constexpr (KF::bf16) {
            hb = f_to_bf16_rne(x); hv = bf16lo_to_f(hb);
            lb = f_to_bf16_rne(x - hv); lv = bf16lo_to_f(lb);
          } else {
            const _Float16 hh = static_cast<_Float16>(x);
            hv = static_cast<float>(hh);
            const _Float16 ll = static_cast<_Float16>(x - hv);
            lv = static_cast<float>(ll);
            hb = half_bits(hh); lb = half_bits(ll);
          }
          q1 += (static_cast<double>(hv) + static_cast<double>(lv)) *
                static_cast<double>(KF::base(c, e) + KF::kCentre * KF::sigma(c, e));
          q2l += static_cast<double>(qt);
          hp |= hb << (16 * half);
          lp |= lb << (16 * half);
        }
        reinterpret_cast<uint32_t*>(&qa[c][lane])[v] = row < 4 ? hp : lp;
      }
    }
    // Sum over the four quarters (lanes row, row+16, row+32, row+48), in fp64.
    q1 += __shfl_xor(q1, 16, 64);
    q1 += __shfl_xor(q1, 32, 64);
    q2l += __shfl_xor(q2l, 16, 64);
    q2l += __shfl_xor(q2l, 32, 64);
    // Per query head constants, broadcast from lane i (row i, a hi row):
    //   biasq_i = sum A * (base + centre*sigma) (scaled units; 1024 * sum A for the
    //   uncentred formats, 0 for centred ones), q2_i = sum_j q~_ij (log2 units).
    inv_qsc = 1.f / qsc;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float q1i = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, static_cast<float>(q1)), i));
      biasq[i] = q1i;
      q2[i] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, static_cast<float>(q2l)), i));
    }
  }
  const uint32_t bias = vconst(0x64006400u);  // fp16 pair (1024, 1024)

  // per-channel keys: the lane's q~ at its two channels, and their code scale
  // and constant (the fragments above keep their zero rows 8-15; rows 0-7,
  // hi and lo, are rewritten per page, zero for heads >= group)
  KcLane kl{};
  if constexpr (KC) {
    const int cw = kc_c < NCK ? kc_c : 0;
    // (lanes with no word, at head_dim 64, contribute nothing)
    const bool own = kc_c < NCK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float f = own && i < G ? qscale : 0.f;
      kl.qk[i][0] = qs[i][kc_ch0] * f;
      kl.qk[i][1] = qs[i][kc_ch1] * f;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float sg = KF::sigma(cw, 2 * kc_v + j);
      kl.isig[j] = 1.f / sg;
      kl.bsig[j] = KF::base(cw, 2 * kc_v + j) / sg;
    }
    kl.word = kc_c < NCK ? (kc_c * 64 + 16 * (lane >> 4)) * 4 + kc_v : -1;
  }

  __syncthreads();  // the A fragments are read by the same wave; order LDS writes before reads

  // ---- main loop: two groups per trip, loads of the next group in flight ----
  SplitState<KB, VB, D> st;
#pragma unroll
  for (int c = 0; c < NCV; ++c) st.acc[c] = float4_t{0.f, 0.f, 0.f, 0.f};
  // A finite floor (not -inf) for the reference max: exp2(z - m) stays 0 for
  // masked tokens (z = -inf) before any token was seen.
#pragma unroll
  for (int i = 0; i < 4; ++i) { st.m_run[i] = -1e30f; st.l_part[i] = 0.f; st.mn_part[i] = 0.f; }

  // Query fragments: held in registers when the register budget allows, else
  // re-read from LDS before each group. The estimate counts the three group
  // buffers, the fragments and the PV accumulators against the 256
  // architectural registers, leaving room for the rest of the loop.
  constexpr int GROUP_WORDS = 4 * KF::kWords + 16 * VRaw<VB, D>::kWords + 4;
  constexpr bool QF_REGS = !KC && !QI8 && KVQ_TUNE_QF_REGS && (DEPTH + 1) * GROUP_WORDS + 4 * NCK + 4 * NCV <= 180;
  u32x4_t qreg[NCK];
  if constexpr (QF_REGS) {
#pragma unroll
    for (int c = 0; c < NCK; ++c) {
      const uint4 v = qa[c][lane];
      qreg[c] = u32x4_t{v.x, v.y, v.z, v.w};
    }
  }
  auto compute = [&](GroupRaw<KB, VB, D>& g) {
    if constexpr (QF_REGS || QI8) {
      compute_group<KB, VB, D, KC>(g, qreg, qi, inv_ql, biasq, q2, inv_qsc, G, lane, bias, wt, wzero, st, kl, qa);
    } else {
      u32x4_t qf[NCK];
#pragma unroll
      for (int c = 0; c < NCK; ++c) {
        const uint4 v = qa[c][lane];
        qf[c] = u32x4_t{v.x, v.y, v.z, v.w};
      }
      compute_group<KB, VB, D, KC>(g, qf, qi, inv_ql, biasq, q2, inv_qsc, G, lane, bias, wt, wzero, st, kl, qa);
    }
  };

  // Rotating group buffers: while position i is computed, positions
  // i+1 .. i+DEPTH are in flight. Each trip covers NB positions, unrolled so
  // that every buffer index is static; positions past the wave's last group
  // are skipped (loads of such positions read masked pages). The loop has a
  // single exit at its bottom, taken when the next trip's first position has
  // no group, so the loads in flight at the back edge are the same at every
  // trip.
  if (gbuf[0].gid < NG) {
    for (;;) {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        load_next(gbuf[(j + DEPTH) % NB]);
        // Of two waves on a SIMD the older is issued first, so one runs up to
        // twice the other's pace, and when the shared tail runs dry the slow
        // wave still has its prefetched groups to finish. Raising each wave's
        // issue priority on every other group (waves out of step by their
        // split) lets the two take turns, which narrows both the spread of
        // groups per wave and of the waves' end times.
        if ((rpos + split) & 1) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
        if (gbuf[j].gid < NG) compute(gbuf[j]);
      }
      if (gbuf[0].gid >= NG) break;
    }
  }

  // ---- epilogue: combine hi/lo rows, add the min term, write the partials ----
  float lsum[4], mnsum[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lsum[i] = wave_sum_scalar(st.l_part[i]);
    mnsum[i] = wave_sum_scalar(st.mn_part[i]);
  }
  float o[NCV][4];
#pragma unroll
  for (int c = 0; c < NCV; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // rows 0-3 (hi weights, lanes 0-15) plus rows 4-7 (lo weights, lanes 16-31)
      o[c][i] = (st.acc[c][i] + __shfl_xor(st.acc[c][i], 16, 64)) / VF::sigma(c) + mnsum[i];
    }
  if (lane < 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i >= G) break;
      const int64_t bg = static_cast<int64_t>(b) * hq + h * G + i;
      float* po = a.part_o + (bg * a.total_slots + slot) * D + v_channel<D>(lane, 0);
      if constexpr (NCV == 8) {
        reinterpret_cast<float4*>(po)[0] = make_float4(o[0][i], o[1][i], o[2][i], o[3][i]);
        reinterpret_cast<float4*>(po)[1] = make_float4(o[4][i], o[5][i], o[6][i], o[7][i]);
      } else {
        reinterpret_cast<float4*>(po)[0] = make_float4(o[0][i], o[1][i], o[2][i], o[3][i]);
      }
      if (lane == 0) {
        float* ml = a.part_ml + (bg * a.total_slots + slot) * 2;
        ml[0] = lsum[i] > 0.f ? st.m_run[i] : NEG_INF;
        ml[1] = lsum[i];
      }
    }
  }
}

// Fused append: a group of LPR lanes per row (lanes [0, LPR): the K row,
// [LPR, 2 LPR): the V row; 16 channels a lane, so 8 lanes per row at head_dim
// 128) quantizes the new token's row of head h as the append kernel does (the
// same rotation, metadata and codes: the shared row routines; any lane split
// of the exact rotation gives the same values), stores it at slot `slot` of
// `page` (null: not stored) and leaves its dequantized rotated values
// x_hat = c * s + mn (a rounded product, then a rounded sum; bf16 rows: the
// rounded value) in `rows` (global memory).
template <int D>
struct AppendLanes {
  static constexpr int CPR = 16, LPR = D / CPR;
};

template <int BITS, int D>
__device__ __forceinline__ void token_append_quant(const TokenAppend& ap, float (&x)[AppendLanes<D>::CPR], int m,
                                                   uint8_t* page, int64_t off, int slot, float* row) {
  constexpr int CPR = AppendLanes<D>::CPR, LPR = AppendLanes<D>::LPR, RB = D * BITS / 8;
  if constexpr (BITS == 16) {
    if (page) store_row_bf16<CPR>(x, page + off + slot * RB + m * (CPR * 2));
#pragma unroll
    for (int j = 0; j < CPR; ++j) row[m * CPR + j] = bf16lo_to_f(f_to_bf16_rne(x[j]));
  } else {
    RowQ<CPR> q;
    quantize_row<BITS, CPR, LPR>(x, ap.meta16 != 0, q);
    if (page)
      store_row<BITS, CPR>(q, page + off + slot * RB + m * (CPR * BITS / 8),
                           page + off + kBlockTokens * RB + slot * (ap.meta16 ? 4 : kMetaBytes), m, ap.meta16 != 0);
#pragma unroll
    for (int j = 0; j < CPR; ++j) row[m * CPR + j] = __fadd_rn(__fmul_rn(__builtin_rintf(q.u[j]), q.s), q.mn);
  }
}

// lane: 0 .. 2 * LPR - 1
template <int D>
__device__ __forceinline__ void token_append_row(const TokenAppend& ap, int had_block, int b, int h, int hkv,
                                                 int lane, uint8_t* page, int slot, float (*rows)[D]) {
  constexpr int CPR = AppendLanes<D>::CPR, LPR = AppendLanes<D>::LPR;
  const int m = lane % LPR, half = lane / LPR;
  float x[CPR];
  const size_t elem = (static_cast<size_t>(b) * hkv + h) * D + m * CPR;
  const void* src = half ? ap.v_new : ap.k_new;
  if (ap.src_bf16) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + elem);
#pragma unroll
    for (int k = 0; k < CPR / 8; ++k) {
      const uint4 w = p[k];
      x[8 * k + 0] = bf16lo_to_f(w.x); x[8 * k + 1] = bf16hi_to_f(w.x);
      x[8 * k + 2] = bf16lo_to_f(w.y); x[8 * k + 3] = bf16hi_to_f(w.y);
      x[8 * k + 4] = bf16lo_to_f(w.z); x[8 * k + 5] = bf16hi_to_f(w.z);
      x[8 * k + 6] = bf16lo_to_f(w.w); x[8 * k + 7] = bf16hi_to_f(w.w);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(src) + elem);
#pragma unroll
    for (int k = 0; k < CPR / 4; ++k) {
      const float4 w = p[k];
      x[4 * k + 0] = w.x; x[4 * k + 1] = w.y; x[4 * k + 2] = w.z; x[4 * k + 3] = w.w;
    }
  }
  rotate_row<CPR, LPR>(x, m, had_block, ap.rs_n);
  const int64_t off = half ? ap.v_off[h] : ap.k_off[h];
  float* row = rows[half];
  switch (half ? ap.bits_v[h] : ap.bits_k[h]) {
    case 2: token_append_quant<2, D>(ap, x, m, page, off, slot, row); break;
    case 3: token_append_quant<3, D>(ap, x, m, page, off, slot, row); break;
    case 4: token_append_quant<4, D>(ap, x, m, page, off, slot, row); break;
    case 8: token_append_quant<8, D>(ap, x, m, page, off, slot, row); break;
    default: token_append_quant<16, D>(ap, x, m, page, off, slot, row); break;  // the host sends 2, 3, 4, 8, 16
  }
}

// The split-0 wave of each (sequence, KV head) of the segment that writes q~
// also appends the call's new token of that head (a fused append), before its
// own pages: one wave per (sequence, KV head) stores it, and the merge reads
// its dequantized rows from the workspace. (Other waves may read the slot's
// old bytes meanwhile; the slot is masked for all of them.)
template <int D>
__device__ __forceinline__ void partial_append_job(const DecodeArgs& a, int si, int L) {
  const DecodeSeg& sg = a.seg[si];
  const TokenAppend& ap = a.ap;
  if (!ap.pool || !sg.write_q) return;
  const int U = sg.n_heads * a.batch;
  if (L % kXcds != 0 || L / kXcds >= U) return;  // not split 0
  const int unit = L / kXcds, b = unit / sg.n_heads;
  const int h = a.heads[sg.head_base + unit % sg.n_heads];
  const int pos = ap.start_pos[b];
  if (pos < 0) return;
  const int pg = pos / kBlockTokens;
  const int32_t blk = pg < ap.table_stride ? ap.table[static_cast<int64_t>(b) * ap.table_stride + pg] : -1;
  uint8_t* page = blk >= 0 && blk < ap.pool_blocks ? ap.pool + blk * ap.block_bytes : nullptr;
  const int lane = threadIdx.x;
  if (lane < 2 * AppendLanes<D>::LPR)
    token_append_row<D>(ap, a.had_block, b, h, a.hkv, lane, page, pos % kBlockTokens,
                        reinterpret_cast<float (*)[D]>(a.anew + (static_cast<int64_t>(b) * a.hkv + h) * 2 * D));
}

template <int KB, int VB, int D, bool M16>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(PartialWaves<KB, VB, D>::value,
                                                                    PartialWaves<KB, VB, D>::value)))
void decode_partial_kernel(DecodeArgs a, const int32_t* __restrict__ table, uint32_t* __restrict__ steal,
                           float qscale) {
  // (table and counters as separate restrict arguments: the counters' atomics
  // cannot alias the block table, so its entries stay scalar loads)
  __shared__ PartialLds<D> lds;
  partial_append_job<D>(a, 0, static_cast<int>(blockIdx.x));
  partial_split<KB, VB, D, M16>(a, 0, static_cast<int>(blockIdx.x), table, steal, qscale, lds);
}

// Keys quantized per channel over each page, values per token: the same split,
// work sharing and partials, with the QK A operand rebuilt per page.
// (8-bit keys, and 8- or 16-bit values at head_dim 128 or 16-bit values at 64,
// need more than half the register file: one wave per SIMD; checked by
// compiling every instance and requiring zero spills)
template <int KB, int VB, int D>
struct KcWaves {
  static constexpr bool wide = D == 128 ? (KB == 8 || VB == 8 || VB == 16) : VB == 16;
  static constexpr int value = wide ? 1 : 2;
};

template <int KB, int VB, int D>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(KcWaves<KB, VB, D>::value,
                                                                    KcWaves<KB, VB, D>::value)))
void decode_partial_kc_kernel(DecodeArgs a, const int32_t* __restrict__ table, uint32_t* __restrict__ steal,
                              float qscale) {
  __shared__ PartialLds<D> lds;
  partial_append_job<D>(a, 0, static_cast<int>(blockIdx.x));
  partial_split<KB, VB, D, false, true>(a, 0, static_cast<int>(blockIdx.x), table, steal, qscale, lds);
}

// Heads of several formats, and of several segments, in one launch: each wave
// finds its segment (the last whose grid range starts at or before its
// workgroup) and runs the body of its head's (key, value) width pair. Covers
// the pairs of 2-, 3- and 4-bit codes, which all run two waves per SIMD. One
// launch fills the device in one dispatch; launches per format or segment on
// concurrent streams start one after another, tens of microseconds apart.
template <int D, bool M16>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_partial_multi_kernel(DecodeArgs a, float qscale) {
  __shared__ PartialLds<D> lds;
  const int blk = static_cast<int>(blockIdx.x);
  int si = 0;
  for (int s = 1; s < a.n_segs; ++s)
    if (blk >= a.seg[s].grid_start) si = s;
  const DecodeSeg& sg = a.seg[si];
  const int L = blk - sg.grid_start;
  const int unit = (L / kXcds) % (sg.n_heads * a.batch);
  const int pair = __builtin_amdgcn_readfirstlane(a.pair[sg.head_base + unit % sg.n_heads]);
  const int32_t* table = sg.table;
  uint32_t* steal = sg.steal;
  partial_append_job<D>(a, si, L);
  switch (pair) {
    case 0x22: partial_split<2, 2, D, M16>(a, si, L, table, steal, qscale, lds); break;
    case 0x23: partial_split<2, 3, D, M16>(a, si, L, table, steal, qscale, lds); break;
    case 0x24: partial_split<2, 4, D, M16>(a, si, L, table, steal, qscale, lds); break;
    case 0x32: partial_split<3, 2, D, M16>(a, si, L, table, steal, qscale, lds); break;
    case 0x33: partial_split<3, 3, D, M16>(a, si, L, table, steal, qscale, lds); break;
    case 0x34: partial_split<3, 4, D, M16>(a, si, L, table, steal, qscale, lds); break;
    case 0x42: partial_split<4, 2, D, M16>(a, si, L, table, steal, qscale, lds); break;
    case 0x43: partial_split<4, 3, D, M16>(a, si, L, table, steal, qscale, lds); break;
    case 0x44: partial_split<4, 4, D, M16>(a, si, L, table, steal, qscale, lds); break;
    default: break;  // the host sends only these pairs
  }
}

// ---------------------------------------------------------------------------
// Merge of the split partials (all segments) and the inverse rotation.
// ---------------------------------------------------------------------------
// One workgroup of NW waves per (sequence, query head): the waves share the
// split slots (wave w takes slots s = w mod NW), so a long list of slots
// (batch 1 at long context has hundreds) is read with NW waves' loads in
// flight; each wave's loop is bound by load latency, not bandwidth.
//
// A short bf16 segment (a.win.pool set: every head 16-bit keys and values, at
// most kMergeWindowMax tokens) is attended to here rather than by a partial
// launch: its scores z_t = q~ . k'_t (q~ written by the partial launch, k'_t
// the stored rotated row, log2 units as in the partials), then its weights
// 2^(z_t - M) and weighted rows enter the same sums as the split partials'.
__device__ __forceinline__ bool ap_pool(const MergeArgs& a) { return a.ap.pool != nullptr; }

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void decode_merge_kernel(MergeArgs a, float rs_n) {
  constexpr int CPL = D / 64;  // channels per lane: [CPL*lane, CPL*lane + CPL)
  constexpr int CHUNK = 1024;  // slots whose weights sit in LDS at a time
  constexpr float NEG_INF = -__builtin_huge_valf();
  __shared__ float wsh[CHUNK];   // split weights 2^(m_s - M) of the current chunk
  __shared__ float red[NW][D];   // per-wave channel sums
  __shared__ float scal[NW][2];  // per-wave max, then per-wave sum of weights * l
  __shared__ float wq[D];        // window segment: q~ of this query head
  __shared__ float wz[kMergeWindowMax];  // window segment: scores, then weights
  __shared__ int32_t wrow[kMergeWindowMax];  // window segment: block of each token (0 when unmapped)
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t bg = blockIdx.x;
  const int S = a.total_slots;
  const float* ml = a.part_ml + bg * S * 2;
  const float* po = a.part_o + bg * S * D;
  const MergeWindow& win = a.win;
  const int b = static_cast<int>(bg / a.hq);
  const int h = static_cast<int>(bg % a.hq) / a.group;
  const int nwin = win.pool ? min(win.seq_lens[b], win.max_len) : 0;
  const uint32_t wblocks = win.pool_blocks > 0x7fffffff ? 0x80000000u : static_cast<uint32_t>(win.pool_blocks);
  // the window row of token t (block 0 for an unmapped page; its weight is 0)
  auto win_row = [&](int t, int64_t off, bool& ok) {
    const int32_t blk = win.table[static_cast<int64_t>(b) * win.table_stride + t / kBlockTokens];
    ok = static_cast<uint32_t>(blk) < wblocks;
    return win.pool + (ok ? blk : 0) * win.block_bytes + off + (t % kBlockTokens) * (D * 2);
  };
  const int wskip = win.pool && win.skip_pos ? win.skip_pos[b] : -1;  // the window slot a fused append fills
  // Read first: the table entry of this thread's first window key row (token
  // tid / 8, eight lanes a token), so that the row's load further down waits
  // for none of the preloads issued in between (loads complete in order), and
  // q~ of this query head (written by the partial launch), whose round trip
  // overlaps the preloads.
  const bool need_q = nwin > 0 || ap_pool(a);
  const int t00 = tid >> 3, tend = (nwin + 7) & ~7;
  int32_t tab0 = 0;
  if (t00 < tend) tab0 = win.table[static_cast<int64_t>(b) * win.table_stride + min(t00, nwin - 1) / kBlockTokens];
  const float qv = need_q && tid < D ? a.qrot[bg * D + tid] : 0.f;
  // Fused append: the partial launch quantized and stored the new token and
  // left its dequantized rows in anew; it is attended to below when its slot
  // is mapped and inside the segment's length.
  const TokenAppend& ap = a.ap;
  bool attend_new = false;
  float anew_k[CPL], anew_v[CPL];  // (wave 0) the new token's rows, CPL channels a lane
  if (ap.pool) {
    const int pos = ap.start_pos[b];
    if (pos >= 0) {
      const int pg = pos / kBlockTokens;
      const int32_t blk = pg < ap.table_stride ? ap.table[static_cast<int64_t>(b) * ap.table_stride + pg] : -1;
      attend_new = blk >= 0 && blk < ap.pool_blocks && pos < min(ap.seq_lens[b], ap.max_len);
    }
    if (attend_new && w == 0) {
      const float* rows = a.anew + (static_cast<int64_t>(b) * (a.hq / a.group) + h) * 2 * D + CPL * lane;
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        anew_k[j] = rows[j];
        anew_v[j] = rows[D + j];
      }
    }
  }
  // This wave's first batch of split slots (w, w + NW, ... of the first chunk,
  // padded with the chunk's last slot) and of window value rows (tokens w,
  // w + NW, ...), loaded before the max is known: the values do not depend
  // on it, so their round trips overlap the max pass and the window scores.
  const int n0 = min(CHUNK, S);
  float v0[8][CPL];
  if (w < n0) {
    const float* pc = po + CPL * lane;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int sc = min(w + u * NW, n0 - 1);
#pragma unroll
      for (int j = 0; j < CPL; ++j) v0[u][j] = pc[static_cast<int64_t>(sc) * D + j];
    }
  }
  const uint8_t* vbase = win.pool ? win.pool + win.v_off[h] + (CPL == 2 ? 4 : 2) * lane : nullptr;
  uint32_t wraw0[8];
  if (w < nwin) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int tc = min(w + u * NW, nwin - 1);
      const int32_t blk = win.table[static_cast<int64_t>(b) * win.table_stride + tc / kBlockTokens];
      const uint8_t* row = vbase + (static_cast<uint32_t>(blk) < wblocks ? blk : 0) * win.block_bytes +
                           (tc % kBlockTokens) * (D * 2);
      if constexpr (CPL == 2) wraw0[u] = *reinterpret_cast<const uint32_t*>(row);
      else wraw0[u] = *reinterpret_cast<const uint16_t*>(row);
      if (tc == wskip) wraw0[u] = 0u;  // (the slot's old bytes may not be a number)
    }
  }
  // global max over splits and window tokens (the splits' maxima read before
  // q~ arrives); a window token's score is summed by eight lanes, D / 8
  // channels each, then over the eight lanes. This thread's first window key
  // row is also read before q~ arrives.
  float mx = NEG_INF;
  for (int s = tid; s < S; s += 64 * NW) mx = fmaxf(mx, ml[2 * s]);
  constexpr int CH = D / 8;  // channels per lane of a token
  const int part = lane & 7;
  uint4 k0[CH / 8];
  int32_t blk0 = 0;
  if (t00 < tend) {
    const int t = min(t00, nwin - 1);
    const bool ok = static_cast<uint32_t>(tab0) < wblocks;
    const uint4* row = reinterpret_cast<const uint4*>(win.pool + (ok ? tab0 : 0) * win.block_bytes + win.k_off[h] +
                                                      (t % kBlockTokens) * (D * 2)) + part * (CH / 8);
#pragma unroll
    for (int c = 0; c < CH / 8; ++c) k0[c] = row[c];
    blk0 = ok ? tab0 : -1;
  }
  if (need_q) {
    if (tid < D) wq[tid] = qv;
    __syncthreads();
  }
  {
    for (int t0 = t00; t0 < tend; t0 += 8 * NW) {
      const int t = min(t0, nwin - 1);  // lanes past the last token repeat it (not stored)
      const bool first = t0 == t00;     // the row read before q~ arrived
      bool ok = blk0 >= 0;
      const uint4* row = first ? nullptr : reinterpret_cast<const uint4*>(win_row(t, win.k_off[h], ok)) + part * (CH / 8);
      float z = 0.f;
#pragma unroll
      for (int c = 0; c < CH / 8; ++c) {
        const uint4 v = first ? k0[c] : row[c];
        const float* qq = &wq[part * CH + 8 * c];
        z = fmaf(qq[0], bf16lo_to_f(v.x), z);
        z = fmaf(qq[1], bf16hi_to_f(v.x), z);
        z = fmaf(qq[2], bf16lo_to_f(v.y), z);
        z = fmaf(qq[3], bf16hi_to_f(v.y), z);
        z = fmaf(qq[4], bf16lo_to_f(v.z), z);
        z = fmaf(qq[5], bf16hi_to_f(v.z), z);
        z = fmaf(qq[6], bf16lo_to_f(v.w), z);
        z = fmaf(qq[7], bf16hi_to_f(v.w), z);
      }
      z += xor_lanes16<1>(z, lane);
      z += xor_lanes16<2>(z, lane);
      z += xor_lanes16<4>(z, lane);
      z = ok && t != wskip ? z : NEG_INF;
      if (part == 0 && t0 < nwin) {
        wz[t] = z;
        wrow[t] = !ok ? 0 : first ? blk0 : win.table[static_cast<int64_t>(b) * win.table_stride + t / kBlockTokens];
      }
      if (t0 < nwin) mx = fmaxf(mx, z);
    }
  }
  // the fused append's token: its score from q~ (in LDS) and its K row
  float z_new = NEG_INF;
  if (attend_new && w == 0) {
    float t = 0.f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) t = fmaf(wq[CPL * lane + j], anew_k[j], t);
    z_new = wave_sum_scalar(t);
    mx = fmaxf(mx, z_new);
  }
  mx = wave_max_scalar(mx);
  if (lane == 0) scal[w][0] = mx;
  __syncthreads();
  mx = scal[0][0];
#pragma unroll
  for (int i = 1; i < NW; ++i) mx = fmaxf(mx, scal[i][0]);

  float x[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) x[j] = 0.f;
  float lpart = 0.f;
  if (mx != NEG_INF) {
    for (int s0 = 0; s0 < S; s0 += CHUNK) {
      const int n = min(CHUNK, S - s0);
      __syncthreads();
      for (int s = tid; s < n; s += 64 * NW) {
        const float ms = ml[2 * (s0 + s)];
        const float wt = ms == NEG_INF ? 0.f : __builtin_amdgcn_exp2f(ms - mx);
        wsh[s] = wt;
        lpart = fmaf(wt, ml[2 * (s0 + s) + 1], lpart);
      }
      __syncthreads();
      const float* pc = po + static_cast<int64_t>(s0) * D + CPL * lane;
      // batches of eight slots (w, w + NW, ...), the last one padded with the
      // list's last slot at weight 0, so no slot waits on another's load
      for (int s = w; s < n; s += 8 * NW) {
        float v[8][CPL], wu[8];
        const bool first = s0 == 0 && s == w;  // the batch loaded at the start
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int su = s + u * NW, sc = min(su, n - 1);
#pragma unroll
          for (int j = 0; j < CPL; ++j) v[u][j] = first ? v0[u][j] : pc[static_cast<int64_t>(sc) * D + j];
          wu[u] = su < n ? wsh[sc] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
          for (int j = 0; j < CPL; ++j) x[j] = fmaf(wu[u], v[u][j], x[j]);
      }
    }
    if (nwin > 0) {
      // window weights 2^(z_t - M) (each thread its own tokens), then each
      // wave adds tokens t = w mod NW of the value rows, CPL channels a lane
      __syncthreads();  // every token's score is stored
      for (int t = tid; t < nwin; t += 64 * NW) {
        const float p = __builtin_amdgcn_exp2f(wz[t] - mx);  // masked: exp2(-inf) = 0
        wz[t] = p;
        lpart += p;
      }
      __syncthreads();
      // tokens t = w, w + NW, ... in batches of eight (the last padded with
      // the last token at weight 0), each token's row read by its CPL-channel
      // lane slices, so a batch's loads are all in flight together
      for (int t = w; t < nwin; t += 8 * NW) {
        uint32_t raw[8];
        float pw[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int tu = t + u * NW, tc = min(tu, nwin - 1);
          if (t == w) {
            raw[u] = wraw0[u];  // loaded at the start
          } else {
            const uint8_t* row = vbase + wrow[tc] * win.block_bytes + (tc % kBlockTokens) * (D * 2);
            if constexpr (CPL == 2) raw[u] = *reinterpret_cast<const uint32_t*>(row);
            else raw[u] = *reinterpret_cast<const uint16_t*>(row);
            if (tc == wskip) raw[u] = 0u;  // (the slot's old bytes may not be a number)
          }
          pw[u] = tu < nwin ? wz[tc] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          x[0] = fmaf(pw[u], bf16lo_to_f(raw[u]), x[0]);
          if constexpr (CPL == 2) x[1] = fmaf(pw[u], bf16hi_to_f(raw[u]), x[1]);
        }
      }
    }
    if (attend_new && w == 0) {
      const float p = __builtin_amdgcn_exp2f(z_new - mx);
      if (lane == 0) lpart += p;
#pragma unroll
      for (int j = 0; j < CPL; ++j) x[j] = fmaf(p, anew_v[j], x[j]);
    }
  }
  // combine the waves
  lpart = wave_sum_scalar(lpart);
  if (lane == 0) scal[w][1] = lpart;
#pragma unroll
  for (int j = 0; j < CPL; ++j) red[w][CPL * lane + j] = x[j];
  __syncthreads();
  if (w != 0) return;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    float t = red[0][CPL * lane + j];
#pragma unroll
    for (int i = 1; i < NW; ++i) t += red[i][CPL * lane + j];
    x[j] = t;
  }
  if (mx != NEG_INF) {
    float lsum = scal[0][1];
#pragma unroll
    for (int i = 1; i < NW; ++i) lsum += scal[i][1];
    const float inv = 1.f / lsum;
#pragma unroll
    for (int j = 0; j < CPL; ++j) x[j] *= inv;
  }
  // o = R^T o' (H symmetric): butterflies in-lane for stride < CPL, else across lanes.
  if constexpr (CPL == 2) {
    if (a.had_block >= 2) {
      const float u = x[0], v = x[1];
      x[0] = u + v;
      x[1] = u - v;
    }
  }
  for (int m = 1; m * CPL < a.had_block; m <<= 1) {
    const bool upper = (lane & m) != 0;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const float y = shfl_xor(x[j], m);
      x[j] = upper ? (y - x[j]) : (x[j] + y);
    }
  }
  float* out = a.out + bg * D + CPL * lane;
  if constexpr (CPL == 2) {
    *reinterpret_cast<float2*>(out) = make_float2(x[0] * rs_n, x[1] * rs_n);
  } else {
    out[0] = x[0] * rs_n;
  }
}

// Workgroups of a single-segment launch (0 if its split count is not a multiple of the XCD count).
unsigned single_grid(const DecodeArgs& a) {
  const DecodeSeg& sg = a.seg[0];
  if (a.n_segs != 1 || sg.n_splits % kXcds != 0 || sg.grid_start != 0) return 0;
  return static_cast<unsigned>(sg.n_splits) * sg.n_heads * a.batch;
}

template <int KB, int VB, int D, bool M16>
hipError_t launch_partial_t(const DecodeArgs& a, float qscale, hipStream_t s) {
  const unsigned grid = single_grid(a);
  if (grid == 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL((decode_partial_kernel<KB, VB, D, M16>), dim3(grid), dim3(64), 0, s, a, a.seg[0].table,
                     a.seg[0].steal, qscale);
  return hipGetLastError();
}

// Formats whose rows carry metadata get a float16-metadata instance too.
template <int KB, int VB, int D>
hipError_t launch_partial_m(const DecodeArgs& a, float qs, hipStream_t s) {
  if constexpr (KB != 16 || VB != 16) {
    if (a.meta16) return launch_partial_t<KB, VB, D, true>(a, qs, s);
  }
  return launch_partial_t<KB, VB, D, false>(a, qs, s);
}

template <int KB, int D>
hipError_t dispatch_v(const DecodeArgs& a, int vbits, float qs, hipStream_t s) {
  switch (vbits) {
    case 2: return launch_partial_m<KB, 2, D>(a, qs, s);
    case 3: return launch_partial_m<KB, 3, D>(a, qs, s);
    case 4: return launch_partial_m<KB, 4, D>(a, qs, s);
    case 8: return launch_partial_m<KB, 8, D>(a, qs, s);
    case 16: return launch_partial_m<KB, 16, D>(a, qs, s);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
hipError_t dispatch_k(const DecodeArgs& a, int kbits, int vbits, float qs, hipStream_t s) {
  switch (kbits) {
    case 2: return dispatch_v<2, D>(a, vbits, qs, s);
    case 3: return dispatch_v<3, D>(a, vbits, qs, s);
    case 4: return dispatch_v<4, D>(a, vbits, qs, s);
    case 8: return dispatch_v<8, D>(a, vbits, qs, s);
    case 16: return dispatch_v<16, D>(a, vbits, qs, s);
    default: return hipErrorInvalidValue;
  }
}

template <int KB, int D>
int waves_v(int vbits) {
  switch (vbits) {
    case 2: return PartialWaves<KB, 2, D>::value;
    case 3: return PartialWaves<KB, 3, D>::value;
    case 4: return PartialWaves<KB, 4, D>::value;
    case 8: return PartialWaves<KB, 8, D>::value;
    default: return PartialWaves<KB, 16, D>::value;
  }
}

template <int D, bool M16>
hipError_t launch_multi_t(const DecodeArgs& a, float qscale, hipStream_t s) {
  unsigned grid = 0;
  for (int i = 0; i < a.n_segs; ++i) {
    const DecodeSeg& sg = a.seg[i];
    if (sg.n_splits % kXcds != 0 || sg.grid_start != static_cast<int>(grid)) return hipErrorInvalidValue;
    grid += static_cast<unsigned>(sg.n_splits) * sg.n_heads * a.batch;
  }
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((decode_partial_multi_kernel<D, M16>), dim3(grid), dim3(64), 0, s, a, qscale);
  return hipGetLastError();
}

template <int KB, int VB, int D>
hipError_t launch_kc_partial_t(const DecodeArgs& a, float qscale, hipStream_t s) {
  const unsigned grid = single_grid(a);
  if (grid == 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL((decode_partial_kc_kernel<KB, VB, D>), dim3(grid), dim3(64), 0, s, a, a.seg[0].table,
                     a.seg[0].steal, qscale);
  return hipGetLastError();
}

template <int KB, int D>
hipError_t dispatch_kc_v(const DecodeArgs& a, int vbits, float qs, hipStream_t s) {
  switch (vbits) {
    case 2: return launch_kc_partial_t<KB, 2, D>(a, qs, s);
    case 3: return launch_kc_partial_t<KB, 3, D>(a, qs, s);
    case 4: return launch_kc_partial_t<KB, 4, D>(a, qs, s);
    case 8: return launch_kc_partial_t<KB, 8, D>(a, qs, s);
    case 16: return launch_kc_partial_t<KB, 16, D>(a, qs, s);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
hipError_t dispatch_kc_k(const DecodeArgs& a, int kbits, int vbits, float qs, hipStream_t s) {
  switch (kbits) {
    case 2: return dispatch_kc_v<2, D>(a, vbits, qs, s);
    case 3: return dispatch_kc_v<3, D>(a, vbits, qs, s);
    case 4: return dispatch_kc_v<4, D>(a, vbits, qs, s);
    case 8: return dispatch_kc_v<8, D>(a, vbits, qs, s);
    default: return hipErrorInvalidValue;
  }
}

template <int KB, int D>
int kc_waves_v(int vbits) {
  switch (vbits) {
    case 2: return KcWaves<KB, 2, D>::value;
    case 3: return KcWaves<KB, 3, D>::value;
    case 4: return KcWaves<KB, 4, D>::value;
    case 8: return KcWaves<KB, 8, D>::value;
    default: return KcWaves<KB, 16, D>::value;
  }
}

template <int D>
int kc_waves_k(int kbits, int vbits) {
  switch (kbits) {
    case 2: return kc_waves_v<2, D>(vbits);
    case 3: return kc_waves_v<3, D>(vbits);
    case 4: return kc_waves_v<4, D>(vbits);
    default: return kc_waves_v<8, D>(vbits);
  }
}

template <int D>
int waves_k(int kbits, int vbits) {
  switch (kbits) {
    case 2: return waves_v<2, D>(vbits);
    case 3: return waves_v<3, D>(vbits);
    case 4: return waves_v<4, D>(vbits);
    case 8: return waves_v<8, D>(vbits);
    default: return waves_v<16, D>(vbits);
  }
}

}  // namespace

int decode_partial_waves_per_simd(int kbits, int vbits, int d, bool kc) {
  if (kc && kbits != 16) return d == 64 ? kc_waves_k<64>(kbits, vbits) : kc_waves_k<128>(kbits, vbits);
  return d == 64 ? waves_k<64>(kbits, vbits) : waves_k<128>(kbits, vbits);
}

hipError_t launch_decode_partial(const DecodeArgs& a, int kbits, int vbits, int d, hipStream_t s) {
  if (a.n_segs != 1 || a.seg[0].n_splits == 0 || a.batch == 0 || a.seg[0].n_heads == 0) return hipSuccess;
  // q~ = (R q) * log2(e) / sqrt(d), with R's 1/sqrt(n) folded in.
  const float qscale = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(a.had_block) * d));
  if (a.kc && kbits != 16) {
    if (d == 128) return dispatch_kc_k<128>(a, kbits, vbits, qscale, s);
    if (d == 64) return dispatch_kc_k<64>(a, kbits, vbits, qscale, s);
    return hipErrorInvalidValue;
  }
  if (d == 128) return dispatch_k<128>(a, kbits, vbits, qscale, s);
  if (d == 64) return dispatch_k<64>(a, kbits, vbits, qscale, s);
  return hipErrorInvalidValue;
}

bool decode_partial_mixable(int kbits, int vbits, int d) {
  return (d == 64 || d == 128) && kbits >= 2 && kbits <= 4 && vbits >= 2 && vbits <= 4;
}

hipError_t launch_decode_partial_multi(const DecodeArgs& a, int d, hipStream_t s) {
  if (a.batch == 0 || a.n_segs == 0) return hipSuccess;
  if (a.kc || a.n_segs > kMaxLaunchSegs) return hipErrorInvalidValue;
  for (int i = 0; i < a.n_segs; ++i)
    for (int j = 0; j < a.seg[i].n_heads; ++j) {
      const int e = a.seg[i].head_base + j;
      if (e < 0 || e >= KVQ_MAX_KV_HEADS || !decode_partial_mixable(a.pair[e] >> 4, a.pair[e] & 15, d))
        return hipErrorInvalidValue;
    }
  const float qscale = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(a.had_block) * d));
  if (d == 128) return a.meta16 ? launch_multi_t<128, true>(a, qscale, s) : launch_multi_t<128, false>(a, qscale, s);
  if (d == 64) return a.meta16 ? launch_multi_t<64, true>(a, qscale, s) : launch_multi_t<64, false>(a, qscale, s);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_merge(const MergeArgs& a, hipStream_t s) {
  if (a.batch * a.hq == 0) return hipSuccess;
  const float rs = static_cast<float>(1.0 / std::sqrt(static_cast<double>(a.had_block)));
  dim3 grid(a.batch * a.hq);
  // long slot lists (batch 1 at long context) get sixteen waves, so the
  // latency-bound loop runs a few trips per wave
  const bool many = a.total_slots >= 128;
  if (a.d == 128 && many) hipLaunchKernelGGL((decode_merge_kernel<128, 16>), grid, dim3(1024), 0, s, a, rs);
  else if (a.d == 128) hipLaunchKernelGGL((decode_merge_kernel<128, 4>), grid, dim3(256), 0, s, a, rs);
  else if (a.d == 64 && many) hipLaunchKernelGGL((decode_merge_kernel<64, 16>), grid, dim3(1024), 0, s, a, rs);
  else if (a.d == 64) hipLaunchKernelGGL((decode_merge_kernel<64, 4>), grid, dim3(256), 0, s, a, rs);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}


namespace {
__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, size_t n) {
  for (size_t i = blockIdx.x * 256ull + threadIdx.x; i < n; i += 256ull * gridDim.x) p[i] = 0u;
}
}  // namespace

hipError_t launch_zero_words(uint32_t* p, size_t n_words, hipStream_t s) {
  const size_t blocks = std::min<size_t>((n_words + 255) / 256, 4096);
  hipLaunchKernelGGL(zero_words_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, p, n_words);
  return hipGetLastError();
}

}  // namespace kvq
