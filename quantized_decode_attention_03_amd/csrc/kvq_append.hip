// Quantize-on-append and dequantize kernels for the paged INT-b KV cache.
//
// What is computed follows the SAW-INT4 summary page (gist.science/ar/paper/
// 2604.19157): section 2 (rotate each head row with a block-diagonal Hadamard
// matrix before quantizing, so outlier channels are spread out) and section 3
// (the rotation and quantization happen in one pass, fused with the cache
// write). Bits per head can differ between K and V and between heads, as in
// the RateQuant summary page (2605.06675), Methodology stage 3.
//
// Layout of work: a row is one (sequence, token, head) vector of head_dim
// values; d/8 consecutive lanes hold one row, 8 channels per lane
// ([8L, 8L+8) on lane L of the row). The Walsh-Hadamard butterflies run in
// registers for strides 1, 2, 4 and across lanes (xor shuffles) for strides
// 8 .. n/2. Row min/max reduce across the same lanes. Each lane then packs its
// 8 codes into b bytes, so a row's codes leave as one coalesced run of d*b/8
// bytes; lane 0 writes the row's {scale, min}.
#include "kvq_device.h"
#include "kvq_internal.h"

#include <cmath>

// Every multiply and add here rounds on its own (no fused multiply-add): the
// stored codes and the dequantized values are defined by separately rounded
// fp32 operations, e.g. x_hat = c * s + mn is a rounded product then a rounded sum.
#pragma clang fp contract(off)

namespace kvq {

namespace {

constexpr int kThreads = 256;

// In-place unnormalised Walsh-Hadamard transform over blocks of n channels,
// natural (Sylvester) order, for 8 channels per lane (fp32, used to undo the
// rotation when reading back).
__device__ __forceinline__ void fwht8(float (&x)[8], int lane_in_row, int n) {
#pragma unroll
  for (int st = 1; st < 8; st <<= 1) {
    if (st < n) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (!(j & st)) {
          const float u = x[j], v = x[j | st];
          x[j] = u + v;
          x[j | st] = u - v;
        }
      }
    }
  }
  for (int m = 1; m * 8 < n; m <<= 1) {
    const bool upper = (lane_in_row & m) != 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float y = shfl_xor(x[j], m);
      x[j] = upper ? (y - x[j]) : (x[j] + y);
    }
  }
}

// The same transform in fp64 for the write path. MI355X issues fp64 adds at
// the fp32 (non-packed) lane rate, and the sums of bf16 or fp32 inputs here are
// exact or nearly so in fp64, so rounding the result to fp32 reproduces the
// rotation's value (an explicit fp64 matrix product rounded to fp32) instead of
// accumulating fp32 rounding over log2(n) stages of cancellation.
__device__ __forceinline__ void fwht8_f64(double (&x)[8], int lane_in_row, int n) {
#pragma unroll
  for (int st = 1; st < 8; st <<= 1) {
    if (st < n) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (!(j & st)) {
          const double u = x[j], v = x[j | st];
          x[j] = u + v;
          x[j | st] = u - v;
        }
      }
    }
  }
  for (int m = 1; m * 8 < n; m <<= 1) {
    const double sgn = (lane_in_row & m) ? -1.0 : 1.0;  // lower: x + y, upper: y - x
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const double y = __shfl_xor(x[j], m, 64);
      x[j] = fma(sgn, x[j], y);
    }
  }
}

__device__ __forceinline__ void load8(const void* src, bool bf16, size_t elem, float (&x)[8]) {
  if (bf16) {
    const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + elem);
    x[0] = bf16lo_to_f(w.x); x[1] = bf16hi_to_f(w.x);
    x[2] = bf16lo_to_f(w.y); x[3] = bf16hi_to_f(w.y);
    x[4] = bf16lo_to_f(w.z); x[5] = bf16hi_to_f(w.z);
    x[6] = bf16lo_to_f(w.w); x[7] = bf16hi_to_f(w.w);
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(src) + elem);
    const float4 a = p[0], b = p[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

// Quantize 8 values with (mn, inv) and store this lane's BITS bytes.
template <int BITS>
__device__ __forceinline__ void quantize_store8(const float (&x)[8], float mn, float inv, uint8_t* dst) {
  float u[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) u[j] = (x[j] - mn) * inv;
  // v_cvt_pk_u8_f32 rounds half to even and saturates to [0, 255]; u lies in
  // [0, 2^b - 1 + 2^-22 (2^b - 1)], so the code is already in range.
  if constexpr (BITS == 8) {
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      w0 = __builtin_amdgcn_cvt_pk_u8_f32(u[j], j, w0);
      w1 = __builtin_amdgcn_cvt_pk_u8_f32(u[4 + j], j, w1);
    }
    *reinterpret_cast<uint2*>(dst) = make_uint2(w0, w1);
  } else if constexpr (BITS == 4) {
    uint32_t ev = 0, od = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ev = __builtin_amdgcn_cvt_pk_u8_f32(u[2 * j], j, ev);
      od = __builtin_amdgcn_cvt_pk_u8_f32(u[2 * j + 1], j, od);
    }
    *reinterpret_cast<uint32_t*>(dst) = ev | (od << 4);
  } else if constexpr (BITS == 2) {
    uint32_t ev = 0, od = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ev = __builtin_amdgcn_cvt_pk_u8_f32(u[2 * j], j, ev);
      od = __builtin_amdgcn_cvt_pk_u8_f32(u[2 * j + 1], j, od);
    }
    const uint32_t t = ev | (od << 2);              // byte m: c[2m] | c[2m+1] << 2
    const uint32_t v = (t | (t >> 4)) & 0x00ff00ffu; // byte 0: c0..c3, byte 2: c4..c7
    *reinterpret_cast<uint16_t*>(dst) = static_cast<uint16_t>((v & 0xffu) | ((v >> 8) & 0xff00u));
  } else {  // BITS == 3: 24 bits per lane, byte stores (lane offsets are 3-byte aligned)
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) w |= static_cast<uint32_t>(__builtin_rintf(u[j])) << (3 * j);
    dst[0] = static_cast<uint8_t>(w);
    dst[1] = static_cast<uint8_t>(w >> 8);
    dst[2] = static_cast<uint8_t>(w >> 16);
  }
}

template <int BITS, int D>
__global__ __launch_bounds__(kThreads) void append_kernel(AppendArgs a, double rs_n) {
  constexpr int LPR = D / 8;             // lanes per row
  constexpr int RPB = kThreads / LPR;    // rows per workgroup
  constexpr int RB = D * BITS / 8;       // bytes per stored row
  const int tid = threadIdx.x;
  const int lane = tid % LPR;
  const int row = blockIdx.x * RPB + tid / LPR;
  const int h = a.heads[blockIdx.y];
  const int64_t area = a.area_off[blockIdx.y];
  const int total = a.batch * a.n_new;
  const bool active = row < total;
  const int r = active ? row : 0;
  const int b = r / a.n_new;
  const int i = r - b * a.n_new;

  float x[8];
  const size_t elem = (static_cast<size_t>(r) * a.hkv + h) * D + lane * 8;
  load8(a.src, a.src_bf16 != 0, elem, x);

  double xd[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) xd[j] = static_cast<double>(x[j]);
  fwht8_f64(xd, lane, a.had_block);
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = static_cast<float>(xd[j] * rs_n);

  // Destination of this row; rows whose page is unmapped are skipped.
  const int p = a.start_pos[b] + i;
  const int page = p / kBlockTokens;
  bool store = active && p >= 0 && page < a.table_stride;
  int64_t blk = -1;
  if (store) {
    blk = a.table[static_cast<int64_t>(b) * a.table_stride + page];
    store = blk >= 0 && blk < a.pool_blocks;
  }
  const int slot = p - page * kBlockTokens;
  uint8_t* base = store ? a.pool + blk * a.block_bytes + area : nullptr;

  if constexpr (BITS == 16) {
    if (store) {
      uint4 w;
      w.x = f_to_bf16_rne(x[0]) | (f_to_bf16_rne(x[1]) << 16);
      w.y = f_to_bf16_rne(x[2]) | (f_to_bf16_rne(x[3]) << 16);
      w.z = f_to_bf16_rne(x[4]) | (f_to_bf16_rne(x[5]) << 16);
      w.w = f_to_bf16_rne(x[6]) | (f_to_bf16_rne(x[7]) << 16);
      *reinterpret_cast<uint4*>(base + slot * RB + lane * 16) = w;
    }
  } else {
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) { mn = fminf(mn, x[j]); mx = fmaxf(mx, x[j]); }
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) {
      mn = fminf(mn, shfl_xor(mn, m));
      mx = fmaxf(mx, shfl_xor(mx, m));
    }
    const float qmax = static_cast<float>((1 << BITS) - 1);
    const float rng = mx - mn;
    float s = 0.f, inv = 0.f;
    if (rng > 0.f) {
      s = rng / qmax;  // IEEE division (correctly rounded)
      inv = qmax / rng;
    }
    if (store) {
      quantize_store8<BITS>(x, mn, inv, base + slot * RB + lane * BITS);
      if (lane == 0)
        *reinterpret_cast<float2*>(base + kBlockTokens * RB + slot * kMetaBytes) = make_float2(s, mn);
    }
  }
}

// Read this lane's 8 stored values of one row back to fp32 (rotated basis).
template <int BITS>
__device__ __forceinline__ void load_row8(const uint8_t* rowp, const uint8_t* metap, int lane, float (&x)[8]) {
  if constexpr (BITS == 16) {
    const uint4 w = *reinterpret_cast<const uint4*>(rowp + lane * 16);
    x[0] = bf16lo_to_f(w.x); x[1] = bf16hi_to_f(w.x);
    x[2] = bf16lo_to_f(w.y); x[3] = bf16hi_to_f(w.y);
    x[4] = bf16lo_to_f(w.z); x[5] = bf16hi_to_f(w.z);
    x[6] = bf16lo_to_f(w.w); x[7] = bf16hi_to_f(w.w);
  } else {
    uint32_t lo = 0, hi = 0;
    const uint8_t* c = rowp + lane * BITS;
    if constexpr (BITS == 8) {
      const uint2 w = *reinterpret_cast<const uint2*>(c);
      lo = w.x; hi = w.y;
    } else if constexpr (BITS == 4) {
      lo = *reinterpret_cast<const uint32_t*>(c);
    } else if constexpr (BITS == 2) {
      lo = *reinterpret_cast<const uint16_t*>(c);
    } else {
      lo = c[0] | (static_cast<uint32_t>(c[1]) << 8) | (static_cast<uint32_t>(c[2]) << 16);
    }
    const float2 meta = *reinterpret_cast<const float2*>(metap);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t code;
      if constexpr (BITS == 8) code = ((j < 4 ? lo : hi) >> (8 * (j & 3))) & 0xffu;
      else code = (lo >> (BITS * j)) & ((1u << BITS) - 1u);
      x[j] = static_cast<float>(code) * meta.x + meta.y;  // two roundings (contraction is off)
    }
  }
}

template <int BITS, int D>
__global__ __launch_bounds__(kThreads) void dequant_kernel(DequantArgs a, float rs_n) {
  constexpr int LPR = D / 8;
  constexpr int RPB = kThreads / LPR;
  constexpr int RB = D * BITS / 8;
  const int tid = threadIdx.x;
  const int lane = tid % LPR;
  const int t = blockIdx.x * RPB + tid / LPR;
  const int h = a.heads[blockIdx.y];
  const int64_t area = a.area_off[blockIdx.y];
  const bool active = t < a.n;
  const int p = a.pos0 + (active ? t : 0);
  const int page = p / kBlockTokens;
  const int slot = p - page * kBlockTokens;
  const int64_t blk = a.table_row[page];
  const bool ok = active && blk >= 0 && blk < a.pool_blocks;

  float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (ok) {
    const uint8_t* base = a.pool + blk * a.block_bytes + area;
    load_row8<BITS>(base + slot * RB, base + kBlockTokens * RB + slot * kMetaBytes, lane, x);
  }
  if (!a.rotated) {
    fwht8(x, lane, a.had_block);  // H is symmetric: R^T applies the same butterflies
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = x[j] * rs_n;
  }
  if (active) {
    float4* o = reinterpret_cast<float4*>(a.out + (static_cast<size_t>(t) * a.hkv + h) * D + lane * 8);
    o[0] = make_float4(x[0], x[1], x[2], x[3]);
    o[1] = make_float4(x[4], x[5], x[6], x[7]);
  }
}

template <int BITS, int D>
hipError_t launch_append_t(const AppendArgs& a, double rs, hipStream_t s) {
  constexpr int RPB = kThreads / (D / 8);
  const int rows = a.batch * a.n_new;
  dim3 grid((rows + RPB - 1) / RPB, a.n_heads);
  hipLaunchKernelGGL((append_kernel<BITS, D>), grid, dim3(kThreads), 0, s, a, rs);
  return hipGetLastError();
}

template <int BITS, int D>
hipError_t launch_dequant_t(const DequantArgs& a, float rs, hipStream_t s) {
  constexpr int RPB = kThreads / (D / 8);
  dim3 grid((a.n + RPB - 1) / RPB, a.n_heads);
  hipLaunchKernelGGL((dequant_kernel<BITS, D>), grid, dim3(kThreads), 0, s, a, rs);
  return hipGetLastError();
}

float rsqrt_exact(int n) { return static_cast<float>(1.0 / std::sqrt(static_cast<double>(n))); }

}  // namespace

#define KVQ_BITS_SWITCH(BITS_VAL, D_VAL, CALL)                                   \
  switch ((BITS_VAL) * 1000 + (D_VAL)) {                                          \
    case 2064: return CALL(2, 64);   case 2128: return CALL(2, 128);             \
    case 3064: return CALL(3, 64);   case 3128: return CALL(3, 128);             \
    case 4064: return CALL(4, 64);   case 4128: return CALL(4, 128);             \
    case 8064: return CALL(8, 64);   case 8128: return CALL(8, 128);             \
    case 16064: return CALL(16, 64); case 16128: return CALL(16, 128);           \
    default: return hipErrorInvalidValue;                                         \
  }

hipError_t launch_append(const AppendArgs& a, int /*unused*/, hipStream_t s) {
  if (a.batch * a.n_new == 0 || a.n_heads == 0) return hipSuccess;
  const double rs = 1.0 / std::sqrt(static_cast<double>(a.had_block));
#define KVQ_APPEND_CALL(B_, D_) launch_append_t<B_, D_>(a, rs, s)
  KVQ_BITS_SWITCH(a.bits, a.d, KVQ_APPEND_CALL)
#undef KVQ_APPEND_CALL
}

hipError_t launch_dequant(const DequantArgs& a, hipStream_t s) {
  if (a.n == 0 || a.n_heads == 0) return hipSuccess;
  const float rs = rsqrt_exact(a.had_block);
#define KVQ_DEQUANT_CALL(B_, D_) launch_dequant_t<B_, D_>(a, rs, s)
  KVQ_BITS_SWITCH(a.bits, a.d, KVQ_DEQUANT_CALL)
#undef KVQ_DEQUANT_CALL
}

}  // namespace kvq
