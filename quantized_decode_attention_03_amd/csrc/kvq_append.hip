// Quantize-on-append and dequantize kernels for the paged INT-b KV cache.
//
// What is computed follows the SAW-INT4 summary page (gist.science/ar/paper/
// 2604.19157): section 2 (rotate each head row with a block-diagonal Hadamard
// matrix before quantizing, so outlier channels are spread out) and section 3
// (the rotation and quantization happen in one pass, fused with the cache
// write). Bits per head can differ between K and V and between heads, as in
// the RateQuant summary page (2605.06675), Methodology stage 3.
//
// Layout of work (append): four lanes per row, each with d/4 contiguous
// channels (see append_rows). Dequantize (a read-back path, not the hot one):
// d/8 lanes per row, 8 channels per lane, butterflies across lanes by xor
// shuffles.
#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_rowq.h"

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

// ---------------------------------------------------------------------------
// Quantize-on-append. A row is one (sequence, token, head) vector of D values;
// four consecutive lanes hold it, lane m taking the contiguous channels
// [m*CPR, (m+1)*CPR), CPR = D/4. So a lane reads 2*CPR (bf16) or 4*CPR (fp32)
// contiguous bytes and writes its CPR*b/8 code bytes contiguously, and 16
// consecutive tokens of one head (one page) leave a wave as one run of codes.
// The Walsh-Hadamard butterflies of stride < CPR run in registers, the (at
// most two) strides CPR and 2*CPR between the four lanes through DPP quad
// permutations. The butterflies run in fp64: MI355X issues fp64 adds at the
// fp32 (non-packed) lane rate, and the +-1 sums of bf16 or fp32 inputs are
// exact in fp64, so scaling by 1/sqrt(n) and rounding to fp32 reproduces the
// rotation's value (an exact matrix product, one rounding).
// ---------------------------------------------------------------------------

// EARLY: the destination's reads go out around the row's load (the start
// position before it, the block-table entry after it), so they overlap the
// load and the rotation; otherwise both follow the rotation (fewer registers
// live across it, for the instance that covers every width).
template <int BITS, int D, bool EARLY = true>
__device__ __forceinline__ void append_rows(const AppendArgs& a, int half, double rs_n) {
  constexpr int LPR = 4, CPR = D / LPR;  // lanes per row, channels per lane
  constexpr int RPB = kThreads / LPR;    // rows per workgroup
  constexpr int RB = D * BITS / 8;       // bytes per stored row
  const int tid = threadIdx.x;
  const int m = tid & (LPR - 1);
  const int row = blockIdx.x * RPB + tid / LPR;
  const int h = a.heads[blockIdx.y];
  const int64_t area = a.area_off[half][blockIdx.y];
  const int total = a.batch * a.n_new;
  const bool active = row < total;
  const int r = active ? row : 0;
  // b = r / n_new by the invariant-divisor multiply: the estimate is the
  // quotient or one less (r < 2^31), so one correction makes it exact
  int b = static_cast<int>(__umulhi(static_cast<uint32_t>(r), a.n_new_magic) >> a.n_new_shift);
  int i = r - b * a.n_new;
  if (i >= a.n_new) {
    ++b;
    i -= a.n_new;
  }

  // destination: start position, then the block-table entry (clamped into the
  // row, read by every lane)
  int p = 0, page = 0;
  int32_t tab = -1;
  auto read_start = [&]() {
    p = a.start_pos[b] + i;
    page = p / kBlockTokens;
  };
  auto read_table = [&]() {
    tab = a.table[static_cast<int64_t>(b) * a.table_stride + min(max(page, 0), a.table_stride - 1)];
  };
  if constexpr (EARLY) read_start();

  // ---- load this lane's CPR channels ----
  float x[CPR];
  const size_t elem = (static_cast<size_t>(r) * a.hkv + h) * D + m * CPR;
  if (a.src_bf16) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.src[half]) + elem);
#pragma unroll
    for (int k = 0; k < CPR / 8; ++k) {
      const uint4 w = p[k];
      x[8 * k + 0] = bf16lo_to_f(w.x); x[8 * k + 1] = bf16hi_to_f(w.x);
      x[8 * k + 2] = bf16lo_to_f(w.y); x[8 * k + 3] = bf16hi_to_f(w.y);
      x[8 * k + 4] = bf16lo_to_f(w.z); x[8 * k + 5] = bf16hi_to_f(w.z);
      x[8 * k + 6] = bf16lo_to_f(w.w); x[8 * k + 7] = bf16hi_to_f(w.w);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(a.src[half]) + elem);
#pragma unroll
    for (int k = 0; k < CPR / 4; ++k) {
      const float4 w = p[k];
      x[4 * k + 0] = w.x; x[4 * k + 1] = w.y; x[4 * k + 2] = w.z; x[4 * k + 3] = w.w;
    }
  }

  if constexpr (EARLY) read_table();

  // ---- rotate ----
  rotate_row<CPR>(x, m, a.had_block, rs_n);

  if constexpr (!EARLY) {
    read_start();
    read_table();
  }
  // ---- destination; rows whose page is unmapped are skipped ----
  const int64_t blk = tab;
  const bool store = active && p >= 0 && page < a.table_stride && blk >= 0 && blk < a.pool_blocks;
  const int slot = p - page * kBlockTokens;
  uint8_t* dst = store ? a.pool + blk * a.block_bytes + area + slot * RB + m * (CPR * BITS / 8) : nullptr;

  if constexpr (BITS == 16) {
    if (store) store_row_bf16<CPR>(x, dst);
  } else {
    // ---- row min / max over the quad, the metadata, then the codes ----
    RowQ<CPR> q;
    quantize_row<BITS, CPR>(x, a.meta16 != 0, q);
    if (store) {
      uint8_t* meta = a.pool + blk * a.block_bytes + area + kBlockTokens * RB + slot * (a.meta16 ? 4 : kMetaBytes);
      store_row<BITS, CPR>(q, dst, meta, m, a.meta16 != 0);
    }
  }
}

// K rows (blockIdx.z == 0) at BK bits and V rows (blockIdx.z == 1) at BV bits
// of the listed heads, in one launch. BK = BV = 0: each workgroup takes its
// head's widths from the arguments (a uniform branch), so heads of different
// widths still share one launch; that instance is held to 168 registers (three
// waves per SIMD, like the fixed-width instances).
template <int BK, int BV, int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(BK == 0 ? 3 : 1)))
void append_kernel(AppendArgs a, double rs_n) {
  const int half = static_cast<int>(blockIdx.z);
  if constexpr (BK != 0) {
    if (half == 0) {
      if (BK == 16 || !a.key_per_channel) append_rows<BK, D>(a, 0, rs_n);  // else append_kc_kernel
    } else {
      append_rows<BV, D>(a, 1, rs_n);
    }
  } else {
    const int bits = a.head_bits[half][blockIdx.y];
    if (half == 0 && bits != 16 && a.key_per_channel) return;  // keys written by append_kc_kernel
    switch (bits) {
      case 2: append_rows<2, D, false>(a, half, rs_n); break;
      case 3: append_rows<3, D, false>(a, half, rs_n); break;
      case 4: append_rows<4, D, false>(a, half, rs_n); break;
      case 8: append_rows<8, D, false>(a, half, rs_n); break;
      default: append_rows<16, D, false>(a, half, rs_n); break;  // the host sends 2, 3, 4, 8 or 16
    }
  }
}

// ---------------------------------------------------------------------------
// Per-channel keys (the KIVI/Quanto key granularity named by the RateQuant
// summary, Methodology 3, and the LogQuant summary, Methodology 5): the 16
// keys of a block are rotated like any row, then every channel is quantized
// over the block's tokens with the row formulas along the token axis
// (fp32 min and max, s = (max - min) / (2^b - 1), codes rounded half to
// even). One wave per (block, head); lane l holds channels
// [l*D/64, (l+1)*D/64) of all 16 rows, so the channel statistics stay in the
// lane and the rotation's butterflies of stride >= D/64 cross lanes by xor
// shuffles (fp64, exact like the row path). Codes go through LDS and are
// packed as each row's bit-stream.
// ---------------------------------------------------------------------------
template <int BITS, int D>
__global__ __launch_bounds__(64) void append_kc_kernel(AppendArgs a, double rs_n) {
  constexpr int CPL = D / 64;
  constexpr int RB = D * BITS / 8;
  constexpr int WPR = RB / 4;  // 32-bit words per row
  __shared__ uint8_t codes[kBlockTokens][D];
  const int lane = threadIdx.x;
  const int blocks_per_seq = a.n_new / kBlockTokens;
  const int b = static_cast<int>(blockIdx.x) / blocks_per_seq;
  const int bi = static_cast<int>(blockIdx.x) % blocks_per_seq;
  const int h = a.heads[blockIdx.y];
  const int64_t area = a.area_off[0][blockIdx.y];
  const int start = a.start_pos[b];
  const int p0 = start + bi * kBlockTokens;
  const int page = p0 / kBlockTokens;
  // whole, mapped blocks only (the condition is the same for the whole wave)
  if (start < 0 || start % kBlockTokens != 0 || page >= a.table_stride) return;
  const int64_t blk = a.table[static_cast<int64_t>(b) * a.table_stride + page];
  if (blk < 0 || blk >= a.pool_blocks) return;
  uint8_t* base = a.pool + blk * a.block_bytes + area;

  float x[kBlockTokens][CPL];
#pragma unroll
  for (int t = 0; t < kBlockTokens; ++t) {
    const size_t elem = ((static_cast<size_t>(b) * a.n_new + bi * kBlockTokens + t) * a.hkv + h) * D + lane * CPL;
    double xd[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c)
      xd[c] = a.src_bf16 ? static_cast<double>(bf16lo_to_f(static_cast<const uint16_t*>(a.src[0])[elem + c]))
                         : static_cast<double>(static_cast<const float*>(a.src[0])[elem + c]);
    if constexpr (CPL == 2) {
      if (a.had_block >= 2) {
        const double u = xd[0], v = xd[1];
        xd[0] = u + v;
        xd[1] = u - v;
      }
    }
    for (int m = 1; m * CPL < a.had_block; m <<= 1) {
      const double sgn = (lane & m) ? -1.0 : 1.0;  // lower lane x + y, upper lane y - x
#pragma unroll
      for (int c = 0; c < CPL; ++c) xd[c] = fma(sgn, xd[c], __shfl_xor(xd[c], m, 64));
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) x[t][c] = static_cast<float>(xd[c] * rs_n);
  }
  const float qmax = static_cast<float>((1 << BITS) - 1);
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    float mn = x[0][c], mx = x[0][c];
#pragma unroll
    for (int t = 1; t < kBlockTokens; ++t) { mn = fminf(mn, x[t][c]); mx = fmaxf(mx, x[t][c]); }
    const float rng = mx - mn;
    float s = 0.f, inv = 0.f;
    if (rng > 0.f) {
      s = rng / qmax;
      inv = qmax / rng;
    }
#pragma unroll
    for (int t = 0; t < kBlockTokens; ++t)
      codes[t][lane * CPL + c] = static_cast<uint8_t>(fminf(fmaxf(__builtin_rintf((x[t][c] - mn) * inv), 0.f), qmax));
    *reinterpret_cast<float2*>(base + kBlockTokens * RB + (lane * CPL + c) * kMetaBytes) = make_float2(s, mn);
  }
  __syncthreads();
  for (int wi = lane; wi < kBlockTokens * WPR; wi += 64) {
    const int t = wi / WPR, w0 = 32 * (wi % WPR);
    uint64_t acc = 0;
    for (int j = w0 / BITS; j < D && j * BITS < w0 + 32; ++j) {
      const int o = j * BITS - w0;
      const uint64_t c = codes[t][j];
      acc |= o >= 0 ? (c << o) : (c >> (-o));
    }
    reinterpret_cast<uint32_t*>(base + t * RB)[wi % WPR] = static_cast<uint32_t>(acc);
  }
}

// ---------------------------------------------------------------------------
// Distortion calibration (RateQuant summary page, Methodology, "distortion
// calibration" and pipeline step 2: the distortion model alpha * beta^-b is
// fitted per quantizer from its measured mean squared error at a few widths).
// Each row goes through exactly the append path's rotation and quantizer, at
// every listed width b: x_hat = code * s + mn, and the error x_hat - x' of
// each element is squared and summed in fp64 (the difference of two fp32
// values and its square are exact there). Rows are spread over a fixed grid;
// each workgroup adds its sums to out[] with one fp64 atomic per width.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void quant_mse_kernel(QuantMseArgs a, double rs_n) {
  constexpr int LPR = 4, CPR = D / LPR, RPB = kThreads / LPR;
  constexpr int NW = kMaxCalibWidths;
  const int tid = threadIdx.x;
  const int m = tid & (LPR - 1);
  double acc[NW];
#pragma unroll
  for (int w = 0; w < NW; ++w) acc[w] = 0.0;
  // every lane runs the same trips (the quad butterflies need whole rows)
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * RPB; base < a.rows;
       base += static_cast<int64_t>(gridDim.x) * RPB) {
    const int64_t row = base + tid / LPR;
    const bool active = row < a.rows;
    const int64_t r = active ? row : 0;
    float x[CPR];
    const size_t elem = static_cast<size_t>(r) * D + m * CPR;
    if (a.x_bf16) {
      const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.x) + elem);
#pragma unroll
      for (int k = 0; k < CPR / 8; ++k) {
        const uint4 w = p[k];
        x[8 * k + 0] = bf16lo_to_f(w.x); x[8 * k + 1] = bf16hi_to_f(w.x);
        x[8 * k + 2] = bf16lo_to_f(w.y); x[8 * k + 3] = bf16hi_to_f(w.y);
        x[8 * k + 4] = bf16lo_to_f(w.z); x[8 * k + 5] = bf16hi_to_f(w.z);
        x[8 * k + 6] = bf16lo_to_f(w.w); x[8 * k + 7] = bf16hi_to_f(w.w);
      }
    } else {
      const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(a.x) + elem);
#pragma unroll
      for (int k = 0; k < CPR / 4; ++k) {
        const float4 w = p[k];
        x[4 * k + 0] = w.x; x[4 * k + 1] = w.y; x[4 * k + 2] = w.z; x[4 * k + 3] = w.w;
      }
    }
    rotate_row<CPR>(x, m, a.had_block, rs_n);
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int j = 1; j < CPR; ++j) { mn = fminf(mn, x[j]); mx = fmaxf(mx, x[j]); }
    mn = fminf(mn, dpp_f32<kDppQuadXor1>(mn));
    mx = fmaxf(mx, dpp_f32<kDppQuadXor1>(mx));
    mn = fminf(mn, dpp_f32<kDppQuadXor2>(mn));
    mx = fmaxf(mx, dpp_f32<kDppQuadXor2>(mx));
    const float rng = mx - mn;
    if (!active) continue;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      if (w >= a.n_widths) break;
      const float qmax = static_cast<float>((1 << a.widths[w]) - 1);
      float s = 0.f, inv = 0.f;
      if (rng > 0.f) {
        s = rng / qmax;
        inv = qmax / rng;
      }
      double sum = 0.0;
#pragma unroll
      for (int j = 0; j < CPR; ++j) {
        const float c = fminf(fmaxf(__builtin_rintf((x[j] - mn) * inv), 0.f), qmax);
        const float xh = c * s + mn;  // a rounded product, then a rounded sum
        const double e = static_cast<double>(xh) - static_cast<double>(x[j]);
        sum += e * e;
      }
      acc[w] += sum;
    }
  }
  // workgroup sums: the wave by xor shuffles, then the four waves through LDS
  __shared__ double part[kThreads / 64][NW];
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    double v = acc[w];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    if ((tid & 63) == 0) part[tid >> 6][w] = v;
  }
  __syncthreads();
  if (tid < a.n_widths) {
    double v = 0.0;
#pragma unroll
    for (int k = 0; k < kThreads / 64; ++k) v += part[k][tid];
    atomicAdd(a.out + tid, v);
  }
}

__global__ void quant_mse_finish_kernel(double* out, int n, double count) {
  if (static_cast<int>(threadIdx.x) < n) out[threadIdx.x] = out[threadIdx.x] / count;
}

// ---------------------------------------------------------------------------
// LogQuant row moves (LogQuant summary page, Methodology 2, dynamic
// adjustment): a token leaving the bf16 window is stored again at the middle
// precision, and a middle token leaving the log-spaced subset at the low
// precision. Workgroup (sequence, KV head), one wave per row: waves 0/1 move
// the K/V window row to the middle segment, waves 2/3 the K/V middle row to
// the low segment. Each source row is turned back into the values it holds
// (bf16, or code * s + mn), then quantized like a new row: token-wise min and
// max in fp32, s = (max - min) / (2^b - 1), codes rounded half to even. All
// four rows are read before any is written (the arriving token may take the
// demoted token's middle slot).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int64_t area_bytes(int d, int b, int meta16) {
  return static_cast<int64_t>(kBlockTokens) * (d * b / 8) + (b == 16 ? 0 : kBlockTokens * (meta16 ? 4 : kMetaBytes));
}

// Byte offset of head h's K (half 0) or V (half 1) area: the K areas of all
// heads come first, then the V areas.
__device__ __forceinline__ int64_t area_offset(const RequantSeg& sg, int hkv, int d, int half, int h) {
  int64_t off = 0;
  for (int i = 0; i < hkv; ++i) {
    if (half == 1) off += area_bytes(d, sg.bits[0][i], sg.meta16);
    else if (i < h) off += area_bytes(d, sg.bits[0][i], sg.meta16);
  }
  if (half == 1)
    for (int i = 0; i < h; ++i) off += area_bytes(d, sg.bits[1][i], sg.meta16);
  return off;
}

// The row of slot `slot` of sequence `seq` in segment sg (null if unmapped).
__device__ __forceinline__ uint8_t* seg_row(const RequantSeg& sg, int seq, int slot, int64_t area, int rb,
                                           uint8_t** meta) {
  const int page = slot / kBlockTokens;
  if (page >= sg.table_stride) return nullptr;
  const int64_t blk = sg.table[static_cast<int64_t>(seq) * sg.table_stride + page];
  if (blk < 0 || blk >= sg.pool_blocks) return nullptr;
  uint8_t* base = sg.pool + blk * sg.block_bytes + area;
  const int t = slot - page * kBlockTokens;
  *meta = base + kBlockTokens * rb + t * (sg.meta16 ? 4 : kMetaBytes);
  return base + t * rb;
}

__device__ __forceinline__ float wave_min_f(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fminf(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

template <int D>
__global__ __launch_bounds__(256) void requant_kernel(RequantArgs a) {
  constexpr int CPL = D / 64;  // channels per lane
  __shared__ uint8_t codes[4][D];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int si = blockIdx.x, h = blockIdx.y, seq = a.seq0 + si;
  const int half = wave & 1;
  const bool demote = wave >= 2;
  const RequantSeg& src = a.seg[demote ? 1 : 0];
  const RequantSeg& dst = a.seg[demote ? 2 : 1];
  const int src_slot = a.moves[si][demote ? 2 : 0], dst_slot = a.moves[si][demote ? 3 : 1];
  const int bs = src.bits[half][h], bd = dst.bits[half][h];
  const int rbs = D * bs / 8, rbd = D * bd / 8;
  uint8_t *smeta = nullptr, *dmeta = nullptr;
  const uint8_t* srow = nullptr;
  uint8_t* drow = nullptr;
  if (src_slot >= 0 && dst_slot >= 0) {
    srow = seg_row(src, seq, src_slot, area_offset(src, a.hkv, D, half, h), rbs, &smeta);
    drow = seg_row(dst, seq, dst_slot, area_offset(dst, a.hkv, D, half, h), rbd, &dmeta);
  }
  const bool active = srow != nullptr && drow != nullptr;  // wave-uniform

  // ---- the values the source row holds ----
  float x[CPL];
  if (active) {
    if (bs == 16) {
#pragma unroll
      for (int c = 0; c < CPL; ++c)
        x[c] = bf16lo_to_f(reinterpret_cast<const uint16_t*>(srow)[lane * CPL + c]);
    } else {
      float2 m;
      if (src.meta16) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(smeta);
        m = make_float2(f16_to_f(w & 0xffffu), f16_to_f(w >> 16));
      } else {
        m = *reinterpret_cast<const float2*>(smeta);
      }
      const uint32_t mask = (1u << bs) - 1u;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int o = (lane * CPL + c) * bs;
        const int byte = o >> 3;
        uint32_t v = srow[byte];
        if (byte + 1 < rbs) v |= static_cast<uint32_t>(srow[byte + 1]) << 8;
        const uint32_t code = (v >> (o & 7)) & mask;
        x[c] = static_cast<float>(code) * m.x + m.y;  // a rounded product, then a rounded sum
      }
    }
  }
  __syncthreads();  // every source row has been read

  // ---- quantize at the destination bits ----
  float s = 0.f, mn = 0.f;
  uint32_t meta_h = 0;
  if (active) {
    if (bd == 16) {
#pragma unroll
      for (int c = 0; c < CPL; ++c)
        reinterpret_cast<uint16_t*>(drow)[lane * CPL + c] = static_cast<uint16_t>(f_to_bf16_rne(x[c]));
    } else {
      float lmn = x[0], lmx = x[0];
#pragma unroll
      for (int c = 1; c < CPL; ++c) { lmn = fminf(lmn, x[c]); lmx = fmaxf(lmx, x[c]); }
      mn = wave_min_f(lmn);
      const float mx = wave_max_f(lmx);
      const float qmax = static_cast<float>((1 << bd) - 1);
      float inv = 0.f;
      if (dst.meta16) {  // float16 metadata: minimum down, scale up (as in the append kernel)
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
          s = rng / qmax;
          inv = qmax / rng;
        }
      }
#pragma unroll
      for (int c = 0; c < CPL; ++c)
        codes[wave][lane * CPL + c] =
            static_cast<uint8_t>(fminf(fmaxf(__builtin_rintf((x[c] - mn) * inv), 0.f), qmax));
    }
  }
  __syncthreads();
  // ---- pack the codes as the row's little-endian bit-stream and store ----
  if (active && bd != 16) {
    const int n_words = rbd / 4;
    if (lane < n_words) {
      const int w0 = 32 * lane;
      uint64_t acc = 0;
      for (int j = w0 / bd; j < D && j * bd < w0 + 32; ++j) {
        const int o = j * bd - w0;
        const uint64_t c = codes[wave][j];
        acc |= o >= 0 ? (c << o) : (c >> (-o));
      }
      reinterpret_cast<uint32_t*>(drow)[lane] = static_cast<uint32_t>(acc);
    }
    if (lane == 0) {
      if (dst.meta16) *reinterpret_cast<uint32_t*>(dmeta) = meta_h;
      else *reinterpret_cast<float2*>(dmeta) = make_float2(s, mn);
    }
  }
}

// Read this lane's 8 stored values of one row back to fp32 (rotated basis).
// metap: the row's {s, mn}, or with kc the first of the area's per-channel pairs.
template <int BITS>
__device__ __forceinline__ void load_row8(const uint8_t* rowp, const uint8_t* metap, bool meta16, bool kc, int lane,
                                          float (&x)[8]) {
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
    float2 meta = make_float2(0.f, 0.f);
    if (kc) {
    } else if (meta16) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(metap);
      meta = make_float2(f16_to_f(w & 0xffffu), f16_to_f(w >> 16));
    } else {
      meta = *reinterpret_cast<const float2*>(metap);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t code;
      if constexpr (BITS == 8) code = ((j < 4 ? lo : hi) >> (8 * (j & 3))) & 0xffu;
      else code = (lo >> (BITS * j)) & ((1u << BITS) - 1u);
      if (kc) meta = reinterpret_cast<const float2*>(metap)[lane * 8 + j];  // channel lane*8 + j
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
    const uint8_t* metap = base + kBlockTokens * RB + (a.kc ? 0 : slot * (a.meta16 ? 4 : kMetaBytes));
    load_row8<BITS>(base + slot * RB, metap, a.meta16 != 0, a.kc != 0, lane, x);
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

template <int BK, int BV, int D>
hipError_t launch_append_t(const AppendArgs& a, double rs, hipStream_t s) {
  constexpr int RPB = kThreads / 4;
  const int rows = a.batch * a.n_new;
  dim3 grid((rows + RPB - 1) / RPB, a.n_heads, 2);
  hipLaunchKernelGGL((append_kernel<BK, BV, D>), grid, dim3(kThreads), 0, s, a, rs);
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

template <int BK>
hipError_t launch_append_k(const AppendArgs& a, double rs, hipStream_t s) {
#define KVQ_APPEND_CALL(B_, D_) launch_append_t<BK, B_, D_>(a, rs, s)
  KVQ_BITS_SWITCH(a.head_bits[1][0], a.d, KVQ_APPEND_CALL)
#undef KVQ_APPEND_CALL
}

hipError_t launch_append(const AppendArgs& args, hipStream_t s) {
  if (args.batch * args.n_new == 0 || args.n_heads == 0) return hipSuccess;
  AppendArgs a = args;
  int l = 0;
  while ((int64_t{2} << l) <= a.n_new) ++l;  // floor(log2 n_new)
  a.n_new_shift = l;
  a.n_new_magic = static_cast<uint32_t>(((uint64_t{1} << (32 + l)) - 1) / static_cast<uint64_t>(a.n_new));
  bool uniform = true;
  for (int half = 0; half < 2; ++half)
    for (int i = 0; i < a.n_heads; ++i) {
      const int b = a.head_bits[half][i];
      if (b != 2 && b != 3 && b != 4 && b != 8 && b != 16) return hipErrorInvalidValue;
      uniform = uniform && b == a.head_bits[half][0];
    }
  const double rs = 1.0 / std::sqrt(static_cast<double>(a.had_block));
  if (!uniform) {
    if (a.d == 64) return launch_append_t<0, 0, 64>(a, rs, s);
    if (a.d == 128) return launch_append_t<0, 0, 128>(a, rs, s);
    return hipErrorInvalidValue;
  }
  switch (a.head_bits[0][0]) {
    case 2: return launch_append_k<2>(a, rs, s);
    case 3: return launch_append_k<3>(a, rs, s);
    case 4: return launch_append_k<4>(a, rs, s);
    case 8: return launch_append_k<8>(a, rs, s);
    default: return launch_append_k<16>(a, rs, s);
  }
}

hipError_t launch_quant_mse(const QuantMseArgs& a, hipStream_t s) {
  hipError_t e = launch_zero_words(reinterpret_cast<uint32_t*>(a.out), 2 * static_cast<size_t>(a.n_widths), s);
  if (e != hipSuccess) return e;
  constexpr int RPB = kThreads / 4;
  const int64_t want = (a.rows + RPB - 1) / RPB;
  const int blocks = static_cast<int>(want < 512 ? want : 512);
  const double rs = 1.0 / std::sqrt(static_cast<double>(a.had_block));
  if (a.d == 64) hipLaunchKernelGGL(quant_mse_kernel<64>, dim3(blocks), dim3(kThreads), 0, s, a, rs);
  else if (a.d == 128) hipLaunchKernelGGL(quant_mse_kernel<128>, dim3(blocks), dim3(kThreads), 0, s, a, rs);
  else return hipErrorInvalidValue;
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(quant_mse_finish_kernel, dim3(1), dim3(64), 0, s, a.out, a.n_widths,
                     static_cast<double>(a.rows) * a.d);
  return hipGetLastError();
}

hipError_t launch_requant(const RequantArgs& a, int n_seqs, hipStream_t s) {
  if (n_seqs <= 0 || a.hkv <= 0) return hipSuccess;
  const dim3 grid(n_seqs, a.hkv);
  if (a.d == 64) hipLaunchKernelGGL(requant_kernel<64>, grid, dim3(256), 0, s, a);
  else if (a.d == 128) hipLaunchKernelGGL(requant_kernel<128>, grid, dim3(256), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int BITS, int D>
hipError_t launch_append_kc_t(const AppendArgs& a, double rs, hipStream_t s) {
  const dim3 grid(a.batch * (a.n_new / kBlockTokens), a.n_heads);
  hipLaunchKernelGGL((append_kc_kernel<BITS, D>), grid, dim3(64), 0, s, a, rs);
  return hipGetLastError();
}

hipError_t launch_append_kc(const AppendArgs& a, hipStream_t s) {
  if (a.batch * a.n_new == 0 || a.n_heads == 0) return hipSuccess;
  if (a.n_new % kBlockTokens != 0) return hipErrorInvalidValue;
  const double rs = 1.0 / std::sqrt(static_cast<double>(a.had_block));
  switch (a.bits[0] * 1000 + a.d) {
    case 2064: return launch_append_kc_t<2, 64>(a, rs, s);
    case 2128: return launch_append_kc_t<2, 128>(a, rs, s);
    case 3064: return launch_append_kc_t<3, 64>(a, rs, s);
    case 3128: return launch_append_kc_t<3, 128>(a, rs, s);
    case 4064: return launch_append_kc_t<4, 64>(a, rs, s);
    case 4128: return launch_append_kc_t<4, 128>(a, rs, s);
    case 8064: return launch_append_kc_t<8, 64>(a, rs, s);
    case 8128: return launch_append_kc_t<8, 128>(a, rs, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_dequant(const DequantArgs& a, hipStream_t s) {
  if (a.n == 0 || a.n_heads == 0) return hipSuccess;
  const float rs = rsqrt_exact(a.had_block);
#define KVQ_DEQUANT_CALL(B_, D_) launch_dequant_t<B_, D_>(a, rs, s)
  KVQ_BITS_SWITCH(a.bits, a.d, KVQ_DEQUANT_CALL)
#undef KVQ_DEQUANT_CALL
}

}  // namespace kvq
