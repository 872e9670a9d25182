// Decode attention over keys quantized per channel (one {s, mn} pair per
// channel and 16-token block) and values per token. Same partial format as
// the MFMA kernel in kvq_decode.hip, so the same merge follows.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

namespace {

// ---------------------------------------------------------------------------
// Decode over per-channel keys (the KIVI/Quanto key granularity of the
// RateQuant summary, Methodology 3, and the LogQuant summary, Methodology 5).
// A key's dequantized value is code * s_c + mn_c with a {s, mn} pair per
// channel and block, so the scale cannot be folded into one offset per token
// as in the row layout; this kernel dequantizes and multiplies on the VALU in
// fp32. One wave per (sequence, KV head, split), each split a contiguous run
// of blocks. Scores: lane = (token t = lane % 16, channel quarter lane / 16),
// summed over the quarters by xor shuffles. Online softmax in log2 units as
// in the MFMA kernel, same partial format, so the same merge follows. Values
// (per token): lane l owns channels [l*D/64, (l+1)*D/64) and accumulates
// p_t * v_hat_t over the block's tokens.
// ---------------------------------------------------------------------------
// Blocks in flight while one is computed: each wave holds a few KB of loads in
// flight, and enough of them keep the memory system busy despite the short
// compute per block.
constexpr int kKcDepth = 4;

// One block's data for one lane, loaded a block ahead of its use.
template <int KB, int VB, int D>
struct KcBlock {
  static constexpr int CPQ = D / 4;
  static constexpr int NWQ = (31 + CPQ * KB) / 32 + 1;            // aligned words a quarter row can span
  static constexpr int CPL = D / 64;
  static constexpr int VW = (32 % (CPL * VB) == 0 || VB == 16) ? 1 : 2;  // words per value token (3-bit straddles)
  float4 kmeta;            // the block's key channel pairs {s, mn} of channels 2 * lane, 2 * lane + 1
  uint32_t kw[NWQ + 1];    // key codes of this lane's (token, quarter)
  uint32_t vw[16][VW];     // per token: the word(s) holding this lane's value channels
  float2 vmeta;            // lane < 16: {s, mn} of value token `lane`
  int ok;                  // the block is mapped
};

// Loads of block `page` of the split [p_lo, p_hi); a position past p_hi loads
// block 0 and is marked empty, so every position issues the same loads.
template <int KB, int VB, int D>
__device__ __forceinline__ void kc_load(const DecodeArgs& a, const int32_t* trow, int page, int p_hi, uint32_t nblk,
                                        int lane, int64_t koff, int64_t voff, KcBlock<KB, VB, D>& g) {
  using KBL = KcBlock<KB, VB, D>;
  constexpr int RBK = D * KB / 8, RBV = D * VB / 8;
  const int32_t blk = page < p_hi ? trow[page] : -1;
  g.ok = static_cast<uint32_t>(blk) < nblk;
  // (an unmapped block reads block 0 and is skipped, so the loads are the same every time)
  const uint8_t* base = a.pool + (g.ok ? blk : 0) * a.block_bytes;
  const uint8_t* kb = base + koff;
  const uint8_t* vb = base + voff;
  const int t = lane & 15, qq = lane >> 4;
  g.kmeta = lane < D / 2 ? reinterpret_cast<const float4*>(kb + kBlockTokens * RBK)[lane] : make_float4(0, 0, 0, 0);
  const uint32_t* kwp = reinterpret_cast<const uint32_t*>(kb + t * RBK) + ((qq * KBL::CPQ * KB) >> 5);
#pragma unroll
  for (int i = 0; i < KBL::NWQ; ++i) g.kw[i] = kwp[i];
  g.kw[KBL::NWQ] = 0u;
  const int bit = lane * KBL::CPL * VB;
#pragma unroll
  for (int tt = 0; tt < 16; ++tt) {
    const uint32_t* row = reinterpret_cast<const uint32_t*>(vb + tt * RBV);
    g.vw[tt][0] = row[bit >> 5];
    if constexpr (KBL::VW == 2) g.vw[tt][1] = ((bit >> 5) + 1) * 4 < RBV ? row[(bit >> 5) + 1] : 0u;
  }
  g.vmeta = (VB != 16 && lane < 16) ? reinterpret_cast<const float2*>(vb + kBlockTokens * RBV)[lane]
                                    : make_float2(1.f, 0.f);
}

template <int KB, int VB, int D>
__global__ __launch_bounds__(64) void decode_kc_kernel(DecodeArgs a, const int32_t* __restrict__ table,
                                                       float qscale, int n_splits) {
  using KBL = KcBlock<KB, VB, D>;
  constexpr int CPQ = KBL::CPQ, CPL = KBL::CPL;
  constexpr float NEG_INF = -__builtin_huge_valf();
  __shared__ float4 qt[D];                 // q~ of the four query rows, channel-major
  __shared__ float qs[4][D];               // (rotation workspace)
  __shared__ __attribute__((aligned(16))) float2 kms[D];  // the current block's key channel metadata
  __shared__ float2 vms[16];               // the current block's value metadata
  const int lane = threadIdx.x;
  const int split = static_cast<int>(blockIdx.x) % n_splits;
  const int unit = static_cast<int>(blockIdx.x) / n_splits;
  const int hidx = unit % a.n_heads, b = unit / a.n_heads;
  const int h = a.heads[hidx], G = a.group, hq = a.hkv * G;
  const int seq_len = a.seq_lens[b];
  const int pages = min((seq_len + kBlockTokens - 1) / kBlockTokens, a.table_stride);
  const int pps = (pages + n_splits - 1) / n_splits;
  const int p_lo = min(split * pps, pages), p_hi = min(p_lo + pps, pages);
  const int32_t* trow = table + static_cast<int64_t>(b) * a.table_stride;
  const uint32_t nblk = a.pool_blocks > 0x7fffffff ? 0x80000000u : static_cast<uint32_t>(a.pool_blocks);
  const int64_t koff = a.k_off[hidx], voff = a.v_off[hidx];

  constexpr int NB = kKcDepth + 1;
  KBL gb[NB];
#pragma unroll
  for (int j = 0; j < kKcDepth; ++j) kc_load<KB, VB, D>(a, trow, p_lo + j, p_hi, nblk, lane, koff, voff, gb[j]);

  // ---- q~ = (R q) * log2(e) / sqrt(d) (R's 1/sqrt(n) folded into qscale) ----
  {
    const int64_t qrow0 = static_cast<int64_t>(b) * hq + h * G;
    for (int e = lane; e < 4 * D; e += 64) {
      const int r = e / D, c = e % D;
      float v = 0.f;
      if (r < G) {
        const int64_t idx = (qrow0 + r) * D + c;
        v = a.q_bf16 ? bf16lo_to_f(static_cast<const uint16_t*>(a.q)[idx]) : static_cast<const float*>(a.q)[idx];
      }
      qs[r][c] = v;
    }
    __syncthreads();
    for (int st = 1; st < a.had_block; st <<= 1) {
      for (int pi = lane; pi < 2 * D; pi += 64) {
        const int r = pi / (D / 2), jj = pi % (D / 2);
        const int j = (jj / st) * 2 * st + (jj % st);
        const float u = qs[r][j], v = qs[r][j + st];
        qs[r][j] = u + v;
        qs[r][j + st] = u - v;
      }
      __syncthreads();
    }
    for (int c = lane; c < D; c += 64)
      qt[c] = make_float4(qs[0][c] * qscale, qs[1][c] * qscale, qs[2][c] * qscale, qs[3][c] * qscale);
    __syncthreads();
  }

  const int t = lane & 15, qq = lane >> 4;
  float m_run[4], l_part[4], o[4][CPL];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m_run[i] = -1e30f;
    l_part[i] = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) o[i][c] = 0.f;
  }
  auto compute = [&](KBL& g, int page) {
    if (!g.ok) return;
    const int tok0 = page * kBlockTokens;
    __syncthreads();  // the previous block's metadata has been read
    if (lane < D / 2) reinterpret_cast<float4*>(kms)[lane] = g.kmeta;
    if (lane < 16) vms[lane] = g.vmeta;
    __syncthreads();
    // ---- scores of the block's 16 tokens ----
    // (the quarter starts at bit 0 of its first word except at head_dim 64 with
    // 3-bit keys, where odd quarters start at bit 16: shift the words once, so
    // every code below sits at a compile-time bit position and the words stay
    // in registers)
    uint32_t kw[KBL::NWQ + 1];
    if constexpr ((CPQ * KB) % 32 == 0) {
#pragma unroll
      for (int i = 0; i <= KBL::NWQ; ++i) kw[i] = g.kw[i];
    } else {
      const int off = (qq * CPQ * KB) & 31;  // 0 or 16
#pragma unroll
      for (int i = 0; i < KBL::NWQ; ++i) kw[i] = off ? (g.kw[i] >> 16) | (g.kw[i + 1] << 16) : g.kw[i];
      kw[KBL::NWQ] = 0u;
    }
    float z[4] = {0.f, 0.f, 0.f, 0.f};
    // word by word (codes that start in word wi), so every register index is static
    constexpr int NWORDS = (CPQ * KB + 31) / 32;
#pragma unroll
    for (int wi = 0; wi < NWORDS; ++wi) {
      const uint64_t two = static_cast<uint64_t>(kw[wi]) | (static_cast<uint64_t>(kw[wi + 1]) << 32);
#pragma unroll
      for (int cl = (32 * wi + KB - 1) / KB; cl < CPQ && cl * KB < 32 * (wi + 1); ++cl) {
        const int c = qq * CPQ + cl;
        const float2 m = kms[c];
        const uint32_t code = static_cast<uint32_t>(two >> (cl * KB - 32 * wi)) & ((1u << KB) - 1u);
        const float kh = static_cast<float>(code) * m.x + m.y;
        const float4 qv = qt[c];
        z[0] = fmaf(qv.x, kh, z[0]);
        z[1] = fmaf(qv.y, kh, z[1]);
        z[2] = fmaf(qv.z, kh, z[2]);
        z[3] = fmaf(qv.w, kh, z[3]);
      }
    }
    const bool valid = tok0 + t < seq_len;
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[i] += __shfl_xor(z[i], 16, 64);
      z[i] += __shfl_xor(z[i], 32, 64);
      z[i] = valid ? z[i] : NEG_INF;
      const float gm = wave_max_scalar(z[i]);
      if (gm > m_run[i]) {  // wave-uniform
        const float alpha = __builtin_amdgcn_exp2f(m_run[i] - gm);
#pragma unroll
        for (int c = 0; c < CPL; ++c) o[i][c] *= alpha;
        l_part[i] *= alpha;
        m_run[i] = gm;
      }
      p[i] = __builtin_amdgcn_exp2f(z[i] - m_run[i]);
      if (qq == 0) l_part[i] += p[i];
    }
    // ---- values ----
    const int nvalid = min(kBlockTokens, seq_len - tok0);
    const int bit = (lane * CPL * VB) & 31;
#pragma unroll
    for (int tt = 0; tt < 16; ++tt) {
      if (tt < nvalid) {  // wave-uniform
        float vh[CPL];
        if constexpr (VB == 16) {
#pragma unroll
          for (int c = 0; c < CPL; ++c) vh[c] = bf16lo_to_f(g.vw[tt][0] >> (16 * ((lane * CPL + c) & 1)));
        } else {
          uint64_t two = g.vw[tt][0];
          if constexpr (KBL::VW == 2) two |= static_cast<uint64_t>(g.vw[tt][1]) << 32;
          const float2 vm = vms[tt];
#pragma unroll
          for (int c = 0; c < CPL; ++c) {
            const uint32_t code = static_cast<uint32_t>(two >> (bit + c * VB)) & ((1u << VB) - 1u);
            vh[c] = static_cast<float>(code) * vm.x + vm.y;
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pt = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, p[i]), tt));
#pragma unroll
          for (int c = 0; c < CPL; ++c) o[i][c] = fmaf(pt, vh[c], o[i][c]);
        }
      }
    }
  };
  // rotating block buffers (static indices: one trip covers NB positions)
  for (int base = p_lo; base < p_hi; base += NB) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      kc_load<KB, VB, D>(a, trow, base + j + kKcDepth, p_hi, nblk, lane, koff, voff, gb[(j + kKcDepth) % NB]);
      if (base + j < p_hi) compute(gb[j], base + j);
    }
  }

  // ---- partials (the MFMA kernel's format) ----
  const int slot = a.slot_base + split;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i >= G) break;
    const float lsum = wave_sum_scalar(l_part[i]);
    const int64_t bg = static_cast<int64_t>(b) * hq + h * G + i;
    float* po = a.part_o + (bg * a.total_slots + slot) * D + lane * CPL;
#pragma unroll
    for (int c = 0; c < CPL; ++c) po[c] = o[i][c];
    if (lane == 0) {
      float* ml = a.part_ml + (bg * a.total_slots + slot) * 2;
      ml[0] = lsum > 0.f ? m_run[i] : NEG_INF;
      ml[1] = lsum;
    }
  }
}

template <int KB, int VB, int D>
hipError_t launch_kc_t(const DecodeArgs& a, int n_splits, int batch, float qscale, hipStream_t s) {
  if (a.batch != batch) return hipErrorInvalidValue;
  dim3 grid(static_cast<unsigned>(n_splits) * a.n_heads * batch);
  hipLaunchKernelGGL((decode_kc_kernel<KB, VB, D>), grid, dim3(64), 0, s, a, a.table, qscale, n_splits);
  return hipGetLastError();
}

template <int KB, int D>
hipError_t dispatch_kc_v(const DecodeArgs& a, int vbits, int n_splits, int batch, float qs, hipStream_t s) {
  switch (vbits) {
    case 2: return launch_kc_t<KB, 2, D>(a, n_splits, batch, qs, s);
    case 3: return launch_kc_t<KB, 3, D>(a, n_splits, batch, qs, s);
    case 4: return launch_kc_t<KB, 4, D>(a, n_splits, batch, qs, s);
    case 8: return launch_kc_t<KB, 8, D>(a, n_splits, batch, qs, s);
    case 16: return launch_kc_t<KB, 16, D>(a, n_splits, batch, qs, s);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
hipError_t dispatch_kc(const DecodeArgs& a, int kbits, int vbits, int n_splits, int batch, float qs, hipStream_t s) {
  switch (kbits) {
    case 2: return dispatch_kc_v<2, D>(a, vbits, n_splits, batch, qs, s);
    case 3: return dispatch_kc_v<3, D>(a, vbits, n_splits, batch, qs, s);
    case 4: return dispatch_kc_v<4, D>(a, vbits, n_splits, batch, qs, s);
    case 8: return dispatch_kc_v<8, D>(a, vbits, n_splits, batch, qs, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_kc(const DecodeArgs& a, int kbits, int vbits, int d, int n_splits, int batch, float qscale,
                            hipStream_t s) {
  if (n_splits == 0 || batch == 0 || a.n_heads == 0) return hipSuccess;
  if (d == 128) return dispatch_kc<128>(a, kbits, vbits, n_splits, batch, qscale, s);
  if (d == 64) return dispatch_kc<64>(a, kbits, vbits, n_splits, batch, qscale, s);
  return hipErrorInvalidValue;
}

}  // namespace kvq
