// Internal interface between the libkvq host code and its kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

// One append launch: the K and V rows of a set of heads that share their
// (K bits, V bits) pair.
struct AppendArgs {
  uint8_t* pool;
  int64_t pool_blocks;
  int64_t block_bytes;
  const int32_t* table;
  int32_t table_stride;
  const int32_t* start_pos;
  const void* src[2];   // K, V: [batch][n_new][hkv][d]
  int32_t src_bf16;
  int32_t meta16;       // 1: float16 {s, mn} (4 bytes per row)
  int32_t key_per_channel;  // 1: keys are written per block by append_kc_kernel, not per row
  int32_t batch, n_new, hkv, d, had_block;
  int32_t n_heads;      // heads in this launch
  int32_t bits[2];      // append_kc_kernel: the key bits of the listed heads
  int32_t heads[KVQ_MAX_KV_HEADS];
  int64_t area_off[2][KVQ_MAX_KV_HEADS];  // byte offset of each listed head's K / V area in a block
  uint8_t head_bits[2][KVQ_MAX_KV_HEADS];  // append_kernel: K / V bits of each listed head
};

struct DequantArgs {
  const uint8_t* pool;
  int64_t pool_blocks;
  int64_t block_bytes;
  const int32_t* table_row;  // this sequence's table row
  int32_t pos0, n, hkv, d, had_block, rotated;
  int32_t meta16;
  int32_t kc;  // rows of a per-channel key area (metadata per channel)
  int32_t n_heads, bits;
  int32_t heads[KVQ_MAX_KV_HEADS];
  int64_t area_off[KVQ_MAX_KV_HEADS];
  float* out;  // [n][hkv][d]
};

// One partial-decode launch: one segment, the heads of that segment whose
// (K bits, V bits) pair is (kbits, vbits).
struct DecodeArgs {
  const uint8_t* pool;
  int64_t pool_blocks;
  int64_t block_bytes;
  const int32_t* table;
  int32_t table_stride;
  const int32_t* seq_lens;
  const void* q;       // [batch][hkv*group][d]
  int32_t q_bf16;
  int32_t meta16;      // 1: float16 {s, mn} (4 bytes per row)
  int32_t kc;          // 1: keys quantized per channel over each block (decode_partial_kc_kernel)
  int32_t hkv, group, had_block;
  int32_t batch;       // sequences (the grid covers batch x n_heads units)
  int32_t slot_base;   // first split slot of this segment
  int32_t total_slots; // split slots over all segments
  uint32_t* steal;     // [batch][hkv][2] work-sharing counters of this segment (zero between calls)
  int32_t share_tail;  // 1: most of each unit's groups go to whichever wave is free; 0: fixed order
  int32_t n_heads;
  int32_t heads[KVQ_MAX_KV_HEADS];
  int64_t k_off[KVQ_MAX_KV_HEADS];
  int64_t v_off[KVQ_MAX_KV_HEADS];
  uint8_t pair[KVQ_MAX_KV_HEADS];  // (key bits << 4) | value bits per listed head (multi-format launch)
  float* part_o;       // [batch][hq][total_slots][d]
  float* part_ml;      // [batch][hq][total_slots][2]  (running max in log2 units, sum)
};

// Distortion calibration: rows [rows][d] of fp32 or bf16, rotated and
// quantized at each listed width; squared errors summed into out[w].
constexpr int kMaxCalibWidths = 8;
struct QuantMseArgs {
  const void* x;
  int32_t x_bf16;
  int64_t rows;
  int32_t d, had_block;
  int32_t n_widths;
  int32_t widths[kMaxCalibWidths];
  double* out;  // [n_widths]
};

// LogQuant row moves: per sequence, window row -> middle row and middle row
// -> low row, re-encoded at the destination bits. Segment 0 window, 1
// middle, 2 low; area offsets are recomputed in the kernel from the bits.
constexpr int kRequantMaxSeqs = 64;
struct RequantSeg {
  uint8_t* pool;
  int64_t pool_blocks;
  int64_t block_bytes;
  const int32_t* table;
  int32_t table_stride;
  int32_t meta16;
  uint8_t bits[2][KVQ_MAX_KV_HEADS];  // K, V bits per head
};
struct RequantArgs {
  RequantSeg seg[3];
  int32_t hkv, d;
  int32_t seq0;                        // sequence index of moves[0]
  int32_t moves[kRequantMaxSeqs][4];   // win_slot, mid_slot, demote_slot, low_slot
};

struct MergeArgs {
  const float* part_o;
  const float* part_ml;
  int32_t batch, hq, d, had_block, total_slots;
  float* out;  // [batch][hq][d]
};

// Launchers return hipSuccess or the launch error; they never synchronise.
hipError_t launch_append(const AppendArgs& a, hipStream_t s);
// Per-channel keys of whole blocks (a.bits[0] < 16, n_new a multiple of 16).
hipError_t launch_append_kc(const AppendArgs& a, hipStream_t s);
hipError_t launch_dequant(const DequantArgs& a, hipStream_t s);
hipError_t launch_decode_partial(const DecodeArgs& a, int kbits, int vbits, int d, int n_splits,
                                 int batch, hipStream_t s);
hipError_t launch_decode_merge(const MergeArgs& a, hipStream_t s);
hipError_t launch_zero_words(uint32_t* p, size_t n_words, hipStream_t s);
// Zeroes out[], accumulates the squared errors, then divides by rows * d.
hipError_t launch_quant_mse(const QuantMseArgs& a, hipStream_t s);
hipError_t launch_requant(const RequantArgs& a, int n_seqs, hipStream_t s);

// Waves per SIMD the partial kernel for (kbits, vbits, d) is compiled to hold
// (kc: keys quantized per channel).
int decode_partial_waves_per_simd(int kbits, int vbits, int d, bool kc);
// Whether heads of this format can share a multi-format launch (2-, 3- and
// 4-bit keys and values, head_dim 64 or 128, per-token keys).
bool decode_partial_mixable(int kbits, int vbits, int d);
// One launch over heads of several formats: a.pair[i] names head i's widths,
// every pair mixable. Same grid, partials and counters as launch_decode_partial.
hipError_t launch_decode_partial_mixed(const DecodeArgs& a, int d, int n_splits, int batch, hipStream_t s);

}  // namespace kvq
