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
  // row r of the launch is new token r % n_new of sequence r / n_new; the
  // quotient is floor(r * n_new_magic / 2^(32 + n_new_shift)) plus at most one
  // for r < 2^31 (filled by launch_append: n_new_shift = floor(log2 n_new),
  // n_new_magic = floor((2^(32 + n_new_shift) - 1) / n_new), below 2^32)
  uint32_t n_new_magic;
  int32_t n_new_shift;
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

// One segment's share of a partial-decode launch: its pool, table and
// lengths, the heads of it the launch covers (entries head_base ..
// head_base + n_heads - 1 of DecodeArgs' head arrays), its splits, and where
// its workgroups start in the launch's one-dimensional grid.
constexpr int kMaxLaunchSegs = 4;
struct DecodeSeg {
  const uint8_t* pool;
  int64_t pool_blocks;
  int64_t block_bytes;
  const int32_t* table;
  int32_t table_stride;
  const int32_t* seq_lens;
  const int32_t* skip_pos;  // [batch] slot to mask (the token a fused append adds; the merge attends to it), or null
  uint32_t* steal;     // [batch][hkv][splits / 8][2] work-sharing counters of this segment (zero between calls)
  int32_t slot_base;   // first split slot of this segment
  int32_t n_splits;    // splits per (sequence, KV head), a multiple of 8
  int32_t grid_start;  // first workgroup of this segment (a multiple of 8)
  int32_t n_heads;
  int32_t head_base;
  int32_t write_q;     // 1: the waves of split 0 write their unit's q~ to qrot
};

// The one token per sequence a fused append adds (kvq_append_decode_attn):
// row b of k_new and v_new is quantized into the segment's pool at slot
// start_pos[b] exactly as the append kernel would, by the partial launch's
// split-0 wave of each (sequence, KV head) (the wave that writes q~), which
// also leaves the token's dequantized rotated K and V rows in the workspace
// (anew); the merge kernel attends to the token from those rows when its slot
// is mapped and below the segment's min(seq_lens[b], max_len). The partial
// launch or the window scan masks that slot.
struct TokenAppend {
  uint8_t* pool;  // null: no fused append
  int64_t pool_blocks;
  int64_t block_bytes;
  const int32_t* table;
  int32_t table_stride;
  const int32_t* seq_lens;
  const int32_t* start_pos;
  const void* k_new;  // [batch][hkv][d], bf16 or fp32
  const void* v_new;
  int32_t src_bf16, meta16, max_len;
  double rs_n;  // 1 / sqrt(had_block)
  int32_t k_off[KVQ_MAX_KV_HEADS];
  int32_t v_off[KVQ_MAX_KV_HEADS];
  uint8_t bits_k[KVQ_MAX_KV_HEADS];
  uint8_t bits_v[KVQ_MAX_KV_HEADS];
};

// One partial-decode launch over the listed heads of one or more segments.
// A single-format launch has one segment whose heads all share (kbits, vbits);
// the multi-format launch takes heads of 2-, 3- and 4-bit pairs from several
// segments (pair[i] names head entry i's widths).
struct DecodeArgs {
  const void* q;       // [batch][hkv*group][d]
  int32_t q_bf16;
  int32_t meta16;      // 1: float16 {s, mn} (4 bytes per row)
  int32_t kc;          // 1: keys quantized per channel over each block (decode_partial_kc_kernel)
  int32_t hkv, group, had_block;
  int32_t batch;
  int32_t total_slots; // split slots over all segments of the call
  int32_t share_tail;  // 1: most of each unit's groups go to whichever wave is free; 0: fixed order
  int32_t n_segs;
  DecodeSeg seg[kMaxLaunchSegs];
  int32_t heads[KVQ_MAX_KV_HEADS];
  int64_t k_off[KVQ_MAX_KV_HEADS];
  int64_t v_off[KVQ_MAX_KV_HEADS];
  uint8_t pair[KVQ_MAX_KV_HEADS];  // (key bits << 4) | value bits per head entry
  float* part_o;       // [batch][hq][total_slots][d]
  float* part_ml;      // [batch][hq][total_slots][2]  (running max in log2 units, sum)
  float* qrot;         // [batch][hq][d]: q~ = (R q) log2(e) / sqrt(d), for a window segment the merge computes
  TokenAppend ap;      // a fused append (ap.pool set): done by the split-0 waves of the write_q segment
  float* anew;         // [batch][hkv][2][d]: the appended token's dequantized rotated K and V rows
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

// A short bf16 segment whose attention the merge kernel computes itself
// (every head 16-bit keys and values), from the q~ the partial launch left.
struct MergeWindow {
  const uint8_t* pool;     // null: no such segment
  int64_t pool_blocks;
  int64_t block_bytes;
  const int32_t* table;
  int32_t table_stride;
  const int32_t* seq_lens;
  const int32_t* skip_pos;  // [batch] slot a fused append fills (masked in the scan), or null
  int32_t max_len;
  int64_t k_off[KVQ_MAX_KV_HEADS];
  int64_t v_off[KVQ_MAX_KV_HEADS];
};

struct MergeArgs {
  const float* part_o;
  const float* part_ml;
  const float* qrot;
  int32_t batch, hq, d, had_block, total_slots, group;
  float* out;  // [batch][hq][d]
  MergeWindow win;
  TokenAppend ap;     // a fused append (ap.pool set): the token is attended to from anew
  const float* anew;  // [batch][hkv][2][d]
};

// Launchers return hipSuccess or the launch error; they never synchronise.
hipError_t launch_append(const AppendArgs& a, hipStream_t s);
// Per-channel keys of whole blocks (a.bits[0] < 16, n_new a multiple of 16).
hipError_t launch_append_kc(const AppendArgs& a, hipStream_t s);
hipError_t launch_dequant(const DequantArgs& a, hipStream_t s);
// One segment (a.seg[0], a.n_segs = 1) whose heads all have widths (kbits, vbits).
hipError_t launch_decode_partial(const DecodeArgs& a, int kbits, int vbits, int d, hipStream_t s);
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
// One launch over heads of several formats and segments: a.pair[i] names
// head entry i's widths, every pair mixable; each segment's workgroups are
// a.seg[s].n_splits * n_heads * batch, from a.seg[s].grid_start.
hipError_t launch_decode_partial_multi(const DecodeArgs& a, int d, hipStream_t s);
// Window segments the merge can take: up to this many tokens.
constexpr int kMergeWindowMax = 512;

// Read-bandwidth references (measurement only): a streaming read of `bytes`
// by `waves` waves, and the partial decode kernel's load pattern over one
// segment with no compute (areas up to 2 KiB per head). Each wave writes one
// word to sink.
hipError_t launch_measure_stream(const void* buf, size_t bytes, uint32_t* sink, int waves, hipStream_t s);
// Whether measure_paged covers the layout: every head's K and V areas 16-byte
// multiples of 16 B to 2 KiB.
bool measure_paged_covers(const kvq_layout& L);
hipError_t launch_measure_paged(const kvq_segment& seg, int batch, int splits, uint32_t* sink, hipStream_t s);

}  // namespace kvq
