/*
 * kvq.h - C ABI of libkvq: quantize-on-append into a paged INT-b KV cache and
 * fused quantized decode attention for AMD Instinct MI355X (gfx950).
 *
 * Conventions (all entry points):
 *  - Every function returns kvq_status. KVQ_OK is 0. An argument error
 *    (KVQ_ERR_ARG, _UNSUPPORTED, _BUDGET, _WORKSPACE, _CAPACITY) is found
 *    before anything is launched or written. kvq_last_error() returns a
 *    message for the calling thread (valid until the next kvq call on that
 *    thread).
 *  - A call that makes several launches and gets KVQ_ERR_DEVICE from one of
 *    them may already have queued the launches before it (they then run). A
 *    decode call that forked work onto side streams joins them back to the
 *    caller's stream on every return path.
 *  - No C++ exception crosses this boundary.
 *  - "device" pointers are HIP device memory owned by the caller; the library
 *    never allocates, frees or retains device memory (the one exception is
 *    kvq_decode_attn_noalloc's fixed scratch array, below).
 *  - Device work is asynchronous on the caller's hipStream_t (0 = the null
 *    stream) with no implicit synchronisation. A launch failure is reported as
 *    KVQ_ERR_DEVICE.
 *  - Host functions are synchronous and need no GPU.
 *  - Process-wide state, all of it created once and then only read, except
 *    where noted: the device's compute-unit count (read once, sizes the split
 *    plan); per device, four side streams and their fork/join events, used by
 *    decode calls that make several partial launches (several segments, or
 *    heads whose widths cannot share one launch). Those calls hold a mutex
 *    while they enqueue, so such calls from different threads serialise on
 *    the host, and their side-stream work queues behind one another on the
 *    device. Calls that write different buffers are otherwise independent.
 *  - Inputs must be finite; results on NaN or Inf inputs are unspecified.
 *
 * Sources for what is computed (page titles as published on gist.science):
 *  [RQ]  "RateQuant" technical summary (paper 2605.06675), Methodology.
 *  [MKV] "Quantize What Counts: More for Keys, Less for Values" (2502.15075).
 *  [LQ]  "LogQuant: Log-Distributed 2-Bit Quantization of KV Cache with
 *        Superior Accuracy Preservation" (2503.19950), technical summary.
 *  [SAW] "SAW-INT4: System-Aware 4-Bit KV-Cache Quantization for Real-World
 *        LLM Serving" (2604.19157).
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_ABI_VERSION 6
#define KVQ_MAX_KV_HEADS 64
#define KVQ_BLOCK_TOKENS 16

typedef enum kvq_status {
  KVQ_OK = 0,
  KVQ_ERR_ARG = 1,         /* a null pointer, a bad size or an inconsistent argument */
  KVQ_ERR_UNSUPPORTED = 2, /* a valid request outside what is built (e.g. head_dim 96) */
  KVQ_ERR_BUDGET = 3,      /* bit budget infeasible or not spent exactly */
  KVQ_ERR_WORKSPACE = 4,   /* workspace smaller than kvq_decode_workspace_bytes */
  KVQ_ERR_DEVICE = 5,      /* a HIP call or kernel launch failed */
  KVQ_ERR_CAPACITY = 6     /* the page free list ran out */
} kvq_status;

typedef enum kvq_dtype {
  KVQ_F32 = 0,
  KVQ_BF16 = 1
} kvq_dtype;

typedef struct hipStream_t_opaque* kvq_stream; /* a hipStream_t */

/*
 * Cache geometry of one pool (one layer, or one precision segment of a layer).
 *
 * A pool is an array of blocks of block_bytes each; a block holds 16
 * consecutive tokens of one sequence for every KV head. Inside a block the K
 * areas of heads 0..Hkv-1 come first, then the V areas. One head's area is
 *     codes[16][head_dim * b / 8]  then  meta[16] { float scale; float min; }
 * where code j of a row occupies bits [j*b, j*b+b) of the row's little-endian
 * bit-stream. For b = 16 the area is bf16[16][head_dim] of the rotated row
 * (round half to even) and has no meta. With meta_fp16 = 1 the meta pairs are
 * { _Float16 scale; _Float16 min; } (4 bytes): the minimum is rounded down
 * and the scale up to float16 before the codes are computed from them, so
 * the codes still fit and the error stays within half a step (the rotated
 * values must lie within the float16 range). With key_per_channel = 1 (and
 * float32 metadata) a K area with b < 16 instead holds codes[16][head_dim*b/8]
 * then kmeta[head_dim] { float scale; float min; }: each channel of the
 * rotated keys is quantized over the block's 16 tokens (the KIVI/Quanto key
 * granularity [RQ: stage 3, KIVI's per-channel keys; LQ: Methodology 5]); V
 * areas stay per token. Per-head b may differ between heads
 * and between K and V [RQ: stage 3, K/V decoupling; MKV: more bits for keys];
 * uniform blocks follow [SAW: section 1, PagedAttention].
 */
typedef struct kvq_layout {
  /* inputs */
  int32_t num_kv_heads; /* Hkv, 1..KVQ_MAX_KV_HEADS */
  int32_t group;        /* G query heads per KV head (q-head g reads KV head g / G), 1..4 */
  int32_t head_dim;     /* d, 64 or 128 */
  int32_t had_block;    /* n, Hadamard block: power of two, 1 <= n <= d (1 = no rotation) */
  int32_t block_tokens; /* must be KVQ_BLOCK_TOKENS */
  int32_t meta_fp16;    /* 0: float32 {s, mn} (8 B per row), 1: float16 {s, mn} (4 B per row) */
  int32_t key_per_channel; /* 0: keys per token; 1: keys per channel over each block (needs meta_fp16 = 0) */
  int32_t bits_k[KVQ_MAX_KV_HEADS]; /* each in {2, 3, 4, 8, 16} */
  int32_t bits_v[KVQ_MAX_KV_HEADS];
  /* outputs of kvq_layout_init */
  int64_t k_off[KVQ_MAX_KV_HEADS]; /* byte offset of head h's K area in a block */
  int64_t v_off[KVQ_MAX_KV_HEADS];
  int64_t block_bytes;
} kvq_layout;

/* One precision segment of the cache, read by decode attention. All segments
 * passed together must share num_kv_heads, group, head_dim and had_block.
 * The attended set is the union of every segment's first seq_lens[b] tokens;
 * token order does not matter [LQ: Methodology 4, A.V = A_P.V_P]. */
typedef struct kvq_segment {
  const kvq_layout* layout;  /* host */
  const void* pool;          /* device, pool_blocks * layout->block_bytes bytes */
  int64_t pool_blocks;
  const int32_t* block_table;/* device, [batch][table_stride] physical block ids */
  int32_t table_stride;
  const int32_t* seq_lens;   /* device, [batch] tokens held by this segment */
  int32_t max_len;           /* host upper bound on seq_lens[] (sizes the grid) */
} kvq_segment;

int kvq_abi_version(void);
const char* kvq_status_str(kvq_status s);
const char* kvq_last_error(void);

/*
 * Host. Fill k_off, v_off and block_bytes from the inputs of *L.
 * Errors: KVQ_ERR_ARG for a null L, block_tokens != 16, meta_fp16 or key_per_channel not 0 or 1,
 * num_kv_heads or group out of range, a bit width outside {2,3,4,8,16}, had_block not a power of
 * two or not dividing head_dim; KVQ_ERR_UNSUPPORTED for head_dim not 64/128
 * or for key_per_channel together with meta_fp16.
 */
kvq_status kvq_layout_init(kvq_layout* L);

/*
 * Host. Greedy marginal-gain integer bit allocation [RQ: Methodology 1 and 3].
 * Minimises sum_i w[i] * D(b_i), D(b) = alpha * beta^-b, subject to
 * sum_i b_i = budget_bits, each b_i taken from ladder[0..n_ladder).
 * Every head starts at the smallest ladder width; each round gives one more
 * ladder step to the head with the largest weighted distortion drop per bit,
 * w_i (D(b) - D(b+)) / (b+ - b), among steps that fit the remaining budget
 * (ties: lowest index), until the budget is spent or no step fits.
 * In:  n >= 1 heads, w[n] > 0 (host), alpha > 0, beta > 1, ladder of
 *      1..16 distinct positive widths (any order), budget_bits.
 * Out: bits_out[n] (host), *leftover_out = unspent bits (may be null).
 * Errors: KVQ_ERR_ARG for bad arguments; KVQ_ERR_BUDGET if budget_bits is below
 * n*min(ladder) or above n*max(ladder) (nothing written), or if bits are left
 * over (the allocation found is still written).
 * Limitation: the rounds only move up, so a budget that some allocation
 * meets exactly can still end with bits left over when the only steps left
 * are wider than the remainder: n = 2, ladder {2,3,4,8}, budget 11 ends at
 * [4,4] with 3 bits left (KVQ_ERR_BUDGET), though [8,3] sums to 11. On
 * {2,3,4,8} a budget of at most 4 bits per head on average is always spent
 * exactly: while bits remain, some head is below 4, where one-bit steps
 * remain.
 */
kvq_status kvq_plan_bits(int32_t n, const float* w, double alpha, double beta,
                         const int32_t* ladder, int32_t n_ladder, int64_t budget_bits,
                         int32_t* bits_out, int64_t* leftover_out);

/*
 * Host. kvq_plan_bits over components that each have their own distortion
 * curve D_i(b) = alpha[i] * beta[i]^-b, sharing one budget [RQ: Methodology 3,
 * K/V decoupling: the keys and the values of every head are 2N separate
 * components with their own fitted curves, so one budget decides the split
 * between keys and values (Key results: 2.85 bits for keys, 2.15 for values
 * at 2.5 on average)]. Rounds, ties and stopping as in kvq_plan_bits, with
 * the drop per bit w_i (D_i(b) - D_i(b+)) / (b+ - b) of each component's own
 * curve. With every alpha[i] and beta[i] equal it returns what kvq_plan_bits
 * returns.
 * In:  alpha[n] > 0, beta[n] > 1 (host), the rest as kvq_plan_bits.
 * Out and errors: as kvq_plan_bits.
 */
kvq_status kvq_plan_bits_components(int32_t n, const float* w, const double* alpha,
                                    const double* beta, const int32_t* ladder, int32_t n_ladder,
                                    int64_t budget_bits, int32_t* bits_out,
                                    int64_t* leftover_out);

/*
 * Host. Least-squares fit of the distortion model D(b) = alpha * beta^-b to
 * measured mean squared errors, as ln mse = ln alpha - b ln beta [RQ:
 * Methodology 1 (the model) and 3 ("distortion calibration": the model is
 * fitted per quantizer, not assumed); Pipeline step 2 (fit at 5 widths)].
 * In:  n >= 2 points (host): widths[n] (not all equal), mse[n] > 0 finite.
 * Out: *alpha_out, *beta_out; *r2_out = coefficient of determination of the
 *      log-linear fit (may be null; 1 when every ln mse is equal).
 * Errors: KVQ_ERR_ARG (nothing written).
 */
kvq_status kvq_fit_distortion(int32_t n, const int32_t* widths, const double* mse,
                              double* alpha_out, double* beta_out, double* r2_out);

/*
 * Host. Ratio of the arithmetic to the geometric mean of the head
 * sensitivities w[n] > 0: the factor by which the optimal per-head
 * allocation lowers the weighted distortion against a uniform one, in the
 * continuous model [RQ: Methodology 1 (AM/GM bound); Significance (the ratio
 * as a predictor of when mixed precision pays)]. Computed in fp64.
 * Errors: KVQ_ERR_ARG (n < 1, null pointers, a w[i] not positive).
 */
kvq_status kvq_amgm_ratio(int32_t n, const float* w, double* ratio_out);

/*
 * Device, async. Calibration measurement for kvq_fit_distortion: the mean
 * squared error of this library's quantizer on `rows` rows of head_dim values
 * at each of the n_widths widths [RQ: Methodology 3, distortion calibration].
 * Each row x is rotated, x' = blockdiag(H_n) x, and quantized exactly as in
 * kvq_quantize_append (fp32 {s, mn}, round half to even), at every width b:
 * mse[w] = sum over rows and channels of (code * s + mn - x')^2 / (rows *
 * head_dim), the errors squared and summed in fp64. Since the rotation is
 * orthonormal this is also the error in the original basis (up to rounding).
 * In:  x device [rows][head_dim] of dtype; widths host [n_widths], each in
 *      1..8, 1 <= n_widths <= 8; had_block a power of two <= head_dim.
 * Out: mse_out device double [n_widths]. The sums are combined with fp64
 *      atomics, so the last bits may vary from call to call.
 * Errors: KVQ_ERR_ARG (null pointers, rows < 1, bad widths or had_block),
 * KVQ_ERR_UNSUPPORTED (head_dim not 64/128), KVQ_ERR_DEVICE.
 */
kvq_status kvq_quant_mse(const void* x, kvq_dtype dtype, int64_t rows, int32_t head_dim,
                         int32_t had_block, const int32_t* widths, int32_t n_widths,
                         double* mse_out, kvq_stream stream);

/*
 * Host. Precision class of each of `total` tokens (position 0 = oldest) for a
 * log-spaced long-context schedule [LQ: Methodology 2]: 0 = the newest
 * `window` tokens (kept in bf16); 1 = the log-spaced subset; 2 = the rest.
 * With r the distance behind the window, span k covers
 * r in [(2^k - 1) window, (2^(k+1) - 1) window) and keeps every 2^k-th token
 * from the span's start in class 1.
 * Out: cls_out[total] (host). Errors: KVQ_ERR_ARG for total < 0, window < 1
 * or a null cls_out with total > 0.
 */
kvq_status kvq_logquant_classes(int32_t total, int32_t window, int8_t* cls_out);

/*
 * LogQuant's dynamic schedule [LQ: Methodology 2, "dynamic adjustment"]: the
 * cache grows one token at a time and keeps three segments per sequence, the
 * newest `window` tokens in a window segment (a ring: position p in slot
 * p mod window), a middle-precision segment holding the log-spaced kept
 * tokens and a low-precision segment holding the rest. A token at position p
 * behind the window lies in span k (as in kvq_logquant_classes) and is kept
 * when p + 1 is a multiple of 2^k, so as it ages into older spans it can only
 * lose precision, and each span still keeps `window` tokens. At a length that
 * is a multiple of 2^K (K the oldest span present) the classes equal
 * kvq_logquant_classes. Appending token T moves token T - window out of the
 * window into the middle segment and demotes at most one middle token,
 * T - 2^k window with k = 1 + (number of trailing zero bits of T + 1), to the
 * low segment; that token's middle slot is reused for the arriving one.
 */
typedef struct kvq_lq_state {
  int32_t total;     /* tokens appended so far */
  int32_t window;    /* window size W >= 1 */
  int32_t n_mid;     /* tokens in the middle segment (slots 0 .. n_mid-1) */
  int32_t n_low;     /* tokens in the low segment (slots 0 .. n_low-1) */
  int32_t* mid_pos;  /* host [cap_mid]: the position each middle slot holds */
  int32_t cap_mid;
} kvq_lq_state;

typedef struct kvq_lq_move {
  int32_t win_slot;    /* window slot of the token leaving the window, -1: none */
  int32_t mid_slot;    /* middle slot it is stored into */
  int32_t demote_slot; /* middle slot of the token moving to the low segment, -1: none */
  int32_t low_slot;    /* low slot it is stored into */
  int32_t new_slot;    /* window slot that receives the appended token */
} kvq_lq_move;

/*
 * Host. Classes (0 window, 1 middle, 2 low) of `total` tokens under the
 * dynamic schedule above. Out: cls_out[total] (host).
 * Errors: KVQ_ERR_ARG for total < 0, window < 1 or a null cls_out (total > 0).
 */
kvq_status kvq_logquant_dynamic_classes(int32_t total, int32_t window, int8_t* cls_out);

/*
 * Host. State of a sequence whose first `total` tokens are already stored by
 * class (prefill): middle slots hold the class-1 positions in ascending
 * order, n_low = the class-2 count. st->mid_pos and st->cap_mid must be set;
 * the other fields are written.
 * Errors: KVQ_ERR_ARG (bad sizes, null pointers), KVQ_ERR_CAPACITY (more
 * middle tokens than cap_mid).
 */
kvq_status kvq_logquant_init(int32_t total, int32_t window, kvq_lq_state* st);

/*
 * Host. Plan the append of one token to each of `batch` sequences and
 * advance their states: moves_out[b] says which stored rows move (for
 * kvq_logquant_requant) and where the new token goes (for
 * kvq_quantize_append into the window segment, start_pos = new_slot).
 * Errors: KVQ_ERR_ARG (null pointers, a state whose mid_pos does not hold the
 * token to demote); KVQ_ERR_CAPACITY (the middle segment needs a slot beyond
 * cap_mid). On an error no state is changed.
 */
kvq_status kvq_logquant_advance(int32_t batch, kvq_lq_state* states, kvq_lq_move* moves_out);

/*
 * Device, async. Apply the row moves of one kvq_logquant_advance step
 * [LQ: Methodology 2]. For every sequence b and KV head: the window row in
 * slot win_slot is stored into middle slot mid_slot, and the middle row in
 * demote_slot into low slot low_slot, each re-encoded at the destination
 * head's bits from the values the source holds (bf16, or code * s + mn):
 * token-wise min/max quantization in fp32, round half to even, exactly as
 * kvq_quantize_append quantizes a rotated row. Every source row is read
 * before any destination row is written, so a demoted token's slot may
 * receive the arriving one in the same call. Run it before appending the new
 * token, whose window slot is the exiting token's.
 * In:  three segments (window, middle, low) of one geometry (heads, head_dim,
 *      had_block); their block tables must map every slot named;
 *      moves host [batch]. seq_lens and max_len of the segments are unused.
 * Errors: KVQ_ERR_ARG (null pointers, geometry mismatch, a slot outside a
 * table row), KVQ_ERR_UNSUPPORTED (a segment with per-channel keys),
 * KVQ_ERR_DEVICE.
 */
kvq_status kvq_logquant_requant(const kvq_segment* window, const kvq_segment* mid,
                                const kvq_segment* low, int32_t batch,
                                const kvq_lq_move* moves, kvq_stream stream);

/*
 * Host. Deterministic page allocation. For seq = 0..batch-1 in order, and
 * within a sequence for logical blocks ceil(old_len/16) .. ceil(new_len/16)-1
 * in order, set block_table[seq * table_stride + lb] = free_list[(*cursor)++].
 * All pointers are host. new_len[s] >= old_len[s] >= 0 and
 * ceil(new_len[s]/16) <= table_stride are required (KVQ_ERR_ARG).
 * KVQ_ERR_CAPACITY if the free list runs out (the table and cursor are then
 * left as they were before the call).
 */
kvq_status kvq_page_alloc(const int32_t* free_list, int32_t n_free, int32_t* cursor,
                          int32_t batch, const int32_t* old_len, const int32_t* new_len,
                          int32_t* block_table, int32_t table_stride);

/*
 * Device, async. Quantize-on-append [SAW: sections 2-3; RQ: stage 3].
 * For every sequence b < batch, new token i < n_new and KV head h, the row
 * x = k[b][i][h][:] (resp. v) is rotated, x' = blockdiag(H_n) x with H_n the
 * orthonormal Sylvester Hadamard matrix, then quantized token-wise in fp32:
 * mn = min x', mx = max x', s = (mx - mn) / (2^b - 1),
 * code = round_half_even((x' - mn) * (2^b - 1) / (mx - mn)) (s = 0 and codes 0
 * for a constant row), packed, and stored with {s, mn} at position
 * p = start_pos[b] + i: block block_table[b * table_stride + p / 16], slot p % 16.
 * For b = 16 the rotated row is stored as bf16. With key_per_channel the keys
 * of each block are quantized together, per channel over its 16 tokens (same
 * formulas along the token axis), so such appends write whole blocks: n_new
 * and every start_pos[b] must be multiples of 16. n_new is checked here; the
 * start positions live in device memory, which this asynchronous call does
 * not read on the host, so for a sequence whose start_pos is not a multiple
 * of 16 the kernel writes its values but no keys. kvq_append_check finds
 * such a sequence on the host copy of the positions before the launch.
 * In:  k, v device [batch][n_new][Hkv][head_dim] of in_dtype; start_pos device
 *      [batch]; block_table device. Every block the new tokens touch must be
 *      mapped; a row whose block id is outside [0, pool_blocks) is skipped.
 * Out: pool (device) rows and meta of the new tokens only.
 * Errors: KVQ_ERR_ARG (null pointers, batch < 0, n_new < 0, bad stride),
 * KVQ_ERR_DEVICE.
 */
kvq_status kvq_quantize_append(const kvq_layout* L, void* pool, int64_t pool_blocks,
                               const int32_t* block_table, int32_t table_stride,
                               int32_t batch, const int32_t* start_pos, int32_t n_new,
                               const void* k, const void* v, kvq_dtype in_dtype,
                               kvq_stream stream);

/*
 * Host. Checks the start positions of a kvq_quantize_append call on their
 * host copy, before the launch: every start_pos_host[b] >= 0, every new
 * token's block inside the table row (start_pos_host[b] + n_new <=
 * 16 * table_stride), and, for a layout with per-channel keys, n_new and
 * every start_pos_host[b] multiples of 16 (whole blocks).
 * Errors: KVQ_ERR_ARG naming the first sequence that fails (nothing else is
 * done; a stale layout or null pointers are KVQ_ERR_ARG too).
 */
kvq_status kvq_append_check(const kvq_layout* L, int32_t batch, const int32_t* start_pos_host,
                            int32_t n_new, int32_t table_stride);

/*
 * Device, async. Read back n tokens [pos0, pos0 + n) of sequence `seq`:
 * x_hat' = code * s + mn in fp32 (a rounded product then a rounded sum), or the
 * bf16 value for b = 16. With rotated = 0 the original basis blockdiag(H_n)^T
 * x_hat' is returned instead (fp32 fast Walsh-Hadamard transform).
 * Out: k_out, v_out device float [n][Hkv][head_dim].
 * Errors: KVQ_ERR_ARG (null pointers, n < 0, pos0 < 0, seq < 0), KVQ_ERR_DEVICE.
 * Rows whose block id is outside [0, pool_blocks) are written as zeros.
 */
kvq_status kvq_dequant(const kvq_layout* L, const void* pool, int64_t pool_blocks,
                       const int32_t* block_table, int32_t table_stride, int32_t seq,
                       int32_t pos0, int32_t n, int32_t rotated,
                       float* k_out, float* v_out, kvq_stream stream);

/*
 * Bytes at the front of every decode workspace that hold the work-sharing
 * counters. Their place and size are fixed (they do not follow the split
 * plan), so one workspace may serve decode calls of any plan, geometry or
 * batch, as long as it is large enough for each.
 */
#define KVQ_DECODE_COUNTER_BYTES 65536

/*
 * Host. Bytes of device workspace kvq_decode_attn needs for these segments
 * and batch size: KVQ_DECODE_COUNTER_BYTES of work-sharing counters at the
 * front, then the split-K partials (o', then max and sum, per query head and
 * split). A call uses two 32-bit counter words per (segment, sequence, KV
 * head, group of eight splits) from the front of the counter area; a call
 * that would need more than the area holds runs in the fixed order
 * (KVQ_DECODE_DETERMINISTIC) and uses none.
 */
kvq_status kvq_decode_workspace_bytes(const kvq_segment* segs, int32_t n_segs,
                                      int32_t batch, size_t* bytes);

/*
 * Device, async. Zeroes a decode workspace (ws_bytes bytes, a multiple of 4,
 * 4-byte aligned). Required once on a new workspace before its first decode
 * call, and again after a decode call that failed on the device; every
 * completed decode call leaves the counters zero, so a workspace is reused
 * without it. Launches a kernel (no memset). It also creates, once per
 * device, the side streams that a decode call with several launches (several
 * segments or per-head bit pairs) runs them on concurrently; so call it
 * outside graph capture, before capturing decode calls.
 * Errors: KVQ_ERR_ARG (null or misaligned), KVQ_ERR_DEVICE.
 */
kvq_status kvq_decode_workspace_init(void* ws, size_t ws_bytes, kvq_stream stream);

/*
 * Device, async. Fused quantized decode attention, one query per q-head:
 *   o[b][g] = softmax(q[b][g] . K_hat^T / sqrt(d)) V_hat
 * over the union of the segments' tokens of KV head g / G, with K_hat, V_hat
 * the dequantized cache in the original basis. Computed in the rotated basis:
 * q' = R q, scores against the stored rotated keys, o' = sum_t p_t v_hat'_t,
 * o = R^T o' (one inverse rotation per output row) [SAW: section 3]. Split-K
 * over pages with an online-softmax merge; fp32 accumulation.
 * A sequence with no tokens in any segment gets a zero output row.
 * In:  q device [batch][Hkv*G][head_dim] of q_dtype, 16-byte aligned.
 * Out: out device float [batch][Hkv*G][head_dim].
 * ws: device workspace of at least kvq_decode_workspace_bytes bytes, zeroed
 * once by kvq_decode_workspace_init before its first use. The waves of one
 * (sequence, KV head) share its pages through counters in ws, so two calls
 * in flight at once must not share a workspace. Every completed call leaves
 * the counters zero, and the counters sit in a fixed area that partials never
 * use, so the workspace is reused as it is by calls of any split plan. The heads of one segment
 * whose key and value widths are 2, 3 or 4 bits share one launch whatever
 * their pairs; a call with several launches (several segments, or heads with
 * 8- or 16-bit codes beside others) runs them concurrently on library side
 * streams forked from and joined back to `stream` with events; graph capture
 * of the call records the same dependencies. The splits of several segments
 * are planned to share one resident round of waves: the segment holding the
 * most gives up the others' share, so the small launches run beside it.
 * Environment (read at each call): KVQ_DECODE_DETERMINISTIC=1 fixes the order
 * in which a unit's waves take its pages, so results are bitwise reproducible
 * (default: most pages go to whichever wave is free, last-bit differences
 * between runs); KVQ_SPLIT_PAGES=n sets the pages per split instead of the
 * planner; KVQ_MIXED_LAUNCH=0 makes one launch per width pair;
 * KVQ_SEGMENT_RESERVE=0 sizes every segment's launch to fill the device alone.
 * The workspace size follows the same plan, so kvq_decode_workspace_bytes
 * must see the same environment (a smaller workspace is KVQ_ERR_WORKSPACE).
 * Errors: KVQ_ERR_ARG, KVQ_ERR_UNSUPPORTED, KVQ_ERR_WORKSPACE, KVQ_ERR_DEVICE.
 */
kvq_status kvq_decode_attn(const kvq_segment* segs, int32_t n_segs, int32_t batch,
                           const void* q, kvq_dtype q_dtype, float* out,
                           void* ws, size_t ws_bytes, kvq_stream stream);

/*
 * The two launches kvq_decode_attn makes, exported so a profiler or caller can
 * time them apart: kvq_decode_partial writes the split partials into ws;
 * kvq_decode_merge combines them and writes out. Same arguments and errors as
 * kvq_decode_attn; calling them in this order on one stream equals one
 * kvq_decode_attn call.
 */
kvq_status kvq_decode_partial(const kvq_segment* segs, int32_t n_segs, int32_t batch,
                              const void* q, kvq_dtype q_dtype,
                              void* ws, size_t ws_bytes, kvq_stream stream);
kvq_status kvq_decode_merge(const kvq_segment* segs, int32_t n_segs, int32_t batch,
                            float* out, void* ws, size_t ws_bytes, kvq_stream stream);

/*
 * Device, async. One decode step in one call: the quantize-on-append of one
 * new token per sequence into segment append_seg, then decode attention over
 * every segment, the new token included [SAW: section 3 (rotation and
 * quantization fused with the cache write; attention read straight from the
 * quantized cache); LQ: Methodology 2 (new tokens enter the full-precision
 * window)]. Equals kvq_quantize_append(segs[append_seg], start_pos, n_new = 1,
 * k_new, v_new) followed by kvq_decode_attn(segs, q): the stored rows and
 * metadata are bit-identical to the append's, and the output equals the two
 * calls' up to the order of fp32 sums. The new token is not read back from the
 * cache: the partial launch masks its slot, its split-0 wave of each
 * (sequence, KV head) quantizes and stores the token and leaves its
 * dequantized rows in ws, and the merge kernel attends to it from those rows,
 * so the step makes no append launch.
 * In:  segs, n_segs, batch, q, q_dtype, ws, ws_bytes: as kvq_decode_attn.
 *      append_seg: index of the segment that receives the token (a row
 *      layout: per-channel keys append whole blocks through
 *      kvq_quantize_append). Its pool is written (the segment's pool pointer
 *      must be writable device memory).
 *      start_pos device int32 [batch]: the token's slot in that segment
 *      (negative: no token for that sequence). Its page must be mapped for the
 *      row to be stored; it is attended to when also below the segment's
 *      min(seq_lens[b], max_len), so seq_lens counts the new token.
 *      k_new, v_new device [batch][Hkv][head_dim] of in_dtype (KVQ_BF16 or
 *      KVQ_F32), 16-byte aligned.
 * Out: out as kvq_decode_attn; the new rows in the append segment's pool.
 * Errors: as kvq_decode_attn; KVQ_ERR_ARG (append_seg out of range, null
 * start_pos / k_new / v_new, misaligned rows, bad in_dtype),
 * KVQ_ERR_UNSUPPORTED (per-channel keys in the append segment).
 */
kvq_status kvq_append_decode_attn(const kvq_segment* segs, int32_t n_segs, int32_t batch,
                                  int32_t append_seg, const int32_t* start_pos,
                                  const void* k_new, const void* v_new, kvq_dtype in_dtype,
                                  const void* q, kvq_dtype q_dtype, float* out,
                                  void* ws, size_t ws_bytes, kvq_stream stream);

/*
 * The two halves of kvq_append_decode_attn, exported so a profiler or caller
 * can time them apart (as kvq_decode_partial and kvq_decode_merge): the
 * partial launch, whose split-0 wave of each (sequence, KV head) quantizes
 * and stores the new token and leaves its dequantized rows in ws (every wave
 * masks its slot), then the merge, which attends to the token from those rows.
 * Same arguments and errors as kvq_append_decode_attn (the merge half takes
 * no rows); calling them in this order on one stream with one workspace
 * equals one kvq_append_decode_attn call.
 */
kvq_status kvq_append_decode_partial(const kvq_segment* segs, int32_t n_segs, int32_t batch,
                                     int32_t append_seg, const int32_t* start_pos,
                                     const void* k_new, const void* v_new, kvq_dtype in_dtype,
                                     const void* q, kvq_dtype q_dtype,
                                     void* ws, size_t ws_bytes, kvq_stream stream);
kvq_status kvq_append_decode_merge(const kvq_segment* segs, int32_t n_segs, int32_t batch,
                                   int32_t append_seg, const int32_t* start_pos,
                                   float* out, void* ws, size_t ws_bytes, kvq_stream stream);

/*
 * Measurement helpers, not part of the decode path: two read-only kernels that
 * give the read bandwidth the decode kernel is measured against on the device
 * it runs on (its roofline in practice, beside the HBM specification).
 *
 * kvq_measure_read_stream: 2048 waves read `bytes` (a multiple of 8192,
 * 16-byte aligned) once, the waves sweeping adjacent 8 KiB chunks, and each
 * wave writes one word to sink (device, sink_words >= 2048).
 *
 * kvq_measure_read_paged: the partial decode kernel's load pattern with no
 * compute, over each of n_segs segments in turn (one launch per segment,
 * back to back on the stream, so a caller can time many launches between two
 * events, e.g. one segment per layer so that no layer's pages are still
 * cached): one wave per (sequence, KV head, split) in the decode's grid
 * order, each split a contiguous range of four-page groups of max_len tokens,
 * reading per page the head's K area and V area through the block table (two
 * groups in flight while one is folded). The segments must share head count,
 * group and head_dim. splits = 0 takes the decode planner's split count for
 * each segment alone and batch; sink (device) receives one word per wave of
 * each launch (sink_words >= the largest launch's splits * num_kv_heads *
 * batch; the launches overwrite each other's words). Covers areas of up to
 * 2 KiB per head (all widths up to 8 bits at head_dim 128); 16-bit rows give
 * KVQ_ERR_UNSUPPORTED. Every segment is checked before the first launch.
 * Errors: KVQ_ERR_ARG, KVQ_ERR_UNSUPPORTED, KVQ_ERR_DEVICE.
 */
kvq_status kvq_measure_read_stream(const void* buf, size_t bytes, uint32_t* sink, int32_t sink_words,
                                   kvq_stream stream);
kvq_status kvq_measure_read_paged(const kvq_segment* segs, int32_t n_segs, int32_t batch, int32_t splits,
                                  uint32_t* sink, int32_t sink_words, kvq_stream stream);

/*
 * Size of kvq_decode_attn_noalloc's fixed scratch array, per GPU: the
 * counter area (KVQ_DECODE_COUNTER_BYTES) and the split-K partials.
 */
#define KVQ_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * Device, async. kvq_decode_attn without a caller workspace, for callers that
 * cannot allocate device memory or hand one in: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. Computes exactly what
 * kvq_decode_attn computes (same kernels), with the workspace in a fixed
 * device array of KVQ_NOALLOC_SCRATCH_BYTES that the library holds per GPU
 * until the process ends. No hipMalloc, hipFree, stream creation or other
 * allocating call is made: the first call on a device looks up the array's
 * address and clears its counter area with a kernel on `stream`. All of a
 * call's partial launches go on `stream`, one after another (no side
 * streams).
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (on different streams without ordering, or from several threads) race
 * and give wrong results. Each completed call leaves the counters zero for
 * the next; after a call that failed on the device the counters may not be
 * zero, and the array cannot be reset.
 * In/Out: as kvq_decode_attn.
 * Errors: as kvq_decode_attn; KVQ_ERR_WORKSPACE when the call's workspace
 * (kvq_decode_workspace_bytes) exceeds KVQ_NOALLOC_SCRATCH_BYTES.
 */
kvq_status kvq_decode_attn_noalloc(const kvq_segment* segs, int32_t n_segs, int32_t batch,
                                   const void* q, kvq_dtype q_dtype, float* out,
                                   kvq_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
