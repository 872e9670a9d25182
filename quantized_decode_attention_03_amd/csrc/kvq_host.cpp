// libkvq host side: argument checks, layout, bit planning, page allocation,
// split planning and kernel dispatch behind the C ABI in include/kvq.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "kvq.h"
#include "kvq_internal.h"

namespace {

thread_local std::string g_last_error;

kvq_status fail(kvq_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

kvq_status ok() {
  g_last_error.clear();
  return KVQ_OK;
}

kvq_status device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(KVQ_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

// Side streams for calls that make several partial-decode launches (one per
// segment and per (K bits, V bits) head group): the launches are independent,
// so they run concurrently, forked from and joined back to the caller's
// stream with events (a pattern graph capture also follows). Created once per
// device, default priority; one enqueue at a time (the events are shared).
constexpr int kSideStreams = 4;
struct SideStreams {
  bool ready = false;
  hipStream_t s[kSideStreams];
  hipEvent_t fork;
  hipEvent_t join[kSideStreams];
};
std::mutex g_side_mutex;
SideStreams g_side[64];

// Creating streams is not allowed while the caller's stream is being captured
// into a graph: kvq_decode_workspace_init creates them ahead of any capture.
hipError_t side_streams(SideStreams** out, hipStream_t caller) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  SideStreams& ss = g_side[dev];
  if (!ss.ready) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (caller && hipStreamIsCapturing(caller, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone)
      return hipErrorStreamCaptureUnsupported;
    for (int i = 0; i < kSideStreams; ++i) {
      if ((e = hipStreamCreateWithFlags(&ss.s[i], hipStreamNonBlocking)) != hipSuccess) return e;
      if ((e = hipEventCreateWithFlags(&ss.join[i], hipEventDisableTiming)) != hipSuccess) return e;
    }
    if ((e = hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming)) != hipSuccess) return e;
    ss.ready = true;
  }
  *out = &ss;
  return hipSuccess;
}

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
bool valid_bits(int b) { return b == 2 || b == 3 || b == 4 || b == 8 || b == 16; }

int64_t row_bytes(int d, int b) { return static_cast<int64_t>(d) * b / 8; }
int64_t area_bytes(int d, int b, int meta_fp16) {
  return KVQ_BLOCK_TOKENS * row_bytes(d, b) + (b == 16 ? 0 : KVQ_BLOCK_TOKENS * (meta_fp16 ? 4 : 8));
}
// A K area with per-channel metadata: 16 code rows, then {s, mn} per channel.
int64_t key_area_bytes(int d, int b, int meta_fp16, int per_channel) {
  if (per_channel && b != 16) return KVQ_BLOCK_TOKENS * row_bytes(d, b) + static_cast<int64_t>(d) * 8;
  return area_bytes(d, b, meta_fp16);
}

// Checks the inputs of a layout and that its outputs match them.
kvq_status check_layout(const kvq_layout* L, const char* who) {
  if (!L) return fail(KVQ_ERR_ARG, "%s: null layout", who);
  if (L->block_tokens != KVQ_BLOCK_TOKENS) return fail(KVQ_ERR_ARG, "%s: block_tokens must be 16", who);
  if (L->meta_fp16 != 0 && L->meta_fp16 != 1) return fail(KVQ_ERR_ARG, "%s: meta_fp16 must be 0 or 1", who);
  if (L->key_per_channel != 0 && L->key_per_channel != 1)
    return fail(KVQ_ERR_ARG, "%s: key_per_channel must be 0 or 1", who);
  if (L->key_per_channel && L->meta_fp16)
    return fail(KVQ_ERR_UNSUPPORTED, "%s: per-channel keys keep float32 metadata", who);
  if (L->num_kv_heads < 1 || L->num_kv_heads > KVQ_MAX_KV_HEADS)
    return fail(KVQ_ERR_ARG, "%s: num_kv_heads %d out of [1, %d]", who, L->num_kv_heads, KVQ_MAX_KV_HEADS);
  if (L->group < 1 || L->group > 4) return fail(KVQ_ERR_ARG, "%s: group %d out of [1, 4]", who, L->group);
  if (L->head_dim != 64 && L->head_dim != 128)
    return fail(KVQ_ERR_UNSUPPORTED, "%s: head_dim %d (built: 64, 128)", who, L->head_dim);
  if (!is_pow2(L->had_block) || L->had_block > L->head_dim)
    return fail(KVQ_ERR_ARG, "%s: had_block %d must be a power of two in [1, head_dim]", who, L->had_block);
  for (int h = 0; h < L->num_kv_heads; ++h) {
    if (!valid_bits(L->bits_k[h]) || !valid_bits(L->bits_v[h]))
      return fail(KVQ_ERR_ARG, "%s: head %d bits (%d, %d) not in {2,3,4,8,16}", who, h, L->bits_k[h], L->bits_v[h]);
  }
  return KVQ_OK;
}

kvq_status check_layout_ready(const kvq_layout* L, const char* who) {
  kvq_status s = check_layout(L, who);
  if (s != KVQ_OK) return s;
  kvq_layout tmp = *L;
  if (kvq_layout_init(&tmp) != KVQ_OK || tmp.block_bytes != L->block_bytes ||
      std::memcmp(tmp.k_off, L->k_off, sizeof(tmp.k_off)) != 0 ||
      std::memcmp(tmp.v_off, L->v_off, sizeof(tmp.v_off)) != 0)
    return fail(KVQ_ERR_ARG, "%s: layout outputs stale; call kvq_layout_init", who);
  return KVQ_OK;
}

// KVQ_DECODE_DETERMINISTIC=1 fixes which wave computes which pages, so the
// result is bitwise reproducible; by default three quarters of each unit's
// pages go to whichever of its waves is free first (faster, last-bit
// differences between runs).
bool deterministic_order() {
  const char* env = std::getenv("KVQ_DECODE_DETERMINISTIC");
  return env && env[0] && env[0] != '0';
}

// KVQ_MIXED_LAUNCH=0: one partial launch per (key, value) width pair of a
// segment, on concurrent streams. By default the heads whose pairs use 2-, 3-
// or 4-bit codes share one launch of the multi-format kernel when the segment
// has several such pairs (same results: each head runs the same code).
bool mixed_launch_enabled() {
  const char* env = std::getenv("KVQ_MIXED_LAUNCH");
  return !(env && env[0] == '0');
}

// KVQ_SEGMENT_RESERVE=0: every segment's launch is sized to fill the device
// alone, as for a single segment.
bool reserve_for_small_segments() {
  const char* env = std::getenv("KVQ_SEGMENT_RESERVE");
  return !(env && env[0] == '0');
}

// Split plan of one segment: nominal pages per split (a multiple of 4) and
// the number of waves (splits) per (sequence, KV head). The kernel shares a
// unit's pages among its waves itself; the nominal size only sets the count.
struct SplitPlan {
  int pages_per_split;
  int n_splits;
};

// Compute units of the current device (0 if no device is visible), read once.
int device_cus() {
  static const int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return n;
  }();
  return cus;
}

// Splits sized so one resident round of waves covers the segment: as many
// splits per (sequence, KV head) as the GPU holds waves of this kernel at
// once, balanced, each a multiple of four pages (one group) and at least two
// groups so the per-split prologue and partial write amortise.
SplitPlan plan_splits(const kvq_segment& s, int batch) {
  const int pages = (std::max(s.max_len, 0) + KVQ_BLOCK_TOKENS - 1) / KVQ_BLOCK_TOKENS;
  SplitPlan p{4, 0};
  if (pages == 0 || batch == 0) return p;
  int pps = 0;
  if (const char* env = std::getenv("KVQ_SPLIT_PAGES")) pps = std::atoi(env);
  if (pps <= 0) {
    // One resident round: a head whose format runs w waves per SIMD takes 1/w
    // of a SIMD per wave, so the splits per unit are the SIMDs of the device
    // over batch * sum_h 1/w_h (heads of different formats share the round).
    const kvq_layout& L = *s.layout;
    double simd_share = 0.0;
    for (int h = 0; h < L.num_kv_heads; ++h)
      simd_share += 1.0 / kvq::decode_partial_waves_per_simd(L.bits_k[h], L.bits_v[h], L.head_dim,
                                                              L.key_per_channel != 0);
    const int cus = device_cus() > 0 ? device_cus() : 256;
    // (rounded down to whole rounds of the eight XCDs, so the round is not overfilled)
    const int64_t fit = static_cast<int64_t>(4.0 * cus / (static_cast<double>(batch) * simd_share));
    const int64_t want_splits = std::max<int64_t>(1, fit >= 8 ? fit / 8 * 8 : fit);
    pps = static_cast<int>((pages + want_splits - 1) / want_splits);
    pps = std::max(pps, 8);
  }
  pps = (pps + 3) / 4 * 4;
  p.pages_per_split = pps;
  // a multiple of the eight XCDs: the kernel spreads each unit's waves evenly
  // over them
  p.n_splits = ((pages + pps - 1) / pps + 7) / 8 * 8;
  return p;
}

kvq_status check_segments(const kvq_segment* segs, int n_segs, int batch, const char* who) {
  if (!segs || n_segs < 1) return fail(KVQ_ERR_ARG, "%s: need at least one segment", who);
  if (batch < 0) return fail(KVQ_ERR_ARG, "%s: batch %d < 0", who, batch);
  for (int i = 0; i < n_segs; ++i) {
    const kvq_segment& s = segs[i];
    kvq_status st = check_layout_ready(s.layout, who);
    if (st != KVQ_OK) return st;
    const kvq_layout& L0 = *segs[0].layout;
    const kvq_layout& L = *s.layout;
    if (L.num_kv_heads != L0.num_kv_heads || L.group != L0.group || L.head_dim != L0.head_dim ||
        L.had_block != L0.had_block)
      return fail(KVQ_ERR_ARG, "%s: segment %d geometry differs from segment 0", who, i);
    if (s.max_len < 0) return fail(KVQ_ERR_ARG, "%s: segment %d max_len < 0", who, i);
    if (s.max_len > 0 && batch > 0) {
      if (!s.pool || !s.block_table || !s.seq_lens) return fail(KVQ_ERR_ARG, "%s: segment %d null pointer", who, i);
      if (s.pool_blocks < 1) return fail(KVQ_ERR_ARG, "%s: segment %d pool_blocks < 1", who, i);
      const int pages = (s.max_len + KVQ_BLOCK_TOKENS - 1) / KVQ_BLOCK_TOKENS;
      if (s.table_stride < pages)
        return fail(KVQ_ERR_ARG, "%s: segment %d table_stride %d < ceil(max_len/16) = %d", who, i, s.table_stride, pages);
    } else if (!s.seq_lens && batch > 0) {
      return fail(KVQ_ERR_ARG, "%s: segment %d null seq_lens", who, i);
    }
  }
  return KVQ_OK;
}

// SIMDs one split of one sequence of segment s holds: a head whose format runs
// w waves per SIMD takes 1/w of one.
double split_simd_share(const kvq_segment& s) {
  const kvq_layout& L = *s.layout;
  double share = 0.0;
  for (int h = 0; h < L.num_kv_heads; ++h)
    share += 1.0 / kvq::decode_partial_waves_per_simd(L.bits_k[h], L.bits_v[h], L.head_dim, L.key_per_channel != 0);
  return share;
}

// KVQ_WINDOW_IN_MERGE=0: a short bf16 segment gets a partial launch of its
// own instead of being attended to by the merge kernel.
bool window_in_merge_enabled() {
  const char* env = std::getenv("KVQ_WINDOW_IN_MERGE");
  return !(env && env[0] == '0');
}

// A segment the merge kernel can attend to itself: 16-bit keys and values in
// every head, at most kMergeWindowMax tokens.
bool window_candidate(const kvq_segment& s) {
  const kvq_layout& L = *s.layout;
  if (L.key_per_channel || s.max_len < 1 || s.max_len > kvq::kMergeWindowMax) return false;
  for (int h = 0; h < L.num_kv_heads; ++h)
    if (L.bits_k[h] != 16 || L.bits_v[h] != 16) return false;
  return true;
}

// The plan of one decode call, shared by the partial and merge calls (and the
// workspace size): the splits of every segment, the segment the merge
// attends to itself, and the segment whose split-0 waves leave q~ for it.
struct CallPlan {
  std::vector<SplitPlan> split;
  int slots = 0;
  int window = -1;
  int q_writer = -1;
};

// need_q: the merge needs q~ (a fused append's token is attended to there),
// so some segment's split-0 waves write it even without a window.
CallPlan plan_call(const kvq_segment* segs, int n_segs, int batch, bool need_q = false) {
  CallPlan c;
  c.split.resize(n_segs);
  for (int i = 0; i < n_segs; ++i) c.split[i] = plan_splits(segs[i], batch);
  // A short bf16 segment beside others: the merge kernel computes its
  // attention from the rotated query one of the other launches leaves, so it
  // needs no partial launch (its waves would need a whole SIMD each and wait
  // for the low-precision waves to retire).
  if (batch > 0 && n_segs > 1 && window_in_merge_enabled()) {
    for (int i = 0; i < n_segs && c.window < 0; ++i)
      if (window_candidate(segs[i])) c.window = i;
    if (c.window >= 0) {
      for (int i = 0; i < n_segs && c.q_writer < 0; ++i)
        if (i != c.window && c.split[i].n_splits > 0) c.q_writer = i;
      if (c.q_writer < 0) c.window = -1;
      else c.split[c.window].n_splits = 0;
    }
  }
  // Several segments' launches run at once, and each was sized to fill one
  // resident round alone. The one holding most SIMDs gives up the others'
  // share (in whole groups of eight splits), so the small launches run beside
  // it rather than after its waves retire.
  if (n_segs > 1 && batch > 0 && !std::getenv("KVQ_SPLIT_PAGES") && reserve_for_small_segments()) {
    const double round = 4.0 * (device_cus() > 0 ? device_cus() : 256);
    int big = 0;
    double big_share = -1.0, all = 0.0;
    for (int i = 0; i < n_segs; ++i) {
      const double sh = static_cast<double>(c.split[i].n_splits) * batch * split_simd_share(segs[i]);
      all += sh;
      if (sh > big_share) { big = i; big_share = sh; }
    }
    const double per_split = batch * split_simd_share(segs[big]);
    if (all > round && per_split > 0.0) {
      const int fit = static_cast<int>((round - (all - big_share)) / per_split) / 8 * 8;
      c.split[big].n_splits = std::min(c.split[big].n_splits, std::max(fit, 8));
    }
  }
  if (need_q && c.q_writer < 0)
    for (int i = 0; i < n_segs && c.q_writer < 0; ++i)
      if (c.split[i].n_splits > 0) c.q_writer = i;
  for (int i = 0; i < n_segs; ++i) c.slots += c.split[i].n_splits;
  return c;
}

// A fused append (kvq_append_decode_attn): one token per sequence into
// segment `seg` at slot start_pos[b]; the partial launch masks that slot and
// the merge kernel quantizes, stores and attends to the token.
struct FusedAppend {
  int seg;
  const int32_t* start_pos;
  const void* k_new;
  const void* v_new;
  kvq_dtype dtype;
};

// The kernels' description of a fused append.
void fill_token_append(const kvq_segment* segs, const FusedAppend& fa, kvq::TokenAppend& ap) {
  const kvq_segment& g = segs[fa.seg];
  const kvq_layout& L = *g.layout;
  // (the segment's pool is const for decoding; a fused append writes the new rows into it)
  ap.pool = static_cast<uint8_t*>(const_cast<void*>(g.pool));
  ap.pool_blocks = g.pool_blocks;
  ap.block_bytes = L.block_bytes;
  ap.table = g.block_table;
  ap.table_stride = g.table_stride;
  ap.seq_lens = g.seq_lens;
  ap.start_pos = fa.start_pos;
  ap.k_new = fa.k_new;
  ap.v_new = fa.v_new;
  ap.src_bf16 = fa.dtype == KVQ_BF16;
  ap.meta16 = L.meta_fp16;
  ap.max_len = g.max_len;
  ap.rs_n = 1.0 / std::sqrt(static_cast<double>(L.had_block));  // (as the append kernel's)
  for (int h = 0; h < L.num_kv_heads; ++h) {
    ap.k_off[h] = static_cast<int32_t>(L.k_off[h]);
    ap.v_off[h] = static_cast<int32_t>(L.v_off[h]);
    ap.bits_k[h] = static_cast<uint8_t>(L.bits_k[h]);
    ap.bits_v[h] = static_cast<uint8_t>(L.bits_v[h]);
  }
}

// Workspace: the work-sharing counter region (KVQ_DECODE_COUNTER_BYTES at the
// front, zero between calls), then partial o' [batch][hq][slots][d], partial
// (max, sum) [batch][hq][slots][2], q~ [batch][hq][d] for a window segment or a
// fused append, and a fused append's dequantized rows [batch][hkv][2][d]. A call's counters are the first words of the region: per segment
// [batch][hkv][splits / 8][2] (uint32); slots is the sum of the segments'
// splits, so a call takes slots / 8 * batch * hkv * 2 words. The region's
// place and size do not depend on the split plan, so no call's partials ever
// land on any call's counters, and one workspace serves calls of any plan.
constexpr size_t kCounterBytes = KVQ_DECODE_COUNTER_BYTES;
struct WsLayout {
  size_t part_o, part_ml, qrot, anew, total;
};
WsLayout ws_layout(int batch, int hkv, int group, int d, int slots) {
  const size_t rows = static_cast<size_t>(batch) * hkv * group, s1 = static_cast<size_t>(std::max(slots, 1));
  WsLayout w;
  w.part_o = kCounterBytes;
  w.part_ml = w.part_o + rows * s1 * d * sizeof(float);
  w.qrot = w.part_ml + rows * s1 * 2 * sizeof(float);
  w.anew = w.qrot + rows * d * sizeof(float);
  w.total = w.anew + static_cast<size_t>(batch) * hkv * 2 * d * sizeof(float);
  return w;
}
// Counter words a call with this plan uses; more than the region holds sends
// the call to the fixed order, which uses none.
size_t counter_words(int batch, int hkv, int slots) { return static_cast<size_t>(slots / 8) * batch * hkv * 2; }

}  // namespace

extern "C" {

int kvq_abi_version(void) { return KVQ_ABI_VERSION; }

const char* kvq_status_str(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "KVQ_OK";
    case KVQ_ERR_ARG: return "KVQ_ERR_ARG";
    case KVQ_ERR_UNSUPPORTED: return "KVQ_ERR_UNSUPPORTED";
    case KVQ_ERR_BUDGET: return "KVQ_ERR_BUDGET";
    case KVQ_ERR_WORKSPACE: return "KVQ_ERR_WORKSPACE";
    case KVQ_ERR_DEVICE: return "KVQ_ERR_DEVICE";
    case KVQ_ERR_CAPACITY: return "KVQ_ERR_CAPACITY";
  }
  return "KVQ_ERR_UNKNOWN";
}

const char* kvq_last_error(void) { return g_last_error.c_str(); }

kvq_status kvq_layout_init(kvq_layout* L) {
  kvq_status s = check_layout(L, "kvq_layout_init");
  if (s != KVQ_OK) return s;
  int64_t off = 0;
  std::memset(L->k_off, 0, sizeof(L->k_off));
  std::memset(L->v_off, 0, sizeof(L->v_off));
  for (int h = 0; h < L->num_kv_heads; ++h) {
    L->k_off[h] = off;
    off += key_area_bytes(L->head_dim, L->bits_k[h], L->meta_fp16, L->key_per_channel);
  }
  for (int h = 0; h < L->num_kv_heads; ++h) {
    L->v_off[h] = off;
    off += area_bytes(L->head_dim, L->bits_v[h], L->meta_fp16);
  }
  L->block_bytes = off;
  return ok();
}

}  // extern "C"

namespace {

// Greedy marginal-gain allocation over components with their own curves
// D_i(b) = alpha[i * stride] * beta[i * stride]^-b (stride 0: one curve for
// all), shared by kvq_plan_bits and kvq_plan_bits_components.
kvq_status plan_bits_greedy(const char* who, int32_t n, const float* w, const double* alpha, const double* beta,
                            int stride, const int32_t* ladder, int32_t n_ladder, int64_t budget_bits,
                            int32_t* bits_out, int64_t* leftover_out) {
  if (n < 1 || !w || !alpha || !beta || !ladder || !bits_out) return fail(KVQ_ERR_ARG, "%s: null pointer or n < 1", who);
  if (n_ladder < 1 || n_ladder > 16) return fail(KVQ_ERR_ARG, "%s: n_ladder %d out of [1, 16]", who, n_ladder);
  for (int i = 0; i < (stride ? n : 1); ++i) {
    const double a = alpha[i * stride], b = beta[i * stride];
    if (!(a > 0.0) || !(b > 1.0) || !std::isfinite(a) || !std::isfinite(b))
      return fail(KVQ_ERR_ARG, "%s: need alpha > 0 and beta > 1 (component %d)", who, i);
  }
  std::vector<int> lad(ladder, ladder + n_ladder);
  std::sort(lad.begin(), lad.end());
  for (int i = 0; i < n_ladder; ++i) {
    if (lad[i] < 1) return fail(KVQ_ERR_ARG, "%s: ladder widths must be positive", who);
    if (i && lad[i] == lad[i - 1]) return fail(KVQ_ERR_ARG, "%s: ladder widths must be distinct", who);
  }
  for (int i = 0; i < n; ++i)
    if (!(w[i] > 0.f) || !std::isfinite(w[i])) return fail(KVQ_ERR_ARG, "%s: w[%d] must be positive", who, i);
  const int64_t lo = static_cast<int64_t>(n) * lad.front(), hi = static_cast<int64_t>(n) * lad.back();
  if (budget_bits < lo || budget_bits > hi)
    return fail(KVQ_ERR_BUDGET, "%s: budget %lld outside [%lld, %lld]", who, static_cast<long long>(budget_bits),
                static_cast<long long>(lo), static_cast<long long>(hi));
  // D_i(b) at every ladder rung, in double.
  const int n_curves = stride ? n : 1;
  std::vector<double> dist(static_cast<size_t>(n_curves) * n_ladder);
  for (int c = 0; c < n_curves; ++c)
    for (int k = 0; k < n_ladder; ++k)
      dist[static_cast<size_t>(c) * n_ladder + k] = alpha[c * stride] * std::pow(beta[c * stride], -static_cast<double>(lad[k]));
  std::vector<int> level(n, 0);
  int64_t remaining = budget_bits - lo;
  while (remaining > 0) {
    int best = -1;
    double best_gain = -1.0;
    for (int i = 0; i < n; ++i) {
      const int lv = level[i];
      if (lv + 1 >= n_ladder) continue;
      const int step = lad[lv + 1] - lad[lv];
      if (step > remaining) continue;
      const double* d = &dist[static_cast<size_t>(stride ? i : 0) * n_ladder];
      const double gain = static_cast<double>(w[i]) * (d[lv] - d[lv + 1]) / step;
      if (gain > best_gain) {
        best = i;
        best_gain = gain;
      }
    }
    if (best < 0) break;
    remaining -= lad[level[best] + 1] - lad[level[best]];
    ++level[best];
  }
  for (int i = 0; i < n; ++i) bits_out[i] = lad[level[i]];
  if (leftover_out) *leftover_out = remaining;
  if (remaining != 0)
    return fail(KVQ_ERR_BUDGET, "%s: %lld bits could not be placed on the ladder", who,
                static_cast<long long>(remaining));
  return ok();
}

}  // namespace

extern "C" {

kvq_status kvq_plan_bits(int32_t n, const float* w, double alpha, double beta, const int32_t* ladder,
                         int32_t n_ladder, int64_t budget_bits, int32_t* bits_out, int64_t* leftover_out) {
  return plan_bits_greedy("kvq_plan_bits", n, w, &alpha, &beta, 0, ladder, n_ladder, budget_bits, bits_out,
                          leftover_out);
}

kvq_status kvq_plan_bits_components(int32_t n, const float* w, const double* alpha, const double* beta,
                                    const int32_t* ladder, int32_t n_ladder, int64_t budget_bits, int32_t* bits_out,
                                    int64_t* leftover_out) {
  return plan_bits_greedy("kvq_plan_bits_components", n, w, alpha, beta, 1, ladder, n_ladder, budget_bits, bits_out,
                          leftover_out);
}

kvq_status kvq_fit_distortion(int32_t n, const int32_t* widths, const double* mse, double* alpha_out,
                              double* beta_out, double* r2_out) {
  if (n < 2 || !widths || !mse || !alpha_out || !beta_out)
    return fail(KVQ_ERR_ARG, "kvq_fit_distortion: null pointer or n < 2");
  double mb = 0.0, my = 0.0;
  for (int i = 0; i < n; ++i) {
    if (!(mse[i] > 0.0) || !std::isfinite(mse[i]))
      return fail(KVQ_ERR_ARG, "kvq_fit_distortion: mse[%d] must be positive and finite", i);
    mb += widths[i];
    my += std::log(mse[i]);
  }
  mb /= n;
  my /= n;
  // least squares of y = ln mse on b: slope = S_by / S_bb, intercept = my - slope * mb
  double sbb = 0.0, sby = 0.0, syy = 0.0;
  for (int i = 0; i < n; ++i) {
    const double db = widths[i] - mb, dy = std::log(mse[i]) - my;
    sbb += db * db;
    sby += db * dy;
    syy += dy * dy;
  }
  if (!(sbb > 0.0)) return fail(KVQ_ERR_ARG, "kvq_fit_distortion: the widths must not all be equal");
  const double slope = sby / sbb, icpt = my - slope * mb;
  double ssr = 0.0;
  for (int i = 0; i < n; ++i) {
    const double e = std::log(mse[i]) - (icpt + slope * widths[i]);
    ssr += e * e;
  }
  *alpha_out = std::exp(icpt);
  *beta_out = std::exp(-slope);
  if (r2_out) *r2_out = syy > 0.0 ? 1.0 - ssr / syy : 1.0;
  return ok();
}

kvq_status kvq_amgm_ratio(int32_t n, const float* w, double* ratio_out) {
  if (n < 1 || !w || !ratio_out) return fail(KVQ_ERR_ARG, "kvq_amgm_ratio: null pointer or n < 1");
  double am = 0.0, lg = 0.0;
  for (int i = 0; i < n; ++i) {
    if (!(w[i] > 0.f) || !std::isfinite(w[i])) return fail(KVQ_ERR_ARG, "kvq_amgm_ratio: w[%d] must be positive", i);
    am += w[i];
    lg += std::log(static_cast<double>(w[i]));
  }
  *ratio_out = (am / n) / std::exp(lg / n);
  return ok();
}

kvq_status kvq_quant_mse(const void* x, kvq_dtype dtype, int64_t rows, int32_t head_dim, int32_t had_block,
                         const int32_t* widths, int32_t n_widths, double* mse_out, kvq_stream stream) {
  if (!x || !widths || !mse_out) return fail(KVQ_ERR_ARG, "kvq_quant_mse: null pointer");
  if (rows < 1) return fail(KVQ_ERR_ARG, "kvq_quant_mse: rows %lld < 1", static_cast<long long>(rows));
  if (dtype != KVQ_F32 && dtype != KVQ_BF16) return fail(KVQ_ERR_ARG, "kvq_quant_mse: bad dtype %d", dtype);
  if (head_dim != 64 && head_dim != 128)
    return fail(KVQ_ERR_UNSUPPORTED, "kvq_quant_mse: head_dim %d (built: 64, 128)", head_dim);
  if (had_block < 1 || had_block > head_dim || (had_block & (had_block - 1)))
    return fail(KVQ_ERR_ARG, "kvq_quant_mse: had_block %d must be a power of two in [1, head_dim]", had_block);
  if (n_widths < 1 || n_widths > kvq::kMaxCalibWidths)
    return fail(KVQ_ERR_ARG, "kvq_quant_mse: n_widths %d out of [1, %d]", n_widths, kvq::kMaxCalibWidths);
  kvq::QuantMseArgs a{};
  for (int i = 0; i < n_widths; ++i) {
    if (widths[i] < 1 || widths[i] > 8) return fail(KVQ_ERR_ARG, "kvq_quant_mse: width %d out of [1, 8]", widths[i]);
    a.widths[i] = widths[i];
  }
  a.x = x;
  a.x_bf16 = dtype == KVQ_BF16;
  a.rows = rows;
  a.d = head_dim;
  a.had_block = had_block;
  a.n_widths = n_widths;
  a.out = mse_out;
  return device_status(kvq::launch_quant_mse(a, reinterpret_cast<hipStream_t>(stream)), "kvq_quant_mse");
}

}  // extern "C"

namespace {

// Class (0 window, 1 middle, 2 low) of position pos at length total under the
// dynamic schedule: span k of the distance r behind the window holds
// 2^k <= r / W + 1 < 2^(k+1); a token there is kept when 2^k divides pos + 1.
int lq_dynamic_class(int64_t pos, int64_t total, int64_t window) {
  const int64_t dist = total - 1 - pos;
  if (dist < window) return 0;
  const uint64_t q = static_cast<uint64_t>((dist - window) / window + 1);
  const int k = 63 - __builtin_clzll(q);
  return ((pos + 1) & ((int64_t{1} << k) - 1)) == 0 ? 1 : 2;
}

}  // namespace

extern "C" {

kvq_status kvq_logquant_dynamic_classes(int32_t total, int32_t window, int8_t* cls_out) {
  if (total < 0 || window < 1) return fail(KVQ_ERR_ARG, "kvq_logquant_dynamic_classes: total < 0 or window < 1");
  if (total > 0 && !cls_out) return fail(KVQ_ERR_ARG, "kvq_logquant_dynamic_classes: null output");
  for (int32_t p = 0; p < total; ++p) cls_out[p] = static_cast<int8_t>(lq_dynamic_class(p, total, window));
  return ok();
}

kvq_status kvq_logquant_init(int32_t total, int32_t window, kvq_lq_state* st) {
  if (!st || total < 0 || window < 1 || st->cap_mid < 0 || (st->cap_mid > 0 && !st->mid_pos))
    return fail(KVQ_ERR_ARG, "kvq_logquant_init: null state, total < 0, window < 1 or bad mid_pos");
  int32_t n_mid = 0, n_low = 0;
  for (int32_t p = 0; p < total; ++p) {
    const int c = lq_dynamic_class(p, total, window);
    n_mid += c == 1;
    n_low += c == 2;
  }
  if (n_mid > st->cap_mid)
    return fail(KVQ_ERR_CAPACITY, "kvq_logquant_init: %d middle tokens exceed cap_mid %d", n_mid, st->cap_mid);
  int32_t slot = 0;
  for (int32_t p = 0; p < total; ++p)
    if (lq_dynamic_class(p, total, window) == 1) st->mid_pos[slot++] = p;
  st->total = total;
  st->window = window;
  st->n_mid = n_mid;
  st->n_low = n_low;
  return ok();
}

kvq_status kvq_logquant_advance(int32_t batch, kvq_lq_state* states, kvq_lq_move* moves_out) {
  if (batch < 0 || (batch > 0 && (!states || !moves_out)))
    return fail(KVQ_ERR_ARG, "kvq_logquant_advance: batch < 0 or null pointers");
  // plan every sequence first, so that an error leaves every state unchanged
  std::vector<kvq_lq_move> plan(batch);
  for (int32_t b = 0; b < batch; ++b) {
    const kvq_lq_state& st = states[b];
    if (st.window < 1 || st.total < 0 || st.total == INT32_MAX || st.n_mid < 0 || st.n_low < 0 ||
        st.n_mid > st.cap_mid || (st.cap_mid > 0 && !st.mid_pos))
      return fail(KVQ_ERR_ARG, "kvq_logquant_advance: sequence %d has an invalid state", b);
    const int64_t t = st.total, w = st.window;
    kvq_lq_move m{-1, -1, -1, -1, static_cast<int32_t>(t % w)};
    if (t >= w) {
      const int32_t e = static_cast<int32_t>(t - w);
      m.win_slot = static_cast<int32_t>(e % w);
      // the token crossing into span k = 1 + tz(t + 1) drops out of the kept set there
      const int k = 1 + __builtin_ctzll(static_cast<uint64_t>(t + 1));
      const int64_t d = k < 62 ? t - (int64_t{1} << k) * w : -1;
      if (d >= 0) {
        int32_t s = -1;
        for (int32_t i = 0; i < st.n_mid; ++i)
          if (st.mid_pos[i] == d) { s = i; break; }
        if (s < 0)
          return fail(KVQ_ERR_ARG, "kvq_logquant_advance: sequence %d: position %lld is not in the middle segment",
                      b, static_cast<long long>(d));
        m.demote_slot = s;
        m.low_slot = st.n_low;
        m.mid_slot = s;
      } else {
        if (st.n_mid >= st.cap_mid)
          return fail(KVQ_ERR_CAPACITY, "kvq_logquant_advance: sequence %d: middle segment full (%d slots)", b,
                      st.cap_mid);
        m.mid_slot = st.n_mid;
      }
    }
    plan[b] = m;
  }
  for (int32_t b = 0; b < batch; ++b) {
    kvq_lq_state& st = states[b];
    const kvq_lq_move& m = plan[b];
    if (m.win_slot >= 0) {
      st.mid_pos[m.mid_slot] = st.total - st.window;
      if (m.demote_slot >= 0) ++st.n_low;
      else ++st.n_mid;
    }
    ++st.total;
    moves_out[b] = m;
  }
  return ok();
}

kvq_status kvq_logquant_requant(const kvq_segment* window, const kvq_segment* mid, const kvq_segment* low,
                                int32_t batch, const kvq_lq_move* moves, kvq_stream stream) {
  const char* who = "kvq_logquant_requant";
  if (!window || !mid || !low || batch < 0 || (batch > 0 && !moves))
    return fail(KVQ_ERR_ARG, "%s: null pointers or batch < 0", who);
  const kvq_segment* segs[3] = {window, mid, low};
  kvq::RequantArgs a{};
  for (int i = 0; i < 3; ++i) {
    kvq_status st = check_layout_ready(segs[i]->layout, who);
    if (st != KVQ_OK) return st;
    const kvq_layout& L = *segs[i]->layout;
    const kvq_layout& L0 = *window->layout;
    if (L.num_kv_heads != L0.num_kv_heads || L.head_dim != L0.head_dim || L.had_block != L0.had_block)
      return fail(KVQ_ERR_ARG, "%s: segment %d geometry differs from the window's", who, i);
    if (L.key_per_channel)
      return fail(KVQ_ERR_UNSUPPORTED, "%s: segment %d has per-channel keys (moved rows are per token)", who, i);
    if (!segs[i]->pool || !segs[i]->block_table || segs[i]->pool_blocks < 1 || segs[i]->table_stride < 1)
      return fail(KVQ_ERR_ARG, "%s: segment %d needs a pool and a block table", who, i);
    kvq::RequantSeg& sg = a.seg[i];
    sg.pool = static_cast<uint8_t*>(const_cast<void*>(segs[i]->pool));
    sg.pool_blocks = segs[i]->pool_blocks;
    sg.block_bytes = L.block_bytes;
    sg.table = segs[i]->block_table;
    sg.table_stride = segs[i]->table_stride;
    sg.meta16 = L.meta_fp16;
    for (int h = 0; h < L.num_kv_heads; ++h) {
      sg.bits[0][h] = static_cast<uint8_t>(L.bits_k[h]);
      sg.bits[1][h] = static_cast<uint8_t>(L.bits_v[h]);
    }
  }
  a.hkv = window->layout->num_kv_heads;
  a.d = window->layout->head_dim;
  for (int32_t b = 0; b < batch; ++b) {
    const kvq_lq_move& m = moves[b];
    const int32_t slots[4] = {m.win_slot, m.mid_slot, m.demote_slot, m.low_slot};
    const int seg_of[4] = {0, 1, 1, 2};
    for (int j = 0; j < 4; ++j)
      if (slots[j] >= static_cast<int64_t>(segs[seg_of[j]]->table_stride) * KVQ_BLOCK_TOKENS)
        return fail(KVQ_ERR_ARG, "%s: sequence %d slot %d outside the table row", who, b, slots[j]);
    if ((m.win_slot >= 0) != (m.mid_slot >= 0) || (m.demote_slot >= 0) != (m.low_slot >= 0))
      return fail(KVQ_ERR_ARG, "%s: sequence %d has a half-specified move", who, b);
  }
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  for (int32_t b0 = 0; b0 < batch; b0 += kvq::kRequantMaxSeqs) {
    const int n = std::min(batch - b0, kvq::kRequantMaxSeqs);
    a.seq0 = b0;
    for (int i = 0; i < n; ++i) {
      const kvq_lq_move& m = moves[b0 + i];
      a.moves[i][0] = m.win_slot;
      a.moves[i][1] = m.mid_slot;
      a.moves[i][2] = m.demote_slot;
      a.moves[i][3] = m.low_slot;
    }
    const hipError_t e = kvq::launch_requant(a, n, s);
    if (e != hipSuccess) return device_status(e, who);
  }
  return ok();
}

kvq_status kvq_logquant_classes(int32_t total, int32_t window, int8_t* cls_out) {
  if (total < 0 || window < 1) return fail(KVQ_ERR_ARG, "kvq_logquant_classes: total < 0 or window < 1");
  if (total > 0 && !cls_out) return fail(KVQ_ERR_ARG, "kvq_logquant_classes: null output");
  for (int32_t pos = 0; pos < total; ++pos) {
    const int64_t dist = static_cast<int64_t>(total) - 1 - pos;
    if (dist < window) {
      cls_out[pos] = 0;
      continue;
    }
    const int64_t r = dist - window;
    // span k: (2^k - 1) W <= r < (2^(k+1) - 1) W, i.e. 2^k <= r/W + 1 < 2^(k+1)
    const int64_t q = r / window + 1;
    int k = 63 - __builtin_clzll(static_cast<unsigned long long>(q));
    const int64_t start = ((int64_t{1} << k) - 1) * window;
    cls_out[pos] = ((r - start) & ((int64_t{1} << k) - 1)) == 0 ? 1 : 2;
  }
  return ok();
}

kvq_status kvq_page_alloc(const int32_t* free_list, int32_t n_free, int32_t* cursor, int32_t batch,
                          const int32_t* old_len, const int32_t* new_len, int32_t* block_table,
                          int32_t table_stride) {
  if (!cursor || batch < 0 || n_free < 0) return fail(KVQ_ERR_ARG, "kvq_page_alloc: bad arguments");
  if (batch > 0 && (!old_len || !new_len || !block_table)) return fail(KVQ_ERR_ARG, "kvq_page_alloc: null pointer");
  if (n_free > 0 && !free_list) return fail(KVQ_ERR_ARG, "kvq_page_alloc: null free list");
  if (*cursor < 0 || *cursor > n_free) return fail(KVQ_ERR_ARG, "kvq_page_alloc: cursor out of range");
  int64_t need = 0;
  for (int s = 0; s < batch; ++s) {
    if (old_len[s] < 0 || new_len[s] < old_len[s])
      return fail(KVQ_ERR_ARG, "kvq_page_alloc: seq %d needs 0 <= old_len <= new_len", s);
    const int have = (old_len[s] + KVQ_BLOCK_TOKENS - 1) / KVQ_BLOCK_TOKENS;
    const int want = (new_len[s] + KVQ_BLOCK_TOKENS - 1) / KVQ_BLOCK_TOKENS;
    if (want > table_stride)
      return fail(KVQ_ERR_ARG, "kvq_page_alloc: seq %d needs %d blocks > table_stride %d", s, want, table_stride);
    need += want - have;
  }
  if (need > n_free - *cursor)
    return fail(KVQ_ERR_CAPACITY, "kvq_page_alloc: need %lld blocks, %d free", static_cast<long long>(need),
                n_free - *cursor);
  for (int s = 0; s < batch; ++s) {
    const int have = (old_len[s] + KVQ_BLOCK_TOKENS - 1) / KVQ_BLOCK_TOKENS;
    const int want = (new_len[s] + KVQ_BLOCK_TOKENS - 1) / KVQ_BLOCK_TOKENS;
    for (int lb = have; lb < want; ++lb)
      block_table[static_cast<int64_t>(s) * table_stride + lb] = free_list[(*cursor)++];
  }
  return ok();
}

kvq_status kvq_quantize_append(const kvq_layout* L, void* pool, int64_t pool_blocks, const int32_t* block_table,
                               int32_t table_stride, int32_t batch, const int32_t* start_pos, int32_t n_new,
                               const void* k, const void* v, kvq_dtype in_dtype, kvq_stream stream) {
  kvq_status st = check_layout_ready(L, "kvq_quantize_append");
  if (st != KVQ_OK) return st;
  if (batch < 0 || n_new < 0) return fail(KVQ_ERR_ARG, "kvq_quantize_append: batch/n_new < 0");
  if (in_dtype != KVQ_F32 && in_dtype != KVQ_BF16) return fail(KVQ_ERR_ARG, "kvq_quantize_append: bad dtype");
  if (batch == 0 || n_new == 0) return ok();
  if (!pool || !block_table || !start_pos || !k || !v) return fail(KVQ_ERR_ARG, "kvq_quantize_append: null pointer");
  if (pool_blocks < 1 || table_stride < 1) return fail(KVQ_ERR_ARG, "kvq_quantize_append: empty pool or table");
  if (static_cast<int64_t>(batch) * n_new > (int64_t{1} << 31) / 8)
    return fail(KVQ_ERR_ARG, "kvq_quantize_append: too many rows in one call");
  if (L->key_per_channel && n_new % KVQ_BLOCK_TOKENS != 0)
    return fail(KVQ_ERR_ARG, "kvq_quantize_append: per-channel keys are appended in whole blocks (n_new %d)", n_new);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // Token-wise rows of every head in one launch (each workgroup takes its
  // head's widths); per-channel keys then in one launch per key width.
  kvq::AppendArgs a{};
  a.pool = static_cast<uint8_t*>(pool);
  a.pool_blocks = pool_blocks;
  a.block_bytes = L->block_bytes;
  a.table = block_table;
  a.table_stride = table_stride;
  a.start_pos = start_pos;
  a.src[0] = k;
  a.src[1] = v;
  a.src_bf16 = in_dtype == KVQ_BF16;
  a.meta16 = L->meta_fp16;
  a.key_per_channel = L->key_per_channel;
  a.batch = batch;
  a.n_new = n_new;
  a.hkv = L->num_kv_heads;
  a.d = L->head_dim;
  a.had_block = L->had_block;
  a.n_heads = L->num_kv_heads;
  for (int h = 0; h < L->num_kv_heads; ++h) {
    a.heads[h] = h;
    a.area_off[0][h] = L->k_off[h];
    a.area_off[1][h] = L->v_off[h];
    a.head_bits[0][h] = static_cast<uint8_t>(L->bits_k[h]);
    a.head_bits[1][h] = static_cast<uint8_t>(L->bits_v[h]);
  }
  hipError_t e = kvq::launch_append(a, s);
  if (e != hipSuccess) return device_status(e, "kvq_quantize_append launch");
  if (L->key_per_channel) {
    bool done[KVQ_MAX_KV_HEADS] = {};
    for (int h0 = 0; h0 < L->num_kv_heads; ++h0) {
      if (done[h0] || L->bits_k[h0] == 16) continue;
      kvq::AppendArgs ak = a;
      ak.n_heads = 0;
      ak.bits[0] = L->bits_k[h0];
      for (int h = h0; h < L->num_kv_heads; ++h) {
        if (!done[h] && L->bits_k[h] == L->bits_k[h0]) {
          ak.heads[ak.n_heads] = h;
          ak.area_off[0][ak.n_heads] = L->k_off[h];
          ak.area_off[1][ak.n_heads] = L->v_off[h];
          ++ak.n_heads;
          done[h] = true;
        }
      }
      e = kvq::launch_append_kc(ak, s);
      if (e != hipSuccess) return device_status(e, "kvq_quantize_append launch (per-channel keys)");
    }
  }
  return ok();
}

kvq_status kvq_append_check(const kvq_layout* L, int32_t batch, const int32_t* start_pos_host, int32_t n_new,
                            int32_t table_stride) {
  kvq_status st = check_layout_ready(L, "kvq_append_check");
  if (st != KVQ_OK) return st;
  if (batch < 0 || n_new < 0 || table_stride < 1)
    return fail(KVQ_ERR_ARG, "kvq_append_check: batch < 0, n_new < 0 or table_stride < 1");
  if (batch > 0 && !start_pos_host) return fail(KVQ_ERR_ARG, "kvq_append_check: null start_pos_host");
  if (L->key_per_channel && n_new % KVQ_BLOCK_TOKENS != 0)
    return fail(KVQ_ERR_ARG, "kvq_append_check: per-channel keys are appended in whole blocks (n_new %d)", n_new);
  const int64_t capacity = static_cast<int64_t>(table_stride) * KVQ_BLOCK_TOKENS;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t p = start_pos_host[b];
    if (p < 0) return fail(KVQ_ERR_ARG, "kvq_append_check: sequence %d start_pos %lld < 0", b, static_cast<long long>(p));
    if (p + n_new > capacity)
      return fail(KVQ_ERR_ARG, "kvq_append_check: sequence %d tokens [%lld, %lld) exceed the table row (%d blocks)", b,
                  static_cast<long long>(p), static_cast<long long>(p + n_new), table_stride);
    if (L->key_per_channel && p % KVQ_BLOCK_TOKENS != 0)
      return fail(KVQ_ERR_ARG,
                  "kvq_append_check: sequence %d start_pos %lld is not a block boundary (per-channel keys)", b,
                  static_cast<long long>(p));
  }
  return ok();
}

kvq_status kvq_dequant(const kvq_layout* L, const void* pool, int64_t pool_blocks, const int32_t* block_table,
                       int32_t table_stride, int32_t seq, int32_t pos0, int32_t n, int32_t rotated, float* k_out,
                       float* v_out, kvq_stream stream) {
  kvq_status st = check_layout_ready(L, "kvq_dequant");
  if (st != KVQ_OK) return st;
  if (n < 0 || pos0 < 0 || seq < 0) return fail(KVQ_ERR_ARG, "kvq_dequant: negative seq, pos0 or n");
  if (n == 0) return ok();
  if (!pool || !block_table || !k_out || !v_out) return fail(KVQ_ERR_ARG, "kvq_dequant: null pointer");
  if (pool_blocks < 1) return fail(KVQ_ERR_ARG, "kvq_dequant: empty pool");
  const int64_t last_page = (static_cast<int64_t>(pos0) + n - 1) / KVQ_BLOCK_TOKENS;
  if (last_page >= table_stride)
    return fail(KVQ_ERR_ARG, "kvq_dequant: tokens [%d, %d) exceed the table row (%d blocks)", pos0, pos0 + n,
                table_stride);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  for (int half = 0; half < 2; ++half) {
    const int32_t* bits = half ? L->bits_v : L->bits_k;
    const int64_t* offs = half ? L->v_off : L->k_off;
    bool done[KVQ_MAX_KV_HEADS] = {};
    for (int h0 = 0; h0 < L->num_kv_heads; ++h0) {
      if (done[h0]) continue;
      kvq::DequantArgs a{};
      a.pool = static_cast<const uint8_t*>(pool);
      a.pool_blocks = pool_blocks;
      a.block_bytes = L->block_bytes;
      a.table_row = block_table + static_cast<int64_t>(seq) * table_stride;
      a.pos0 = pos0;
      a.n = n;
      a.hkv = L->num_kv_heads;
      a.d = L->head_dim;
      a.had_block = L->had_block;
      a.rotated = rotated != 0;
      a.meta16 = L->meta_fp16;
      a.bits = bits[h0];
      a.kc = half == 0 && L->key_per_channel && bits[h0] != 16;
      a.out = half ? v_out : k_out;
      for (int h = h0; h < L->num_kv_heads; ++h) {
        if (!done[h] && bits[h] == bits[h0]) {
          a.heads[a.n_heads] = h;
          a.area_off[a.n_heads] = offs[h];
          ++a.n_heads;
          done[h] = true;
        }
      }
      hipError_t e = kvq::launch_dequant(a, s);
      if (e != hipSuccess) return device_status(e, "kvq_dequant launch");
    }
  }
  return ok();
}

kvq_status kvq_decode_workspace_bytes(const kvq_segment* segs, int32_t n_segs, int32_t batch, size_t* bytes) {
  if (!bytes) return fail(KVQ_ERR_ARG, "kvq_decode_workspace_bytes: null output");
  kvq_status st = check_segments(segs, n_segs, batch, "kvq_decode_workspace_bytes");
  if (st != KVQ_OK) return st;
  const kvq_layout& L = *segs[0].layout;
  *bytes = ws_layout(batch, L.num_kv_heads, L.group, L.head_dim, plan_call(segs, n_segs, batch).slots).total;
  return ok();
}

kvq_status kvq_decode_workspace_init(void* ws, size_t ws_bytes, kvq_stream stream) {
  if (ws_bytes == 0) return ok();
  if (!ws) return fail(KVQ_ERR_ARG, "kvq_decode_workspace_init: null workspace");
  if (ws_bytes % 4 != 0 || reinterpret_cast<uintptr_t>(ws) % 4 != 0)
    return fail(KVQ_ERR_ARG, "kvq_decode_workspace_init: workspace not 4-byte aligned and sized");
  {
    std::lock_guard<std::mutex> lock(g_side_mutex);
    SideStreams* ss = nullptr;
    hipError_t e = side_streams(&ss, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_status(e, "kvq_decode_workspace_init side streams");
  }
  return device_status(kvq::launch_zero_words(static_cast<uint32_t*>(ws), ws_bytes / 4,
                                              reinterpret_cast<hipStream_t>(stream)),
                       "kvq_decode_workspace_init launch");
}

// The partial launches of one decode call. serial: every launch goes on the
// caller's stream, one after another (no side streams are created or used).
static kvq_status decode_partial_impl(const kvq_segment* segs, int32_t n_segs, int32_t batch, const void* q,
                                      kvq_dtype q_dtype, void* ws, size_t ws_bytes, kvq_stream stream, bool serial,
                                      const FusedAppend* fa = nullptr) {
  kvq_status st = check_segments(segs, n_segs, batch, "kvq_decode_partial");
  if (st != KVQ_OK) return st;
  if (q_dtype != KVQ_F32 && q_dtype != KVQ_BF16) return fail(KVQ_ERR_ARG, "kvq_decode_partial: bad q dtype");
  if (batch == 0) return ok();
  if (!q || !ws) return fail(KVQ_ERR_ARG, "kvq_decode_partial: null q or workspace");
  if (reinterpret_cast<uintptr_t>(q) % 16 != 0) return fail(KVQ_ERR_ARG, "kvq_decode_partial: q not 16-byte aligned");
  const kvq_layout& L0 = *segs[0].layout;
  const int hq = L0.num_kv_heads * L0.group;
  const int d = L0.head_dim;
  const CallPlan plan = plan_call(segs, n_segs, batch, fa != nullptr);
  const WsLayout wl = ws_layout(batch, L0.num_kv_heads, L0.group, d, plan.slots);
  if (ws_bytes < wl.total)
    return fail(KVQ_ERR_WORKSPACE, "kvq_decode_partial: workspace %zu < %zu bytes", ws_bytes, wl.total);
  uint32_t* steal = static_cast<uint32_t*>(ws);
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  const bool share_tail =
      !deterministic_order() && counter_words(batch, L0.num_kv_heads, plan.slots) * sizeof(uint32_t) <= kCounterBytes;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);

  kvq::DecodeArgs base{};
  base.q = q;
  base.q_bf16 = q_dtype == KVQ_BF16;
  base.hkv = L0.num_kv_heads;
  base.group = L0.group;
  base.had_block = L0.had_block;
  base.batch = batch;
  base.total_slots = plan.slots;
  base.share_tail = share_tail ? 1 : 0;
  base.part_o = reinterpret_cast<float*>(wsb + wl.part_o);
  base.part_ml = reinterpret_cast<float*>(wsb + wl.part_ml);
  base.qrot = reinterpret_cast<float*>(wsb + wl.qrot);
  if (fa) {
    fill_token_append(segs, *fa, base.ap);
    base.anew = reinterpret_cast<float*>(wsb + wl.anew);
  }

  std::vector<int> slot_base(n_segs, 0);
  for (int i = 1; i < n_segs; ++i) slot_base[i] = slot_base[i - 1] + plan.split[i - 1].n_splits;
  // segment i's part of a launch, over head entries [head_base, head_base + n_heads)
  auto seg_desc = [&](int i, int head_base, int n_heads, int grid_start) {
    const kvq_segment& sg = segs[i];
    kvq::DecodeSeg ds{};
    ds.pool = static_cast<const uint8_t*>(sg.pool);
    ds.pool_blocks = sg.pool_blocks;
    ds.block_bytes = sg.layout->block_bytes;
    ds.table = sg.block_table;
    ds.table_stride = sg.table_stride;
    ds.seq_lens = sg.seq_lens;
    ds.steal = steal + static_cast<size_t>(slot_base[i] / 8) * batch * L0.num_kv_heads * 2;
    ds.slot_base = slot_base[i];
    ds.n_splits = plan.split[i].n_splits;
    ds.grid_start = grid_start;
    ds.n_heads = n_heads;
    ds.head_base = head_base;
    ds.write_q = i == plan.q_writer;
    ds.skip_pos = fa && i == fa->seg ? fa->start_pos : nullptr;
    return ds;
  };
  struct Launch {
    kvq::DecodeArgs a;
    int kbits, vbits;
    bool multi;
    // a wave's share of the launch: pages per split times the bytes of a
    // page of its heaviest head (orders the launches: the longest first)
    int64_t bytes;
  };
  std::vector<Launch> launches;
  // bytes one wave reads for head h of segment i: its pages per split times
  // the head's K and V codes and metadata per page
  auto wave_bytes = [&](int i, int h) {
    const kvq_layout& L = *segs[i].layout;
    const int64_t page = static_cast<int64_t>(KVQ_BLOCK_TOKENS) * (L.bits_k[h] + L.bits_v[h]) * d / 8 +
                         2 * KVQ_BLOCK_TOKENS * (L.meta_fp16 ? 4 : 8);
    const int pages = (std::max(segs[i].max_len, 0) + KVQ_BLOCK_TOKENS - 1) / KVQ_BLOCK_TOKENS;
    const int splits = std::max(plan.split[i].n_splits, 1);
    return page * ((pages + splits - 1) / splits);
  };
  auto add_head = [&](kvq::DecodeArgs& a, const kvq_layout& L, int h, int e) {
    a.heads[e] = h;
    a.k_off[e] = L.k_off[h];
    a.v_off[e] = L.v_off[h];
    a.pair[e] = static_cast<uint8_t>(L.bits_k[h] << 4 | L.bits_v[h]);
  };
  const bool allow_mixed = mixed_launch_enabled();
  auto mixable = [&](const kvq_layout& L, int h) {
    return allow_mixed && !L.key_per_channel && kvq::decode_partial_mixable(L.bits_k[h], L.bits_v[h], d);
  };
  // Heads of 2-, 3- and 4-bit pairs, over every segment (of one metadata
  // width), share one multi-format launch when they make more than one
  // (segment, pair) group; the rest get one launch per (segment, pair).
  int meta16_multi = -1;  // the metadata width whose heads go into the multi launch
  {
    int groups = 0, segs_in = 0, entries = 0, first_meta = -1;
    for (int i = 0; i < n_segs; ++i) {
      const kvq_layout& L = *segs[i].layout;
      if (plan.split[i].n_splits == 0) continue;
      if (first_meta < 0) first_meta = L.meta_fp16;
      if (L.meta_fp16 != first_meta) continue;
      int pairs[KVQ_MAX_KV_HEADS], np = 0, here = 0;
      for (int h = 0; h < L.num_kv_heads; ++h) {
        if (!mixable(L, h)) continue;
        ++here;
        const int pr = L.bits_k[h] << 4 | L.bits_v[h];
        bool seen = false;
        for (int k = 0; k < np; ++k) seen = seen || pairs[k] == pr;
        if (!seen) pairs[np++] = pr;
      }
      if (here) ++segs_in;
      groups += np;
      entries += here;
    }
    if (groups >= 2 && segs_in <= kvq::kMaxLaunchSegs && entries <= KVQ_MAX_KV_HEADS) meta16_multi = first_meta;
  }
  if (meta16_multi >= 0) {
    Launch l{base, 0, 0, true, 0};
    int e = 0, grid = 0;
    for (int i = 0; i < n_segs; ++i) {
      const kvq_layout& L = *segs[i].layout;
      if (plan.split[i].n_splits == 0 || L.meta_fp16 != meta16_multi) continue;
      const int e0 = e;
      for (int h = 0; h < L.num_kv_heads; ++h)
        if (mixable(L, h)) {
          add_head(l.a, L, h, e++);
          l.bytes = std::max(l.bytes, wave_bytes(i, h));
        }
      if (e == e0) continue;
      l.a.seg[l.a.n_segs++] = seg_desc(i, e0, e - e0, grid);
      grid += plan.split[i].n_splits * (e - e0) * batch;
    }
    l.a.meta16 = meta16_multi;
    launches.push_back(l);
  }
  for (int i = 0; i < n_segs; ++i) {
    const kvq_layout& L = *segs[i].layout;
    if (plan.split[i].n_splits == 0) continue;
    const bool in_multi = meta16_multi >= 0 && L.meta_fp16 == meta16_multi;
    bool done[KVQ_MAX_KV_HEADS] = {};
    for (int h0 = 0; h0 < L.num_kv_heads; ++h0) {
      if (done[h0] || (in_multi && mixable(L, h0))) continue;
      Launch l{base, L.bits_k[h0], L.bits_v[h0], false, 0};
      l.a.meta16 = L.meta_fp16;
      l.a.kc = L.key_per_channel;
      int e = 0;
      for (int h = h0; h < L.num_kv_heads; ++h) {
        if (!done[h] && L.bits_k[h] == L.bits_k[h0] && L.bits_v[h] == L.bits_v[h0] && !(in_multi && mixable(L, h))) {
          add_head(l.a, L, h, e++);
          done[h] = true;
        }
      }
      l.a.seg[0] = seg_desc(i, 0, e, 0);
      l.a.n_segs = 1;
      l.bytes = wave_bytes(i, h0);
      launches.push_back(l);
    }
  }
  auto launch = [&](const Launch& l, hipStream_t st) {
    return l.multi ? kvq::launch_decode_partial_multi(l.a, d, st)
                   : kvq::launch_decode_partial(l.a, l.kbits, l.vbits, d, st);
  };
  if (launches.empty()) return ok();
  if (launches.size() == 1) return device_status(launch(launches[0], s), "kvq_decode_partial launch");
  if (serial) {
    for (const Launch& l : launches) {
      const hipError_t e = launch(l, s);
      if (e != hipSuccess) return device_status(e, "kvq_decode_partial launch");
    }
    return ok();
  }
  // Several launches (width groups that cannot share a launch) run
  // concurrently: the one whose waves have most to read on the caller's
  // stream, which starts it first (side-stream launches start 10-25 us
  // later), the others on side streams forked from it and joined back before
  // the call returns. (One after another on one stream is slower: small
  // launches are latency-bound and then add up.)
  std::stable_sort(launches.begin(), launches.end(),
                   [](const Launch& x, const Launch& y) { return x.bytes > y.bytes; });
  std::lock_guard<std::mutex> lock(g_side_mutex);
  SideStreams* ss = nullptr;
  hipError_t e = side_streams(&ss, s);
  if (e != hipSuccess)
    return device_status(e, "kvq_decode_partial side streams (call kvq_decode_workspace_init before capturing)");
  const int n_side = std::min<int>(kSideStreams, static_cast<int>(launches.size()) - 1);
  if ((e = hipEventRecord(ss->fork, s)) != hipSuccess) return device_status(e, "kvq_decode_partial fork");
  // Every side stream that was forked is joined back, also after a failed
  // launch, so the caller's stream (or a capture of it) never leaves work of
  // this call behind on a side stream.
  int forked = 0;
  hipError_t first = hipSuccess;
  const char* what = "kvq_decode_partial launch";
  for (; forked < n_side; ++forked) {
    if ((e = hipStreamWaitEvent(ss->s[forked], ss->fork, 0)) != hipSuccess) {
      first = e;
      what = "kvq_decode_partial fork";
      break;
    }
  }
  for (size_t j = 0; j < launches.size() && first == hipSuccess; ++j) {
    hipStream_t st = j == 0 ? s : ss->s[(j - 1) % n_side];
    first = launch(launches[j], st);
  }
  for (int i = 0; i < forked; ++i) {
    hipError_t ej = hipEventRecord(ss->join[i], ss->s[i]);
    if (ej == hipSuccess) ej = hipStreamWaitEvent(s, ss->join[i], 0);
    if (ej != hipSuccess && first == hipSuccess) {
      first = ej;
      what = "kvq_decode_partial join";
    }
  }
  return device_status(first, what);
}

kvq_status kvq_decode_partial(const kvq_segment* segs, int32_t n_segs, int32_t batch, const void* q,
                              kvq_dtype q_dtype, void* ws, size_t ws_bytes, kvq_stream stream) {
  return decode_partial_impl(segs, n_segs, batch, q, q_dtype, ws, ws_bytes, stream, false);
}

kvq_status kvq_measure_read_stream(const void* buf, size_t bytes, uint32_t* sink, int32_t sink_words,
                                   kvq_stream stream) {
  constexpr int kWaves = 2048;
  if (!buf || !sink) return fail(KVQ_ERR_ARG, "kvq_measure_read_stream: null pointer");
  if (bytes < 8192 || bytes % 8192 != 0 || reinterpret_cast<uintptr_t>(buf) % 16 != 0)
    return fail(KVQ_ERR_ARG, "kvq_measure_read_stream: bytes must be a positive multiple of 8192, buf 16-byte aligned");
  if (sink_words < kWaves) return fail(KVQ_ERR_ARG, "kvq_measure_read_stream: sink_words %d < %d", sink_words, kWaves);
  return device_status(kvq::launch_measure_stream(buf, bytes, sink, kWaves, reinterpret_cast<hipStream_t>(stream)),
                       "kvq_measure_read_stream");
}

kvq_status kvq_measure_read_paged(const kvq_segment* segs, int32_t n_segs, int32_t batch, int32_t splits,
                                  uint32_t* sink, int32_t sink_words, kvq_stream stream) {
  const char* who = "kvq_measure_read_paged";
  kvq_status st = check_segments(segs, n_segs, batch, who);
  if (st != KVQ_OK) return st;
  if (batch < 1) return fail(KVQ_ERR_ARG, "%s: need batch >= 1", who);
  if (!sink) return fail(KVQ_ERR_ARG, "%s: null sink", who);
  if (splits != 0 && (splits < 8 || splits % 8 != 0))
    return fail(KVQ_ERR_ARG, "%s: splits %d not a positive multiple of 8", who, splits);
  std::vector<int> plan(n_segs);
  for (int i = 0; i < n_segs; ++i) {
    const kvq_segment& sg = segs[i];
    if (sg.max_len < 1) return fail(KVQ_ERR_ARG, "%s: segment %d: max_len %d < 1", who, i, sg.max_len);
    if (!kvq::measure_paged_covers(*sg.layout))
      return fail(KVQ_ERR_UNSUPPORTED, "%s: segment %d: areas of more than 2 KiB per head (16-bit rows) are not "
                  "covered", who, i);
    plan[i] = splits != 0 ? splits : plan_splits(sg, batch).n_splits;
    const int64_t waves = static_cast<int64_t>(plan[i]) * sg.layout->num_kv_heads * batch;
    if (sink_words < waves)
      return fail(KVQ_ERR_ARG, "%s: segment %d: sink_words %d < %lld waves", who, i, sink_words,
                  static_cast<long long>(waves));
  }
  for (int i = 0; i < n_segs; ++i) {
    const hipError_t e = kvq::launch_measure_paged(segs[i], batch, plan[i], sink, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_status(e, who);
  }
  return ok();
}

}  // extern "C"

static kvq_status decode_merge_impl(const kvq_segment* segs, int32_t n_segs, int32_t batch, float* out, void* ws,
                                    size_t ws_bytes, kvq_stream stream, const FusedAppend* fa) {
  kvq_status st = check_segments(segs, n_segs, batch, "kvq_decode_merge");
  if (st != KVQ_OK) return st;
  if (batch == 0) return ok();
  if (!out || !ws) return fail(KVQ_ERR_ARG, "kvq_decode_merge: null output or workspace");
  const kvq_layout& L0 = *segs[0].layout;
  const int hq = L0.num_kv_heads * L0.group;
  const CallPlan plan = plan_call(segs, n_segs, batch, fa != nullptr);
  const WsLayout wl = ws_layout(batch, L0.num_kv_heads, L0.group, L0.head_dim, plan.slots);
  if (ws_bytes < wl.total)
    return fail(KVQ_ERR_WORKSPACE, "kvq_decode_merge: workspace %zu < %zu bytes", ws_bytes, wl.total);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // With no split at all the merge kernel still runs and writes zero rows
  // (no memset node, so the call stays safe to capture in a graph).
  const uint8_t* wsb = static_cast<const uint8_t*>(ws);
  kvq::MergeArgs a{};
  a.part_o = reinterpret_cast<const float*>(wsb + wl.part_o);
  a.part_ml = reinterpret_cast<const float*>(wsb + wl.part_ml);
  a.qrot = reinterpret_cast<const float*>(wsb + wl.qrot);
  a.batch = batch;
  a.hq = hq;
  a.d = L0.head_dim;
  a.had_block = L0.had_block;
  a.total_slots = plan.slots;
  a.group = L0.group;
  a.out = out;
  if (plan.window >= 0) {
    const kvq_segment& w = segs[plan.window];
    a.win.pool = static_cast<const uint8_t*>(w.pool);
    a.win.pool_blocks = w.pool_blocks;
    a.win.block_bytes = w.layout->block_bytes;
    a.win.table = w.block_table;
    a.win.table_stride = w.table_stride;
    a.win.seq_lens = w.seq_lens;
    a.win.skip_pos = fa && fa->seg == plan.window ? fa->start_pos : nullptr;
    a.win.max_len = w.max_len;
    for (int h = 0; h < w.layout->num_kv_heads; ++h) {
      a.win.k_off[h] = w.layout->k_off[h];
      a.win.v_off[h] = w.layout->v_off[h];
    }
  }
  if (fa) {
    fill_token_append(segs, *fa, a.ap);
    a.anew = reinterpret_cast<const float*>(wsb + wl.anew);
  }
  return device_status(kvq::launch_decode_merge(a, s), "kvq_decode_merge launch");
}

extern "C" {

kvq_status kvq_decode_merge(const kvq_segment* segs, int32_t n_segs, int32_t batch, float* out, void* ws,
                            size_t ws_bytes, kvq_stream stream) {
  return decode_merge_impl(segs, n_segs, batch, out, ws, ws_bytes, stream, nullptr);
}

kvq_status kvq_decode_attn(const kvq_segment* segs, int32_t n_segs, int32_t batch, const void* q, kvq_dtype q_dtype,
                           float* out, void* ws, size_t ws_bytes, kvq_stream stream) {
  kvq_status st = kvq_decode_partial(segs, n_segs, batch, q, q_dtype, ws, ws_bytes, stream);
  if (st != KVQ_OK) return st;
  return kvq_decode_merge(segs, n_segs, batch, out, ws, ws_bytes, stream);
}

}  // extern "C"

// The fused append's own argument checks (before any launch); the segments
// are checked by the partial and merge calls.
static kvq_status check_fused(const kvq_segment* segs, int32_t n_segs, int32_t batch, int32_t append_seg,
                              const int32_t* start_pos, const void* k_new, const void* v_new, kvq_dtype in_dtype,
                              bool rows, const char* who) {
  kvq_status st = check_segments(segs, n_segs, batch, who);
  if (st != KVQ_OK) return st;
  if (append_seg < 0 || append_seg >= n_segs)
    return fail(KVQ_ERR_ARG, "%s: append_seg %d outside [0, %d)", who, append_seg, n_segs);
  const kvq_segment& g = segs[append_seg];
  if (g.layout->key_per_channel)
    return fail(KVQ_ERR_UNSUPPORTED, "%s: per-channel keys are appended in whole blocks (kvq_quantize_append)", who);
  if (batch == 0) return ok();
  if (!start_pos) return fail(KVQ_ERR_ARG, "%s: null start_pos", who);
  if (!rows) return ok();
  if (in_dtype != KVQ_F32 && in_dtype != KVQ_BF16) return fail(KVQ_ERR_ARG, "%s: bad input dtype", who);
  if (!k_new || !v_new) return fail(KVQ_ERR_ARG, "%s: null k_new or v_new", who);
  if (reinterpret_cast<uintptr_t>(k_new) % 16 != 0 || reinterpret_cast<uintptr_t>(v_new) % 16 != 0)
    return fail(KVQ_ERR_ARG, "%s: k_new and v_new must be 16-byte aligned", who);
  if (!g.pool || !g.block_table || !g.seq_lens) return fail(KVQ_ERR_ARG, "%s: null pool, table or lengths", who);
  return ok();
}

extern "C" {

// The partial half quantizes and stores the new token (its split-0 waves) and
// needs the new rows; the merge half reads the token's dequantized rows from
// the workspace and needs only where the token went.
kvq_status kvq_append_decode_partial(const kvq_segment* segs, int32_t n_segs, int32_t batch, int32_t append_seg,
                                     const int32_t* start_pos, const void* k_new, const void* v_new,
                                     kvq_dtype in_dtype, const void* q, kvq_dtype q_dtype, void* ws,
                                     size_t ws_bytes, kvq_stream stream) {
  kvq_status st = check_fused(segs, n_segs, batch, append_seg, start_pos, k_new, v_new, in_dtype, true,
                              "kvq_append_decode_partial");
  if (st != KVQ_OK || batch == 0) return st;
  const FusedAppend fa{append_seg, start_pos, k_new, v_new, in_dtype};
  return decode_partial_impl(segs, n_segs, batch, q, q_dtype, ws, ws_bytes, stream, false, &fa);
}

kvq_status kvq_append_decode_merge(const kvq_segment* segs, int32_t n_segs, int32_t batch, int32_t append_seg,
                                   const int32_t* start_pos, float* out, void* ws, size_t ws_bytes,
                                   kvq_stream stream) {
  kvq_status st = check_fused(segs, n_segs, batch, append_seg, start_pos, nullptr, nullptr, KVQ_BF16, false,
                              "kvq_append_decode_merge");
  if (st != KVQ_OK || batch == 0) return st;
  // (the merge kernel reads no new row: only the slot, its page and the lengths)
  const FusedAppend fa{append_seg, start_pos, nullptr, nullptr, KVQ_BF16};
  return decode_merge_impl(segs, n_segs, batch, out, ws, ws_bytes, stream, &fa);
}

kvq_status kvq_append_decode_attn(const kvq_segment* segs, int32_t n_segs, int32_t batch, int32_t append_seg,
                                  const int32_t* start_pos, const void* k_new, const void* v_new, kvq_dtype in_dtype,
                                  const void* q, kvq_dtype q_dtype, float* out, void* ws, size_t ws_bytes,
                                  kvq_stream stream) {
  // (every argument checked before the first launch)
  kvq_status st = check_fused(segs, n_segs, batch, append_seg, start_pos, k_new, v_new, in_dtype, true,
                              "kvq_append_decode_attn");
  if (st != KVQ_OK || batch == 0) return st;
  st = kvq_append_decode_partial(segs, n_segs, batch, append_seg, start_pos, k_new, v_new, in_dtype, q, q_dtype,
                                 ws, ws_bytes, stream);
  if (st != KVQ_OK) return st;
  return kvq_append_decode_merge(segs, n_segs, batch, append_seg, start_pos, out, ws, ws_bytes, stream);
}

}  // extern "C"

namespace {

// Scratch memory of kvq_decode_attn_noalloc: the decode workspace (counter
// area, then partials) in a fixed device array, one copy per GPU the library
// runs on, held until the process ends. Host code never uses the array's name
// as an address (on the host it is only a stand-in): the device address comes
// from hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kNoallocScratchBytes = KVQ_NOALLOC_SCRATCH_BYTES;
static_assert(kNoallocScratchBytes % 256 == 0 && kNoallocScratchBytes > kCounterBytes, "scratch size");
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address; on the first call for a device its
// counter area is cleared on `s` (a kernel, not a memset node), which every
// later call on that device's streams follows in stream order or by the
// caller's synchronisation.
hipError_t noalloc_scratch(void** out, hipStream_t s) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if ((e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    if ((e = kvq::launch_zero_words(static_cast<uint32_t*>(ptr), kCounterBytes / 4, s)) != hipSuccess) return e;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

kvq_status kvq_decode_attn_noalloc(const kvq_segment* segs, int32_t n_segs, int32_t batch, const void* q,
                                   kvq_dtype q_dtype, float* out, kvq_stream stream) {
  const char* who = "kvq_decode_attn_noalloc";
  kvq_status st = check_segments(segs, n_segs, batch, who);
  if (st != KVQ_OK) return st;
  if (q_dtype != KVQ_F32 && q_dtype != KVQ_BF16) return fail(KVQ_ERR_ARG, "%s: bad q dtype", who);
  if (batch == 0) return ok();
  if (!q || !out) return fail(KVQ_ERR_ARG, "%s: null q or output", who);
  const kvq_layout& L0 = *segs[0].layout;
  const size_t need =
      ws_layout(batch, L0.num_kv_heads, L0.group, L0.head_dim, plan_call(segs, n_segs, batch).slots).total;
  if (need > kNoallocScratchBytes)
    return fail(KVQ_ERR_WORKSPACE, "%s: this call needs %zu bytes of scratch, more than the fixed %zu", who, need,
                kNoallocScratchBytes);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void* ws = nullptr;
  const hipError_t e = noalloc_scratch(&ws, s);
  if (e != hipSuccess) return device_status(e, "kvq_decode_attn_noalloc scratch");
  st = decode_partial_impl(segs, n_segs, batch, q, q_dtype, ws, kNoallocScratchBytes, stream, true);
  if (st != KVQ_OK) return st;
  return kvq_decode_merge(segs, n_segs, batch, out, ws, kNoallocScratchBytes, stream);
}

}  // extern "C"
