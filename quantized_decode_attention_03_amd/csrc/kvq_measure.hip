// Read-bandwidth references for measuring the decode kernel on the device it
// runs on. Neither is part of the decode path: they read and discard.
//
//  * measure_stream_kernel: a plain streaming read of a buffer, every wave
//    sweeping adjacent 8 KiB chunks (the device reads one contiguous window at
//    a time), 16 bytes per lane per load, eight loads in flight per wave.
//  * measure_paged_kernel: the partial decode kernel's load pattern with no
//    compute: one wave per (sequence, KV head, split) in the same
//    XCD-interleaved one-dimensional grid, each split a contiguous range of
//    four-page groups, and per page the head's key area (codes and metadata)
//    and value area, read through the block table (its entries one group
//    ahead), with the next two groups' loads in flight while one is folded. Its rate is what the cache's own
//    access pattern allows on this device.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

namespace {

constexpr int kStreamChunk = 8192;  // bytes per wave step (eight 1 KiB loads)

__global__ __launch_bounds__(64) void measure_stream_kernel(const uint8_t* buf, size_t chunks, uint32_t* sink) {
  const int lane = threadIdx.x;
  uint32_t acc = 0;
  for (size_t c = blockIdx.x; c < chunks; c += gridDim.x) {
    const uint8_t* p = buf + c * kStreamChunk + lane * 16;
    uint4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = ld_cache_u4(p + i * 1024);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  }
  // one word per wave, so the loads are not dropped
  acc = __builtin_amdgcn_readfirstlane(acc) ^ __builtin_amdgcn_readlane(acc, 63);
  if (lane == 0) sink[blockIdx.x] = acc;
}

struct PagedArgs {
  const uint8_t* pool;
  int64_t pool_blocks, block_bytes;
  const int32_t* table;
  int32_t table_stride;
  int32_t batch, n_heads, splits, pages;
  int32_t last16[2][KVQ_MAX_KV_HEADS];    // index of the last 16-byte chunk of each head's K / V area
  int64_t area_off[2][KVQ_MAX_KV_HEADS];
  uint32_t* sink;
};

// A head's K and V areas of one page are read as 16-byte chunks, lane l taking
// chunk l and, for areas of more than 1 KiB, chunk l + 64 (clamped to the
// area's last chunk: areas of up to 2 KiB, every width up to 8 bits at
// head_dim 128); an area of at most 1 KiB takes one load. A group is four
// pages.
struct PagedBuf {
  uint4 v[4][2][2];
};

// The four block-table entries of group g (clamped into the sequence's row),
// read one group before the group's pages, as the decode kernel does.
struct GroupTab {
  int32_t blk[4];
};

__device__ __forceinline__ GroupTab paged_tab(const PagedArgs& a, const int32_t* trow, int g) {
  GroupTab t;
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) t.blk[pp] = trow[max(min(4 * g + pp, a.pages - 1), 0)];
  return t;
}

__device__ __forceinline__ void paged_load(const PagedArgs& a, const GroupTab& t, int h, int lane, uint32_t nblk,
                                           PagedBuf& r) {
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) {
    const int32_t blk = t.blk[pp];
    const int64_t bo = static_cast<uint32_t>(blk) < nblk ? blk * a.block_bytes : 0;  // unmapped: block 0
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const uint4* base = reinterpret_cast<const uint4*>(a.pool + bo + a.area_off[half][h]);
      const int last = a.last16[half][h];
      r.v[pp][half][0] = ld_cache_u4(base + min(lane, last));
      // (the area's size is the same in every lane: a uniform branch)
      r.v[pp][half][1] = last >= 64 ? ld_cache_u4(base + min(lane + 64, last)) : make_uint4(0u, 0u, 0u, 0u);
    }
  }
}

__device__ __forceinline__ uint32_t paged_fold(const PagedBuf& r) {
  uint32_t x = 0;
#pragma unroll
  for (int pp = 0; pp < 4; ++pp)
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int i = 0; i < 2; ++i) x ^= r.v[pp][half][i].x ^ r.v[pp][half][i].y ^ r.v[pp][half][i].z ^ r.v[pp][half][i].w;
  return x;
}

__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2))) void measure_paged_kernel(PagedArgs a) {
  const int lane = threadIdx.x;
  const int U = a.n_heads * a.batch;
  const int m = static_cast<int>(blockIdx.x) / 8;
  const int unit = m % U;
  const int split = static_cast<int>(blockIdx.x) % 8 + 8 * (m / U);
  const int h = unit % a.n_heads, b = unit / a.n_heads;
  const int groups = (a.pages + 3) / 4;
  const int g0 = static_cast<int>(static_cast<int64_t>(groups) * split / a.splits);
  const int g1 = static_cast<int>(static_cast<int64_t>(groups) * (split + 1) / a.splits);
  const int32_t* trow = a.table + static_cast<int64_t>(b) * a.table_stride;
  const uint32_t nblk = a.pool_blocks > 0x7fffffff ? 0x80000000u : static_cast<uint32_t>(a.pool_blocks);
  // a ring of three groups: two in flight while one is folded; each group's
  // table entries are read one group ahead of its pages
  PagedBuf r0, r1, r2;
  uint32_t acc = 0;
  int g = g0;
  GroupTab t = paged_tab(a, trow, g);
  if (g < g1) paged_load(a, t, h, lane, nblk, r0);
  t = paged_tab(a, trow, g + 1);
  if (g + 1 < g1) paged_load(a, t, h, lane, nblk, r1);
  t = paged_tab(a, trow, g + 2);
  for (; g < g1; g += 3) {
    GroupTab tn = paged_tab(a, trow, g + 3);
    if (g + 2 < g1) paged_load(a, t, h, lane, nblk, r2);
    acc ^= paged_fold(r0);
    if (g + 1 >= g1) break;
    t = paged_tab(a, trow, g + 4);
    if (g + 3 < g1) paged_load(a, tn, h, lane, nblk, r0);
    acc ^= paged_fold(r1);
    if (g + 2 >= g1) break;
    tn = paged_tab(a, trow, g + 5);
    if (g + 4 < g1) paged_load(a, t, h, lane, nblk, r1);
    acc ^= paged_fold(r2);
    t = tn;
  }
  acc = __builtin_amdgcn_readfirstlane(acc) ^ __builtin_amdgcn_readlane(acc, 63);
  if (lane == 0) a.sink[blockIdx.x] = acc;
}

}  // namespace

hipError_t launch_measure_stream(const void* buf, size_t bytes, uint32_t* sink, int waves, hipStream_t s) {
  const size_t chunks = bytes / kStreamChunk;
  if (chunks == 0 || waves < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(measure_stream_kernel, dim3(static_cast<unsigned>(waves)), dim3(64), 0, s,
                     static_cast<const uint8_t*>(buf), chunks, sink);
  return hipGetLastError();
}

namespace {
int64_t area_bytes(const kvq_layout& L, int half, int h) {
  if (half == 0) return (h + 1 < L.num_kv_heads ? L.k_off[h + 1] : L.v_off[0]) - L.k_off[h];
  return (h + 1 < L.num_kv_heads ? L.v_off[h + 1] : L.block_bytes) - L.v_off[h];
}
}  // namespace

bool measure_paged_covers(const kvq_layout& L) {
  for (int h = 0; h < L.num_kv_heads; ++h)
    for (int half = 0; half < 2; ++half) {
      const int64_t n = area_bytes(L, half, h);
      if (n % 16 != 0 || n < 16 || n > 2048) return false;
    }
  return true;
}

hipError_t launch_measure_paged(const kvq_segment& seg, int batch, int splits, uint32_t* sink, hipStream_t s) {
  const kvq_layout& L = *seg.layout;
  PagedArgs a{};
  a.pool = static_cast<const uint8_t*>(seg.pool);
  a.pool_blocks = seg.pool_blocks;
  a.block_bytes = L.block_bytes;
  a.table = seg.block_table;
  a.table_stride = seg.table_stride;
  a.batch = batch;
  a.n_heads = L.num_kv_heads;
  a.splits = splits;
  a.pages = (seg.max_len + KVQ_BLOCK_TOKENS - 1) / KVQ_BLOCK_TOKENS;
  if (a.pages == 0 || batch == 0 || splits < 8 || splits % 8 != 0 || !measure_paged_covers(L))
    return hipErrorInvalidValue;
  for (int h = 0; h < L.num_kv_heads; ++h) {
    a.area_off[0][h] = L.k_off[h];
    a.area_off[1][h] = L.v_off[h];
    a.last16[0][h] = static_cast<int32_t>(area_bytes(L, 0, h) / 16 - 1);
    a.last16[1][h] = static_cast<int32_t>(area_bytes(L, 1, h) / 16 - 1);
  }
  a.sink = sink;
  hipLaunchKernelGGL(measure_paged_kernel, dim3(static_cast<unsigned>(splits) * a.n_heads * batch), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvq
