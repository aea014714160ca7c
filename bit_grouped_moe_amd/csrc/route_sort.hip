// Token-to-expert grouping on the device: a deterministic stable counting
// sort, one launch.  The pages require every active expert to run in one
// launch without a host round trip ("grouped-nf4-gemm 0.43.0", page
// header; "flashrt/grouped-moe-gemv", "Functions": no host
// synchronisation); the grouping itself is this library's design.
//
// Launch: E + 1 workgroups of 1024 threads.  Workgroup b < E owns expert b,
// workgroup E owns the dropped pairs.  Each workgroup
//   1. builds the full expert histogram in LDS (integer LDS atomics: the
//      counts do not depend on their order),
//   2. reduces it to its own segment start and tile base,
//   3. compacts its pairs in ascending pair order with one block-wide
//      exclusive scan over contiguous per-thread chunks, and
//   4. writes its offsets entry and its tiles.
// No global atomics, no workspace; the result is the unique stable order.
#include "gq_device.hpp"
#include "gq_host.hpp"
#include "../../include/gq.h"

namespace gq {

constexpr int kSortThreads = 1024;
constexpr int kSortWaves = kSortThreads / kWave;

// Block-wide sum of v (all threads get the result).
__device__ __forceinline__ int block_sum(int v, int* red) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  int s = 0;
#pragma unroll
  for (int i = 0; i < kSortWaves; ++i) s += red[i];
  return s;
}

// Block-wide exclusive scan of v; *total gets the sum.
__device__ __forceinline__ int block_exclusive_scan(int v, int* red, int* total) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  int inc = wave_inclusive_scan(v);
  __syncthreads();
  if (lane == kWave - 1) red[w] = inc;
  __syncthreads();
  int base = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kSortWaves; ++i) {
    int r = red[i];
    base += (i < w) ? r : 0;
    all += r;
  }
  *total = all;
  return base + inc - v;
}

constexpr int kIdsPerThread = 16;
constexpr int kSuperChunk = kSortThreads * kIdsPerThread;
constexpr int kPastEnd = INT32_MIN;  // marks slots beyond the last pair

// Load the kIdsPerThread contiguous ids of this thread in super-chunk sc.
// All loads are issued before any is used.
__device__ __forceinline__ void load_ids(const int32_t* __restrict__ ids, int32_t P, int sc,
                                         int v[kIdsPerThread]) {
  const int64_t base = (int64_t)sc * kSuperChunk + (int64_t)threadIdx.x * kIdsPerThread;
#pragma unroll
  for (int j = 0; j < kIdsPerThread; ++j) {
    int64_t idx = base + j;
    v[j] = idx < P ? ids[idx] : kPastEnd;
  }
}

__global__ __launch_bounds__(kSortThreads) void route_sort_kernel(
    const int32_t* __restrict__ ids, int32_t P, int32_t E, int32_t tile_m,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pairs,
    int32_t* __restrict__ tiles, int32_t max_tiles, int32_t* __restrict__ num_tiles) {
  __shared__ int hist[1024];
  __shared__ int red[kSortWaves];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const unsigned uE = (unsigned)E;
  const int n_super = (P + kSuperChunk - 1) / kSuperChunk;

  for (int e = tid; e < E; e += kSortThreads) hist[e] = 0;
  __syncthreads();
  for (int sc = 0; sc < n_super; ++sc) {
    int v[kIdsPerThread];
    load_ids(ids, P, sc, v);
#pragma unroll
    for (int j = 0; j < kIdsPerThread; ++j)
      if ((unsigned)v[j] < uE) atomicAdd(&hist[v[j]], 1);
  }
  __syncthreads();

  // Segment start / tile base of expert b, and the grand totals.
  const int c = (tid < E) ? hist[tid] : 0;
  const int t = (c + tile_m - 1) / tile_m;
  const int seg_start = block_sum(tid < b ? c : 0, red);
  const int tile_base = block_sum(tid < b ? t : 0, red);
  const int valid_total = block_sum(c, red);
  const int tile_total = block_sum(t, red);

  // Stable compaction of this workgroup's pairs: thread-contiguous chunks
  // in ascending pair order, placed by a block-wide exclusive scan.
  int cursor = (b < E) ? seg_start : valid_total;
  for (int sc = 0; sc < n_super; ++sc) {
    int v[kIdsPerThread];
    load_ids(ids, P, sc, v);
    int mine = 0;
#pragma unroll
    for (int j = 0; j < kIdsPerThread; ++j) {
      bool hit = (b < E) ? (v[j] == b) : (v[j] != kPastEnd && (unsigned)v[j] >= uE);
      mine += hit ? 1 : 0;
    }
    int total = 0;
    int pos = cursor + block_exclusive_scan(mine, red, &total);
    const int base = sc * kSuperChunk + tid * kIdsPerThread;
#pragma unroll
    for (int j = 0; j < kIdsPerThread; ++j) {
      bool hit = (b < E) ? (v[j] == b) : (v[j] != kPastEnd && (unsigned)v[j] >= uE);
      if (hit) sorted_pairs[pos++] = base + j;
    }
    cursor += total;
  }

  if (b < E) {
    if (tid == 0) offsets[b] = seg_start;
    const int nt = (hist[b] + tile_m - 1) / tile_m;
    for (int j = tid; j < nt; j += kSortThreads) {
      tiles[2 * (tile_base + j)] = b;
      tiles[2 * (tile_base + j) + 1] = seg_start + j * tile_m;
    }
  } else {
    if (tid == 0) {
      offsets[E] = valid_total;
      num_tiles[0] = tile_total;
    }
    for (int j = tile_total + tid; j < max_tiles; j += kSortThreads) {
      tiles[2 * j] = -1;
      tiles[2 * j + 1] = -1;
    }
  }
}

}  // namespace gq

extern "C" int32_t gq_route_max_tiles(int32_t rows, int32_t topk, int32_t num_experts,
                                      int32_t tile_m) {
  if (rows < 0 || topk < 0 || num_experts < 1 || tile_m < 1) return -1;
  int64_t P = (int64_t)rows * topk;
  int64_t m = gq::ceil_div64(P, tile_m) + num_experts + 1;
  return m > INT32_MAX ? -1 : (int32_t)m;
}

extern "C" int gq_route_sort(const int32_t* topk_ids, int32_t rows, int32_t topk,
                             int32_t num_experts, int32_t tile_m, int32_t* expert_offsets,
                             int32_t* sorted_pairs, int32_t* tiles, int32_t max_tiles,
                             int32_t* num_tiles, hipStream_t stream) {
  using namespace gq;
  if (rows < 0 || topk < 0 || num_experts < 1 || tile_m < 1) return kInvalid;
  int64_t P = (int64_t)rows * topk;
  if (!expert_offsets || !tiles || !num_tiles) return kInvalid;
  if (P > 0 && (!topk_ids || !sorted_pairs)) return kInvalid;   // may be NULL when empty
  if (P >= INT32_MAX) return kNotSupported;
  if (num_experts > 1024) return kNotSupported;
  int32_t need = gq_route_max_tiles(rows, topk, num_experts, tile_m);
  if (need < 0 || max_tiles < need) return kInvalid;
  hipLaunchKernelGGL(route_sort_kernel, dim3(num_experts + 1), dim3(kSortThreads), 0, stream,
                     topk_ids, (int32_t)P, num_experts, tile_m, expert_offsets, sorted_pairs,
                     tiles, max_tiles, num_tiles);
  return launch_status();
}
