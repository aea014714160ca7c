// Token-to-expert grouping on the device: a deterministic stable counting
// sort, one launch.  The pages require every active expert to run in one
// launch without a host round trip ("grouped-nf4-gemm 0.43.0", page
// header; "flashrt/grouped-moe-gemv", "Functions": no host
// synchronisation); the grouping itself is this library's design.
//
// Launch: E + 1 workgroups of 1024 threads.  Workgroup b < E owns expert b,
// workgroup E owns the dropped pairs.  Each workgroup
//   1. stages the ids in LDS with coalesced loads (32768 per pass),
//   2. builds the full expert histogram in LDS (integer LDS atomics: the
//      counts do not depend on their order) and reduces it to its own
//      segment start and tile base,
//   3. compacts its pairs in ascending pair order: wave w owns a contiguous
//      range of 2048 ids, lane l takes ids range + 64j + l (conflict-free LDS
//      reads) and the wave keeps the 32 match ballots in scalar registers;
//      a pair's place is the workgroup's cursor + the earlier waves' counts
//      + the wave's running count + its rank among the matching lanes
//      (ballot bit count), and
//   4. writes its offsets entry and its tiles.
// No global atomics, no workspace; the result is the unique stable order.
#include "gq_device.hpp"
#include "gq_host.hpp"
#include "../../include/gq.h"

namespace gq {

constexpr int kSortThreads = 1024;
constexpr int kSortWaves = kSortThreads / kWave;
constexpr int kChunkIds = 32768;                          // ids staged in LDS per pass
constexpr int kPerLane = kChunkIds / kSortThreads;        // 32
constexpr int kPastEnd = INT32_MIN;                       // slots beyond the last pair

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

// Stage ids [c0, c0 + kChunkIds) in LDS (kPastEnd past P); loads issued first.
__device__ __forceinline__ void stage_ids(const int32_t* __restrict__ ids, int32_t P, int64_t c0,
                                          int* s_ids) {
  int v[kPerLane];
#pragma unroll
  for (int j = 0; j < kPerLane; ++j) {
    const int64_t idx = c0 + (int64_t)j * kSortThreads + threadIdx.x;
    v[j] = idx < P ? ids[idx] : kPastEnd;
  }
#pragma unroll
  for (int j = 0; j < kPerLane; ++j) s_ids[j * kSortThreads + threadIdx.x] = v[j];
}

__global__ __launch_bounds__(kSortThreads) void route_sort_kernel(
    const int32_t* __restrict__ ids, int32_t P, int32_t E, int32_t tile_m,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pairs,
    int32_t* __restrict__ tiles, int32_t max_tiles, int32_t* __restrict__ num_tiles) {
  __shared__ int s_ids[kChunkIds];                        // 128 KB
  __shared__ int hist[1024];
  __shared__ int red[kSortWaves];
  __shared__ int wcount[kSortWaves];
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const unsigned uE = (unsigned)E;
  const int n_chunks = (P + kChunkIds - 1) / kChunkIds;

  for (int e = tid; e < E; e += kSortThreads) hist[e] = 0;
  for (int ch = 0; ch < n_chunks; ++ch) {
    __syncthreads();                                       // s_ids free, hist zeroed
    stage_ids(ids, P, (int64_t)ch * kChunkIds, s_ids);
    __syncthreads();
#pragma unroll 8
    for (int j = 0; j < kPerLane; ++j) {
      const int v = s_ids[j * kSortThreads + tid];
      if ((unsigned)v < uE) atomicAdd(&hist[v], 1);
    }
  }
  __syncthreads();

  // Segment start / tile base of expert b, and the grand totals.
  const int c = (tid < E) ? hist[tid] : 0;
  const int t = (c + tile_m - 1) / tile_m;
  const int seg_start = block_sum(tid < b ? c : 0, red);
  const int tile_base = block_sum(tid < b ? t : 0, red);
  const int valid_total = block_sum(c, red);
  const int tile_total = block_sum(t, red);

  // Stable compaction of this workgroup's pairs (see the file comment).
  int cursor = (b < E) ? seg_start : valid_total;
  for (int ch = 0; ch < n_chunks; ++ch) {
    if (n_chunks > 1) {                                    // one chunk: still staged
      __syncthreads();
      stage_ids(ids, P, (int64_t)ch * kChunkIds, s_ids);
      __syncthreads();
    }
    const int wbase = wave * (kChunkIds / kSortWaves);     // the wave's 2048 ids
    uint64_t bal[kPerLane];                                // the wave's matches, kept for pass 2
    int mine = 0;
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
      const int v = s_ids[wbase + j * kWave + lane];
      const bool hit = (b < E) ? (v == b) : (v != kPastEnd && (unsigned)v >= uE);
      bal[j] = __ballot(hit);
      mine += __popcll(bal[j]);
    }
    if (lane == 0) wcount[wave] = mine;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int i = 0; i < kSortWaves; ++i) {
      const int n = wcount[i];
      before += i < wave ? n : 0;
      total += n;
    }
    int pos = cursor + before;
    const int64_t pbase = (int64_t)ch * kChunkIds + wbase;
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
      const uint64_t m = bal[j];
      if ((m >> lane) & 1ull)
        sorted_pairs[pos + __popcll(m & ((1ull << lane) - 1ull))] = (int)(pbase + j * kWave + lane);
      pos += __popcll(m);
    }
    cursor += total;
    __syncthreads();                                       // wcount reused
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
