// Token-to-expert grouping on the device: a deterministic stable counting
// sort, one launch.  The pages require every active expert to run in one
// launch without a host round trip ("grouped-nf4-gemm 0.43.0", page
// header; "flashrt/grouped-moe-gemv", "Functions": no host
// synchronisation); the grouping itself is this library's design.
//
// Launch: E + 1 workgroups of 1024 threads.  Workgroup b < E owns expert b,
// workgroup E owns the dropped pairs.  The ids are taken in chunks of 32768;
// wave w of a workgroup owns ids [chunk + 2048 w, chunk + 2048 (w + 1)) and
// lane l holds ids chunk + 2048 w + 64 j + l, j < 32, in registers (each
// load instruction reads 256 contiguous bytes).  Each workgroup
//   1. builds the full expert histogram with integer LDS atomics into
//      several copies of the histogram, lane l adding to copy l mod C (C = 64
//      for E <= 128, fewer for larger E; at most 8192 counters): a skewed
//      routing makes many lanes of one instruction hit the same expert, and
//      same-address lanes of an LDS atomic serialise; the copies are summed
//      by groups of lanes (integer counts: the order does not matter),
//   2. lets every wave read the histogram and form its segment start, tile
//      base and the totals itself (lane partial sums and a butterfly sum, no
//      barrier),
//   3. compacts its pairs in ascending pair order from the same registers:
//      the wave's 32 match ballots are taken once to count (for the first
//      chunk during the histogram pass, so the two share a barrier) and once
//      to place, rows without a match skipped; a pair's place is the
//      workgroup's cursor + the earlier waves' counts + the wave's running
//      count + its rank among the matching lanes (ballot bit count), and
//   4. writes its offsets entry and its tiles.
// No global atomics, no workspace; the result is the unique stable order.
#include "gq_device.hpp"
#include "gq_host.hpp"
#include "../../include/gq.h"

namespace gq {

constexpr int kSortThreads = 1024;
constexpr int kSortWaves = kSortThreads / kWave;
constexpr int kChunkIds = 32768;                          // ids per pass
constexpr int kPerLane = kChunkIds / kSortThreads;        // 32
constexpr int kWaveIds = kChunkIds / kSortWaves;          // 2048 contiguous ids per wave
constexpr int kHistCounters = 8192;                       // LDS counters over all copies
constexpr int kPastEnd = INT32_MIN;                       // slots beyond the last pair

// The lane's 32 ids of chunk c0 (kPastEnd past P), all loads issued first:
// unconditional where the wave's 2048 ids are all in range, clamped
// addresses then a select on the last partial range, none past P.
__device__ __forceinline__ void load_ids(const int32_t* __restrict__ ids, int32_t P, int64_t c0,
                                         int (&v)[kPerLane]) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int64_t wbase = c0 + (int64_t)wave * kWaveIds;
  if (wbase + kWaveIds <= P) {
    const int32_t* p = ids + wbase + lane;
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) v[j] = p[j * kWave];
  } else if (wbase < P) {
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
      const int64_t idx = wbase + (int64_t)j * kWave + lane;
      const int x = ids[idx < P ? idx : P - 1];
      v[j] = idx < P ? x : kPastEnd;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) v[j] = kPastEnd;
  }
}

// Sum over the wave with DPP lane moves (total on lane 63), read back into a
// scalar register: a fixed order, no LDS traffic.
__device__ __forceinline__ int wave_total(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
  v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);  // row_mirror
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0x8, 0xF, false);  // row_bcast:31
  return __builtin_amdgcn_readlane(v, kWave - 1);
}

// One workgroup's whole share of the sort.  kDropped selects the pairs it
// compacts at compile time (expert b's, or the dropped ones for b = E), so
// the match test in the loops is one compare with no branch.
template <bool kDropped>
__device__ __forceinline__ void sort_workgroup(
    const int32_t* __restrict__ ids, int32_t P, int32_t E, int32_t tile_m,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pairs,
    int32_t* __restrict__ tiles, int32_t max_tiles, int32_t* __restrict__ num_tiles,
    int* __restrict__ hist_c, int* __restrict__ hist, int* __restrict__ wcount) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const unsigned uE = (unsigned)E;
  const int n_chunks = (P + kChunkIds - 1) / kChunkIds;
  // copies: the largest power of two <= 64 with C * E <= kHistCounters
  int C = 64;
  while (C > 1 && C * E > kHistCounters) C >>= 1;
  const int cl = lane & (C - 1);

  auto hit = [&](int x) { return kDropped ? (x != kPastEnd && (unsigned)x >= uE) : (x == b); };
  for (int i = tid; i < C * (E + 1); i += kSortThreads) hist_c[i] = 0;
  int v[kPerLane];
  for (int ch = 0; ch < n_chunks; ++ch) {
    load_ids(ids, P, (int64_t)ch * kChunkIds, v);
    if (ch == 0) __syncthreads();                          // copies zeroed
#pragma unroll
    for (int j = 0; j < kPerLane; ++j)
      atomicAdd(&hist_c[((unsigned)v[j] < uE ? v[j] : E) * C + cl], 1);
    if (ch == 0) {                     // the wave's matches in chunk 0, for the compaction
      int mine = 0;
#pragma unroll
      for (int j = 0; j < kPerLane; ++j) mine += __popcll(__ballot(hit(v[j])));
      if (lane == 0) wcount[wave] = mine;
    }
  }
  __syncthreads();
  // Sum the copies: G lanes per expert (G the largest power of two with
  // G * E <= 1024, so a group lies inside one wave), each over copies
  // part, part + G, ... (rotated by e so neighbouring experts start in
  // different banks), then a butterfly over the group.
  {
    int G = kWave;
    while (G > 1 && G * E > kSortThreads) G >>= 1;
    const int e = tid / G, part = tid & (G - 1);
    int s = 0;
    if (e < E)
      for (int k = part; k < C; k += G) s += hist_c[e * C + ((k + e) & (C - 1))];
    for (int off = G >> 1; off > 0; off >>= 1) s += __shfl_xor(s, off, kWave);
    if (e < E && part == 0) hist[e] = s;
  }
  __syncthreads();

  // Segment start / tile base of expert b, and the grand totals: every wave
  // forms them from the histogram on its own.
  int seg_start = 0, tile_base = 0, valid_total = 0, tile_total = 0;
  for (int e = lane; e < E; e += kWave) {
    const int c = hist[e], t = (c + tile_m - 1) / tile_m;
    seg_start += e < b ? c : 0;
    tile_base += e < b ? t : 0;
    valid_total += c;
    tile_total += t;
  }
  seg_start = wave_total(seg_start);
  tile_base = wave_total(tile_base);
  valid_total = wave_total(valid_total);
  tile_total = wave_total(tile_total);

  // Stable compaction of this workgroup's pairs (see the file comment).  One
  // chunk: the ids are still in registers.
  int cursor = kDropped ? valid_total : seg_start;
  for (int ch = 0; ch < n_chunks; ++ch) {
    if (n_chunks > 1) load_ids(ids, P, (int64_t)ch * kChunkIds, v);
    if (ch > 0) {                      // chunk 0's counts came with the histogram
      int mine = 0;
#pragma unroll
      for (int j = 0; j < kPerLane; ++j) mine += __popcll(__ballot(hit(v[j])));
      if (lane == 0) wcount[wave] = mine;
      __syncthreads();
    }
    int before = 0, total = 0;
#pragma unroll
    for (int i = 0; i < kSortWaves; ++i) {
      const int n = wcount[i];
      before += i < wave ? n : 0;
      total += n;
    }
    int pos = cursor + before;
    const int64_t pbase = (int64_t)ch * kChunkIds + (int64_t)wave * kWaveIds;
    // The ballots are taken again rather than kept (64 scalar registers);
    // the empty asm keeps the compiler from reusing the first ones.
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) asm volatile("" : "+v"(v[j]));
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
      const bool h = hit(v[j]);
      const uint64_t m = __ballot(h);
      if (m == 0ull) continue;                             // uniform: most rows match nothing
      if (h) {
        const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        sorted_pairs[pos + rank] = (int)(pbase + j * kWave + lane);
      }
      pos += __popcll(m);
    }
    cursor += total;
    if (ch + 1 < n_chunks) __syncthreads();               // wcount reused
  }

  if (!kDropped) {
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

__global__ __launch_bounds__(kSortThreads) void route_sort_kernel(
    const int32_t* __restrict__ ids, int32_t P, int32_t E, int32_t tile_m,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pairs,
    int32_t* __restrict__ tiles, int32_t max_tiles, int32_t* __restrict__ num_tiles) {
  __shared__ int hist_c[kHistCounters + kWave];           // [E + 1][C] copies (row E: ids
                                                          // outside [0, E)), 32 KB
  __shared__ int hist[1024];
  __shared__ int wcount[kSortWaves];
  if ((int)blockIdx.x < E)
    sort_workgroup<false>(ids, P, E, tile_m, offsets, sorted_pairs, tiles, max_tiles, num_tiles,
                          hist_c, hist, wcount);
  else
    sort_workgroup<true>(ids, P, E, tile_m, offsets, sorted_pairs, tiles, max_tiles, num_tiles,
                         hist_c, hist, wcount);
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
