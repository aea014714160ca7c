// Decode-time grouped GEMV on 4-bit packed experts (a few token rows: 1..8
// tokens in gather mode, or their routed pairs in flatten mode; <= 256 pairs).
//
// Pages: "grouped-nf4-gemm 0.43.0" -- page header (one launch for the
// active experts, no full-size bf16 weight copies) and "Which entry
// point?" (the single-row decode bandwidth route); "flashrt/grouped-moe-gemv"
// -- "Functions" (one product per routed slot, [M, top_k] routing,
// [M, top_k, N] output).  The kernel design is this library's own.
//
// Design (HBM-bound: the weight bytes of the active experts are the cost):
//  * grid (ceil(N / R), P): workgroup (x, p) owns rows [x*R, x*R + R) of the
//    expert of pair p.  Only the FIRST pair routed to an expert does the
//    work and it serves every pair of that expert, so each active expert's
//    bytes cross HBM once.  No sort, no host sync: topk_ids is read here.
//  * a thread owns one 16-byte segment (32 weights) of the rows it handles,
//    at a fixed K offset, so the activation slice it needs sits in 32
//    float registers; several rows per thread, all loads issued up front.
//    Consecutive threads read consecutive 16-byte pieces of contiguous rows
//    (fully coalesced).
//  * NF4: codebook value pairs from a 256-entry LDS table indexed by the
//    code byte, the 64-block absmax factored out of each 32-weight partial
//    sum; MXFP4: the
//    gfx950 e2m1 converter to bf16 pairs and bf16-pair dot products, the
//    e8m0 factor applied to the partial sum with ldexp.  Both keep the
//    decoded weight and its products exact (float32 sums).
//  * partial sums are reduced in a fixed order (DPP lane moves inside a wave,
//    LDS across waves): no atomics, bitwise reproducible.
#include <algorithm>

#include "gq_device.hpp"
#include "gq_host.hpp"
#include "../../include/gq.h"

namespace gq {

constexpr int kGemvMaxThreads = 256;
constexpr int kGemvMaxPairs = 256;
constexpr int kGemvMaxK = 8192;     // 256 segments of 32 weights

// Partial dot product of one 32-weight segment with the activation slice
// (xf: as float32; xr: the raw bf16 pairs).  NF4: codebook values (float32)
// against xf.  MXFP4: the converter turns each code byte into its two
// weights as a bf16 pair (exact: every e2m1 value is a bf16 value) and
// v_dot2_f32_bf16 multiplies it with the matching activation pair (the
// products are exact in float32; two per instruction, float32 sums): 25%
// fewer VALU instructions than float32 FMAs on converted weights, and no
// activation conversion; one-token gpt-oss gate_up 9.99 -> 9.70 us, down
// 7.34 -> 7.01 us (graph-replayed, same-box A/B).
//
// NF4 values come from a 256-entry table of codebook value pairs indexed by
// the code byte (one 8-byte LDS read per two weights, the table at LDS
// address 0 so its byte offset is one shift).  Against the 16-entry table
// (one 4-byte read per weight) this halves the LDS reads at the end of each
// workgroup, where the decode follows the last weight bytes; same-box A/B
// over three alternations, graph-replayed: one-token gate_up 6.05-6.08 ->
// 5.92-5.97 us, down 4.97-5.05 -> 4.78-4.81 us, decode step 11.1 -> 10.7-10.8
// us, M = 4 down 10.8 -> 10.4 us.
using LutT = f32x2;
constexpr int kLutN = 256;
__device__ __forceinline__ void lut_init(LutT* lut, int tid, int nt) {
  for (int t = tid; t < kLutN; t += nt) nf4_pairs_init(lut, t);
}
template <bool kMx>
__device__ __forceinline__ float segment_dot(const LutT* lut, u32x4 c, float am, uint32_t sb,
                                             const float (&xf)[32], const u32x4 (&xr)[4]) {
  float acc = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t d = c[w];
    // The decode does not depend on the pair: without this the compiler
    // hoists every row's decoded weights out of the pair loop and needs one
    // register per weight.  (No instruction is emitted.)
    asm volatile("" : "+v"(d));
    if constexpr (kMx) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint32_t wv = e2m1_pair_bf16_scaled(d, b, 1.0f);   // element 2j: low half
        // a scalar copy first: a bit_cast of a vector element reads element 0
        const uint32_t xv = xr[w][b];
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wv),
                                              __builtin_bit_cast(bf16x2, xv), acc, false);
      }
    } else {
      float q[8];
      nf4_pairs8(lut, d, q);                        // element 2j: high nibble
#pragma unroll
      for (int j = 0; j < 8; ++j) acc = __builtin_fmaf(q[j], xf[8 * w + j], acc);
    }
  }
  if constexpr (kMx) return e8m0_apply(acc, sb);
  else return acc * am;
}

// kIter rows per thread.  Memory round trips on the critical path: (1) the
// expert id of pair p0 (a scalar load), issued together with the routing
// table and p0's activation slice; (2) the weight bytes.  Routing decisions
// are taken per wave from ballots (no barrier), after p0's rows are
// computed.  Pairs that share p0's expert (rare at decode) cost one more
// activation load each.
//
// kWaveRows: a row's S segments lie inside one wave (64 % S == 0) and are
// summed with DPP lane moves; otherwise partial sums meet in LDS.  Both
// orders are fixed, so results are reproducible.
// Argument order: what the first loads need (routing ids, activations,
// weights, sizes) comes first, in the first 14 dwords, which are preloaded
// into SGPRs (every kernel here is compiled with kernel-argument preload),
// so the expert-id load issues without waiting for a kernel-argument load;
// the segment layout is derived from K rather than passed.
// kAct: 0 plain product; 1 SwiGLU with gate rows [0, N/2) and up rows
// [N/2, N); 2 the gpt-oss gated unit with gate row 2j and up row 2j + 1
// (alpha, limit).  With an activation a workgroup takes output columns
// [n0, n0 + R/2) and the gate and up rows of each.  kHostBank: the same code
// for a bank in pinned host memory (a separate instance, so that profiles
// keep the host-link launches apart from the HBM ones).
template <bool kMx, int kIter, bool kWaveRows, int kAct, bool kHostBank = false>
__global__ __launch_bounds__(kGemvMaxThreads) void grouped_gemv_kernel(
    const int32_t* __restrict__ ids, const uint16_t* __restrict__ x,
    const uint8_t* __restrict__ codes, const void* __restrict__ scl, int K, int N, int E,
    int x_stride, int topk, int P, const float* __restrict__ pair_scale,
    uint16_t* __restrict__ out, float alpha, float limit) {
  constexpr bool kGlu = kAct != 0;
  __shared__ __attribute__((aligned(4096))) LutT lut[kLutN];
  __shared__ float red[kWaveRows ? 1 : kIter * (kGemvMaxThreads + 32)];

  // segment layout (the host's segment_layout, derived from K)
  const int S = K >> 5;
  int W, G, NT;
  if constexpr (kWaveRows) {
    const int lgW = S > 1 ? 32 - __builtin_clz(S - 1) : 0;
    W = 1 << lgW;
    G = kGemvMaxThreads >> lgW;
    NT = kGemvMaxThreads;
  } else {
    W = S;
    G = S >= kGemvMaxThreads ? 1 : kGemvMaxThreads / S;
    NT = ((S * G + kWave - 1) / kWave) * kWave;
  }
  const int tid = threadIdx.x;                      // NT == blockDim.x
  const int lane = tid & (kWave - 1);
  const int p0 = blockIdx.y;
  const int R = G * kIter;                          // weight rows per workgroup
  constexpr int kHalf = kIter / 2;
  const int Nout = kGlu ? N / 2 : N;                // output columns per pair
  const int Rout = kGlu ? R / 2 : R;
  const int n0 = blockIdx.x * Rout;
  const int g = tid / W;                            // row slot
  const int s = tid - g * W;                        // segment
  const bool active = kWaveRows ? s < S : tid < S * G;
  // weight row of row slot gg, iteration i (clamped into the matrix)
  auto wrow = [&](int gg, int i) -> int {
    if constexpr (kAct == 1) {
      const int j = min(n0 + gg + G * (i % kHalf), Nout - 1);
      return i < kHalf ? j : Nout + j;
    } else if constexpr (kAct == 2) {
      if constexpr (!kWaveRows) {
        // rows reduced through LDS: the workgroup's 2 Rout weight rows in
        // order, so that each load instruction reads neighbouring rows (row
        // slot r = gg + G i takes row 2 n0 + r: the gate of output n0 + r/2
        // for even r, its up row for odd r; ~0.3 us faster on the one-token
        // gpt-oss gate_up than gate and up rows in separate halves)
        return min(2 * n0 + gg + G * i, N - 1);
      }
      const int j = min(n0 + gg + G * (i % kHalf), Nout - 1);
      return 2 * j + (i < kHalf ? 0 : 1);
    } else {
      return min(n0 + gg + G * i, N - 1);
    }
  };

  // ---- round trip 1: expert of p0, routing table (per wave), p0's activations ----
  const int e = ids[p0];
  int idl[kGemvMaxPairs / kWave];
#pragma unroll
  for (int c = 0; c < kGemvMaxPairs / kWave; ++c) {
    const int q = lane + kWave * c;
    idl[c] = (kWave * c < P && q < P) ? ids[q] : -1;
  }
  u32x4 xr[4];
  {
    const u32x4* xp =
        reinterpret_cast<const u32x4*>(x + (int64_t)(p0 / topk) * x_stride + (active ? s : 0) * 32);
#pragma unroll
    for (int v = 0; v < 4; ++v) xr[v] = xp[v];
  }

  // ---- round trip 2: the weight bytes of expert e ----
  // Everything but the expert's base address is formed while the id is in
  // flight, so that once it arrives only the scalar base remains before the
  // loads issue (offsets from a scalar base: the loads take the base in
  // SGPRs).  Offsets inside one expert fit 32 bits (host check: an expert's
  // codes are < 2^31 bytes); rows < 2^24 and row bytes <= 4096 allow 24-bit
  // multiplies.  No branch on the id before the loads: with one, the
  // compiler sinks every address computation and the activation loads below
  // the id wait.  A dropped pair reads expert 0 and stores zeros.  Measured
  // under graph replay against the form with a dropped-pair return and the
  // addresses formed after the id: one-token gate_up 6.37-6.40 -> 6.09-6.13
  // us, down 5.20-5.24 -> 4.99 us, M=4 gate_up 15.2-15.4 -> 14.9-15.0 us.
  //
  // Unconditional loads from clamped addresses (rows past N and idle lanes
  // re-read valid bytes whose results are never stored): a conditional load
  // would zero its registers first and stall on every older load in flight.
  // The weight bytes are read once per launch: non-temporal loads (measured
  // ~2% faster on the one-token gate_up launch than default-policy loads).
  const uint32_t row_bytes = (uint32_t)K / 2;
  const uint32_t s_cl = active ? s : 0;
  constexpr uint32_t kScaleBytes = kMx ? 1u : 4u;             // e8m0 byte / fp32 absmax
  const uint32_t spr = kMx ? (uint32_t)(K / 32) : (uint32_t)(K / 64);   // scales per row
  uint32_t woff[kIter], soff[kIter];
#pragma unroll
  for (int i = 0; i < kIter; ++i) {
    const uint32_t r = (uint32_t)wrow(g, i);
    woff[i] = __umul24(r, row_bytes) + s_cl * 16u;
    soff[i] = (__umul24(r, spr) + (kMx ? s_cl : s_cl / 2)) * kScaleBytes;
    // opaque: otherwise refolded into multiply-adds with the base after the
    // id has arrived
    asm volatile("" : "+v"(woff[i]), "+v"(soff[i]));
  }
  size_t ebytes = (size_t)N * row_bytes, escl = (size_t)N * spr * kScaleBytes;
  asm volatile("" : "+s"(ebytes), "+s"(escl));
  const bool dropped = (unsigned)e >= (unsigned)E;             // uniform
  const size_t ec = dropped ? 0 : (size_t)(uint32_t)e;
  const uint8_t* cbase = codes + ec * ebytes;
  const uint8_t* sbase = static_cast<const uint8_t*>(scl) + ec * escl;
  u32x4 cw[kIter];
  float am[kIter];
  uint32_t sb[kIter];
#pragma unroll
  for (int i = 0; i < kIter; ++i) {
    cw[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(cbase + woff[i]));
    if constexpr (kMx) {
      sb[i] = (uint32_t)sbase[soff[i]];
      am[i] = 0.f;
    } else {
      am[i] = *reinterpret_cast<const float*>(sbase + soff[i]);
      sb[i] = 0u;
    }
  }

  if constexpr (!kMx) {
    lut_init(lut, tid, blockDim.x);
    lds_barrier();
  }

  // ---- the rows of one pair: kWaveRows -> row i's total on the last lane of
  // its segment group; otherwise thread r < R holds row r's total ----
  float vals[kWaveRows ? kIter : 1];
  auto act_pair = [&](float gate, float up) {
    if constexpr (kAct == 2) {
      const float gc = fminf(gate, limit);
      const float uc = fminf(fmaxf(up, -limit), limit);
      return gc * sigmoid_f32(alpha * gc) * (uc + 1.0f);
    } else {
      return silu_f32(gate) * up;
    }
  };
  auto compute_pair = [&]() {
    float xf[32];
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        xf[8 * v + 2 * cc] = bf16lo_to_f32(xr[v][cc]);
        xf[8 * v + 2 * cc + 1] = bf16hi_to_f32(xr[v][cc]);
      }
    if constexpr (kWaveRows) {
#pragma unroll
      for (int i = 0; i < kIter; ++i) {
        const float part = active ? segment_dot<kMx>(lut, cw[i], am[i], sb[i], xf, xr) : 0.f;
        vals[i] = group_sum_last(part, W);                     // total on lane s == W-1
      }
      if constexpr (kGlu) {
#pragma unroll
        for (int i = 0; i < kHalf; ++i) vals[i] = act_pair(vals[i], vals[i + kHalf]);
      }
    } else {
      constexpr int kStride = kGemvMaxThreads + 32;            // pad: spreads banks
#pragma unroll
      for (int i = 0; i < kIter; ++i)
        red[i * kStride + tid] = active ? segment_dot<kMx>(lut, cw[i], am[i], sb[i], xf, xr) : 0.f;
      lds_barrier();
      vals[0] = 0.f;
      bool unit_done = false;                // the gated unit already applied (uniform)
      if (8 * R <= NT) {
        // eight threads per row (segments part, part + 8, ...), then an
        // 8-lane DPP sum; the total goes through LDS to thread r
        const int rr = tid >> 3, part = tid & 7;
        float v = 0.f;
        if (rr < R) {
          const int gg = rr % G, ii = rr / G;                  // weight row wrow(gg, ii)
          const float* src = red + ii * kStride + gg * S;
          float s0 = 0.f, s1 = 0.f;
          int j = part;
          for (; j + 8 < S; j += 16) {
            s0 += src[j];
            s1 += src[j + 8];
          }
          if (j < S) s0 += src[j];
          v = s0 + s1;
        }
        v = group_sum_last(v, 8);                              // on the lane with part == 7
        lds_barrier();                                         // every partial read
        if (rr < R && part == 7) red[rr] = v;
        lds_barrier();
        if constexpr (kGlu) {                // the row totals are in LDS already
          vals[0] = tid >= Rout ? 0.f
                    : kAct == 2 ? act_pair(red[2 * tid], red[2 * tid + 1])
                                : act_pair(red[tid], red[tid + Rout]);
          unit_done = true;
        } else {
          if (tid < R) vals[0] = red[tid];
        }
      } else if (tid < R) {                                    // R <= NT (host check)
        const int gg = tid % G, ii = tid / G;                  // weight row wrow(gg, ii)
        const float* src = red + ii * kStride + gg * S;
        float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;          // fixed order, 4 chains
        int j = 0;
        for (; j + 4 <= S; j += 4) {
          s0 += src[j];
          s1 += src[j + 1];
          s2 += src[j + 2];
          s3 += src[j + 3];
        }
        for (; j < S; ++j) s0 += src[j];
        vals[0] = (s0 + s1) + (s2 + s3);
      }
      lds_barrier();
      if constexpr (kGlu) {                  // gate row r with up row r + R/2 (kAct 2: 2r, 2r + 1)
        if (!unit_done) {
          if (tid < R) red[tid] = vals[0];
          lds_barrier();
          vals[0] = tid >= Rout ? 0.f
                    : kAct == 2 ? act_pair(red[2 * tid], red[2 * tid + 1])
                                : act_pair(red[tid], red[tid + Rout]);
          lds_barrier();
        }
      }
    }
  };
  auto store_pair = [&](int p) {
    const float sc = pair_scale ? pair_scale[p] : 1.f;
    if constexpr (kWaveRows) {
#pragma unroll
      for (int i = 0; i < (kGlu ? kHalf : kIter); ++i) {
        const int n = n0 + g + G * i;
        if (s == W - 1 && n < Nout)
          out[(int64_t)p * Nout + n] = f32_to_bf16_bits(dropped ? 0.f : vals[i] * sc);
      }
    } else {
      const int n = n0 + tid;
      if (tid < Rout && n < Nout)
        out[(int64_t)p * Nout + n] = f32_to_bf16_bits(dropped ? 0.f : vals[0] * sc);
    }
  };

  // ---- p0's rows are computed before the routing table is inspected: with
  // the decision first, the compiler holds the weight loads back until the
  // table has arrived (a full extra memory round trip) ----
  compute_pair();

  // ---- is p0 the first pair of expert e?  (same answer in every wave) ----
  uint64_t match[kGemvMaxPairs / kWave];
  bool dup = false;
#pragma unroll
  for (int c = 0; c < kGemvMaxPairs / kWave; ++c) {
    const int q = lane + kWave * c;
    match[c] = __ballot(idl[c] == e && q < P);   // q < P: the padding (-1) may equal e
    dup |= __ballot(idl[c] == e && q < p0) != 0ull;
  }
  if (dup) return;                           // an earlier pair's workgroup serves p0
  store_pair(p0);

  // ---- then every later pair routed to e, ascending ----
  for (int c = 0; c < kGemvMaxPairs / kWave; ++c) {
    uint64_t m = match[c];
    if (c == p0 / kWave) m &= ~(1ull << (p0 % kWave));
    while (m) {
      const int p = kWave * c + __builtin_ctzll(m);
      m &= m - 1ull;
      const u32x4* xp = reinterpret_cast<const u32x4*>(x + (int64_t)(p / topk) * x_stride +
                                                        (active ? s : 0) * 32);
#pragma unroll
      for (int v = 0; v < 4; ++v) xr[v] = xp[v];
      if (!dropped) compute_pair();          // a dropped pair stores zeros
      store_pair(p);
    }
  }
}

template <bool kMx, int kIter, int kAct, bool kHostBank>
static void launch_gemv_iter(dim3 grid, int NT, bool wave_rows, hipStream_t stream,
                             const uint16_t* x, int x_stride, int K, const uint8_t* codes,
                             const void* scl, int N, int E, const int32_t* ids, int topk, int P,
                             const float* pair_scale, uint16_t* out, float alpha, float limit) {
  if (wave_rows)
    hipLaunchKernelGGL((grouped_gemv_kernel<kMx, kIter, true, kAct, kHostBank>), grid, dim3(NT),
                       0, stream,
                       ids, x, codes, scl, K, N, E, x_stride, topk, P, pair_scale, out, alpha,
                       limit);
  else
    hipLaunchKernelGGL((grouped_gemv_kernel<kMx, kIter, false, kAct, kHostBank>), grid, dim3(NT),
                       0, stream,
                       ids, x, codes, scl, K, N, E, x_stride, topk, P, pair_scale, out, alpha,
                       limit);
}

// Segment lanes: S segments of 32 weights per row.  S <= 64: a row's
// segments go to a group of W = S rounded up to a power of two lanes inside
// one wave (lanes s >= S idle); longer rows: S consecutive threads, reduced
// through LDS.
static void segment_layout(int K, int& S, int& W, int& G, int& NT) {
  S = K / 32;
  W = S;
  if (S <= kWave)
    while (W & (W - 1)) W += W & -W;
  G = S > kWave ? (S >= kGemvMaxThreads ? 1 : kGemvMaxThreads / S) : kGemvMaxThreads / W;
  NT = S > kWave ? ((S * G + kWave - 1) / kWave) * kWave : kGemvMaxThreads;
}

template <bool kMx, int kAct, bool kHostBank = false>
static int launch_gemv(const uint16_t* x, int32_t rows, int32_t K, int64_t x_stride,
                       const uint8_t* codes, const void* scl, int32_t E, int32_t N,
                       const int32_t* ids, int32_t topk, const float* pair_scale, uint16_t* out,
                       hipStream_t stream, float alpha = 0.f, float limit = 0.f) {
  if (!x || !codes || !scl || !ids || !out) return kInvalid;
  if (rows < 1 || topk < 1 || E < 1 || N < 1 || K <= 0) return kInvalid;
  if (K % (kMx ? 32 : 64)) return kInvalid;
  if (kAct != 0 && N % 2) return kInvalid;
  if (kAct == 2 && !(limit >= 0.f && limit < 3.4e38f && alpha == alpha && alpha > -3.4e38f &&
                     alpha < 3.4e38f))
    return kInvalid;                                       // finite alpha, limit >= 0
  if (x_stride < K || x_stride % 8) return kInvalid;
  if (!aligned16(x) || !aligned16(codes) || !aligned4(ids) || !aligned4(out)) return kInvalid;
  if (!kMx && !aligned4(scl)) return kInvalid;
  if (pair_scale && !aligned4(pair_scale)) return kInvalid;
  const int64_t P = (int64_t)rows * topk;
  if (P > kGemvMaxPairs || K > kGemvMaxK || N >= (1 << 24)) return kNotSupported;
  if ((int64_t)N * (K / 2) >= ((int64_t)1 << 31)) return kNotSupported;   // 32-bit offsets
  if (x_stride > INT32_MAX) return kNotSupported;
  int S, W, G, NT;
  segment_layout(K, S, W, G, NT);
  // Rows per thread: the largest count (8, 4, 2) that still gives enough
  // workgroups.  With in-wave reductions many small workgroups stream better
  // (about eight per CU: on the one-token gate_up GEMV 1536 workgroups of 2
  // rows per thread beat 768 of 4 by 8%); the LDS-reduced long rows prefer
  // more rows per thread (two workgroups per CU).
  const int64_t want_blocks = S <= kWave ? 2048 : 512;
  int iter = 8;
  while (iter > 2 && (int64_t)((N + G * iter - 1) / (G * iter)) * P < want_blocks) iter >>= 1;
  const int R = G * iter;
  if (S > kWave && R > NT) return kNotSupported;     // one reduced row per thread
  const dim3 grid((N + R - 1) / R, (unsigned)P);
  switch (iter) {
    case 8:
      launch_gemv_iter<kMx, 8, kAct, kHostBank>(grid, NT, S <= kWave, stream, x, (int)x_stride, K, codes, scl,
                                     N, E, ids, topk, (int)P, pair_scale, out, alpha, limit);
      break;
    case 4:
      launch_gemv_iter<kMx, 4, kAct, kHostBank>(grid, NT, S <= kWave, stream, x, (int)x_stride, K, codes, scl,
                                     N, E, ids, topk, (int)P, pair_scale, out, alpha, limit);
      break;
    default:
      launch_gemv_iter<kMx, 2, kAct, kHostBank>(grid, NT, S <= kWave, stream, x, (int)x_stride, K, codes, scl,
                                     N, E, ids, topk, (int)P, pair_scale, out, alpha, limit);
      break;
  }
  return launch_status();
}

// ---------------------------------------------------------------------------
// Down projection of every routed pair with the router-weighted combine
// fused in (decode: a few tokens).  y[t, n] = sum_s w[t, s] * (act[t*k+s] .
// W_{ids[t, s]}[n, :]), slots in order, float32, one bf16 rounding.
//
// A workgroup owns output rows [n0, n0 + Rb) for EVERY pair, so a token's
// k products meet in its LDS and are reduced there: no atomics, no second
// launch.  Wave w takes pairs w, w + NWv, ... (kPPW of them; the expert id is
// one scalar load per pair, as in the GEMV); its lane groups (W lanes) take
// kR consecutive rows each, one 16-byte weight segment per lane and row, all
// against the pair's 64-byte activation slice.  A pair whose expert is
// outside [0, E) contributes 0.
constexpr int kCombineMaxPairs = 64;
constexpr int kCombineMaxWaves = 16;
constexpr int kCombineMaxYs = 1024;

// kSeg = 2 (rows of 65..128 segments, I <= 4096): a row takes the whole
// wave and lane s also takes segment s + 64.
template <bool kMx, int kR, int kPPW, int kSeg>
__global__ __launch_bounds__(kWave * kCombineMaxWaves) void gemv_down_combine_kernel(
    const int32_t* __restrict__ ids, const uint16_t* __restrict__ act,
    const uint8_t* __restrict__ codes, const void* __restrict__ scl, int I, int H, int E,
    int a_stride, int topk, int P, const float* __restrict__ tw, uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(4096))) LutT lut[kLutN];
  __shared__ float ys[kCombineMaxYs];                      // [P][Rb]
  __shared__ float tws[kCombineMaxPairs];                  // router weights

  // layout derived from I and P as on the host (arguments ordered as in
  // grouped_gemv_kernel)
  const int S = I >> 5;
  const int W = kSeg == 2 ? kWave : (S > 1 ? 1 << (32 - __builtin_clz(S - 1)) : 1);
  const int NWv = min(P, kCombineMaxWaves);
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  // uniform by construction; said so, the pair ids below become scalar loads
  // and their addresses scalar arithmetic (as a vector load, every lane
  // fetched the same id and the 64-bit address math ran on the VALU):
  // graph-replayed NF4 decode layer 11.5 -> 11.3 us
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int slots = kWave / W;                             // lane groups per wave
  const int Rb = slots * kR;                               // rows per workgroup
  const int n0 = blockIdx.x * Rb;
  const int g = lane / W, s = lane - g * W;
  bool active[kSeg];
  int s_cl[kSeg];
#pragma unroll
  for (int j = 0; j < kSeg; ++j) {
    active[j] = s + kWave * j < S;
    s_cl[j] = active[j] ? s + kWave * j : 0;
  }
  const size_t row_bytes = (size_t)I / 2;

  // ---- round trip 1: the wave's experts (scalar) and activation slices; the
  // router weight of pair tid too, kept in a register until the combine (a
  // load there, after the arithmetic, put a memory round trip at the end of
  // every workgroup; into LDS at once, its wait held the weight loads back)
  const float tw_own = (tw && tid < P) ? tw[tid] : 1.f;
  int pp[kPPW], ee[kPPW];
  u32x4 xr[kPPW][kSeg][4];
#pragma unroll
  for (int q = 0; q < kPPW; ++q) {
    pp[q] = min(wave + NWv * q, P - 1);                    // surplus pairs repeat the last
    ee[q] = ids[pp[q]];
#pragma unroll
    for (int j = 0; j < kSeg; ++j) {
      const u32x4* ap =
          reinterpret_cast<const u32x4*>(act + (int64_t)pp[q] * a_stride + s_cl[j] * 32);
#pragma unroll
      for (int v = 0; v < 4; ++v) xr[q][j][v] = ap[v];
    }
  }
  // ---- round trip 2: weight segments (dropped pairs read expert 0) ----
  u32x4 cw[kPPW][kR][kSeg];
  float am[kPPW][kR][kSeg];
  uint32_t sb[kPPW][kR][kSeg];
#pragma unroll
  for (int q = 0; q < kPPW; ++q) {
    const int e = (unsigned)ee[q] < (unsigned)E ? ee[q] : 0;
#pragma unroll
    for (int i = 0; i < kR; ++i) {
      const size_t row = (size_t)e * H + min(n0 + g * kR + i, H - 1);
#pragma unroll
      for (int j = 0; j < kSeg; ++j) {
        cw[q][i][j] =
            *reinterpret_cast<const u32x4*>(codes + row * row_bytes + (size_t)s_cl[j] * 16);
        if constexpr (kMx) {
          sb[q][i][j] =
              (uint32_t)static_cast<const uint8_t*>(scl)[row * (size_t)(I / 32) + s_cl[j]];
          am[q][i][j] = 0.f;
        } else {
          am[q][i][j] = static_cast<const float*>(scl)[row * (size_t)(I / 64) + s_cl[j] / 2];
          sb[q][i][j] = 0u;
        }
      }
    }
  }
  if constexpr (!kMx) {
    lut_init(lut, tid, blockDim.x);
    lds_barrier();
  }
#pragma unroll
  for (int q = 0; q < kPPW; ++q) {
    float part[kR];
#pragma unroll
    for (int i = 0; i < kR; ++i) part[i] = 0.f;
#pragma unroll
    for (int j = 0; j < kSeg; ++j) {
      float xf[32];
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          xf[8 * v + 2 * cc] = bf16lo_to_f32(xr[q][j][v][cc]);
          xf[8 * v + 2 * cc + 1] = bf16hi_to_f32(xr[q][j][v][cc]);
        }
#pragma unroll
      for (int i = 0; i < kR; ++i)
        if (active[j])
          part[i] += segment_dot<kMx>(lut, cw[q][i][j], am[q][i][j], sb[q][i][j], xf, xr[q][j]);
    }
    const int p = wave + NWv * q;
#pragma unroll
    for (int i = 0; i < kR; ++i) {
      const float tot = group_sum_last(part[i], W);
      if (s == W - 1 && p < P) ys[p * Rb + g * kR + i] = (unsigned)ee[q] < (unsigned)E ? tot : 0.f;
    }
  }
  if (tid < P) tws[tid] = tw_own;
  lds_barrier();
  // ---- combine: thread (t, r) sums its token's slots in order ----
  const int rows = P / topk;
  for (int idx = tid; idx < rows * Rb; idx += kWave * NWv) {
    const int t = idx / Rb, r = idx - t * Rb;
    const int n = n0 + r;
    if (n >= H) continue;
    float acc = 0.f;
    for (int sl = 0; sl < topk; ++sl) {
      const int p = t * topk + sl;
      acc = __builtin_fmaf(tws[p], ys[p * Rb + r], acc);
    }
    y[(int64_t)t * H + n] = f32_to_bf16_bits(acc);
  }
}

template <bool kMx, int kR, int kPPW, int kSeg>
static void launch_dc(dim3 grid, int NWv, hipStream_t stream, const uint16_t* act, int a_stride,
                      int I, const uint8_t* codes, const void* scl, int H, int E,
                      const int32_t* ids, int topk, int P, const float* tw, uint16_t* y) {
  hipLaunchKernelGGL((gemv_down_combine_kernel<kMx, kR, kPPW, kSeg>), grid, dim3(kWave * NWv), 0,
                     stream, ids, act, codes, scl, I, H, E, a_stride, topk, P, tw, y);
}

template <bool kMx>
static int launch_down_combine(const uint16_t* act, int32_t rows, int32_t I, int64_t a_stride,
                               const uint8_t* codes, const void* scl, int32_t E, int32_t H,
                               const int32_t* ids, int32_t topk, const float* tw, uint16_t* y,
                               hipStream_t stream) {
  if (!act || !codes || !scl || !ids || !y) return kInvalid;
  if (rows < 1 || topk < 1 || E < 1 || H < 1 || I <= 0 || I % (kMx ? 32 : 64)) return kInvalid;
  if (a_stride < I || a_stride % 8) return kInvalid;
  if (!aligned16(act) || !aligned16(codes) || !aligned4(ids) || !aligned4(y)) return kInvalid;
  if (!kMx && !aligned4(scl)) return kInvalid;
  if (tw && !aligned4(tw)) return kInvalid;
  const int64_t P = (int64_t)rows * topk;
  if (P > kCombineMaxPairs || I > 64 * kWave || H >= (1 << 24)) return kNotSupported;
  if (a_stride > INT32_MAX) return kNotSupported;
  const int NWv = (int)std::min<int64_t>(P, kCombineMaxWaves);
  const int ppw = (int)((P + NWv - 1) / NWv);               // 1..4
  const bool two_seg = I > 32 * kWave;                      // 65..128 segments per row
  if (two_seg && ppw > 2) return kNotSupported;              // registers: <= 32 pairs
  int S, W, G, NT;
  segment_layout(I, S, W, G, NT);
  if (two_seg) W = kWave;
  // rows per lane group: 2 for one pair per wave (as the GEMV; 4 when a row
  // takes the whole wave: half the workgroups, gpt-oss decode layer 18.6 ->
  // 17.7 us, while 8 rows ran at 31 us), 1 otherwise
  const int kr = ppw == 1 ? (two_seg ? 4 : 2) : 1;
  const int Rb = (kWave / W) * kr;
  if (P * Rb > kCombineMaxYs) return kNotSupported;
  const dim3 grid((H + Rb - 1) / Rb);
  if (two_seg) {
    if (ppw == 1)
      launch_dc<kMx, 4, 1, 2>(grid, NWv, stream, act, (int)a_stride, I, codes, scl, H, E, ids,
                              topk, (int)P, tw, y);
    else
      launch_dc<kMx, 1, 2, 2>(grid, NWv, stream, act, (int)a_stride, I, codes, scl, H, E, ids,
                              topk, (int)P, tw, y);
  } else if (ppw == 1) {
    launch_dc<kMx, 2, 1, 1>(grid, NWv, stream, act, (int)a_stride, I, codes, scl, H, E, ids,
                            topk, (int)P, tw, y);
  } else if (ppw == 2) {
    launch_dc<kMx, 1, 2, 1>(grid, NWv, stream, act, (int)a_stride, I, codes, scl, H, E, ids,
                            topk, (int)P, tw, y);
  } else {
    launch_dc<kMx, 1, 4, 1>(grid, NWv, stream, act, (int)a_stride, I, codes, scl, H, E, ids,
                            topk, (int)P, tw, y);
  }
  return launch_status();
}

// ---------------------------------------------------------------------------
// Combine of per-pair outputs (prefill): y[t, :] = sum_s w[t, s] * yp[t*k+s, :]
// in slot order, float32, one bf16 rounding.  Thread = 8 columns of a token.
__global__ __launch_bounds__(256) void moe_combine_kernel(const uint16_t* __restrict__ yp,
                                                          int64_t stride, int rows, int topk,
                                                          int H, const float* __restrict__ tw,
                                                          uint16_t* __restrict__ y) {
  const int chunks = H / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)rows * chunks) return;
  const int t = (int)(idx / chunks), c = (int)(idx - (int64_t)t * chunks);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int sl = 0; sl < topk; ++sl) {
    const int64_t p = (int64_t)t * topk + sl;
    const float w = tw ? tw[p] : 1.f;
    const u32x4 v = *reinterpret_cast<const u32x4*>(yp + p * stride + c * 8);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] = __builtin_fmaf(w, bf16lo_to_f32(v[q]), acc[2 * q]);
      acc[2 * q + 1] = __builtin_fmaf(w, bf16hi_to_f32(v[q]), acc[2 * q + 1]);
    }
  }
  const u32x4 o{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
  *reinterpret_cast<u32x4*>(y + (int64_t)t * H + c * 8) = o;
}

// Expert banks resident in pinned host memory: the device address of each
// bank, from the runtime's mapping of the pinned allocation.  Memory the
// runtime has not pinned and mapped is rejected here, before any launch
// (a device read of an unmapped host address would fault).
static int host_bank_ptrs(const void* a, const void* b, const void*& da, const void*& db) {
  if (!a || !b) return kInvalid;
  void* pa = nullptr;
  void* pb = nullptr;
  if (hipHostGetDevicePointer(&pa, const_cast<void*>(a), 0) != hipSuccess || !pa ||
      hipHostGetDevicePointer(&pb, const_cast<void*>(b), 0) != hipSuccess || !pb) {
    (void)hipGetLastError();                               // do not leave it for the next call
    return kInvalid;
  }
  da = pa;
  db = pb;
  return kOk;
}

}  // namespace gq

extern "C" int gq_nf4_grouped_gemv_host(const uint16_t* x, int32_t rows, int32_t K,
                                        int64_t x_stride, const uint8_t* codes,
                                        const float* absmax, int32_t num_experts, int32_t N,
                                        const int32_t* topk_ids, int32_t topk,
                                        const float* pair_scale, uint16_t* out,
                                        hipStream_t stream) {
  const void *dc = nullptr, *da = nullptr;
  const int st = gq::host_bank_ptrs(codes, absmax, dc, da);
  if (st != gq::kOk) return st;
  return gq::launch_gemv<false, 0, true>(x, rows, K, x_stride, static_cast<const uint8_t*>(dc), da,
                                   num_experts, N, topk_ids, topk, pair_scale, out, stream);
}

extern "C" int gq_mxfp4_grouped_gemv_host(const uint16_t* x, int32_t rows, int32_t K,
                                          int64_t x_stride, const uint8_t* blocks,
                                          const uint8_t* scales, int32_t num_experts, int32_t N,
                                          const int32_t* topk_ids, int32_t topk,
                                          const float* pair_scale, uint16_t* out,
                                          hipStream_t stream) {
  const void *db = nullptr, *ds = nullptr;
  const int st = gq::host_bank_ptrs(blocks, scales, db, ds);
  if (st != gq::kOk) return st;
  return gq::launch_gemv<true, 0, true>(x, rows, K, x_stride, static_cast<const uint8_t*>(db), ds,
                                  num_experts, N, topk_ids, topk, pair_scale, out, stream);
}

extern "C" int gq_nf4_grouped_gemv(const uint16_t* x, int32_t rows, int32_t K, int64_t x_stride,
                                   const uint8_t* codes, const float* absmax, int32_t num_experts,
                                   int32_t N, const int32_t* topk_ids, int32_t topk,
                                   const float* pair_scale, uint16_t* out, hipStream_t stream) {
  return gq::launch_gemv<false, 0>(x, rows, K, x_stride, codes, absmax, num_experts, N,
                                       topk_ids, topk, pair_scale, out, stream);
}

extern "C" int gq_nf4_grouped_gemv_swiglu(const uint16_t* x, int32_t rows, int32_t K,
                                          int64_t x_stride, const uint8_t* codes,
                                          const float* absmax, int32_t num_experts, int32_t N,
                                          const int32_t* topk_ids, int32_t topk, uint16_t* act,
                                          hipStream_t stream) {
  return gq::launch_gemv<false, 1>(x, rows, K, x_stride, codes, absmax, num_experts, N,
                                      topk_ids, topk, nullptr, act, stream);
}

extern "C" int gq_nf4_grouped_gemv_down_combine(const uint16_t* act, int32_t rows, int32_t I,
                                                int64_t act_stride, const uint8_t* codes,
                                                const float* absmax, int32_t num_experts,
                                                int32_t H, const int32_t* topk_ids, int32_t topk,
                                                const float* topk_weights, uint16_t* y,
                                                hipStream_t stream) {
  return gq::launch_down_combine<false>(act, rows, I, act_stride, codes, absmax, num_experts, H,
                                        topk_ids, topk, topk_weights, y, stream);
}

extern "C" int gq_mxfp4_grouped_gemv_down_combine(const uint16_t* act, int32_t rows, int32_t I,
                                                  int64_t act_stride, const uint8_t* blocks,
                                                  const uint8_t* scales, int32_t num_experts,
                                                  int32_t H, const int32_t* topk_ids,
                                                  int32_t topk, const float* topk_weights,
                                                  uint16_t* y, hipStream_t stream) {
  return gq::launch_down_combine<true>(act, rows, I, act_stride, blocks, scales, num_experts, H,
                                       topk_ids, topk, topk_weights, y, stream);
}

extern "C" int gq_moe_combine(const uint16_t* y_pairs, int32_t rows, int32_t topk, int32_t H,
                              int64_t stride, const float* topk_weights, uint16_t* y,
                              hipStream_t stream) {
  using namespace gq;
  if (rows < 0 || topk < 1 || H < 1 || H % 8 || stride < H || stride % 8) return kInvalid;
  if (rows == 0) return kOk;
  if (!y_pairs || !y || !aligned16(y_pairs) || !aligned16(y)) return kInvalid;
  if (topk_weights && !aligned4(topk_weights)) return kInvalid;
  const int64_t threads = (int64_t)rows * (H / 8);
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > INT32_MAX || (int64_t)rows * topk >= INT32_MAX) return kNotSupported;
  hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, y_pairs,
                     stride, rows, topk, H, topk_weights, y);
  return launch_status();
}

extern "C" int gq_mxfp4_grouped_gemv(const uint16_t* x, int32_t rows, int32_t K, int64_t x_stride,
                                     const uint8_t* blocks, const uint8_t* scales,
                                     int32_t num_experts, int32_t N, const int32_t* topk_ids,
                                     int32_t topk, const float* pair_scale, uint16_t* out,
                                     hipStream_t stream) {
  return gq::launch_gemv<true, 0>(x, rows, K, x_stride, blocks, scales, num_experts, N,
                                  topk_ids, topk, pair_scale, out, stream);
}

extern "C" int gq_mxfp4_grouped_gemv_swiglu(const uint16_t* x, int32_t rows, int32_t K,
                                            int64_t x_stride, const uint8_t* blocks,
                                            const uint8_t* scales, int32_t num_experts, int32_t N,
                                            const int32_t* topk_ids, int32_t topk, float alpha,
                                            float limit, uint16_t* act, hipStream_t stream) {
  return gq::launch_gemv<true, 2>(x, rows, K, x_stride, blocks, scales, num_experts, N,
                                  topk_ids, topk, nullptr, act, stream, alpha, limit);
}
