// Pieces shared by the prefill grouped GEMM kernels (gemm.hip: bf16 matrix
// cores on exactly decoded weights; gemm_mx8.hip: the block-scaled fp4
// matrix instruction on raw MXFP4 bytes): the argument block, the tile-list
// head (block -> tile mapping, rows of dropped pairs), the per-column code
// loads of the 256-column kernels and the row-store epilogue.
#pragma once

#include "gq_device.hpp"
#include "gq_host.hpp"

namespace gq {

constexpr int kTM = 256;          // tile rows (routed pairs)
constexpr int kTK = 64;           // contraction per step
constexpr int kGemmThreads = 256;
constexpr int kXN = 256;          // B columns per tile of the one-wave-per-SIMD kernels
constexpr int kNarrowRows = 128;  // tiles up to here: 4 sub-tiles per wave

// kFwdNF4Glu: NF4 forward on a fused gate_up weight (gate rows [0, I), up
// rows [I, 2I)) whose epilogue writes SwiGLU(gate, up) = silu(gate) * up.
// kFwdMX8: MXFP4 forward on the block-scaled matrix instruction, activations
// given as their two-term e4m3 split.
enum BMode { kFwdNF4 = 0, kFwdMX = 1, kDgradNF4 = 2, kDgradMX = 3, kFwdNF4Glu = 4, kFwdMX8 = 5 };

struct GemmArgs {
  const uint16_t* x;           // activations (forward) or output gradient (dgrad); kFwdMX8:
                               // the split codes (bytes)
  int64_t x_stride;            // elements of x per row (kFwdMX8: bytes / 2)
  const uint8_t* xs;           // kFwdMX8: split scales [rows, Kp/16] bytes
  int64_t xs_stride;           // bytes per row of xs
  const uint8_t* codes;        // [E, Nw, Kw/2]
  const void* scl;             // NF4 absmax float [E, Nw, Kw/64] / MXFP4 e8m0 [E, Nw, Kw/32]
  int Nw, Kw;                  // expert weight shape [Nw, Kw]
  int Kc;                      // contraction length (Kw forward, Nw dgrad)
  int Nout;                    // output columns (Nw forward, Kw dgrad)
  int E, topk, P;
  const float* pair_scale;
  const int32_t* offsets;
  const int32_t* sorted_pairs;
  const int32_t* tiles;
  const int32_t* num_tiles;
  int n_col_tiles;             // ceil(Nout / output columns per tile)
  int n_logical;               // max_tiles * n_col_tiles
  uint16_t* out;               // [P, Nout]
  float act_alpha, act_limit;  // gpt-oss gated unit (kernels with the activation epilogue)
  uint8_t* out_q;              // gated unit written as its two-term e4m3 split instead of
  uint8_t* out_s;              // bf16: codes [P, 2 Nout], scales [P, Nout / 16] (Nout % 64 == 0)
};

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void glb_void_t;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// The tile a workgroup owns.  Block index -> logical tile is XCD-aware: the
// hardware deals blocks round-robin to the 8 XCDs, and consecutive blocks of
// one XCD get all column tiles of a row tile, so the gathered activation
// rows are reused from that XCD's L2.  Tiles past the last expert tile
// zero the rows of dropped pairs (ids outside [0, E)) in their column range
// and report no work.  A tile entry that cannot come from gq_route_sort is
// rejected rather than read through.
struct TileInfo {
  int e, start, valid, n0;
};

// kSplitOut: the output is the e4m3 split (out_q, out_s); a dropped pair's
// row gets zero codes and zero scale bytes in the tile's column range, which
// is what the split of a zero row is.
template <int kTNo, bool kSplitOut = false>
__device__ __forceinline__ bool tile_head(const GemmArgs& g, int tid, TileInfo& t) {
  const int C = g.n_col_tiles;
  const int bid = blockIdx.x;
  const int q = bid >> 3, xcd = bid & 7;
  const int logical = (q / C) * (8 * C) + xcd * C + (q % C);
  if (logical >= g.n_logical) return false;
  const int tile = logical / C;
  t.n0 = (logical % C) * kTNo;
  const int T = *g.num_tiles;
  if (tile >= T) {
    const int dstart = g.offsets[g.E] + (tile - T) * kTM;
    if (dstart >= g.P || dstart < 0) return false;
    const int dvalid = min(kTM, g.P - dstart);
    if constexpr (kSplitOut) {
      // columns [n0, n0 + ncols): 2 ncols code bytes from byte 2 n0 of the
      // row, ncols / 16 scale bytes from byte n0 / 16 (multiples of 64)
      const int ncols = min(kTNo, g.Nout - t.n0);
      const int per = ncols / 8 + ncols / 64;              // 16-byte code pieces + scale dwords
      for (int idx = tid; idx < dvalid * per; idx += kGemmThreads) {
        const int r = idx / per, c = idx % per;
        const int p = g.sorted_pairs[dstart + r];
        if ((unsigned)p >= (unsigned)g.P) continue;
        if (c < ncols / 8)
          *reinterpret_cast<u32x4*>(g.out_q + (int64_t)p * (2 * g.Nout) + 2 * t.n0 + 16 * c) =
              u32x4{0u, 0u, 0u, 0u};
        else
          *reinterpret_cast<uint32_t*>(g.out_s + (int64_t)p * (g.Nout / 16) + t.n0 / 16 +
                                       4 * (c - ncols / 8)) = 0u;
      }
      return false;
    }
    for (int idx = tid; idx < dvalid * (kTNo / 8); idx += kGemmThreads) {
      const int r = idx / (kTNo / 8), c8 = idx % (kTNo / 8);
      const int col = t.n0 + c8 * 8;
      const int p = g.sorted_pairs[dstart + r];
      if (col < g.Nout && (unsigned)p < (unsigned)g.P)
        *reinterpret_cast<u32x4*>(g.out + (int64_t)p * g.Nout + col) = u32x4{0u, 0u, 0u, 0u};
    }
    return false;
  }
  t.e = g.tiles[2 * tile];
  t.start = g.tiles[2 * tile + 1];
  if ((unsigned)t.e >= (unsigned)g.E || (unsigned)t.start >= (unsigned)g.P) return false;
  t.valid = min(kTM, min(g.offsets[t.e + 1], g.P) - t.start);
  return t.valid > 0;
}

// Per-lane weight loads of the 256-column kernels: column jcol (column
// blocks 0 and 1 are jcol and jcol + 32; SwiGLU: gate row jcol and up row
// Nout + jcol), the 16 code bytes of K step ks at byte 16 * half of the
// step's 32-byte chunk, and their factor (NF4 absmax of the step; MXFP4 e8m0
// byte of scale block 2 ks + half).  Rows past the matrix re-read its last
// row (their results are never stored).
struct NLoad {
  u32x4 c[2];      // 32 codes of column blocks 0 and 1
  float a[2];      // NF4 absmax
  uint32_t s[2];   // MXFP4 scale bytes
};

template <int kMode>
__device__ __forceinline__ NLoad n_load(const GemmArgs& g, int e, int jcol, int ks, int half) {
  constexpr bool kMx = kMode == kFwdMX || kMode == kFwdMX8;
  NLoad L;
  const int k0 = ks * kTK;
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    int n;
    if constexpr (kMode == kFwdNF4Glu) n = min(jcol, g.Nout - 1) + (cb ? g.Nout : 0);
    else n = min(jcol + 32 * cb, g.Nw - 1);
    const size_t row = (size_t)e * g.Nw + n;
    L.c[cb] = *reinterpret_cast<const u32x4*>(g.codes + row * (size_t)(g.Kw / 2) + k0 / 2 +
                                              16 * half);
    if constexpr (kMx) {
      L.s[cb] = static_cast<const uint8_t*>(g.scl)[row * (size_t)(g.Kw / 32) + k0 / 32 + half];
      L.a[cb] = 0.f;
    } else {
      L.a[cb] = static_cast<const float*>(g.scl)[row * (size_t)(g.Kw / 64) + ks];
      L.s[cb] = 0u;
    }
  }
  return L;
}

// Epilogue shared by the forward and dgrad kernels.  A transposed
// accumulator block (32 columns x 32 rows, weights as the first MFMA
// operand) gives lane (lr, lh) the row lr of the sub-tile at columns
// 8q + 4 lh + [0, 4), q = r / 4.  The lane scales by its row's pair weight,
// rounds to bf16 and swaps half of its words with the partner lane 32 away
// (v_permlane32_swap), after which each lane holds 8 consecutive columns and
// writes them as one 16-byte piece of the output row.
__device__ __forceinline__ void store_block_t(const float (&v)[16], uint16_t* orow, int lh) {
  uint32_t w[4][2];                                        // columns 8q + 4 lh + [0, 4)
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    w[q][0] = pack_bf16x2(v[4 * q], v[4 * q + 1]);
    w[q][1] = pack_bf16x2(v[4 * q + 2], v[4 * q + 3]);
  }
#pragma unroll
  for (int jp = 0; jp < 2; ++jp) {
    // after the swap: lane half 0 holds columns 16 jp + [0, 8), half 1
    // columns 16 jp + [8, 16)
    const auto s0 = __builtin_amdgcn_permlane32_swap(w[2 * jp][0], w[2 * jp + 1][0], false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(w[2 * jp][1], w[2 * jp + 1][1], false, false);
    *reinterpret_cast<u32x4*>(orow + 16 * jp + 8 * lh) = u32x4{s0[0], s1[0], s0[1], s1[1]};
  }
}

// Epilogue of the 256-column kernels: wave w owns the columns
// n0 + 64 w + [0, 64) (column blocks cb = 0, 1) of every active 32-row
// sub-tile; each lane writes its row's 32 columns per block, scaled by the
// row's pair weight.
template <int kSub>
__device__ __forceinline__ void store_wide_rows(const f32x16 (&acc)[kSub][2], int nrows,
                                                int valid, const int* pair_s,
                                                const float* scale_s, const GemmArgs& g, int n0,
                                                int wave, int lr, int lh) {
#pragma unroll
  for (int i = 0; i < kSub; ++i) {
    if (i >= nrows) continue;
    const int m = 32 * i + lr;
    const int p = pair_s[m];
    const float sc = scale_s[m];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int col = n0 + 64 * wave + 32 * cb;
      if (m < valid && col < g.Nout) {
        float v[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] = acc[i][cb][r] * sc;
        store_block_t(v, g.out + (int64_t)p * g.Nout + col, lh);
      }
    }
  }
}

// gpt-oss gated unit of one (gate, up) pair: the gate clamped above at
// `limit`, the up value clipped to [-limit, limit],
//   act = gc * sigmoid(alpha * gc) * (uc + 1),  float32.
__device__ __forceinline__ float oss_act(float gate, float up, float alpha, float limit) {
  const float gc = fminf(gate, limit);
  const float uc = fminf(fmaxf(up, -limit), limit);
  return gc * sigmoid_f32(alpha * gc) * (uc + 1.0f);
}

// Activation epilogue of one transposed accumulator block whose 32 columns
// are 16 interleaved (gate, up) weight-row pairs: lane (lr, lh) holds its
// row at columns 8q + 4 lh + [0, 4), i.e. the pairs of output columns
// 4q + 2 lh and 4q + 2 lh + 1.  Two v_permlane32_swap exchanges give lane
// half h the output columns 8h + [0, 8), written as one 16-byte piece.
__device__ __forceinline__ void store_block_act(const float (&v)[16], uint16_t* orow, int lh,
                                                float alpha, float limit) {
  uint32_t o[4];                                           // output columns 4q + 2 lh + [0, 2)
#pragma unroll
  for (int q = 0; q < 4; ++q)
    o[q] = pack_bf16x2(oss_act(v[4 * q], v[4 * q + 1], alpha, limit),
                       oss_act(v[4 * q + 2], v[4 * q + 3], alpha, limit));
  // half 0: own o0 | partner o0 | own o1 | partner o1 = columns 0..7;
  // half 1: partner o2 | own o2 | partner o3 | own o3 = columns 8..15
  const auto a = __builtin_amdgcn_permlane32_swap(o[0], o[2], false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(o[1], o[3], false, false);
  *reinterpret_cast<u32x4*>(orow + 8 * lh) = u32x4{a[0], a[1], b[0], b[1]};
}

// Host: argument checks shared by the grouped GEMM entry points.
static inline int common_gemm_checks(const void* x, int64_t x_rows, int64_t x_stride, int32_t Kc,
                                     const uint8_t* codes, const void* scl, const int32_t* offsets,
                                     const int32_t* sorted_pairs, const int32_t* tiles,
                                     const int32_t* num_tiles, const uint16_t* out) {
  if (!x || !codes || !scl || !offsets || !sorted_pairs || !tiles || !num_tiles || !out)
    return kInvalid;
  if (x_stride < Kc || x_stride % 8) return kInvalid;
  if (x_rows * x_stride >= INT32_MAX) return kNotSupported;   // 32-bit activation offsets
  if (!aligned16(x) || !aligned16(codes) || !aligned16(out)) return kInvalid;
  if (!aligned4(offsets) || !aligned4(sorted_pairs) || !aligned4(tiles) || !aligned4(num_tiles))
    return kInvalid;
  return kOk;
}

}  // namespace gq
