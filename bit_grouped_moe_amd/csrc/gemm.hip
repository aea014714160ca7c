// Prefill grouped GEMM on 4-bit packed experts (NF4, MXFP4) and their
// input gradients, on gfx950 bf16 matrix cores.
//
// Pages: "grouped-nf4-gemm 0.43.0" -- page header (one GPU launch for the
// active experts, no full-size bf16 weight copies) and "Which entry point?"
// (grouped NF4 forward and backward, native MXFP4 expert math);
// "Receipts-driven engineering" -- opening summary (the codebook is decoded
// in registers inside the GEMM mainloop; the NF4 path is differentiable).
// The tiling below is this library's own design for CDNA4.
//
// One launch covers every tile of every expert (tile list from
// gq_route_sort): a workgroup takes 256 routed pairs of one expert (gathered
// activation rows) times a column tile, and the K loop runs in steps of 64.
// Two kernels share the tile list, the decode routines and the epilogue:
//  * contractions of at least 1024 (grouped_gemm_fwd_kernel): 256 columns
//    per tile, one wave per SIMD, activation tiles loaded straight into LDS
//    (see the comment above that kernel);
//  * shorter contractions and the input gradient (grouped_gemm_body): 128
//    columns per tile, two workgroups per CU so that one workgroup's
//    prologue and epilogue overlap the other's matrix work.
// The B tile (weights x 64 K) is decoded ONCE per workgroup from packed
// codes into bf16: in the first kernel each wave owns 64 of the 256 columns
// for all rows and decodes them straight into MFMA operand registers; in the
// second B goes through LDS (double-buffered, one barrier per step), shared
// by the waves.  The K order inside a step is permuted identically for A and
// B (lane half h takes k in [32h, 32h+32)), so every operand load
// is a contiguous 16-byte piece; the weights are the first MFMA operand, so
// a lane accumulates one output row and the epilogue writes rows from
// registers.  Block index -> tile is XCD-aware: the hardware deals blocks
// round-robin to the 8 XCDs, and consecutive blocks of one XCD get all
// column tiles of a row tile, so the gathered activation rows are reused
// from that XCD's L2.  Tiles past the last expert tile zero the rows of
// dropped pairs, in the same launch.  Every output element is written once:
// no atomics.
#include <type_traits>
#include <utility>

#include "gemm_common.hpp"
#include "gq_device.hpp"
#include "gq_host.hpp"
#include "../../include/gq.h"

namespace gq {

constexpr int kTN = 128;          // tile columns (output features)
constexpr int kBStride = 72;      // bf16 per LDS row of B (64 + 8 pad: conflict-free 16-B reads)
constexpr int kCStride = 64;      // bytes per LDS row of raw codes (dgrad staging)

// ---- B producers: fill Bs[col][k] (bf16, row stride kBStride) for step ks ----

// Forward: B[k][col] = W[n0 + col][ks*64 + k].  Thread t decodes 32 weights:
// col = t / 2, half h = t % 2 (k in [32h, 32h+32)), so the two halves of a
// row's 32 code bytes are neighbouring lanes and a load instruction touches
// 32 rows rather than 64 (down GEMM 188 -> 185 us).
struct FwdLoad {
  u32x4 c;
  float a;      // NF4 absmax
  uint32_t s;   // MXFP4 scale byte
  bool ok;
};

// Loads are unconditional, from addresses clamped into the bank; elements
// outside the matrix are zeroed when decoded.  (A conditional load would
// first zero its destination registers, and the hardware wait-count logic
// then stalls on every older load in flight before that write.)
template <int kMode>
__device__ __forceinline__ FwdLoad fwd_load(const GemmArgs& g, int e, int n0, int ks, int tid) {
  FwdLoad L;
  const int col = tid >> 1, h = tid & 1;
  const int k0 = ks * kTK + h * 32;
  int n;
  if constexpr (kMode == kFwdNF4Glu) {
    // columns [0, 64): gate rows n0 + col; [64, 128): the matching up rows
    const int j = n0 + (col & 63);
    L.ok = j < g.Nout && k0 < g.Kw;
    n = min(j, g.Nout - 1) + (col >= 64 ? g.Nout : 0);
  } else {
    n = n0 + col;
    L.ok = n < g.Nw && k0 < g.Kw;
  }
  const size_t row = (size_t)e * g.Nw + min(n, g.Nw - 1);
  const size_t kk = (size_t)min(k0, g.Kw - 32);
  L.c = *reinterpret_cast<const u32x4*>(g.codes + row * (size_t)(g.Kw / 2) + kk / 2);
  if constexpr (kMode == kFwdMX) {
    L.s = (uint32_t)static_cast<const uint8_t*>(g.scl)[row * (size_t)(g.Kw / 32) + kk / 32];
    L.a = 0.f;
  } else {
    L.a = static_cast<const float*>(g.scl)[row * (size_t)(g.Kw / 64) + kk / 64];
    L.s = 0u;
  }
  return L;
}

// Decode one code dword (8 weights, chunk q of the thread's 32) of a forward
// B tile into Bs[col][h*32 + 8q .. +8].
template <int kMode>
__device__ __forceinline__ void fwd_decode_chunk(const FwdLoad& L, int q, const float* lut,
                                                 uint16_t* Bs, int tid) {
  const int col = tid >> 1, h = tid & 1;
  uint32_t p[4];
  // Elements outside the matrix get a zero factor (their codes are a clamped
  // re-read): one select per chunk instead of one per output dword.
  if constexpr (kMode == kFwdMX) {
    const float sc = L.ok ? e8m0_to_f32(L.s) : 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b) p[b] = e2m1_pair_bf16_scaled(L.c[q], b, sc);
  } else {
    nf4_decode8_bf16(lut, L.c[q], L.ok ? L.a : 0.f, p);
  }
  *reinterpret_cast<u32x4*>(Bs + col * kBStride + h * 32 + 8 * q) = u32x4{p[0], p[1], p[2], p[3]};
}

// Dgrad: B[k][col] = W[ks*64 + k][k0 + col], i.e. a 64 x 128 block of W
// consumed transposed.  Raw codes (64 rows x 64 bytes) are staged in LDS,
// then thread t decodes rows 8*(t/32) .. +8 of the column quad 4*(t%32) ..
// +4 and writes four 16-byte runs of 8 consecutive contraction values.
// The 128 columns span 2 NF4 absmax blocks or 4 MXFP4 scale blocks per row;
// their factors are staged as float ([64 rows][kBlk]).
template <int kMode>
struct DgFmt {
  static constexpr bool kMx = kMode == kDgradMX;
  static constexpr int kBlkK = kMx ? 32 : 64;             // weights per scale block
  static constexpr int kBlk = kTN / kBlkK;                 // scale blocks per tile row
};

struct DgLoad {
  u32x4 c;
  float a;      // NF4 absmax of (row t/kBlk, block t%kBlk), t < 64*kBlk
  uint32_t s;   // MXFP4 scale byte of the same
  bool aok;     // the scale block lies inside the matrix
};

template <int kMode>
__device__ __forceinline__ DgLoad dg_load(const GemmArgs& g, int e, int k0, int ks, int tid) {
  using F = DgFmt<kMode>;
  DgLoad L;
  const int r = tid >> 2, q = tid & 3;                    // row in step, 16-byte quarter
  const int n = ks * kTK + r;                             // W row (< Nw since Nw % 64 == 0)
  const int kb = k0 + q * 32;                             // first weight of this quarter
  const size_t row = (size_t)e * g.Nw + n;
  L.c = *reinterpret_cast<const u32x4*>(g.codes + row * (size_t)(g.Kw / 2) +
                                        min(kb, g.Kw - 32) / 2);
  // scale of (row t/kBlk, block t%kBlk); threads past 64*kBlk reload a valid one
  const int t = tid & (F::kBlk * kTK - 1);
  const int ar = t / F::kBlk, ablk = k0 / F::kBlkK + t % F::kBlk;
  const int nblk = g.Kw / F::kBlkK;
  L.aok = ablk < nblk;
  const size_t aidx = ((size_t)e * g.Nw + ks * kTK + ar) * (size_t)nblk + min(ablk, nblk - 1);
  if constexpr (F::kMx) {
    L.s = (uint32_t)static_cast<const uint8_t*>(g.scl)[aidx];
    L.a = 0.f;
  } else {
    L.a = static_cast<const float*>(g.scl)[aidx];
    L.s = 0u;
  }
  return L;
}

template <int kMode>
__device__ __forceinline__ void dg_stage(const DgLoad& L, uint8_t* Cs, float* As, int tid) {
  using F = DgFmt<kMode>;
  // Cs: 64 rows x kCStride bytes of raw codes; As: [64 rows][kBlk] factors
  const int r = tid >> 2, q = tid & 3;
  // Quarters past the matrix width keep their (clamped, re-read) codes:
  // their scale blocks get a zero factor below, so they decode to zeros.
  // (A select here on the loaded codes is hoisted by the compiler to the
  // start of the step and makes it wait for the code load just issued.)
  *reinterpret_cast<u32x4*>(Cs + r * kCStride + q * 16) = L.c;
  if (tid < F::kBlk * kTK) {
    float f;
    if constexpr (F::kMx) f = e8m0_to_f32(L.s);
    else f = L.a;
    // factor of (row tid / kBlk, block tid % kBlk), stored block-major so a
    // thread's 8 consecutive rows are 32 contiguous bytes
    As[(tid % F::kBlk) * kTK + tid / F::kBlk] = L.aok ? f : 0.f;
  }
}

// Dgrad decode.  Thread (j4, r8) = (tid % 32, tid / 32) produces rows
// r8*8 .. +8 of the column quad 4*j4 .. +3: it reads its two code bytes of
// each of the 8 rows from LDS once per step, the rows' factors (one scale
// block covers the quad) as 32 contiguous bytes, and writes each column's 8
// consecutive contraction values as one 16-byte run.  Both formats take two
// passes of two columns.
//  * NF4: codebook values from the 16-entry LDS table; weight =
//    float32(value * absmax), then bf16 RNE.
//  * MXFP4 (code byte cp of each row holds
//    columns 4*j4 + 2cp and + 2cp + 1, the even one in the low nibble): the
//    hardware converter turns the byte into the two bf16 weights with the
//    e8m0 factor applied, exactly; a byte permute then pairs rows i and
//    i + 1 of one column.
struct DgCodes {
  uint32_t two[4];   // bytes j4*2, j4*2+1 of rows r8*8 + 2i (low half) and + 2i+1 (high half)
};

// The dgrad B tile stores column col at LDS row dg_brow(col), a permutation
// inside each group of four rows.  The decode writes columns 4 apart in one
// instruction (a thread owns a column quad) and the MFMA operand reads take 32
// consecutive columns; with 72-element rows the plain order put four lanes of
// every 16-byte write group on the same banks.  XOR-ing the row's low two
// bits with bit 4 and with bits 3 ^ 5 keeps both access groups on distinct
// banks (checked for 64 banks x 16 lanes and 32 banks x 8 lanes per cycle).
__device__ __forceinline__ int dg_brow(int col) {
  return col ^ ((col >> 4) & 1) ^ ((((col >> 3) ^ (col >> 5)) & 1) << 1);
}

template <int kMode>
__device__ __forceinline__ void dg_read_codes(const uint8_t* Cs, const float* As, int tid,
                                              DgCodes& R) {
  const int j4 = tid & 31, r8 = tid >> 5;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = r8 * 8 + i;
    const uint32_t v = *reinterpret_cast<const uint16_t*>(Cs + r * kCStride + j4 * 2);
    R.two[i >> 1] = (i & 1) ? (R.two[i >> 1] | (v << 16)) : v;
  }
}

template <int kMode>
__device__ __forceinline__ void dg_decode_pair(const DgCodes& R, const float* As, int cp,
                                               uint16_t* Bs, int tid) {
  using F = DgFmt<kMode>;
  const int j4 = tid & 31, r8 = tid >> 5;
  // factors of the 8 rows for the quad's scale block (32 contiguous bytes)
  const f32x4* fp = reinterpret_cast<const f32x4*>(As + ((j4 * 4) / F::kBlkK) * kTK + r8 * 8);
  const f32x4 f0 = fp[0], f1 = fp[1];
  const float f[8] = {f0[0], f0[1], f0[2], f0[3], f1[0], f1[1], f1[2], f1[3]};
  uint32_t ce[4], co[4];                 // columns 4 j4 + 2cp (even) and + 1 (odd), rows paired
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    // rows 2h (low half of two[h]) and 2h + 1 (high half): byte cp and 2 + cp
    const uint32_t r0 = e2m1_pair_bf16_scaled(R.two[h], cp, f[2 * h]);
    const uint32_t r1 = e2m1_pair_bf16_scaled(R.two[h], 2 + cp, f[2 * h + 1]);
    ce[h] = __builtin_amdgcn_perm(r1, r0, 0x05040100u);     // low halves: even column
    co[h] = __builtin_amdgcn_perm(r1, r0, 0x07060302u);     // high halves: odd column
  }
  const int c0 = j4 * 4 + 2 * cp;
  *reinterpret_cast<u32x4*>(Bs + dg_brow(c0) * kBStride + r8 * 8) = u32x4{ce[0], ce[1], ce[2], ce[3]};
  *reinterpret_cast<u32x4*>(Bs + dg_brow(c0 + 1) * kBStride + r8 * 8) =
      u32x4{co[0], co[1], co[2], co[3]};
}

// NF4: columns 2*part and 2*part + 1 of the quad per call (part 0, 1: the
// decode is spread over two MFMA slices), from the 16-entry codebook table
// (16 distinct banks: conflict-free); code dword h holds rows 2h and 2h + 1,
// its 8 nibbles in element order are the quad's columns of row 2h then of
// row 2h + 1 (high nibble = even column).
__device__ __forceinline__ void dg_decode_nf4(const DgCodes& R, const float* As, const float* lut,
                                              uint16_t* Bs, int tid, int part) {
  const int j4 = tid & 31, r8 = tid >> 5;
  const f32x4* fp = reinterpret_cast<const f32x4*>(As + (j4 / 16) * kTK + r8 * 8);
  const f32x4 f0 = fp[0], f1 = fp[1];
  const float f[8] = {f0[0], f0[1], f0[2], f0[3], f1[0], f1[1], f1[2], f1[3]};
  uint32_t c[2][4];                      // [column of the pair][row pair]
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    float q[8];
    nf4_lookup8(lut, R.two[h], q);       // the other pair's lookups are dead code
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int col = 2 * part + k;
      c[k][h] = pack_bf16x2(q[col] * f[2 * h], q[4 + col] * f[2 * h + 1]);
    }
  }
#pragma unroll
  for (int k = 0; k < 2; ++k)
    *reinterpret_cast<u32x4*>(Bs + dg_brow(j4 * 4 + 2 * part + k) * kBStride + r8 * 8) =
        u32x4{c[k][0], c[k][1], c[k][2], c[k][3]};
}

// one step's B tile in two passes (slices 1 and 2), two columns of the quad each
template <int kMode>
__device__ __forceinline__ void dg_decode(const DgCodes& R, const float* As, int part,
                                          const float* lut, uint16_t* Bs, int tid) {
  if constexpr (kMode == kDgradNF4) {
    dg_decode_nf4(R, As, lut, Bs, tid, part);
  } else {
    dg_decode_pair<kMode>(R, As, part, Bs, tid);
  }
}

// Rows of sub-tiles ms0, ms1 (32 rows each) for the 128 B columns of a
// 256 x 128 tile (SwiGLU: 64 outputs from gate blocks 0, 1 and up blocks 2, 3).
template <bool kGlu, int kTNo>
__device__ __forceinline__ void store_rows_t(const f32x16 (&acc)[2][4], bool act0, bool act1,
                                             int ms0, int ms1, int valid, const int* pair_s,
                                             const GemmArgs& g, int n0, int lr, int lh) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if (!(j ? act1 : act0)) continue;
    const int m = (j ? ms1 : ms0) * 32 + lr;
    const int p = pair_s[m];
    const float sc = (g.pair_scale && m < valid) ? g.pair_scale[p] : 1.f;
#pragma unroll
    for (int c = 0; c < kTNo / 32; ++c) {
      const int col = n0 + 32 * c;
      if (m < valid && col < g.Nout) {
        float v[16];
#pragma unroll
        for (int r = 0; r < 16; ++r)
          v[r] = kGlu ? silu_f32(acc[j][c][r]) * acc[j][c + 2][r] * sc : acc[j][c][r] * sc;
        store_block_t(v, g.out + (int64_t)p * g.Nout + col, lh);
      }
    }
  }
}

// ---- the 256 x 128 kernel (short contractions, input gradient) ----
// Wave w owns the 32-row sub-tiles w and w+4 (interleaved so that short
// expert segments still spread over all four SIMDs) across all 128 columns:
// 2 x 4 v_mfma_f32_32x32x16_bf16 per 16-wide K slice.
// Software pipeline, one barrier per K step.  Iteration ks:
//   issue the global loads that step ks+1 (activations) and ks+2 (codes)
//   need; decode step ks+1 into the LDS buffer the MFMAs are not reading;
//   run the MFMAs of step ks from the other buffer; barrier.
// The decode (VALU + LDS) and the matrix-core work of different steps are
// independent inside an iteration, so they overlap.  Dgrad stages raw codes
// through LDS first (transposed consumption), one step further ahead.
template <int kMode>
__device__ __forceinline__ void grouped_gemm_body(const GemmArgs& g) {
  constexpr bool kDg = kMode == kDgradNF4 || kMode == kDgradMX;
  // Activation (dY) operand of the input gradient.  MXFP4: staged like the
  // forward operand (coalesced 128-byte row loads, per-wave swizzled LDS
  // area); fragment-shaped loads straight into registers make every load
  // instruction touch 32 rows and kept the address unit ~80% busy (gpt-oss
  // dgrad gate_up 513 -> 433 us staged).  NF4: LDS-direct loads into the
  // same area (on the Qwen3 shapes tiles are half full, ~128 rows per
  // expert, and staging through registers costs more LDS issue than the
  // address unit saves: 227 vs 220 us with fragment-shaped loads; LDS-direct
  // 213 us).  For MXFP4 the LDS-direct form is not faster (434 vs 426 us).
  constexpr bool kDmaA = kMode == kDgradNF4;
  constexpr bool kGlu = kMode == kFwdNF4Glu;
  constexpr int kTNo = kGlu ? kTN / 2 : kTN;               // output columns per tile
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kTN * kBStride];
  __shared__ __attribute__((aligned(16))) uint8_t Cs[kDg ? 2 : 1][kDg ? kTK * kCStride : 16];
  __shared__ float As[kDg ? 2 : 1][kDg ? DgFmt<kMode>::kBlk * kTK : 1];
  __shared__ __attribute__((aligned(16))) uint16_t Aw[4][64 * kTK];
  __shared__ int pair_s[kTM];
  // dgrad rows are the pairs themselves: row_s aliases pair_s (saves 1 KB of
  // LDS, which lets two dgrad workgroups share a CU)
  __shared__ int row_s_buf[kDg ? 1 : kTM];
  int* const row_s = kDg ? pair_s : row_s_buf;
  __shared__ float lut[16];

  const int tid = threadIdx.x;
  TileInfo ti;
  if (!tile_head<kTNo>(g, tid, ti)) return;
  const int e = ti.e, start = ti.start, valid = ti.valid, n0 = ti.n0;
  for (int r = tid; r < kTM; r += kGemmThreads) {
    int p = g.sorted_pairs[start + min(r, valid - 1)];
    p = ((unsigned)p < (unsigned)g.P) ? p : 0;
    pair_s[r] = p;
    if constexpr (!kDg) row_s[r] = p / g.topk;
  }
  if constexpr (kMode != kFwdMX && kMode != kDgradMX) nf4_lut_init(lut, tid);
  lds_barrier();

  const int wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 31, lh = lane >> 5;
  const int ms0 = wave, ms1 = wave + 4;                    // owned 32-row sub-tiles
  const bool act0 = ms0 * 32 < valid, act1 = ms1 * 32 < valid;
  const int nsteps = (g.Kc + kTK - 1) / kTK;
  const bool ktail = (g.Kc % kTK) != 0;                   // MXFP4 only: last step half full
  // valid B columns: the SwiGLU tile decodes all 128 (missing ones as zeros)
  const int ncols = kGlu ? kTN : min(kTN, g.Nout - n0);     // multiple of 32

  f32x16 acc[2][4];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][c][r] = 0.f;

  // ---- A operand: the gathered activation rows, staged per wave through LDS.
  // Global loads are coalesced: load i (0..7) of a lane reads 16 bytes, chunk
  // lane%8 of the K step, of the wave's local row
  //   r(i) = (i/4)*32 + (i%4)*8 + lane/8   (rows 0..31: sub-tile ms0, 32..63: ms1)
  // so 8 lanes cover one row's 128 bytes (MFMA-fragment-shaped loads touch 32
  // rows per instruction and were the kernel's largest cost).  The wave writes
  // them into its own LDS area with the chunk slot XOR-swizzled by
  // (row >> 1) & 7 and reads MFMA fragments (row lr, chunk lh*4 + sl) back;
  // both directions are free of bank conflicts, and no other wave touches the
  // area, so no barrier.  Loads are unconditional within a wave's loop
  // variant (chunks past a K tail re-read the last valid chunk and are zeroed
  // when read), see the note at fwd_load; a wave loads the rows of sub-tile
  // ms1 only in the variants where ms1 is active (kNa = 8 loads) and none in
  // the variant for a wave without active rows.
  uint16_t* aw = &Aw[wave][0];
  // The lane's row offsets are re-read from LDS at every step (registers
  // are short); element offsets fit 32 bits (host check).
  auto load_a = [&](auto na_c, int ks, u32x4 (&Ar)[8]) {
    constexpr int kNa = decltype(na_c)::value;
    const int k = min(ks * kTK + (lane & 7) * 8, g.Kc - 8);
#pragma unroll
    for (int i = 0; i < kNa; ++i) {
      const int off = row_s[(i < 4 ? ms0 : ms1) * 32 + (i & 3) * 8 + (lane >> 3)] * (int)g.x_stride;
      Ar[i] = *reinterpret_cast<const u32x4*>(g.x + off + k);
    }
  };
  auto stage_a = [&](auto na_c, const u32x4 (&Ar)[8]) {
    constexpr int kNa = decltype(na_c)::value;
#pragma unroll
    for (int i = 0; i < kNa; ++i) {
      const int r = (i >> 2) * 32 + (i & 3) * 8 + (lane >> 3);
      const int slot = (lane & 7) ^ ((r >> 1) & 7);
      *reinterpret_cast<u32x4*>(aw + r * kTK + slot * 8) = Ar[i];
    }
  };
  auto read_a = [&](int nj, int sl, u32x4 (&a)[2], bool zero_hi) {
#pragma unroll
    for (int j = 0; j < nj; ++j) {
      const int r = j * 32 + lr;
      const int slot = (lh * 4 + sl) ^ ((r >> 1) & 7);
      a[j] = *reinterpret_cast<const u32x4*>(aw + r * kTK + slot * 8);
      if constexpr (kMode == kFwdMX) {                     // K tail: zero the missing half
        if (zero_hi) a[j] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  // NF4 dgrad: the same rows and swizzle, written by LDS-direct loads.
  // Instruction j (j < 4: sub-tile ms0, else ms1) fills the wave's local rows
  // r0(j) .. r0(j) + 8, r0(j) = (j / 4) * 32 + (j % 4) * 8; lane L writes
  // slot L % 8 of row r0(j) + L / 8 and so fetches global chunk
  // (L % 8) ^ ((row >> 1) & 7).  A step's fragments are all read into
  // registers at its start, then the next step's rows are loaded over them
  // (one area per wave: no barrier).  Rows are the pairs; the contraction
  // (N) is a multiple of 64, so no K tail.  Byte offsets fit 32 bits (host
  // check on the element offsets).
  uint32_t voff[kDmaA ? 8 : 1];
  if constexpr (kDmaA) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = (j >> 2) * 32 + (j & 3) * 8 + (lane >> 3);
      const int c = (lane & 7) ^ ((r >> 1) & 7);
      voff[j] = (uint32_t)row_s[(j < 4 ? ms0 : ms1) * 32 + (j & 3) * 8 + (lane >> 3)] *
                    (uint32_t)(g.x_stride * 2) + 16u * (uint32_t)c;
    }
  }
  auto dma_a = [&](auto na_c, int ks) {
    constexpr int kNa = decltype(na_c)::value;             // 8: both sub-tiles, 4: ms0 only
    const char* xb = reinterpret_cast<const char*>(g.x) + (size_t)ks * (kTK * 2);
#pragma unroll
    for (int j = 0; j < kNa; ++j) {
      uint32_t vo = voff[j];
      // opaque: otherwise the compiler keeps all offsets widened to 64 bits
      // (16 registers) and spills
      asm volatile("" : "+v"(vo));
      __builtin_amdgcn_global_load_lds((glb_void_t*)(xb + vo),
                                       (lds_void_t*)(aw + ((j >> 2) * 32 + (j & 3) * 8) * kTK),
                                       16, 0, 0);
    }
  };
  auto read_frags = [&](auto na_c, u32x4 (&F)[2][4]) {
    constexpr int kNj = decltype(na_c)::value / 4;
#pragma unroll
    for (int j = 0; j < kNj; ++j)
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
        const int slot = (lh * 4 + sl) ^ ((lr >> 1) & 7);
        F[j][sl] = *reinterpret_cast<const u32x4*>(aw + (j * 32 + lr) * kTK + slot * 8);
      }
  };
  auto load_b_slice = [&](const uint16_t* B, int sl, bf16x8 (&b)[4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int row = kDg ? dg_brow(c * 32 + lr) : c * 32 + lr;
      b[c] = as_bf16x8(
          *reinterpret_cast<const u32x4*>(B + row * kBStride + lh * 32 + sl * 8));
    }
  };
  // kRows = number of active 32-row sub-tiles of this wave (1 or 2) with all
  // 128 columns valid: unguarded MFMAs.  kRows == 0: generic guarded path.
  // kRows == -1 (no active sub-tile): the wave only decodes its share of B.
  auto mfma_slice = [&](auto rows_c, const u32x4 (&a)[2], const bf16x8 (&b)[4]) {
    constexpr int kRows = decltype(rows_c)::value;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      // weights as the first operand: the accumulator holds the transposed
      // tile, one output row per lane
      if constexpr (kRows == 0) {
        if (c * 32 >= ncols) continue;
        if (act0)
          acc[0][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[c], as_bf16x8(a[0]), acc[0][c],
                                                              0, 0, 0);
        if (act1)
          acc[1][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[c], as_bf16x8(a[1]), acc[1][c],
                                                              0, 0, 0);
      } else {
        acc[0][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[c], as_bf16x8(a[0]), acc[0][c],
                                                            0, 0, 0);
        if constexpr (kRows == 2)
          acc[1][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[c], as_bf16x8(a[1]), acc[1][c],
                                                              0, 0, 0);
      }
    }
  };

  u32x4 Ar[kDmaA ? 1 : 8];                                 // staged A prefetch
  u32x4 Ad[2][kDmaA ? 4 : 1];                              // a step's A fragments (LDS-direct)
  FwdLoad F0{}, F1{};
  DgLoad D{};
  DgCodes R{};

  // Loop variant of the wave (uniform): rows of activations it loads per
  // step (8 loads: both sub-tiles, 4: sub-tile ms0, 0: none).
  using I2 = std::integral_constant<int, 2>;
  using I1 = std::integral_constant<int, 1>;
  using I0 = std::integral_constant<int, 0>;
  using Im = std::integral_constant<int, -1>;
  const int variant = !act0 ? -1 : (ncols == kTN ? (act1 ? 2 : 1) : 0);
  const int na = variant == -1 ? 0 : (variant == 1 ? 4 : 8);

  // ---- prologue: step 0 decoded into Bs[0] and staged in Aw; step 1's
  // activations and codes in flight ----
  auto prologue_a = [&](auto na_c) {
    if constexpr (decltype(na_c)::value > 0) {
      if constexpr (kDmaA) {
        dma_a(na_c, 0);
      } else {
        load_a(na_c, 0, Ar);
        stage_a(na_c, Ar);
        load_a(na_c, min(1, nsteps - 1), Ar);
      }
    }
  };
  if (na == 8) prologue_a(std::integral_constant<int, 8>{});
  else if (na == 4) prologue_a(std::integral_constant<int, 4>{});
  if constexpr (kDg) {
    D = dg_load<kMode>(g, e, n0, 0, tid);
    dg_stage<kMode>(D, Cs[0], As[0], tid);
    D = dg_load<kMode>(g, e, n0, min(1, nsteps - 1), tid);
    lds_barrier();
    dg_read_codes<kMode>(Cs[0], As[0], tid, R);
    dg_decode<kMode>(R, As[0], 0, lut, Bs[0], tid);
    dg_decode<kMode>(R, As[0], 1, lut, Bs[0], tid);
    dg_stage<kMode>(D, Cs[1], As[1], tid);
    D = dg_load<kMode>(g, e, n0, min(2, nsteps - 1), tid);
  } else {
    F0 = fwd_load<kMode>(g, e, n0, 0, tid);
    F1 = fwd_load<kMode>(g, e, n0, min(1, nsteps - 1), tid);
#pragma unroll
    for (int q = 0; q < 4; ++q) fwd_decode_chunk<kMode>(F0, q, lut, Bs[0], tid);
  }
  lds_barrier();

  // ---- main loop: step ks runs its MFMAs slice by slice, its operands read
  // from LDS one slice ahead; between slices it decodes a quarter of step
  // ks+1 into the other B buffer.  After the last slice it stages step ks+1's
  // activations (loaded during step ks-1) and loads step ks+2's.  All
  // prefetches and decodes are unconditional (indices clamped to the last
  // step): loads under a branch make the compiler wait for them early.
  // Unrolled by two so the two code register sets swap roles without copies. ----
  auto run_loop = [&](auto rows_c) {
    constexpr int kRows = decltype(rows_c)::value;
    constexpr int kNa = kRows < 0 ? 0 : (kRows == 1 ? 4 : 8);
    using NaC = std::integral_constant<int, kNa>;
    auto step = [&](int ks, FwdLoad& F_dec, FwdLoad& F_fill) {
      const uint16_t* B = Bs[ks & 1];
      uint16_t* Bn = Bs[(ks + 1) & 1];
      const bool zero_hi = ktail && ks == nsteps - 1 && lh == 1;
      if constexpr (!kDg) F_fill = fwd_load<kMode>(g, e, n0, min(ks + 2, nsteps - 1), tid);
      // B fragments ping-pong between two register sets (no copies): slice
      // sl's MFMAs read one set while slice sl+1's load into the other.  The
      // slice's A fragments are read at its start (registers are short).
      bf16x8 b0[4], b1[4];
      auto slice = [&](int sl, const bf16x8 (&bc)[4], bf16x8 (&bn)[4]) {
        u32x4 ac[2];
        if constexpr (kRows >= 0) {
          constexpr int kNj = kRows == 1 ? 1 : 2;          // sub-tiles with operands
          if constexpr (kDmaA) {
            ac[0] = Ad[0][sl];
            if constexpr (kNj == 2) ac[1] = Ad[1][sl];
          } else {
            read_a(kNj, sl, ac, zero_hi);
          }
          if (sl < 3) load_b_slice(B, sl + 1, bn);
        }
        if constexpr (kDg) {
          if (sl == 0) dg_read_codes<kMode>(Cs[(ks + 1) & 1], As[(ks + 1) & 1], tid, R);
          if (sl == 1 || sl == 2) dg_decode<kMode>(R, As[(ks + 1) & 1], sl - 1, lut, Bn, tid);
          if (sl == 3) {                                   // codes of step ks+2, then ks+3
            dg_stage<kMode>(D, Cs[ks & 1], As[ks & 1], tid);
            D = dg_load<kMode>(g, e, n0, min(ks + 3, nsteps - 1), tid);
          }
        } else {
          fwd_decode_chunk<kMode>(F_dec, sl, lut, Bn, tid);
        }
        if constexpr (kRows >= 0) mfma_slice(rows_c, ac, bc);
        if constexpr (kDmaA && kNa > 0) {
          if (sl == 0) {        // every fragment of step ks has arrived: load step ks+1 over them
            __builtin_amdgcn_s_waitcnt(0xC07F);            // lgkmcnt(0)
            dma_a(NaC{}, min(ks + 1, nsteps - 1));
          }
        }
      };
      if constexpr (kDmaA && kNa > 0) read_frags(NaC{}, Ad);  // waits for step ks's rows
      if constexpr (kRows >= 0) load_b_slice(B, 0, b0);
      slice(0, b0, b1);
      slice(1, b1, b0);
      slice(2, b0, b1);
      slice(3, b1, b0);
      if constexpr (!kDmaA && kNa > 0) {
        stage_a(NaC{}, Ar);                              // step ks+1 (own area: no barrier)
        load_a(NaC{}, min(ks + 2, nsteps - 1), Ar);
      }
      if constexpr (kDmaA) {
        // Barrier without a fence: a release fence would also wait for the
        // LDS-direct loads in flight (they count as pending LDS writes) and
        // with them for the code loads just issued.  Those loads write only
        // this wave's own area, which only this wave reads, after the wait
        // the compiler inserts for them; lgkmcnt(0) completes this wave's
        // LDS writes, and the empty asm statements keep every memory access
        // on its side of the barrier.
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0xC07F);                // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      } else {
        lds_barrier();
      }
    };
    for (int ks = 0; ks < nsteps; ks += 2) {
      step(ks, F1, F0);
      if (ks + 1 < nsteps) step(ks + 1, F0, F1);
    }
  };
  if (variant == 2) run_loop(I2{});
  else if (variant == 1) run_loop(I1{});
  else if (variant == 0) run_loop(I0{});
  else run_loop(Im{});

  // ---- epilogue: one output row per lane, written from registers ----
  store_rows_t<kGlu, kTNo>(acc, act0, act1, ms0, ms1, valid, pair_s, g, n0, lr, lh);
}

// The dgrad fits 2 waves per SIMD (2 workgroups per CU): it keeps its code
// words two rows per register.
template <int kMode>
__global__ __launch_bounds__(kGemmThreads, 2) void grouped_dgrad_kernel(GemmArgs g) {
  grouped_gemm_body<kMode>(g);
}
// Forward products with a short contraction (few K steps per tile) run on
// the two-workgroups-per-CU kernel: one workgroup's prologue and epilogue
// then overlap the other's matrix work.
template <int kMode>
__global__ __launch_bounds__(kGemmThreads, 2) void grouped_gemm_fwd_shortk_kernel(GemmArgs g) {
  grouped_gemm_body<kMode>(g);
}

// ---- forward kernel: 256 x 256 output tile, one wave per SIMD ----
// Workgroup = 4 waves on one CU (256 accumulator registers per lane, ~70 KB
// of LDS); the tile loop is fwd_columns below.

// Instruction interleave for one K slice of kM MFMAs: after each MFMA, an
// even share of the slice's LDS reads, VALU ops and LDS writes, so that the
// single wave of a SIMD keeps the matrix core fed while it decodes.
template <int kM, int kDs, int kValu, int kDsw, int m>
__device__ __forceinline__ void sched_one() {
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  constexpr int ds = kDs * (m + 1) / kM - kDs * m / kM;
  constexpr int va = kValu * (m + 1) / kM - kValu * m / kM;
  constexpr int dw = kDsw * (m + 1) / kM - kDsw * m / kM;
  if constexpr (ds > 0) __builtin_amdgcn_sched_group_barrier(0x100, ds, 0);
  if constexpr (va > 0) __builtin_amdgcn_sched_group_barrier(0x002, va, 0);
  if constexpr (dw > 0) __builtin_amdgcn_sched_group_barrier(0x200, dw, 0);
}
template <int kM, int kDs, int kValu, int kDsw, int... I>
__device__ __forceinline__ void sched_slice_seq(std::integer_sequence<int, I...>) {
  (sched_one<kM, kDs, kValu, kDsw, I>(), ...);
}
template <int kM, int kDs, int kValu, int kDsw>
__device__ __forceinline__ void sched_slice() {
  sched_slice_seq<kM, kDs, kValu, kDsw>(std::make_integer_sequence<int, kM>{});
}

// ---- the 256-column tile loop: one B column per wave, decoded in registers ----
// Wave w owns the B columns 64 w + [0, 64) for ALL of the tile's 32-row
// sub-tiles (up to 4 on tiles of at most 128 rows, up to 8 otherwise: 8 x 2
// blocks of 32 x 32 accumulators fill the 256 AGPRs), so each B column feeds
// exactly one wave, which decodes it straight into MFMA operand registers:
// no B tile in LDS, no B fragment reads, no B barrier traffic.  (A 2 x 2
// layout with B decoded once into LDS and read by two waves each was 2-4%
// slower on every workload measured, 8-10% on tiles of at most 64 rows.)
// Lane (lr, lh) of column block cb holds column 64 w + 32 cb + lr
// (SwiGLU: block 0 is gate row j = 32 w + lr of the tile's outputs, block 1
// the matching up row) and, in slice sl, k = 32 lh + 8 sl + [0, 8): the K
// order of the A fragments, so the lane's operand for the whole step is the
// 16 code bytes at byte 16 lh of the column's 32-byte step chunk (the
// step's 64 K are one NF4 absmax block; each lane half's 32 K one MXFP4
// scale block).  The activation tile goes from global memory straight into
// LDS (LDS-direct loads, double-buffered, one barrier per step); each wave
// reads the A fragments of every active sub-tile.  Per 16-wide K slice a
// wave runs (active sub-tiles) x 2 v_mfma_f32_32x32x16_bf16, interleaved
// (NF4) with its fragment reads, table reads and decode VALU work.
// The SwiGLU epilogue combines blocks 0 and 1, which sit in the same lanes.
template <int kMode, int kSub>
__device__ __forceinline__ void fwd_columns(const GemmArgs& g, int e, int n0, int start, int valid,
                                           int tid, uint16_t* A0, uint16_t* A1, f32x2* lut2,
                                           int* pair_s, int* row_s, float* scale_s) {
  constexpr bool kGlu = kMode == kFwdNF4Glu;
  constexpr bool kMx = kMode == kFwdMX;
  const int nsteps = (g.Kc + kTK - 1) / kTK;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int lr = lane & 31, lh = lane >> 5;
  const bool ktail = kMx && (g.Kc % kTK) != 0;             // MXFP4: last step half full
  // this lane's column (SwiGLU: its output column) and whether it exists
  const int jcol = kGlu ? n0 + 32 * wave + lr : n0 + 64 * wave + lr;
  bool cok[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) cok[cb] = kGlu ? jcol < g.Nout : jcol + 32 * cb < g.Nw;
  // K tail: lane half 1 has no weights in the last step; it re-reads half 0
  // (in bounds) and decodes with a zero factor.
  auto load = [&](int ks) {
    const bool full = ks * kTK + kTK <= g.Kw;
    return n_load<kMode>(g, e, jcol, ks, full ? lh : 0);
  };
  NLoad X = load(0);
  NLoad Y = load(min(1, nsteps - 1));
  // The pair weight of this thread's row is loaded here but put into LDS only
  // after the main loop: written now, its dependent load would be waited for
  // before the prologue barrier (gate_up 312 -> 307 us).
  float psc;
  {
    int p = g.sorted_pairs[start + min(tid, valid - 1)];
    p = ((unsigned)p < (unsigned)g.P) ? p : 0;
    pair_s[tid] = p;
    row_s[tid] = p / g.topk;
    psc = g.pair_scale ? g.pair_scale[p] : 1.f;
  }
  if constexpr (!kMx) nf4_pairs_init(lut2, tid);
  lds_barrier();

  // LDS-direct activation loads: instruction j of wave w fills the 8-row
  // group arow(j) (128-row tiles: the wave's own 32 rows; 256-row tiles:
  // groups dealt round-robin to the waves).  Rows are 128 bytes with the
  // 16-byte chunk slot XOR-swizzled by (row >> 1) & 7 (conflict-free
  // fragment reads): lane L fills slot L % 8 of row L / 8 of the group, so it
  // fetches the global chunk (L % 8) ^ swizzle(row).
  auto arow = [&](int j) { return kSub == 4 ? 32 * wave + 8 * j : 8 * (4 * j + wave); };
  uint32_t voff[kSub];
  uint32_t tailbits = 0;
#pragma unroll
  for (int j = 0; j < kSub; ++j) {
    const int R = arow(j) + (lane >> 3);
    const int c = (lane & 7) ^ ((R >> 1) & 7);
    voff[j] = (uint32_t)row_s[R] * (uint32_t)(g.x_stride * 2) + 16u * (uint32_t)c;
    tailbits |= (c >= 4 ? 1u : 0u) << j;
  }
  auto dma_a = [&](int ks, uint16_t* Adst) {
    const char* xb = reinterpret_cast<const char*>(g.x) + (size_t)ks * (kTK * 2);
    const bool tail = ktail && ks == nsteps - 1;
#pragma unroll
    for (int j = 0; j < kSub; ++j) {
      if (arow(j) < valid) {                               // groups past the segment: skipped
        uint16_t* dst = Adst + arow(j) * kTK;
        if (kMx && tail && ((tailbits >> j) & 1u)) {
          *reinterpret_cast<u32x4*>(dst + lane * 8) = u32x4{0u, 0u, 0u, 0u};
        } else {
          __builtin_amdgcn_global_load_lds((glb_void_t*)(xb + voff[j]), (lds_void_t*)dst, 16, 0,
                                           0);
        }
      }
    }
  };
  const int aslot_x = (lr >> 1) & 7;
  auto read_a = [&](const uint16_t* A, int i, int sl) -> u32x4 {
    const int R = 32 * i + lr;
    return *reinterpret_cast<const u32x4*>(A + R * kTK + (((lh * 4 + sl) ^ aslot_x) * 8));
  };
  // B operand of slice sl, column block cb, for the step whose codes are L
  auto decode = [&](const NLoad& L, int ks, int cb, int sl) -> bf16x8 {
    const uint32_t cw = L.c[cb][sl];
    uint32_t w[4];
    if constexpr (kMx) {
      const bool live = cok[cb] && (!(ktail && ks == nsteps - 1) || lh == 0);
      const float f = live ? e8m0_to_f32(L.s[cb]) : 0.f;
#pragma unroll
      for (int b = 0; b < 4; ++b) w[b] = e2m1_pair_bf16_scaled(cw, b, f);
    } else {
      float q[8];
      nf4_pairs8(lut2, cw, q);
      const float a = cok[cb] ? L.a[cb] : 0.f;
#pragma unroll
      for (int b = 0; b < 4; ++b) w[b] = pack_bf16x2(q[2 * b] * a, q[2 * b + 1] * a);
    }
    return as_bf16x8(u32x4{w[0], w[1], w[2], w[3]});
  };

  f32x16 acc[kSub][2];
#pragma unroll
  for (int i = 0; i < kSub; ++i)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][c][r] = 0.f;
  const int nrows = (valid + 31) / 32;                     // active sub-tiles (all waves)
  // A column block (32 columns from a multiple of 32; the matrix width is a
  // multiple of 32) is valid for all lanes or for none: wave-uniform flags.
  const bool allcols = __builtin_amdgcn_readfirstlane((cok[0] && cok[1]) ? 1 : 0) != 0;
  const bool anycol = __builtin_amdgcn_readfirstlane((cok[0] || cok[1]) ? 1 : 0) != 0;

  // ---- prologue: step 0's activations staged, its B decoded; step 1's
  // codes in flight ----
  bf16x8 B0[2][4], B1[2][4];
  dma_a(0, A0);
#pragma unroll
  for (int sl = 0; sl < 4; ++sl)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) B0[cb][sl] = decode(X, 0, cb, sl);
  __builtin_amdgcn_s_waitcnt(0);
  lds_barrier();

  auto run_loop = [&](auto rows_c) {
    constexpr int kRows = decltype(rows_c)::value;         // -1: guarded generic path
    auto step = [&](int ks, const uint16_t* Ac, uint16_t* An, const bf16x8 (&Bc)[2][4],
                    bf16x8 (&Bn)[2][4], const NLoad& Ldec, NLoad& Lfill) {
      dma_a(min(ks + 1, nsteps - 1), An);
      Lfill = load(min(ks + 2, nsteps - 1));
      __builtin_amdgcn_sched_barrier(0);                   // keep the loads at the step start
      u32x4 fa[2][kSub];
      auto frags = [&](int sl, u32x4 (&a)[kSub]) {
#pragma unroll
        for (int i = 0; i < kSub; ++i) {
          if (kRows >= 0 ? i < kRows : true) a[i] = read_a(Ac, i, sl);
        }
      };
      frags(0, fa[0]);
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
        if (sl < 3) frags(sl + 1, fa[(sl + 1) & 1]);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) Bn[cb][sl] = decode(Ldec, min(ks + 1, nsteps - 1), cb, sl);
#pragma unroll
        for (int i = 0; i < kSub; ++i)
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) {
            if constexpr (kRows >= 0) {
              if (i < kRows)
                acc[i][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    Bc[cb][sl], as_bf16x8(fa[sl & 1][i]), acc[i][cb], 0, 0, 0);
            } else {
              if (i < nrows && anycol)
                acc[i][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    Bc[cb][sl], as_bf16x8(fa[sl & 1][i]), acc[i][cb], 0, 0, 0);
            }
          }
        // NF4: interleave the slice's MFMAs with its fragment reads, table
        // reads and decode VALU work (one wave per SIMD)
        if constexpr (kRows > 0 && !kMx) sched_slice<2 * kRows, kRows + 8, 36, 0>();
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);                  // vmcnt(0): this step's loads landed
      lds_barrier();
    };
    for (int ks = 0; ks < nsteps; ks += 2) {
      step(ks, A0, A1, B0, B1, Y, X);
      if (ks + 1 < nsteps) step(ks + 1, A1, A0, B1, B0, X, Y);
    }
  };
  // loop variants by active sub-tiles (1..4 on 128-row tiles, 5..8 on
  // 256-row tiles), all columns valid; else the guarded generic loop
  using I8 = std::integral_constant<int, kSub == 8 ? 8 : 4>;
  using I7 = std::integral_constant<int, kSub == 8 ? 7 : 3>;
  using I6 = std::integral_constant<int, kSub == 8 ? 6 : 2>;
  using I5 = std::integral_constant<int, kSub == 8 ? 5 : 1>;
  if (allcols && nrows == I8::value) run_loop(I8{});
  else if (allcols && nrows == I7::value) run_loop(I7{});
  else if (allcols && nrows == I6::value) run_loop(I6{});
  else if (allcols && nrows == I5::value) run_loop(I5{});
  else run_loop(std::integral_constant<int, -1>{});
  scale_s[tid] = psc;
  lds_barrier();

  // ---- epilogue: one output row per lane ----
  if constexpr (kGlu) {
#pragma unroll
    for (int i = 0; i < kSub; ++i) {
      if (i >= nrows) continue;
      const int m = 32 * i + lr;
      const int p = pair_s[m];
      const float sc = scale_s[m];
      const int col = n0 + 32 * wave;
      if (m < valid && col < g.Nout) {
        float v[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] = silu_f32(acc[i][0][r]) * acc[i][1][r] * sc;
        store_block_t(v, g.out + (int64_t)p * g.Nout + col, lh);
      }
    }
  } else {
    store_wide_rows<kSub>(acc, nrows, valid, pair_s, scale_s, g, n0, wave, lr, lh);
  }
}

template <int kMode>
__global__ __launch_bounds__(kGemmThreads, 1) void grouped_gemm_fwd_kernel(GemmArgs g) {
  constexpr bool kGlu = kMode == kFwdNF4Glu;
  constexpr int kTNo = kGlu ? kXN / 2 : kXN;               // output columns per tile
  // Separate arrays: the compiler then knows that an LDS-direct load into one
  // buffer does not alias reads of the other (no extra waits).
  __shared__ __attribute__((aligned(16))) uint16_t A0[kTM * kTK];
  __shared__ __attribute__((aligned(16))) uint16_t A1[kTM * kTK];
  __shared__ int pair_s[kTM];                              // pair of each tile row
  __shared__ int row_s[kTM];                               // its activation row (pair / topk)
  __shared__ float scale_s[kTM];                           // its pair weight (1 if none)
  // NF4 code-byte pair table; the alignment places it at LDS address 0
  __shared__ __attribute__((aligned(4096))) f32x2 lut2[256];

  const int tid = threadIdx.x;
  TileInfo t;
  if (!tile_head<kTNo>(g, tid, t)) return;
  if (t.valid <= kNarrowRows)
    fwd_columns<kMode, 4>(g, t.e, t.n0, t.start, t.valid, tid, A0, A1, lut2, pair_s, row_s,
                          scale_s);
  else
    fwd_columns<kMode, 8>(g, t.e, t.n0, t.start, t.valid, tid, A0, A1, lut2, pair_s, row_s,
                          scale_s);
}

// Contractions of at least this many elements use the 256 x 256 kernel
// (one wave per SIMD); shorter ones the 256 x 128 kernel, two workgroups per CU.
constexpr int kLongK = 1024;

template <int kMode>
static int launch_gemm(GemmArgs g, int32_t max_tiles, int32_t tile_m, hipStream_t stream) {
  if (tile_m != kTM) return kNotSupported;
  const int64_t need = (int64_t)(g.P + kTM - 1) / kTM + g.E + 1;
  if (max_tiles < need) return kInvalid;
  constexpr bool kDgMode = kMode == kDgradNF4 || kMode == kDgradMX;
  const bool wide = !kDgMode && g.Kc >= kLongK;
  const int kW = wide ? kXN : kTN;                          // B columns per tile
  const int kTNo = kMode == kFwdNF4Glu ? kW / 2 : kW;       // output columns per tile
  g.n_col_tiles = (g.Nout + kTNo - 1) / kTNo;
  const int64_t n_logical = (int64_t)max_tiles * g.n_col_tiles;
  const int64_t group = 8LL * g.n_col_tiles;
  const int64_t grid = ((n_logical + group - 1) / group) * group;
  if (grid > INT32_MAX) return kNotSupported;
  g.n_logical = (int)n_logical;
  if constexpr (kDgMode)
    hipLaunchKernelGGL(grouped_dgrad_kernel<kMode>, dim3((unsigned)grid), dim3(kGemmThreads), 0,
                       stream, g);
  else if (wide)
    hipLaunchKernelGGL(grouped_gemm_fwd_kernel<kMode>, dim3((unsigned)grid), dim3(kGemmThreads),
                       0, stream, g);
  else
    hipLaunchKernelGGL(grouped_gemm_fwd_shortk_kernel<kMode>, dim3((unsigned)grid),
                       dim3(kGemmThreads), 0, stream, g);
  return launch_status();
}

template <bool kMx, bool kGlu = false>
static int forward_entry(const uint16_t* x, int32_t rows, int32_t K, int64_t x_stride,
                         const uint8_t* codes, const void* scl, int32_t E, int32_t N,
                         int32_t topk, const float* pair_scale, const int32_t* offsets,
                         const int32_t* sorted_pairs, const int32_t* tiles,
                         const int32_t* num_tiles, int32_t max_tiles, int32_t tile_m,
                         uint16_t* out, hipStream_t stream) {
  if (rows < 0 || topk < 1 || E < 1 || N < 1 || N % (kGlu ? 64 : 32) || K <= 0 ||
      K % (kMx ? 32 : 64))
    return kInvalid;
  if (x_stride < K || x_stride % 8) return kInvalid;
  if (tile_m != kTM) return kNotSupported;
  const int64_t P = (int64_t)rows * topk;
  if (P >= INT32_MAX) return kNotSupported;
  if (P == 0) return kOk;                                  // nothing to enqueue
  int st = common_gemm_checks(x, rows, x_stride, K, codes, scl, offsets, sorted_pairs, tiles,
                              num_tiles, out);
  if (st != kOk) return st;
  if (!kMx && !aligned4(scl)) return kInvalid;
  if (pair_scale && !aligned4(pair_scale)) return kInvalid;
  GemmArgs g{};
  g.x = x; g.x_stride = x_stride; g.codes = codes; g.scl = scl;
  g.Nw = N; g.Kw = K; g.Kc = K; g.Nout = kGlu ? N / 2 : N;
  g.E = E; g.topk = topk; g.P = (int)P; g.pair_scale = pair_scale;
  g.offsets = offsets; g.sorted_pairs = sorted_pairs; g.tiles = tiles; g.num_tiles = num_tiles;
  g.out = out;
  if constexpr (kGlu) return launch_gemm<kFwdNF4Glu>(g, max_tiles, tile_m, stream);
  else return launch_gemm<kMx ? kFwdMX : kFwdNF4>(g, max_tiles, tile_m, stream);
}

}  // namespace gq

extern "C" int gq_nf4_grouped_gemm(const uint16_t* x, int32_t rows, int32_t K, int64_t x_stride,
                                   const uint8_t* codes, const float* absmax, int32_t num_experts,
                                   int32_t N, int32_t topk, const float* pair_scale,
                                   const int32_t* expert_offsets, const int32_t* sorted_pairs,
                                   const int32_t* tiles, const int32_t* num_tiles,
                                   int32_t max_tiles, int32_t tile_m, uint16_t* out,
                                   hipStream_t stream) {
  return gq::forward_entry<false>(x, rows, K, x_stride, codes, absmax, num_experts, N, topk,
                                  pair_scale, expert_offsets, sorted_pairs, tiles, num_tiles,
                                  max_tiles, tile_m, out, stream);
}

extern "C" int gq_nf4_grouped_gemm_swiglu(const uint16_t* x, int32_t rows, int32_t K,
                                          int64_t x_stride, const uint8_t* codes,
                                          const float* absmax, int32_t num_experts, int32_t N,
                                          int32_t topk, const int32_t* expert_offsets,
                                          const int32_t* sorted_pairs, const int32_t* tiles,
                                          const int32_t* num_tiles, int32_t max_tiles,
                                          int32_t tile_m, uint16_t* act, hipStream_t stream) {
  return gq::forward_entry<false, true>(x, rows, K, x_stride, codes, absmax, num_experts, N, topk,
                                        nullptr, expert_offsets, sorted_pairs, tiles, num_tiles,
                                        max_tiles, tile_m, act, stream);
}

extern "C" int gq_mxfp4_grouped_gemm(const uint16_t* x, int32_t rows, int32_t K,
                                     int64_t x_stride, const uint8_t* blocks,
                                     const uint8_t* scales, int32_t num_experts, int32_t N,
                                     int32_t topk, const float* pair_scale,
                                     const int32_t* expert_offsets, const int32_t* sorted_pairs,
                                     const int32_t* tiles, const int32_t* num_tiles,
                                     int32_t max_tiles, int32_t tile_m, uint16_t* out,
                                     hipStream_t stream) {
  return gq::forward_entry<true>(x, rows, K, x_stride, blocks, scales, num_experts, N, topk,
                                 pair_scale, expert_offsets, sorted_pairs, tiles, num_tiles,
                                 max_tiles, tile_m, out, stream);
}

namespace gq {

template <bool kMx>
static int dgrad_entry(const uint16_t* dy, int32_t P, int32_t N, int64_t dy_stride,
                       const uint8_t* codes, const void* scl, int32_t E, int32_t K,
                       const int32_t* offsets, const int32_t* sorted_pairs, const int32_t* tiles,
                       const int32_t* num_tiles, int32_t max_tiles, int32_t tile_m, uint16_t* dx,
                       hipStream_t stream) {
  if (P < 0 || E < 1 || N < 1 || N % 64 || K <= 0 || K % (kMx ? 32 : 64)) return kInvalid;
  if (dy_stride < N || dy_stride % 8) return kInvalid;
  if (tile_m != kTM) return kNotSupported;
  if (P == 0) return kOk;                                  // nothing to enqueue
  int st = common_gemm_checks(dy, P, dy_stride, N, codes, scl, offsets, sorted_pairs, tiles,
                              num_tiles, dx);
  if (st != kOk) return st;
  if (!kMx && !aligned4(scl)) return kInvalid;
  GemmArgs g{};
  g.x = dy; g.x_stride = dy_stride; g.codes = codes; g.scl = scl;
  g.Nw = N; g.Kw = K; g.Kc = N; g.Nout = K;
  g.E = E; g.topk = 1; g.P = P; g.pair_scale = nullptr;
  g.offsets = offsets; g.sorted_pairs = sorted_pairs; g.tiles = tiles;
  g.num_tiles = num_tiles; g.out = dx;
  return launch_gemm<kMx ? kDgradMX : kDgradNF4>(g, max_tiles, tile_m, stream);
}

}  // namespace gq

extern "C" int gq_nf4_grouped_dgrad(const uint16_t* dy, int32_t P, int32_t N, int64_t dy_stride,
                                    const uint8_t* codes, const float* absmax,
                                    int32_t num_experts, int32_t K,
                                    const int32_t* expert_offsets, const int32_t* sorted_pairs,
                                    const int32_t* tiles, const int32_t* num_tiles,
                                    int32_t max_tiles, int32_t tile_m, uint16_t* dx,
                                    hipStream_t stream) {
  return gq::dgrad_entry<false>(dy, P, N, dy_stride, codes, absmax, num_experts, K,
                                expert_offsets, sorted_pairs, tiles, num_tiles, max_tiles, tile_m,
                                dx, stream);
}

extern "C" int gq_mxfp4_grouped_dgrad(const uint16_t* dy, int32_t P, int32_t N, int64_t dy_stride,
                                      const uint8_t* blocks, const uint8_t* scales,
                                      int32_t num_experts, int32_t K,
                                      const int32_t* expert_offsets, const int32_t* sorted_pairs,
                                      const int32_t* tiles, const int32_t* num_tiles,
                                      int32_t max_tiles, int32_t tile_m, uint16_t* dx,
                                      hipStream_t stream) {
  return gq::dgrad_entry<true>(dy, P, N, dy_stride, blocks, scales, num_experts, K,
                               expert_offsets, sorted_pairs, tiles, num_tiles, max_tiles, tile_m,
                               dx, stream);
}
