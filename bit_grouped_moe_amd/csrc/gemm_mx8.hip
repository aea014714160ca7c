// MXFP4 prefill grouped GEMM on the gfx950 block-scaled matrix instruction
// (v_mfma_scale_f32_32x32x64_f8f6f4): the e2m1 weight codes and their e8m0
// scales go from memory straight into the instruction's fp4 operand, with
// no decode; the activations go in as a two-term e4m3 split.
//
// Pages: "Receipts-driven engineering", opening summary (MXFP4 as OCP e2m1
// on a checkpoint's released bytes, decoded inside the mainloop) and
// "grouped-nf4-gemm 0.43.0", "Which entry point?" (native MXFP4 expert
// math); the MXFP4 inference record "How do I run MoE expert inference
// natively on MXFP4 (e2m1 + e8m0) weights ...", summary.  The pages keep
// activations in bf16 (weights-only 4-bit); the fp4 instruction takes its
// other operand in an MX format, so each bf16 activation is written as
// hi * 2^Xh + lo * 2^Xl (two e4m3 terms, each with an e8m0 scale per 32 of a
// row, the second holding the first's rounding residual): close to bf16
// precision, and the product stays within the bf16 path's tolerance.
//
// Operand layout of the instruction (32 x 32 x 64, measured on the device):
//  * fp4 operand: lane (c, h) = (lane % 32, lane / 32) holds column c's
//    32-element K block h as 16 bytes, element 2j in the low nibble of byte
//    j -- exactly one stored MXFP4 block -- and the e8m0 byte of that block
//    as its scale;
//  * e4m3 operand: lane (m, h) holds row m's elements 16 h + [0, 16) of K
//    block 0 in bytes 0..15 and of K block 1 in bytes 16..31; the scale of
//    (row m, block b) comes from lane m + 32 b.
// The split kernel below writes the activations in exactly that order, so
// an activation row of a 64-K step is one 128-byte piece (hi 64 B, lo 64 B)
// staged like the bf16 kernel's activation tile.
#include <type_traits>
#include <utility>

#include "gemm_common.hpp"
#include "../../include/gq.h"

namespace gq {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// ---- two-term e4m3 split of bf16 activations --------------------------------
// Kp = K rounded up to 64.  codes [rows, 2 Kp] bytes: per row and 64-K step
// s, 128 bytes: hi codes [0, 64), lo codes [64, 128); in each 64, lane half
// h's 32 bytes at 32 h: elements 16 h + [0, 16) of block 2s, then of block
// 2s + 1.  scales [rows, Kp / 16] bytes: per step s_hi(2s), s_lo(2s),
// s_hi(2s+1), s_lo(2s+1).  A block past K (K % 64 == 32) is written as
// zeros with scale byte 0.
//
// Block exponent X: the smallest integer with amax * 2^-X <= 448 (the
// largest e4m3 magnitude), clamped to [-127, 127]; -127 for an all-zero
// block.  For amax = 1.f * 2^E (normal): X = E - 8, plus 1 when 1.f > 1.75.
__device__ __forceinline__ int split_exponent(float amax) {
  const uint32_t b = __float_as_uint(amax);
  if (b == 0u) return -127;
  const int e = (int)(b >> 23);
  const int X = e - 135 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return max(-127, min(127, X));
}

// e4m3 codes of v[i] * 2^-X (round to nearest even; |v * 2^-X| <= 448 by the
// choice of X), packed 4 per dword in element order; also returns the
// values the codes represent, times 2^X.
__device__ __forceinline__ void split_term(const float (&v)[32], int X, uint32_t (&q)[8],
                                           float (&back)[32]) {
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    const float a0 = __builtin_amdgcn_ldexpf(v[4 * d], -X);
    const float a1 = __builtin_amdgcn_ldexpf(v[4 * d + 1], -X);
    const float a2 = __builtin_amdgcn_ldexpf(v[4 * d + 2], -X);
    const float a3 = __builtin_amdgcn_ldexpf(v[4 * d + 3], -X);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(a2, a3, w, true);
    q[d] = (uint32_t)w;
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
    back[4 * d] = __builtin_amdgcn_ldexpf(lo.x, X);
    back[4 * d + 1] = __builtin_amdgcn_ldexpf(lo.y, X);
    back[4 * d + 2] = __builtin_amdgcn_ldexpf(hi.x, X);
    back[4 * d + 3] = __builtin_amdgcn_ldexpf(hi.y, X);
  }
}

__global__ __launch_bounds__(256) void act_split_kernel(const uint16_t* __restrict__ x,
                                                        int64_t rows, int K, int64_t x_stride,
                                                        int Kp, uint8_t* __restrict__ q,
                                                        uint8_t* __restrict__ sc) {
  const int nb = Kp / 32;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;     // one 32-block
  if (t >= rows * nb) return;
  const int64_t r = t / nb;
  const int b = (int)(t - r * nb);
  const int s = b >> 1, j = b & 1;
  uint32_t qh[8], ql[8];
  uint32_t sbytes = 0u;
  if (b * 32 < K) {
    const u32x4* xp = reinterpret_cast<const u32x4*>(x + r * x_stride + b * 32);
    float v[32];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4 w = xp[c];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[8 * c + 2 * k] = bf16lo_to_f32(w[k]);
        v[8 * c + 2 * k + 1] = bf16hi_to_f32(w[k]);
      }
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const int Xh = split_exponent(amax);
    float back[32];
    split_term(v, Xh, qh, back);
    float rmax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      v[i] = v[i] - back[i];                                     // exact residual
      rmax = fmaxf(rmax, fabsf(v[i]));
    }
    const int Xl = split_exponent(rmax);
    split_term(v, Xl, ql, back);
    sbytes = (uint32_t)(Xh + 127) | ((uint32_t)(Xl + 127) << 8);
  } else {
#pragma unroll
    for (int d = 0; d < 8; ++d) qh[d] = ql[d] = 0u;
  }
  uint8_t* qrow = q + r * (2 * (int64_t)Kp) + (int64_t)s * 128;
  // elements [0, 16) of the block belong to lane half 0, [16, 32) to half 1
  *reinterpret_cast<u32x4*>(qrow + 16 * j) = u32x4{qh[0], qh[1], qh[2], qh[3]};
  *reinterpret_cast<u32x4*>(qrow + 32 + 16 * j) = u32x4{qh[4], qh[5], qh[6], qh[7]};
  *reinterpret_cast<u32x4*>(qrow + 64 + 16 * j) = u32x4{ql[0], ql[1], ql[2], ql[3]};
  *reinterpret_cast<u32x4*>(qrow + 96 + 16 * j) = u32x4{ql[4], ql[5], ql[6], ql[7]};
  *reinterpret_cast<uint16_t*>(sc + r * (int64_t)(Kp / 16) + s * 4 + 2 * j) = (uint16_t)sbytes;
}

// The gated unit of one output row's 32-column block, written as its split
// (the activation epilogue with kSplit).  The block is the two transposed
// accumulator blocks v0, v1 (32 interleaved gate/up weight rows each) of a
// row: after the exchanges of store_block_act, lane half h holds the bf16
// results of block columns 8h + [0, 8) (from v0) and 16 + 8h + [0, 8) (from
// v1); the two halves' maxima are exchanged once per term, and each lane
// converts its 16 values exactly as act_split_kernel converts them (so the
// bytes equal those of the bf16 output split afterwards).  qrow: the row's
// 128 code bytes of the block's 64-K step; blk: the block's index within it.
__device__ __forceinline__ void store_block_act_split(const float (&v0)[16], const float (&v1)[16],
                                                      uint8_t* qrow, uint8_t* srow, int blk,
                                                      int lh, float alpha, float limit) {
  float y[16];                                             // this lane's 16 block values
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const float (&v)[16] = cb ? v1 : v0;
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      o[q] = pack_bf16x2(oss_act(v[4 * q], v[4 * q + 1], alpha, limit),
                         oss_act(v[4 * q + 2], v[4 * q + 3], alpha, limit));
    const auto a = __builtin_amdgcn_permlane32_swap(o[0], o[2], false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(o[1], o[3], false, false);
    const uint32_t w[4] = {a[0], a[1], b[0], b[1]};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      y[8 * cb + 2 * k] = bf16lo_to_f32(w[k]);
      y[8 * cb + 2 * k + 1] = bf16hi_to_f32(w[k]);
    }
  }
  // the block maximum over both lane halves (lanes l and l ^ 32)
  auto block_max = [&](const float (&u)[16]) {
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(u[i]));
    // one element of the result is this lane's own value, the other its
    // partner's (which is which depends on the lane half)
    const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m),
                                                    false, false);
    return fmaxf(__uint_as_float(x[0]), __uint_as_float(x[1]));
  };
  // e4m3 codes of u * 2^-X (4 dwords, element order) and the residual
  auto term = [&](float (&u)[16], int X, uint32_t (&q)[4]) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(u[4 * d], -X),
                                              __builtin_amdgcn_ldexpf(u[4 * d + 1], -X), 0,
                                              false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(u[4 * d + 2], -X),
                                          __builtin_amdgcn_ldexpf(u[4 * d + 3], -X), w, true);
      q[d] = (uint32_t)w;
      const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
      const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
      u[4 * d] -= __builtin_amdgcn_ldexpf(lo.x, X);
      u[4 * d + 1] -= __builtin_amdgcn_ldexpf(lo.y, X);
      u[4 * d + 2] -= __builtin_amdgcn_ldexpf(hi.x, X);
      u[4 * d + 3] -= __builtin_amdgcn_ldexpf(hi.y, X);
    }
  };
  uint32_t qh[4], ql[4];
  const int Xh = split_exponent(block_max(y));
  term(y, Xh, qh);                                         // y is now the exact residual
  const int Xl = split_exponent(block_max(y));
  term(y, Xl, ql);
  // elements [0, 16) at byte 16 blk, [16, 32) at 32 + 16 blk; lo codes + 64
  const int o0 = 16 * blk + 8 * lh, o1 = 32 + 16 * blk + 8 * lh;
  *reinterpret_cast<uint2*>(qrow + o0) = uint2{qh[0], qh[1]};
  *reinterpret_cast<uint2*>(qrow + o1) = uint2{qh[2], qh[3]};
  *reinterpret_cast<uint2*>(qrow + 64 + o0) = uint2{ql[0], ql[1]};
  *reinterpret_cast<uint2*>(qrow + 64 + o1) = uint2{ql[2], ql[3]};
  if (lh == 0)
    *reinterpret_cast<uint16_t*>(srow + 2 * blk) =
        (uint16_t)((uint32_t)(Xh + 127) | ((uint32_t)(Xl + 127) << 8));
}

// ---- the grouped GEMM: 256 pairs x 256 columns per workgroup ----------------
// One wave per SIMD; wave w owns the columns n0 + 64 w + [0, 64) (two
// column blocks of 32) for every 32-row sub-tile of the tile (4 or 8
// sub-tiles as in the bf16 kernel), so each weight byte is loaded by exactly
// one lane, straight into the operand registers.  Per 64-K step a wave
// issues (active sub-tiles) x 2 column blocks x 2 terms instructions.  The
// activation codes (128 bytes per row and step, 16-byte chunks XOR-swizzled
// by (row >> 1) & 7 for conflict-free reads) and their scale dwords go from
// global memory straight into LDS (double-buffered, one barrier per step);
// the weight codes and scales load two steps ahead into registers.
// (Measured on gpt-oss gate_up: the same kernel on 128-row half tiles, two
// workgroups per CU, is slower -- 400 vs 362 us -- because every half tile
// loads the whole weight slice again.)
constexpr int kMx8Rows = 128;                              // tiles up to here: 4 sub-tiles

// End of a K step: wait until at most the newest kBLoads vector-memory
// instructions (the next-but-one step's weight loads, issued last) are
// outstanding and every LDS read has returned, then a workgroup barrier.
// The wait is the s_waitcnt builtin, which the compiler's own wait
// insertion takes into account (so it adds no full wait before the next
// step's LDS reads); empty asm statements with a memory clobber keep every
// memory access on its side of the barrier, and no fence forces a wait for
// the weight loads that may stay in flight.
constexpr int kBLoads = 4;                                 // 2 x 16 code bytes + 2 scale bytes
__device__ __forceinline__ void step_barrier() {
  asm volatile("" ::: "memory");
  // s_waitcnt vmcnt(kBLoads) expcnt(7) lgkmcnt(0)
  __builtin_amdgcn_s_waitcnt(kBLoads | (7 << 4) | (0 << 8));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int kSub, bool kAct, bool kSplit>
__device__ __forceinline__ void mx8_columns(const GemmArgs& g, const TileInfo& t, int tid,
                                            uint8_t* A0, uint8_t* A1, uint32_t* S0, uint32_t* S1,
                                            int* pair_s, int* row_s, float* scale_s) {
  const int nsteps = (g.Kc + kTK - 1) / kTK;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int lr = lane & 31, lh = lane >> 5;
  const int valid = t.valid;
  // weight rows of the tile: t.n0 counts output columns, two weight rows
  // (gate, up) per output column with the activation epilogue
  const int wn0 = kAct ? 2 * t.n0 : t.n0;
  const int jcol = wn0 + 64 * wave + lr;
  // K tail (K % 64 == 32): lane half 1 has no weights in the last step; it
  // re-reads half 0 (in bounds) against the zero activations of the pad.
  auto load = [&](int ks) {
    const bool full = ks * kTK + kTK <= g.Kw;
    return n_load<kFwdMX8>(g, t.e, jcol, ks, full ? lh : 0);
  };
  NLoad X = load(0), Y = load(min(1, nsteps - 1));
  // the row's pair weight goes to LDS after the main loop (as in the bf16
  // kernel: the prologue barrier then does not wait for its dependent load)
  float psc;
  {
    int p = g.sorted_pairs[t.start + min(tid, valid - 1)];
    p = ((unsigned)p < (unsigned)g.P) ? p : 0;
    pair_s[tid] = p;
    row_s[tid] = p / g.topk;
    psc = g.pair_scale ? g.pair_scale[p] : 1.f;
  }
  lds_barrier();

  auto arow = [&](int j) { return kSub == 4 ? 32 * wave + 8 * j : 8 * (4 * j + wave); };
  const uint32_t row_bytes = (uint32_t)(g.x_stride * 2);
  uint32_t voff[kSub];
#pragma unroll
  for (int j = 0; j < kSub; ++j) {
    const int R = arow(j) + (lane >> 3);
    const int c = (lane & 7) ^ ((R >> 1) & 7);
    voff[j] = (uint32_t)row_s[R] * row_bytes + 16u * (uint32_t)c;
  }
  const uint32_t soff = (uint32_t)row_s[tid] * (uint32_t)g.xs_stride;
  auto dma = [&](int ks, uint8_t* Adst, uint32_t* Sdst) {
    const char* xb = reinterpret_cast<const char*>(g.x) + (size_t)ks * 128;
#pragma unroll
    for (int j = 0; j < kSub; ++j) {
      if (arow(j) < valid)                                 // groups past the segment: skipped
        __builtin_amdgcn_global_load_lds((glb_void_t*)(xb + voff[j]),
                                         (lds_void_t*)(Adst + arow(j) * 128), 16, 0, 0);
    }
    if (64 * wave < valid)
      __builtin_amdgcn_global_load_lds((glb_void_t*)(g.xs + soff + (size_t)ks * 4),
                                       (lds_void_t*)(Sdst + 64 * wave), 4, 0, 0);
  };
  const int aslot_x = (lr >> 1) & 7;
  // e4m3 operand of sub-tile i, term t (0: hi codes in chunks 2 lh, 2 lh + 1;
  // 1: lo codes in chunks 4 + 2 lh, 5 + 2 lh) of row 32 i + lr
  auto read_a = [&](const uint8_t* A, int i, int term) -> i32x8 {
    const uint8_t* row = A + (32 * i + lr) * 128;
    const u32x4 c0 = *reinterpret_cast<const u32x4*>(row + 16 * ((4 * term + 2 * lh) ^ aslot_x));
    const u32x4 c1 =
        *reinterpret_cast<const u32x4*>(row + 16 * ((4 * term + 2 * lh + 1) ^ aslot_x));
    return i32x8{(int)c0[0], (int)c0[1], (int)c0[2], (int)c0[3],
                 (int)c1[0], (int)c1[1], (int)c1[2], (int)c1[3]};
  };

  f32x16 acc[kSub][2];
#pragma unroll
  for (int i = 0; i < kSub; ++i)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][c][r] = 0.f;
  const int nrows = (valid + 31) / 32;                     // active sub-tiles (all waves)
  const bool allcols =
      __builtin_amdgcn_readfirstlane((jcol < g.Nw && jcol + 32 < g.Nw) ? 1 : 0) != 0;
  const bool anycol = __builtin_amdgcn_readfirstlane(jcol < g.Nw ? 1 : 0) != 0;

  dma(0, A0, S0);
  __builtin_amdgcn_s_waitcnt(0);
  lds_barrier();

  auto run_loop = [&](auto rows_c) {
    constexpr int kRows = decltype(rows_c)::value;         // -1: guarded generic path
    // Step ks: the activation tile of step ks + 1 goes into the other LDS
    // buffer and the weight codes of step ks + 2 into registers while the
    // instructions of step ks run.  The step ends with a wait for everything
    // but the newest weight loads (kBLoads instructions, issued last) and a
    // barrier: the next step's tile is then in LDS for every wave, and every
    // wave has finished reading this step's buffer before it is refilled.
    auto step = [&](int ks, const uint8_t* Ac, const uint32_t* Sc, uint8_t* An, uint32_t* Sn,
                    const NLoad& Lc, NLoad& Ln) {
      dma(min(ks + 1, nsteps - 1), An, Sn);
      __builtin_amdgcn_sched_barrier(0);                   // the tile loads first
      Ln = load(min(ks + 2, nsteps - 1));
      __builtin_amdgcn_sched_barrier(0);                   // then the weight loads
      const i32x8 b0{(int)Lc.c[0][0], (int)Lc.c[0][1], (int)Lc.c[0][2], (int)Lc.c[0][3], 0, 0, 0, 0};
      const i32x8 b1{(int)Lc.c[1][0], (int)Lc.c[1][1], (int)Lc.c[1][2], (int)Lc.c[1][3], 0, 0, 0, 0};
      const int sb0 = (int)Lc.s[0], sb1 = (int)Lc.s[1];
      // Units u = (term, sub-tile): the hi terms of all active sub-tiles,
      // then the lo terms, so that 2 x (active sub-tiles) independent
      // instructions separate two uses of an accumulator.  A unit's fragment
      // is read two units ahead (a ring of three), and the reads are placed
      // between the instructions of earlier units.
      constexpr int kN = kRows > 0 ? kRows : kSub;         // sub-tiles in the sequence
      constexpr int kU = 2 * kN;
      uint32_t sw[kSub];
#pragma unroll
      for (int i = 0; i < kSub; ++i)
        if (kRows >= 0 ? i < kRows : i < nrows) sw[i] = Sc[32 * i + lr] >> (16 * lh);
      const bool run = kRows >= 0 || anycol;
      auto live = [&](int u) { return kRows >= 0 || (u % kN) < nrows; };
      i32x8 f[3];
#pragma unroll
      for (int u = 0; u < 2 && u < kU; ++u)
        if (live(u)) f[u] = read_a(Ac, u % kN, u / kN);
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        if (u + 2 < kU && live(u + 2)) f[(u + 2) % 3] = read_a(Ac, (u + 2) % kN, (u + 2) / kN);
        const int i = u % kN, term = u / kN;
        if (run && live(u)) {
          const int sa = (int)(term ? sw[i] >> 8 : sw[i]);
          acc[i][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b0, f[u % 3], acc[i][0], 4, 0,
                                                                      0, sb0, 0, sa);
          acc[i][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b1, f[u % 3], acc[i][1], 4, 0,
                                                                      0, sb1, 0, sa);
        }
      }
      if constexpr (kRows > 0) {
        // first two fragments and the scales, then per unit: its two
        // instructions and the reads of the unit two ahead
        __builtin_amdgcn_sched_group_barrier(0x100, 4 + kRows, 0);
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          if (u + 2 < kU) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
      }
      step_barrier();
    };
    // the weight registers rotate X (step ks) <- Y (ks + 1) <- Z (ks + 2)
    NLoad Z;
    for (int ks = 0; ks < nsteps; ks += 2) {
      step(ks, A0, S0, A1, S1, X, Z);
      X = Y;
      Y = Z;
      if (ks + 1 < nsteps) {
        step(ks + 1, A1, S1, A0, S0, X, Z);
        X = Y;
        Y = Z;
      }
    }
  };
  // loop variants by active sub-tiles (1..4 on 128-row tiles, 5..8 on
  // 256-row tiles) with all columns valid; else the guarded generic loop
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

  if constexpr (kSplit) {
    // the wave's 32 output columns are one split block of each row
    const int col = t.n0 + 32 * wave;                      // output column (Nout % 64 == 0)
#pragma unroll
    for (int i = 0; i < kSub; ++i) {
      if (i >= nrows) continue;
      const int m = 32 * i + lr;
      const int p = pair_s[m];
      if (m < valid && col < g.Nout) {
        float v0[16], v1[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          v0[r] = acc[i][0][r];
          v1[r] = acc[i][1][r];
        }
        store_block_act_split(v0, v1, g.out_q + (int64_t)p * (2 * g.Nout) + 2 * (col & ~63),
                              g.out_s + (int64_t)p * (g.Nout / 16) + (col & ~63) / 16,
                              (col >> 5) & 1, lh, g.act_alpha, g.act_limit);
      }
    }
  } else if constexpr (kAct) {
#pragma unroll
    for (int i = 0; i < kSub; ++i) {
      if (i >= nrows) continue;
      const int m = 32 * i + lr;
      const int p = pair_s[m];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const int col = t.n0 + 32 * wave + 16 * cb;         // output column (Nout % 16 == 0)
        if (m < valid && col < g.Nout) {
          float v[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) v[r] = acc[i][cb][r];
          store_block_act(v, g.out + (int64_t)p * g.Nout + col, lh, g.act_alpha, g.act_limit);
        }
      }
    }
  } else {
    store_wide_rows<kSub>(acc, nrows, valid, pair_s, scale_s, g, t.n0, wave, lr, lh);
  }
}

// kAct: gate_up product with the gpt-oss gated unit applied in the epilogue
// (weight rows 2j, 2j + 1 -> output column j of an [P, N/2] result); kSplit:
// that result written as its two-term e4m3 split (the next product's input).
template <bool kAct, bool kSplit = false>
__global__ __launch_bounds__(kGemmThreads, 1) void grouped_gemm_mx8_kernel(GemmArgs g) {
  // separate arrays: an LDS-direct load into one buffer does not alias reads
  // of the other
  __shared__ __attribute__((aligned(16))) uint8_t A0[kTM * 128];
  __shared__ __attribute__((aligned(16))) uint8_t A1[kTM * 128];
  __shared__ __attribute__((aligned(16))) uint32_t S0[kTM];
  __shared__ __attribute__((aligned(16))) uint32_t S1[kTM];
  __shared__ int pair_s[kTM];                              // pair of each tile row
  __shared__ int row_s[kTM];                               // its activation row (pair / topk)
  __shared__ float scale_s[kTM];                           // its pair weight (1 if none)
  const int tid = threadIdx.x;
  TileInfo t;
  if (!tile_head<kAct ? kXN / 2 : kXN, kSplit>(g, tid, t)) return;
  if (t.valid <= kMx8Rows)
    mx8_columns<4, kAct, kSplit>(g, t, tid, A0, A1, S0, S1, pair_s, row_s, scale_s);
  else
    mx8_columns<8, kAct, kSplit>(g, t, tid, A0, A1, S0, S1, pair_s, row_s, scale_s);
}

static inline int64_t split_kp(int64_t K) { return (K + kTK - 1) / kTK * kTK; }

}  // namespace gq

extern "C" int gq_act_split_e4m3(const uint16_t* x, int32_t rows, int32_t K, int64_t x_stride,
                                 uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  using namespace gq;
  if (rows < 0 || K <= 0 || K % 32 || x_stride < K || x_stride % 8) return kInvalid;
  if (rows == 0) return kOk;
  if (!x || !codes || !scales || !aligned16(x) || !aligned16(codes) || !aligned4(scales))
    return kInvalid;
  const int64_t Kp = split_kp(K);
  const int64_t threads = (int64_t)rows * (Kp / 32);
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > INT32_MAX) return kNotSupported;
  hipLaunchKernelGGL(act_split_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x,
                     (int64_t)rows, K, x_stride, (int)Kp, codes, scales);
  return launch_status();
}

namespace gq {

// kSplit (with kAct): the result goes to out_q / out_s as its split instead
// of to out.
template <bool kAct, bool kSplit = false>
static int mx8_entry(const uint8_t* x_codes, const uint8_t* x_scales, int32_t rows, int32_t K,
                     const uint8_t* blocks, const uint8_t* scales, int32_t num_experts, int32_t N,
                     int32_t topk, const float* pair_scale, float alpha, float limit,
                     const int32_t* expert_offsets, const int32_t* sorted_pairs,
                     const int32_t* tiles, const int32_t* num_tiles, int32_t max_tiles,
                     int32_t tile_m, uint16_t* out, hipStream_t stream, uint8_t* out_q = nullptr,
                     uint8_t* out_s = nullptr) {
  if (rows < 0 || topk < 1 || num_experts < 1 || N < 1 || N % 32 || K <= 0 || K % 32)
    return kInvalid;
  if (kSplit && N % 128) return kNotSupported;             // whole 64-column split steps
  if (kAct && !(limit >= 0.f && limit < 3.4e38f && alpha == alpha && alpha > -3.4e38f &&
                alpha < 3.4e38f))
    return kInvalid;                                       // finite alpha, limit >= 0
  if (tile_m != kTM) return kNotSupported;
  const int64_t P = (int64_t)rows * topk;
  if (P >= INT32_MAX) return kNotSupported;
  if (P == 0) return kOk;                                  // nothing to enqueue
  const int64_t Kp = split_kp(K);
  if ((int64_t)rows * 2 * Kp >= INT32_MAX) return kNotSupported;   // 32-bit row offsets
  if (!x_codes || !x_scales || !blocks || !scales || !expert_offsets || !sorted_pairs || !tiles ||
      !num_tiles)
    return kInvalid;
  if (kSplit ? (!out_q || !out_s || !aligned16(out_q) || !aligned4(out_s))
             : (!out || !aligned16(out)))
    return kInvalid;
  if (!aligned16(x_codes) || !aligned4(x_scales) || !aligned16(blocks)) return kInvalid;
  if (!aligned4(expert_offsets) || !aligned4(sorted_pairs) || !aligned4(tiles) ||
      !aligned4(num_tiles) || (pair_scale && !aligned4(pair_scale)))
    return kInvalid;
  const int64_t need = (P + kTM - 1) / kTM + num_experts + 1;
  if (max_tiles < need) return kInvalid;
  GemmArgs g{};
  g.x = reinterpret_cast<const uint16_t*>(x_codes);
  g.x_stride = Kp;                                         // 2 Kp bytes per row
  g.xs = x_scales;
  g.xs_stride = Kp / 16;
  g.codes = blocks; g.scl = scales;
  g.Nw = N; g.Kw = K; g.Kc = K; g.Nout = kAct ? N / 2 : N;
  g.E = num_experts; g.topk = topk; g.P = (int)P; g.pair_scale = pair_scale;
  g.offsets = expert_offsets; g.sorted_pairs = sorted_pairs; g.tiles = tiles;
  g.num_tiles = num_tiles; g.out = out;
  g.act_alpha = alpha; g.act_limit = limit;
  g.out_q = out_q; g.out_s = out_s;
  g.n_col_tiles = (N + kXN - 1) / kXN;                     // 256 weight rows per tile
  const int64_t n_logical = (int64_t)max_tiles * g.n_col_tiles;
  const int64_t group = 8LL * g.n_col_tiles;
  const int64_t grid = ((n_logical + group - 1) / group) * group;
  if (grid > INT32_MAX) return kNotSupported;
  g.n_logical = (int)n_logical;
  hipLaunchKernelGGL((grouped_gemm_mx8_kernel<kAct, kSplit>), dim3((unsigned)grid),
                     dim3(kGemmThreads), 0, stream, g);
  return launch_status();
}

}  // namespace gq

extern "C" int gq_mxfp4_grouped_gemm_scaled(const uint8_t* x_codes, const uint8_t* x_scales,
                                            int32_t rows, int32_t K, const uint8_t* blocks,
                                            const uint8_t* scales, int32_t num_experts, int32_t N,
                                            int32_t topk, const float* pair_scale,
                                            const int32_t* expert_offsets,
                                            const int32_t* sorted_pairs, const int32_t* tiles,
                                            const int32_t* num_tiles, int32_t max_tiles,
                                            int32_t tile_m, uint16_t* out, hipStream_t stream) {
  return gq::mx8_entry<false>(x_codes, x_scales, rows, K, blocks, scales, num_experts, N, topk,
                              pair_scale, 0.f, 0.f, expert_offsets, sorted_pairs, tiles,
                              num_tiles, max_tiles, tile_m, out, stream);
}

extern "C" int gq_mxfp4_grouped_gemm_scaled_swiglu(
    const uint8_t* x_codes, const uint8_t* x_scales, int32_t rows, int32_t K,
    const uint8_t* blocks, const uint8_t* scales, int32_t num_experts, int32_t N, int32_t topk,
    float alpha, float limit, const int32_t* expert_offsets, const int32_t* sorted_pairs,
    const int32_t* tiles, const int32_t* num_tiles, int32_t max_tiles, int32_t tile_m,
    uint16_t* act, hipStream_t stream) {
  return gq::mx8_entry<true>(x_codes, x_scales, rows, K, blocks, scales, num_experts, N, topk,
                             nullptr, alpha, limit, expert_offsets, sorted_pairs, tiles,
                             num_tiles, max_tiles, tile_m, act, stream);
}

extern "C" int gq_mxfp4_grouped_gemm_scaled_swiglu_split(
    const uint8_t* x_codes, const uint8_t* x_scales, int32_t rows, int32_t K,
    const uint8_t* blocks, const uint8_t* scales, int32_t num_experts, int32_t N, int32_t topk,
    float alpha, float limit, const int32_t* expert_offsets, const int32_t* sorted_pairs,
    const int32_t* tiles, const int32_t* num_tiles, int32_t max_tiles, int32_t tile_m,
    uint8_t* act_codes, uint8_t* act_scales, hipStream_t stream) {
  return gq::mx8_entry<true, true>(x_codes, x_scales, rows, K, blocks, scales, num_experts, N,
                                   topk, nullptr, alpha, limit, expert_offsets, sorted_pairs,
                                   tiles, num_tiles, max_tiles, tile_m, nullptr, stream,
                                   act_codes, act_scales);
}
