// Device-side building blocks shared by the libgq kernels (gfx950, wave64).
//
// Decode routines live here once so that the decode probes and the matmul
// kernels run the same code:
//  * NF4 (pages: "Receipts-driven engineering", opening summary -- 16-entry
//    normal-float codebook, bitsandbytes packed layout; "grouped-nf4-gemm
//    0.43.0", "Try the packers and byte checks on CPU" -- one float32
//    absmax per 64 weights): weight = float32(codebook[code] * absmax).
//    The codebook is read from a 16-entry table in LDS; 16 consecutive
//    dwords sit in 16 distinct banks, so every lookup is conflict-free
//    (lanes that hit the same bank read the same address).
//  * MXFP4 (same summary -- OCP e2m1 codes; e8m0 block scales): the gfx950
//    hardware converter turns two e2m1 codes into exact float32 / bf16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gq {

constexpr int kWave = 64;

// NF4 data type of QLoRA (Dettmers et al. 2023) as float32 bit patterns,
// index = 4-bit code.
__device__ constexpr uint32_t kNF4Bits[16] = {
    0xBF800000u, 0xBF3239B1u, 0xBF066B30u, 0xBECA32A0u, 0xBE91A24Du, 0xBE3D353Fu,
    0xBDBA7871u, 0x00000000u, 0x3DA2FAFFu, 0x3E24CAE3u, 0x3E7C04DDu, 0x3EAD033Au,
    0x3EE1A4B8u, 0x3F1007ABu, 0x3F3913B3u, 0x3F800000u};

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Fill a 16-entry float LUT in LDS with the NF4 codebook (threads 0..15).
// The value is selected from immediates rather than loaded from memory, so
// the LDS write never waits on (in-order) global loads issued before it.
__device__ __forceinline__ void nf4_lut_init(float* lut, int tid) {
  uint32_t v = 0u;
#pragma unroll
  for (int i = 0; i < 16; ++i) v = (tid == i) ? kNF4Bits[i] : v;
  if (tid < 16) lut[tid] = __uint_as_float(v);
}

// OCP e2m1 magnitudes (codes 0..7) as float32 bit patterns; bit 3 of a code
// is the sign.
__device__ constexpr uint32_t kE2M1Bits[8] = {0x00000000u, 0x3F000000u, 0x3F800000u,
                                              0x3FC00000u, 0x40000000u, 0x40400000u,
                                              0x40800000u, 0x40C00000u};

// Fill a 16-entry float LUT in LDS with the e2m1 values (threads 0..15),
// selected from immediates like nf4_lut_init.  Code 8 is -0.
__device__ __forceinline__ void e2m1_lut_init(float* lut, int tid) {
  uint32_t v = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) v = ((tid & 7) == i) ? kE2M1Bits[i] : v;
  if (tid < 16) lut[tid] = __uint_as_float(v | ((tid & 8) ? 0x80000000u : 0u));
}

// bf16 bit pattern of x, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  __bf16 b = (__bf16)x;
  return __builtin_bit_cast(uint16_t, b);
}

// Two floats -> packed bf16 pair (lo in bits 0..15), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// bf16 bits (low / high half of a dword) -> float, exact.
__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---- NF4 -----------------------------------------------------------------
// Byte j of a row holds element 2j in its high nibble, 2j+1 in its low one.
// nf4_q_hi/lo return the (unscaled) codebook value of byte `byte_idx` of
// dword `d`.
__device__ __forceinline__ float nf4_q_hi(const float* lut, uint32_t d, int byte_idx) {
  return lut[(d >> (8 * byte_idx + 4)) & 15u];
}
__device__ __forceinline__ float nf4_q_lo(const float* lut, uint32_t d, int byte_idx) {
  return lut[(d >> (8 * byte_idx)) & 15u];
}

// NF4 codebook values of the 8 weights of one code dword, in element order.
// Addressing costs 1.25 ops per weight: the nibbles are first spread into
// bytes already multiplied by 4 (byte offsets into the 16-float LDS table),
// then each lookup extracts one byte.
__device__ __forceinline__ void nf4_lookup8(const float* lut, uint32_t d, float q[8]) {
  uint32_t hi4 = (d >> 2) & 0x3C3C3C3Cu;           // byte j: 4 * code of element 2j
  uint32_t lo4 = (d << 2) & 0x3C3C3C3Cu;           // byte j: 4 * code of element 2j+1
  // Opaque to the optimizer: otherwise it folds the spread back into a shift
  // and a mask per lookup (two ops) instead of one byte extract.
  asm("" : "+v"(hi4), "+v"(lo4));
  const char* base = reinterpret_cast<const char*>(lut);
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    q[2 * b] = *reinterpret_cast<const float*>(base + __builtin_amdgcn_ubfe(hi4, 8 * b, 8));
    q[2 * b + 1] = *reinterpret_cast<const float*>(base + __builtin_amdgcn_ubfe(lo4, 8 * b, 8));
  }
}

// Decode the 8 weights of one dword of NF4 codes to bf16 pairs (element
// order preserved: out[i] holds elements 2i (low half) and 2i+1 (high half)).
// weight = float32(q * absmax), then bf16 RNE.
__device__ __forceinline__ void nf4_decode8_bf16(const float* lut, uint32_t d, float absmax,
                                                 uint32_t out[4]) {
  float q[8];
  nf4_lookup8(lut, d, q);
#pragma unroll
  for (int b = 0; b < 4; ++b) out[b] = pack_bf16x2(q[2 * b] * absmax, q[2 * b + 1] * absmax);
}

// 256-entry table of codebook value pairs indexed by a code byte: entry b
// holds {value of the high nibble (element 2j), value of the low nibble
// (element 2j+1)}.  One 8-byte LDS read yields both weights of a byte; with
// the table at LDS address 0 its byte offset (b << 3) is a single shift.
__device__ __forceinline__ void nf4_pairs_init(f32x2* tab, int t) {
  uint32_t hi = 0u, lo = 0u;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    hi = ((t >> 4) == i) ? kNF4Bits[i] : hi;
    lo = ((t & 15) == i) ? kNF4Bits[i] : lo;
  }
  if (t < 256) tab[t] = f32x2{__uint_as_float(hi), __uint_as_float(lo)};
}

// NF4 codebook values of the 8 weights of one code dword, in element order,
// from the pair table.
__device__ __forceinline__ void nf4_pairs8(const f32x2* tab, uint32_t d, float q[8]) {
  const char* base = reinterpret_cast<const char*>(tab);
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const f32x2 v =
        *reinterpret_cast<const f32x2*>(base + (__builtin_amdgcn_ubfe(d, 8 * b, 8) << 3));
    q[2 * b] = v.x;
    q[2 * b + 1] = v.y;
  }
}

// sigmoid(z) = 1 / (1 + e^-z) in float32 from the hardware base-2
// exponential and reciprocal (e^-z = 2^(-z log2 e); about 1 ulp each, so a
// few ulp of float32 in all): the gated units sit at the end of short,
// latency-bound kernels, where the correctly rounded expf and division
// sequences cost ~0.9 us on the one-token gpt-oss gate_up GEMV.  Large |z|
// gives exactly 0 or 1.
__device__ __forceinline__ float sigmoid_f32(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * 1.44269504088896341f));
}

// SiLU, z * sigmoid(z), in float32.
__device__ __forceinline__ float silu_f32(float z) { return z * sigmoid_f32(z); }

// ---- MXFP4 ---------------------------------------------------------------
// Byte j of a 16-byte block holds element 2j in its low nibble, 2j+1 in its
// high nibble.  e2m1 -> float32 is exact; the e8m0 factor 2^(s-127) is then
// applied with ldexp (exact, denormals kept); s == 255 is NaN.
__device__ __forceinline__ f32x2 e2m1_pair_f32(uint32_t d, int byte_idx) {
  switch (byte_idx) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 3);
  }
}

__device__ __forceinline__ float e8m0_apply(float v, uint32_t s) {
  float r = __builtin_amdgcn_ldexpf(v, (int)s - 127);
  return s == 255u ? __uint_as_float(0x7FC00000u) : r;
}

// Two e2m1 codes of byte `byte_idx` straight to a bf16 pair with the e8m0
// factor folded in by the converter (exact for every scale the
// representable range allows; checked bit for bit by the decode probe).
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  // 2^(s-127): s in 1..254 is a normal float; s == 0 is the subnormal 2^-127.
  uint32_t bits = (s == 0u) ? 0x00400000u : (s << 23);
  return __uint_as_float(s == 255u ? 0x7FC00000u : bits);
}

__device__ __forceinline__ uint32_t e2m1_pair_bf16_scaled(uint32_t d, int byte_idx, float scale) {
  bf16x2 v;
  switch (byte_idx) {
    case 0: v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 0); break;
    case 1: v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 1); break;
    case 2: v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 2); break;
    default: v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 3); break;
  }
  return __builtin_bit_cast(uint32_t, v);
}

// ---- wave / block helpers ---------------------------------------------------
// Workgroup barrier that orders LDS only.  __syncthreads() fences every
// address space, which makes each wave wait for ALL of its outstanding
// global loads (s_waitcnt vmcnt(0)) at every barrier and defeats prefetching.
// The kernels here exchange data between threads through LDS only, so an
// LDS-scoped release/acquire around s_barrier is sufficient.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// v from lane (lane pattern kCtrl) through a DPP move; rows (16 lanes) not in
// kRowMask read 0.
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, kRowMask, 0xF, false));
}

// Sum over aligned groups of `width` lanes (a power of two, 1..64) with DPP
// lane moves only (no LDS traffic, no waits), in a fixed order.  The last
// lane of each group receives the group total (width <= 16: every lane).
//   quad_perm [1,0,3,2], [2,3,0,1]: pairs, then quads
//   row_half_mirror, row_mirror: 8 and 16 lanes
//   row_bcast:15 into rows 1 and 3, row_bcast:31 into row 3: 32 and 64 lanes
__device__ __forceinline__ float group_sum_last(float v, int width) {
  if (width >= 2) v += dpp_f32<0xB1>(v);
  if (width >= 4) v += dpp_f32<0x4E>(v);
  if (width >= 8) v += dpp_f32<0x141>(v);
  if (width >= 16) v += dpp_f32<0x140>(v);
  if (width >= 32) v += dpp_f32<0x142, 0xA>(v);
  if (width >= 64) v += dpp_f32<0x143, 0x8>(v);
  return v;
}

__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

}  // namespace gq
