// Decode probes: write packed weights out as float32 and/or bf16 with the
// same device decode routines the matmul kernels use, so the decoding can
// be compared bit for bit.  Packed shapes follow "grouped-nf4-gemm 0.43.0",
// section "Try the packers and byte checks on CPU"; the codebooks follow
// "Receipts-driven engineering", opening summary.  Not on the hot path.
#include "gq_device.hpp"
#include "gq_host.hpp"
#include "../../include/gq.h"

namespace gq {

constexpr int kDecodeThreads = 256;

// One thread per dword of codes (8 weights).
__global__ __launch_bounds__(kDecodeThreads) void nf4_decode_kernel(
    const uint32_t* __restrict__ codes, const float* __restrict__ absmax, int64_t n_dwords,
    int K, float* __restrict__ out_f32, uint32_t* __restrict__ out_bf16) {
  __shared__ float lut[16];
  nf4_lut_init(lut, threadIdx.x);
  __syncthreads();
  const int64_t i = (int64_t)blockIdx.x * kDecodeThreads + threadIdx.x;
  if (i >= n_dwords) return;
  const int dw_per_row = K / 8;
  const int64_t row = i / dw_per_row;
  const int col8 = (int)(i - row * dw_per_row);          // weights col8*8 .. +8
  const uint32_t d = codes[i];
  const float a = absmax[row * (K / 64) + col8 / 8];
  if (out_f32) {
    float w[8];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      w[2 * b] = nf4_q_hi(lut, d, b) * a;
      w[2 * b + 1] = nf4_q_lo(lut, d, b) * a;
    }
    f32x4* o = reinterpret_cast<f32x4*>(out_f32 + i * 8);
    o[0] = f32x4{w[0], w[1], w[2], w[3]};
    o[1] = f32x4{w[4], w[5], w[6], w[7]};
  }
  if (out_bf16) {
    uint32_t p[4];
    nf4_decode8_bf16(lut, d, a, p);
    reinterpret_cast<u32x4*>(out_bf16)[i] = u32x4{p[0], p[1], p[2], p[3]};
  }
}

__global__ __launch_bounds__(kDecodeThreads) void mxfp4_decode_kernel(
    const uint32_t* __restrict__ blocks, const uint8_t* __restrict__ scales, int64_t n_dwords,
    float* __restrict__ out_f32, uint32_t* __restrict__ out_bf16) {
  const int64_t i = (int64_t)blockIdx.x * kDecodeThreads + threadIdx.x;
  if (i >= n_dwords) return;
  const uint32_t d = blocks[i];
  const uint32_t s = scales[i / 4];                     // 4 dwords per 32-block
  if (out_f32) {
    float w[8];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      f32x2 v = e2m1_pair_f32(d, b);
      w[2 * b] = e8m0_apply(v.x, s);
      w[2 * b + 1] = e8m0_apply(v.y, s);
    }
    f32x4* o = reinterpret_cast<f32x4*>(out_f32 + i * 8);
    o[0] = f32x4{w[0], w[1], w[2], w[3]};
    o[1] = f32x4{w[4], w[5], w[6], w[7]};
  }
  if (out_bf16) {
    const float sc = e8m0_to_f32(s);
    uint32_t p[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) p[b] = e2m1_pair_bf16_scaled(d, b, sc);
    reinterpret_cast<u32x4*>(out_bf16)[i] = u32x4{p[0], p[1], p[2], p[3]};
  }
}

}  // namespace gq

static int decode_common_checks(const void* a, const void* b, int64_t n_rows, int32_t K,
                                int block, const void* f32, const void* bf16) {
  using namespace gq;
  if (!a || !b || (!f32 && !bf16)) return kInvalid;
  if (n_rows < 0 || K <= 0 || K % block) return kInvalid;
  if (!aligned4(a) || (f32 && !aligned16(f32)) || (bf16 && !aligned16(bf16))) return kInvalid;
  if (n_rows > (INT64_MAX / K)) return kNotSupported;
  return kOk;
}

extern "C" int gq_nf4_decode(const uint8_t* codes, const float* absmax, int64_t n_rows,
                             int32_t K, float* out_f32, uint16_t* out_bf16, hipStream_t stream) {
  using namespace gq;
  int st = decode_common_checks(codes, absmax, n_rows, K, 64, out_f32, out_bf16);
  if (st != kOk) return st;
  if (!aligned4(absmax)) return kInvalid;
  const int64_t n_dwords = n_rows * (K / 8);
  if (n_dwords == 0) return kOk;
  const int64_t grid = ceil_div64(n_dwords, kDecodeThreads);
  if (grid > INT32_MAX) return kNotSupported;
  hipLaunchKernelGGL(nf4_decode_kernel, dim3((unsigned)grid), dim3(kDecodeThreads), 0, stream,
                     reinterpret_cast<const uint32_t*>(codes), absmax, n_dwords, K, out_f32,
                     reinterpret_cast<uint32_t*>(out_bf16));
  return launch_status();
}

extern "C" int gq_mxfp4_decode(const uint8_t* blocks, const uint8_t* scales, int64_t n_rows,
                               int32_t K, float* out_f32, uint16_t* out_bf16,
                               hipStream_t stream) {
  using namespace gq;
  int st = decode_common_checks(blocks, scales, n_rows, K, 32, out_f32, out_bf16);
  if (st != kOk) return st;
  const int64_t n_dwords = n_rows * (K / 8);
  if (n_dwords == 0) return kOk;
  const int64_t grid = ceil_div64(n_dwords, kDecodeThreads);
  if (grid > INT32_MAX) return kNotSupported;
  hipLaunchKernelGGL(mxfp4_decode_kernel, dim3((unsigned)grid), dim3(kDecodeThreads), 0, stream,
                     reinterpret_cast<const uint32_t*>(blocks), scales, n_dwords, out_f32,
                     reinterpret_cast<uint32_t*>(out_bf16));
  return launch_status();
}

extern "C" const char* gq_status_string(int status) {
  switch (status) {
    case 0: return "gq: success";
    case (int)hipErrorInvalidValue: return "gq: invalid argument (hipErrorInvalidValue)";
    case (int)hipErrorNotSupported: return "gq: not supported (hipErrorNotSupported)";
    default: return "gq: HIP launch error";
  }
}
