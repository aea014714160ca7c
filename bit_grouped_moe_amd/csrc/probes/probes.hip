// Measurement controls for the benchmark: an empty launch, a coalesced
// streaming read, a plain copy and matrix-instruction issue-rate loops.
// Declared in include/gq_probes.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../../include/gq_probes.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
constexpr int kThreads = 256;

__global__ void empty_kernel() {}

template <int kPerThread>
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ p,
                                                               int64_t n16,
                                                               uint32_t* __restrict__ sink) {
  const int64_t base = (int64_t)blockIdx.x * kThreads * kPerThread + threadIdx.x;
  u32x4 v[kPerThread];
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int64_t j = base + (int64_t)i * kThreads;
    v[i] = p[j < n16 ? j : n16 - 1];                     // unconditional, clamped
  }
  u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) acc ^= v[i];
  const uint32_t r = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (r == 0x9E3779B9u) sink[0] = r;
}

__global__ __launch_bounds__(kThreads) void copy_kernel(const u32x4* __restrict__ src,
                                                        u32x4* __restrict__ dst, int64_t n16) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < n16) dst[i] = src[i];
}

// ---- matrix-instruction rate loops ----
// Each wave keeps kAcc independent 32 x 32 accumulators and issues kAcc
// matrix instructions per iteration, cycling through kSets operand sets of
// random (finite) values so the data toggles as in a real GEMM.
constexpr int kAcc = 8;
constexpr int kSets = 4;

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16; x *= 0x7FEB352Du; x ^= x >> 15; x *= 0x846CA68Bu; x ^= x >> 16;
  return x;
}

// kind: 0 bf16 32x32x16; 1 scaled 32x32x64 e4m3 x e2m1; 2 e2m1 x e2m1;
// 3 e4m3 x e4m3 (scale operands = 1.0, e8m0 byte 127)
template <int kKind>
__global__ __launch_bounds__(kThreads) void mfma_rate_kernel(int64_t iters, uint32_t* sink) {
  const uint32_t seed = (blockIdx.x * kThreads + threadIdx.x) * 2654435761u;
  i32x8 a[kSets], b[kSets];
#pragma unroll
  for (int s = 0; s < kSets; ++s)
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      uint32_t u = mix32(seed + 97u * (uint32_t)(s * 8 + r));
      uint32_t v = mix32(u ^ 0x5bd1e995u);
      if constexpr (kKind == 0) {              // bf16 pairs, exponents near 1
        u = (u & 0x807F807Fu) | 0x3F003F00u;
        v = (v & 0x807F807Fu) | 0x3F003F00u;
      } else {                                 // e4m3 without NaN codes; e2m1 any
        if constexpr (kKind == 1 || kKind == 3) u &= 0xFEFEFEFEu;
        if constexpr (kKind == 3) v &= 0xFEFEFEFEu;
      }
      a[s][r] = (int)u;
      b[s][r] = (int)v;
    }
  f32x16 acc[kAcc];
#pragma unroll
  for (int i = 0; i < kAcc; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
  // iterations in groups of kSets so every operand index is static
  for (int64_t it = 0; it < iters; it += kSets) {
#pragma unroll
    for (int j = 0; j < kSets; ++j)
#pragma unroll
    for (int i = 0; i < kAcc; ++i) {
      const i32x8& A = a[i % kSets];
      const i32x8& B = b[(i + j) % kSets];
      if constexpr (kKind == 0) {
        typedef int i32x4 __attribute__((ext_vector_type(4)));
        const i32x4 a4{A[0], A[1], A[2], A[3]}, b4{B[0], B[1], B[2], B[3]};
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a4),
                                                         __builtin_bit_cast(bf16x8, b4), acc[i],
                                                         0, 0, 0);
      } else if constexpr (kKind == 1) {
        acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, acc[i], 0, 4, 0, 0x7F7F7F7F,
                                                                 0, 0x7F7F7F7F);
      } else if constexpr (kKind == 2) {
        acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, acc[i], 4, 4, 0, 0x7F7F7F7F,
                                                                 0, 0x7F7F7F7F);
      } else {
        acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, acc[i], 0, 0, 0, 0x7F7F7F7F,
                                                                 0, 0x7F7F7F7F);
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kAcc; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[i][r];
  if (__float_as_uint(s) == 0x9E3779B9u) sink[0] = 1u;
}

}  // namespace

extern "C" int gq_probe_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream) {
  if (!src || !dst || bytes <= 0 || bytes % 16 || (reinterpret_cast<uintptr_t>(src) & 15u) ||
      (reinterpret_cast<uintptr_t>(dst) & 15u))
    return (int)hipErrorInvalidValue;
  const int64_t n16 = bytes / 16;
  const int64_t blocks = (n16 + kThreads - 1) / kThreads;
  if (blocks > INT32_MAX) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16);
  return (int)hipGetLastError();
}

extern "C" int gq_probe_empty(hipStream_t stream) {
  hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, stream);
  return (int)hipGetLastError();
}

extern "C" int gq_probe_stream_read(const void* buf, int64_t bytes, int32_t loads_per_thread,
                                    uint32_t* sink, hipStream_t stream) {
  if (!buf || !sink || bytes <= 0 || bytes % 16 || (reinterpret_cast<uintptr_t>(buf) & 15u))
    return (int)hipErrorInvalidValue;
  const int L = loads_per_thread;
  if (L != 1 && L != 2 && L != 4 && L != 8 && L != 16) return (int)hipErrorInvalidValue;
  const int64_t n16 = bytes / 16;
  const int64_t blocks = (n16 + (int64_t)kThreads * L - 1) / ((int64_t)kThreads * L);
  if (blocks > INT32_MAX) return (int)hipErrorInvalidValue;
  const u32x4* p = static_cast<const u32x4*>(buf);
  const dim3 grid((unsigned)blocks);
  switch (L) {
    case 1: hipLaunchKernelGGL(stream_read_kernel<1>, grid, dim3(kThreads), 0, stream, p, n16, sink); break;
    case 2: hipLaunchKernelGGL(stream_read_kernel<2>, grid, dim3(kThreads), 0, stream, p, n16, sink); break;
    case 4: hipLaunchKernelGGL(stream_read_kernel<4>, grid, dim3(kThreads), 0, stream, p, n16, sink); break;
    case 8: hipLaunchKernelGGL(stream_read_kernel<8>, grid, dim3(kThreads), 0, stream, p, n16, sink); break;
    default: hipLaunchKernelGGL(stream_read_kernel<16>, grid, dim3(kThreads), 0, stream, p, n16, sink); break;
  }
  return (int)hipGetLastError();
}

extern "C" int64_t gq_probe_mfma_flops(int32_t kind) {
  switch (kind) {
    case 0: return 2LL * 32 * 32 * 16;
    case 1: case 2: case 3: return 2LL * 32 * 32 * 64;
    default: return -1;
  }
}

extern "C" int gq_probe_mfma(int32_t kind, int64_t iters, int32_t blocks, uint32_t* sink,
                             hipStream_t stream) {
  if (!sink || iters < 1 || iters % 4 || blocks < 1 || kind < 0 || kind > 3)
    return (int)hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks);
  switch (kind) {
    case 0: hipLaunchKernelGGL(mfma_rate_kernel<0>, grid, dim3(kThreads), 0, stream, iters, sink); break;
    case 1: hipLaunchKernelGGL(mfma_rate_kernel<1>, grid, dim3(kThreads), 0, stream, iters, sink); break;
    case 2: hipLaunchKernelGGL(mfma_rate_kernel<2>, grid, dim3(kThreads), 0, stream, iters, sink); break;
    default: hipLaunchKernelGGL(mfma_rate_kernel<3>, grid, dim3(kThreads), 0, stream, iters, sink); break;
  }
  return (int)hipGetLastError();
}

extern "C" int32_t gq_probe_mfma_per_wave_iter(void) { return kAcc; }
