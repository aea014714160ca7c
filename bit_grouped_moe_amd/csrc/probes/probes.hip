// Measurement controls for the benchmark: an empty launch and a coalesced
// streaming read.  Declared in include/gq_probes.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../../include/gq_probes.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kPerThread = 16;

__global__ void empty_kernel() {}

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

extern "C" int gq_probe_stream_read(const void* buf, int64_t bytes, uint32_t* sink,
                                    hipStream_t stream) {
  if (!buf || !sink || bytes <= 0 || bytes % 16 || (reinterpret_cast<uintptr_t>(buf) & 15u))
    return (int)hipErrorInvalidValue;
  const int64_t n16 = bytes / 16;
  const int64_t blocks = (n16 + (int64_t)kThreads * kPerThread - 1) / ((int64_t)kThreads * kPerThread);
  if (blocks > INT32_MAX) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                     static_cast<const u32x4*>(buf), n16, sink);
  return (int)hipGetLastError();
}
