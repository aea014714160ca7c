// Host-side argument checks shared by the libgq entry points.  Every check
// runs before anything is enqueued; a failed check returns
// hipErrorInvalidValue (malformed) or hipErrorNotSupported (well-formed but
// outside the kernels' supported range), following the native C-ABI error
// convention of the GPTQModel wiki page "NF12".
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gq {

constexpr int kOk = 0;
constexpr int kInvalid = (int)hipErrorInvalidValue;
constexpr int kNotSupported = (int)hipErrorNotSupported;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? kOk : (int)e;
}

inline int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace gq
