// Device-side position bookkeeping: pos[i] += delta, so that a captured HIP
// graph of decode steps replays with every step at the next position.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "swa_internal.h"

namespace swa {
namespace {

__global__ void add_i32_kernel(int32_t* dst, size_t n, int32_t delta) {
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x) {
    const int64_t v = static_cast<int64_t>(dst[i]) + delta;
    dst[i] = static_cast<int32_t>(v > INT32_MAX ? INT32_MAX : (v < INT32_MIN ? INT32_MIN : v));
  }
}

}  // namespace

hipError_t launch_add_i32(int32_t* dst, size_t n, int32_t delta, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256;
  const unsigned grid = static_cast<unsigned>(blocks < 4096 ? blocks : 4096);
  add_i32_kernel<<<grid, 256, 0, stream>>>(dst, n, delta);
  return hipGetLastError();
}

}  // namespace swa
