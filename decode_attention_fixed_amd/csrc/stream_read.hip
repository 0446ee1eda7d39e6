// Reads a device buffer once, as fast as the chip allows: the achievable HBM
// read rate, against which the decode kernels' fractions of the 8 TB/s peak
// can be read.  No page defines it; it is a measuring aid of the library.
//
// Workgroup w streams its own contiguous share of 16-byte units with
// nontemporal loads, kUnroll loads in flight per thread; the XOR of what a
// wave read goes to sink[w * kWaves + wave] so that no load can be dropped.
// Workgroup w runs on XCD w mod 8, and the even XCDs stream faster: shares
// of 17/16 of an equal one on even w and 15/16 on odd w read 4 GiB ~1.3%
// faster than equal shares (7.12 against 7.03 TB/s, in one run), the same
// weights as the paged decode's balanced grid.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "swa_internal.h"

namespace swa {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kUnroll = 8;
static_assert(kStreamReadGrid * kWaves * sizeof(uint32_t) == kStreamReadSinkBytes,
              "one sink word per wave");

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4_t* src, size_t units,
                                                               uint32_t* sink) {
  auto start = [&](size_t w) {  // first unit of workgroup w's share
    return (16 * w + (w & 1)) * units / (16 * static_cast<size_t>(gridDim.x));
  };
  const size_t u0 = start(blockIdx.x);
  const size_t u1 = blockIdx.x + 1 == gridDim.x ? units : start(blockIdx.x + 1);
  uint32_t acc = 0;
  size_t u = u0 + threadIdx.x;
  for (; u + static_cast<size_t>(kUnroll - 1) * kThreads < u1; u += kUnroll * kThreads) {
    u32x4_t v[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) v[k] = __builtin_nontemporal_load(src + u + k * kThreads);
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (; u < u1; u += kThreads) {
    const u32x4_t v = __builtin_nontemporal_load(src + u);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * kWaves + (threadIdx.x >> 6)] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream) {
  const size_t units = bytes / 16;
  stream_read_kernel<<<kStreamReadGrid, kThreads, 0, stream>>>(static_cast<const u32x4_t*>(src),
                                                              units, sink);
  return hipGetLastError();
}

}  // namespace swa
