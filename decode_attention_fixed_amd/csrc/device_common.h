// Device helpers shared by the HIP kernels: bf16 <-> f32, exact f64 -> bf16
// rounding, 16-byte vector access.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swa {

// bf16 halves of a 32-bit word -> f32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// f32 -> bf16, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// f64 -> bf16, round to nearest, ties to even, without double rounding:
// first round to float32 with round-to-odd (truncate, then set the last bit
// if anything was lost), then round that to bf16.  Round-to-odd into a
// format with at least two more bits than the target makes the second
// rounding exact (Boldo and Melquiond, "Emulation of FMA and correctly
// rounded sums: proved algorithms using rounding to odd", 2008).
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double x) {
  float f = static_cast<float>(x);  // nearest
  uint32_t u = __float_as_uint(f);
  const double back = static_cast<double>(f);
  if (fabs(back) > fabs(x)) u -= 1u;          // one step toward zero: truncation
  if (static_cast<double>(__uint_as_float(u)) != x) u |= 1u;  // inexact: make odd
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

struct alignas(16) Vec16 {
  uint32_t w[4];
};

__device__ __forceinline__ Vec16 load16(const void* p) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  Vec16 r;
  r.w[0] = v.x;
  r.w[1] = v.y;
  r.w[2] = v.z;
  r.w[3] = v.w;
  return r;
}

__device__ __forceinline__ void store16(void* p, const Vec16& r) {
  *reinterpret_cast<uint4*>(p) = make_uint4(r.w[0], r.w[1], r.w[2], r.w[3]);
}

}  // namespace swa
