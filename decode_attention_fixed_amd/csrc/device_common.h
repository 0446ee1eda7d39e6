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

// cos / sin of the RoPE angle pos * theta_i of one pair (theta_i =
// base^(-2i/d), computed once on the host in float64).  The angle is formed
// in float64 and reduced modulo 2 pi with a two-part 2 pi (Cody and Waite)
// before the float64 sincos, which then stays on its short-argument path.
// Every kernel that rotates a row takes its angles from here, so rows
// written by different entry points are bit-identical.
__device__ __forceinline__ void rope_sincos(double pos, double theta, double* s, double* c) {
  constexpr double kTwoPiHi = 6.283185307179586232;       // 2 pi rounded to float64
  constexpr double kTwoPiLo = 2.4492935982947064e-16;     // 2 pi - kTwoPiHi
  constexpr double kInvTwoPi = 0.15915494309189533577;
  const double a = pos * theta;
  const double k = rint(a * kInvTwoPi);
  double r = fma(-k, kTwoPiHi, a);
  r = fma(-k, kTwoPiLo, r);
  sincos(r, s, c);
}

// Rotation of one RoPE pair (x0, x1) by the angle with cosine c and sine s,
// in float64 with explicit fused multiply-adds (no contraction choice is left
// to the compiler, so every kernel computes the same bits).
__device__ __forceinline__ void rope_rotate_pair(double x0, double x1, double c, double s,
                                                 double* o0, double* o1) {
  *o0 = fma(x0, c, -(x1 * s));
  *o1 = fma(x0, s, x1 * c);
}

// int8 rows ([kvc] §5.1: INT8 cache).  A wave quantises one row of d values:
// lane l < d/2 holds the row's elements e0 and e1 (a RoPE pair) as float64.
//   a = max |x|,  s = float32(a / 127),  c = clamp(rint(x / s), -127, 127)
// (s = 0 gives codes 0).  Every lane of the wave calls it; it returns s and
// the lane's two codes (exact integers in float64).  Every kernel that
// stores an int8 row takes its codes from here, so rows written by different
// entry points are bit-identical.
__device__ __forceinline__ float quantize_pair_row(double x0, double x1, bool active, double* c0,
                                                   double* c1) {
  double a = active ? fmax(fabs(x0), fabs(x1)) : 0.0;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) a = fmax(a, __shfl_xor(a, o));
  const float s = static_cast<float>(a / 127.0);
  const double sd = static_cast<double>(s);
  *c0 = 0.0;
  *c1 = 0.0;
  if (active && sd > 0.0) {
    *c0 = fmin(fmax(rint(x0 / sd), -127.0), 127.0);
    *c1 = fmin(fmax(rint(x1 / sd), -127.0), 127.0);
  }
  return s;
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
