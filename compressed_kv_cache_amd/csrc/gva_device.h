// Device-side helpers shared by the libgva kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gva {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bfloat16 stored as its 16-bit pattern.
typedef uint16_t bf16_t;

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// float -> bf16, round to nearest, ties to even; NaN stays a (quiet) NaN,
// magnitudes past the largest bf16 round to infinity.
__device__ __forceinline__ bf16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

// double -> bf16 with a single round-to-nearest-even.  The double is first
// narrowed to float with round-to-odd (truncate, then set the last bit when
// anything was dropped); float keeps 16 more bits than bf16, so the second
// rounding cannot create a false tie (Boldo & Melquiond, "Emulation of FMA
// and correctly rounded sums: proved algorithms using rounding to odd").
__device__ __forceinline__ bf16_t f64_to_bf16_rne(double x) {
  if (x != x) return static_cast<bf16_t>(0x7fc0u);
  float t = __double2float_rz(x);
  uint32_t u = __float_as_uint(t);
  if (static_cast<double>(t) != x && (u & 0x7f800000u) != 0x7f800000u) u |= 1u;
  return f32_to_bf16_rne(__uint_as_float(u));
}

template <typename CT> struct Cache;
template <> struct Cache<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ float from_f32(float x) { return x; }
  static __device__ __forceinline__ float from_f64(double x) { return static_cast<float>(x); }
};
template <> struct Cache<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ bf16_t from_f32(float x) { return f32_to_bf16_rne(x); }
  static __device__ __forceinline__ bf16_t from_f64(double x) { return f64_to_bf16_rne(x); }
};

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace gva
