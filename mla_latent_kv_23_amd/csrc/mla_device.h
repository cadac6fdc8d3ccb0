// Device-side helpers shared by the libmla kernels: storage conversions
// (bf16, OCP E4M3FN) and the RoPE rotation rule.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla.h"

namespace mla {

// Largest supported d_rope (the host passes one inverse frequency per pair).
constexpr int kMaxRopePairs = 64;

// Inverse RoPE frequencies base^(-2i/d_rope), formed on the host in float64
// and passed by value to the kernels that rotate.
struct RopeFreqs {
  double inv_freq[kMaxRopePairs];
};

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Logistic output gate sigma(g) = 1 / (1 + e^-g) in float32: 0 for g -> -inf
// (e^-g overflows to inf), 1 for g -> +inf.
__device__ __forceinline__ float sigmoid_f32(float g) { return 1.0f / (1.0f + expf(-g)); }

// float32 -> bf16, round to nearest even; NaN stays NaN (quiet bit set).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// OCP E4M3FN: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits, no infinity,
// largest finite magnitude 448.  Round to nearest even, saturating at 448.
__device__ __forceinline__ uint8_t f32_to_e4m3fn(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  float a = fminf(fabsf(v), 448.0f);
  uint32_t mag;
  if (a < 0.015625f) {                       // below 2^-6: subnormal grid of 2^-9
    mag = static_cast<uint32_t>(rintf(a * 512.0f));   // 8 -> the smallest normal code
  } else {
    int e;
    float f = frexpf(a, &e);                 // a = f * 2^e, f in [0.5, 1)
    float m = rintf((f * 2.0f - 1.0f) * 8.0f);   // mantissa in eighths, exact scaling
    int ef = e - 1 + 7;
    uint32_t mi = static_cast<uint32_t>(m);
    if (mi == 8u) { mi = 0u; ef += 1; }
    mag = (static_cast<uint32_t>(ef) << 3) | mi;
  }
  return static_cast<uint8_t>(sign | mag);
}

__device__ __forceinline__ float e4m3fn_to_f32(uint8_t c) {
  const int e = (c >> 3) & 0xF, m = c & 0x7;
  float v = (e == 0) ? ldexpf(static_cast<float>(m), -9) : ldexpf(static_cast<float>(8 + m), e - 10);
  return (c & 0x80) ? -v : v;
}

// cos/sin of pos * inv_freq, angle in float64, results rounded to float32.
__device__ __forceinline__ void rope_cos_sin(int32_t pos, double inv_freq, float* c, float* s) {
  double sn, cs;
  sincos(static_cast<double>(pos) * inv_freq, &sn, &cs);
  *c = static_cast<float>(cs);
  *s = static_cast<float>(sn);
}

// Rotate one pair; inputs are exact float32 values, products are exact in
// float64, the sums are rounded once to float64, then to float32.
__device__ __forceinline__ void rope_pair(float x, float y, float c, float s, float* ox, float* oy) {
  const double dx = x, dy = y, dc = c, ds = s;
  *ox = static_cast<float>(dx * dc - dy * ds);
  *oy = static_cast<float>(dx * ds + dy * dc);
}

// Activation element access for the two activation dtypes.
template <typename T> struct Act;
template <> struct Act<float> {
  static __device__ __forceinline__ float ld(const float* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ void st(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Act<uint16_t> {
  static __device__ __forceinline__ float ld(const uint16_t* p, int64_t i) { return bf16_bits_to_f32(p[i]); }
  static __device__ __forceinline__ void st(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16_bits(v); }
};

}  // namespace mla
