// fg_e4m3.hpp -- device-side OCP E4M3 encoding shared by the quantisers and
// the fused GEMM epilogue, so that both produce the same codes and scales.
//
// Per 1x128 or 128x128 block (the 2kiu.com DeepGEMM explainer, section 4.4:
// scales from the data's statistics, out-of-range values saturated; the
// zwzgs.cn DeepGEMM page, "Features > fine-grained scaling"): scale =
// amax / 448 (1 for an all-zero block), optionally rounded up to a power of
// two (the MX / micro-scaling block scales of the explainer's section 7);
// code = nearest E4M3 of clamp(x / scale, -448, 448), ties to the even code,
// sign kept.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fg {

constexpr float kE4M3Max = 448.0f;

// Nearest E4M3 code of y (|y| <= 448, finite), ties to the even code; the
// sign bit is copied from y.
__device__ __forceinline__ uint32_t e4m3_rne(float y) {
  const uint32_t bits = __float_as_uint(y);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const float a = __uint_as_float(bits & 0x7fffffffu);
  uint32_t mag;
  if (a < 0.015625f) {
    // below the smallest normal 2^-6 the codes 0..8 are the multiples
    // c * 2^-9; a * 512 is exact, rintf rounds half to even
    mag = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    // keep 3 mantissa bits: round the fp32 significand at bit 20, half to even
    uint32_t u = bits & 0x7fffffffu;
    u += 0x7ffffu + ((u >> 20) & 1u);
    const uint32_t e = (u >> 23) - 127u + 7u;  // E4M3 exponent field (1..15)
    mag = (e << 3) | ((u >> 20) & 7u);
  }
  return sign | mag;
}

__device__ __forceinline__ float block_scale(float amax) {
  return amax == 0.0f ? 1.0f : amax / kE4M3Max;   // IEEE division
}

// The smallest power of two >= s (s positive, finite), and at least 2^-126.
// A normal s with a zero mantissa is already one; otherwise clear the
// mantissa and step the exponent up (a subnormal s has exponent field 0 and
// becomes 2^-126).
__device__ __forceinline__ float pow2_up(float s) {
  const uint32_t u = __float_as_uint(s);
  const uint32_t e = u & 0x7f800000u;
  if (e != 0u && (u & 0x007fffffu) == 0u) return s;
  return __uint_as_float(e + 0x00800000u);
}

// Code of x in a block with scale s: x / s (IEEE division), saturated.
__device__ __forceinline__ uint32_t e4m3_scaled(float x, float s) {
  return e4m3_rne(fminf(fmaxf(x / s, -kE4M3Max), kE4M3Max));
}

}  // namespace fg
