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

// Nearest E4M3 codes, ties to the even code, sign kept (so -tiny -> 0x80),
// for finite inputs with |y| <= 448: gfx950's v_cvt_pk_fp8_f32 (OCP E4M3).
// On every finite fp32 value in that range it gives the same byte as a
// software round-to-nearest-even encoder (the E4M3 significand rounded at
// fp32 bit 20, and the subnormal codes as multiples of 2^-9) -- checked
// exhaustively on the device, all 2^32 bit patterns. Codes of y0, y1 land in
// bytes 0, 1 (HI = false) or 2, 3 (HI = true) of the result; the other half
// is kept from `old`.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3_pk(float y0, float y1, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, (int)old, HI);
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

__device__ __forceinline__ float sat448(float y) { return fminf(fmaxf(y, -kE4M3Max), kE4M3Max); }

// Codes of four values of a block with scale s: x / s (IEEE division),
// saturated to +-448, rounded to nearest E4M3; bytes in input order.
__device__ __forceinline__ uint32_t e4m3x4_div(float x0, float x1, float x2, float x3, float s) {
  const uint32_t lo = e4m3_pk<false>(sat448(x0 / s), sat448(x1 / s), 0u);
  return e4m3_pk<true>(sat448(x2 / s), sat448(x3 / s), lo);
}

// The same for a power-of-two scale, given inv = 1 / s: x * inv is then the
// correctly rounded x / s (1/s is a power of two; for scales from amax / 448
// of finite fp32 data it is a normal number).
__device__ __forceinline__ uint32_t e4m3x4_mul(float x0, float x1, float x2, float x3, float inv) {
  const uint32_t lo = e4m3_pk<false>(sat448(x0 * inv), sat448(x1 * inv), 0u);
  return e4m3_pk<true>(sat448(x2 * inv), sat448(x3 * inv), lo);
}

}  // namespace fg
