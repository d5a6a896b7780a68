// act_math.h - the float32 arithmetic of the FP8 1x128 activation cast and of SwiGLU,
// shared by the stand-alone quantization kernels (quantize.hip) and the GEMM epilogue
// that applies them to its own output, so that both take every float32 decision the
// same way and produce the same codes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mgg {

// Smallest u with 2^(u - 127) >= s (s > 0), from the float32 bits of s.
__device__ __forceinline__ uint32_t ue8m0_at_least(float s) {
  const uint32_t b = __float_as_uint(s);
  return ((b >> 23) & 0xffu) + ((b & 0x7fffffu) != 0u ? 1u : 0u);
}

// Four float32 values -> four E4M3 codes (round to nearest even), packed little-endian.
__device__ __forceinline__ uint32_t to_e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// Scale of one 128-element group from its absolute maximum: s = amax / 448 (IEEE
// division); an all-zero group takes `sf_zero`. F32 scales are floored at 1e-30 and the
// codes are x * (1 / s); UE8M0 scales are the smallest power of two not below s and the
// codes are x * 2^-e (exact). Returns the multiplier; `bits` receives the stored scale
// (float32 bits or the UE8M0 code).
template <bool UE8M0>
__device__ __forceinline__ float group_scale_1x128(float amax, float sf_zero, uint32_t& bits) {
  float s = amax / 448.0f;
  if constexpr (UE8M0) {
    const uint32_t code = ue8m0_at_least(s == 0.f ? sf_zero : s);
    bits = code;
    return ldexpf(1.0f, 127 - (int)code);
  } else {
    if (s == 0.f) s = sf_zero;
    s = fmaxf(s, 1e-30f);
    bits = __float_as_uint(s);
    return 1.0f / s;
  }
}

// Taylor coefficients (ln 2)^k / k!, k = 0..7, of 2^r = e^(r ln 2): each built in double
// as c_k = c_(k-1) * ln 2 / k and rounded once to float.
struct ExpPoly {
  float c[8];
};
constexpr ExpPoly make_exp_poly() {
  ExpPoly p{};
  double c = 1.0;
  p.c[0] = 1.0f;
  for (int k = 1; k < 8; ++k) {
    c = c * 0.6931471805599453 / k;
    p.c[k] = (float)c;
  }
  return p;
}
constexpr ExpPoly kExpPoly = make_exp_poly();

// e^y as one fixed float32 evaluation, so that every rounding is specified: t = y log2(e)
// (one float multiply), n = t rounded to the nearest integer (ties to even), r = t - n
// (exact, |r| <= 1/2), 2^r by the degree-7 Taylor polynomial in Horner form with every
// multiply and add rounded separately (contraction into fused multiply-adds is switched
// off here), then an exact scaling by 2^n. t is clamped to [-150, 128]: above 128 the
// result is +inf, below -150 it is 0. Relative error below 1e-5 on the range silu uses.
__device__ __forceinline__ float exp_fixed(float y) {
#pragma clang fp contract(off)
  float t = y * (float)1.4426950408889634;
  const bool big = t > 128.0f, small = t < -150.0f;
  t = fminf(fmaxf(t, -150.0f), 128.0f);
  const float n = __builtin_rintf(t);
  const float r = t - n;
  float p = kExpPoly.c[7];
#pragma unroll
  for (int k = 6; k >= 0; --k) p = p * r + kExpPoly.c[k];
  float out = ldexpf(p, (int)n);
  out = big ? __builtin_huge_valf() : out;
  return small ? 0.0f : out;
}

// silu(x) = x / (1 + e^-x): one float add and one IEEE float division.
__device__ __forceinline__ float silu_fixed(float x) {
#pragma clang fp contract(off)
  const float d = 1.0f + exp_fixed(-x);
  return x / d;
}

}  // namespace mgg
