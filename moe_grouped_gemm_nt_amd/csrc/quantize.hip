// quantize.hip - FP8 E4M3 activation quantization with 1x128 per-token scales, the step
// that feeds the M-grouped GEMMs their FP8 activations (C ABI in
// include/moe_grouped_gemm_nt.h: quantize_fp8_1x128).
//
// Per row and 128-column group: amax = max |x|; scale s = amax / 448 (an all-zero group
// takes the caller's `sf_zero`; F32 scales are floored at 1e-30), codes = E4M3(x / s)
// computed as x * (1 / s) — the float32 arithmetic of the cast printed in the repro
// script of the DeepGEMM issue "Non-deterministic numerical problem of
// k_grouped_fp8_gemm_nt_contiguous", applied along K per token. UE8M0 scales are the
// smallest power of two not below amax / 448 (exact scaling, no code can overflow).
//
// Layout: X bf16 [M][K] (K contiguous), Q E4M3 bytes [M][K], SF [K/128][M] (float32 or one
// byte per scale) — the activation-scale layout the GEMM entry points read.
//
// One workgroup handles 16 rows x 512 columns (see quant_rows_1x128); the group maximum
// is a 16-lane butterfly. The kernel is HBM-bound (3 bytes per element).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_grouped_gemm_nt.h"

namespace {

constexpr int kRowsPerBlock = 16;  // 4 waves x 4 rows
constexpr int kColsPerBlock = 512;  // one wave instruction covers 512 contiguous columns
constexpr int kThreadsQ = 256;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

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

// One workgroup: 16 rows x 512 columns. Wave w takes rows 4w .. 4w + 3 of the block; in
// each, lanes 16 g .. 16 g + 15 cover 128-column group g (8 elements per lane), so one
// load instruction reads 1 KB of a row contiguously. The 64 scales of the block are
// collected in LDS and written as four runs of 16 consecutive rows.
template <bool UE8M0>
__global__ __launch_bounds__(kThreadsQ) void quant_rows_1x128(const uint16_t* __restrict__ X,
                                                              uint8_t* __restrict__ Q,
                                                              void* __restrict__ SF, int M,
                                                              int K, float sf_zero) {
  __shared__ uint32_t s_sf[4][kRowsPerBlock];  // [group][row] scale bits or codes
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane >> 4, l16 = lane & 15;
  const int m0 = blockIdx.x * kRowsPerBlock;
  const int kb = blockIdx.y * 4 + grp;  // this lane's 128-column group
  const bool col_ok = kb * 128 < K;     // uniform per 16-lane group
  const long col = (long)kb * 128 + l16 * 8;
  u32x4 w[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = m0 + 4 * wave + r;
    w[r] = (u32x4){0u, 0u, 0u, 0u};
    if (m < M && col_ok) w[r] = *reinterpret_cast<const u32x4*>(X + (long)m * K + col);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int rl = 4 * wave + r, m = m0 + rl;
    float v[8] = {bf16_lo(w[r].x), bf16_hi(w[r].x), bf16_lo(w[r].y), bf16_hi(w[r].y),
                  bf16_lo(w[r].z), bf16_hi(w[r].z), bf16_lo(w[r].w), bf16_hi(w[r].w)};
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 16));
    float s = amax / 448.0f;  // IEEE float32 division
    float inv;
    uint32_t sfbits;
    if constexpr (UE8M0) {
      const uint32_t code = ue8m0_at_least(s == 0.f ? sf_zero : s);
      inv = ldexpf(1.0f, 127 - (int)code);  // exact
      sfbits = code;
    } else {
      if (s == 0.f) s = sf_zero;
      s = fmaxf(s, 1e-30f);
      inv = 1.0f / s;  // IEEE float32 division
      sfbits = __float_as_uint(s);
    }
    u32x2 out;
    out.x = to_e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
    out.y = to_e4m3x4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
    if (m < M && col_ok) *reinterpret_cast<u32x2*>(Q + (long)m * K + col) = out;
    if (l16 == 0) s_sf[grp][rl] = sfbits;
  }
  __syncthreads();
  if (threadIdx.x < 4 * kRowsPerBlock) {
    const int g = threadIdx.x / kRowsPerBlock, rl = threadIdx.x % kRowsPerBlock;
    const int m = m0 + rl, k2 = blockIdx.y * 4 + g;
    if (m < M && k2 * 128 < K) {
      if constexpr (UE8M0)
        reinterpret_cast<uint8_t*>(SF)[(long)k2 * M + m] = (uint8_t)s_sf[g][rl];
      else
        reinterpret_cast<uint32_t*>(SF)[(long)k2 * M + m] = s_sf[g][rl];
    }
  }
}

}  // namespace

// Called by the public entry point in grouped_gemm.hip (which owns the error text).
extern "C" __attribute__((visibility("hidden"))) mgg_status quantize_fp8_1x128_impl(
    int M, int K, const void* X, void* Q, void* SF, mgg_sf_fmt sf, float sf_zero,
    hipStream_t stream, const char** err) {
  if (M < 1 || K < 128 || K % 128 != 0) {
    *err = "M must be positive and K a positive multiple of 128";
    return MGG_EINVAL;
  }
  if (!X || !Q || !SF) {
    *err = "null pointer";
    return MGG_EINVAL;
  }
  if ((uintptr_t)X % 16 || (uintptr_t)Q % 8 || (sf == MGG_SF_F32 && (uintptr_t)SF % 4)) {
    *err = "X must be 16-byte, Q 8-byte and float32 scales 4-byte aligned";
    return MGG_EINVAL;
  }
  if (sf != MGG_SF_F32 && sf != MGG_SF_UE8M0) {
    *err = "unknown scale format";
    return MGG_EINVAL;
  }
  if (!(sf_zero > 0.f) || !(sf_zero < 3.0e38f)) {
    *err = "sf_zero must be a positive finite float";
    return MGG_EINVAL;
  }
  if (K / 128 > 65535) {
    *err = "K too large";
    return MGG_EUNSUPPORTED;
  }
  const dim3 grid((unsigned)((M + kRowsPerBlock - 1) / kRowsPerBlock),
                  (unsigned)((K + kColsPerBlock - 1) / kColsPerBlock));
  if (sf == MGG_SF_UE8M0)
    hipLaunchKernelGGL(quant_rows_1x128<true>, grid, dim3(kThreadsQ), 0, stream,
                       (const uint16_t*)X, (uint8_t*)Q, SF, M, K, sf_zero);
  else
    hipLaunchKernelGGL(quant_rows_1x128<false>, grid, dim3(kThreadsQ), 0, stream,
                       (const uint16_t*)X, (uint8_t*)Q, SF, M, K, sf_zero);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    *err = hipGetErrorString(e);
    return MGG_EHIP;
  }
  return MGG_OK;
}
