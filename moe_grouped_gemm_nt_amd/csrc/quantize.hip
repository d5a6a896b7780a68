// quantize.hip - FP8 E4M3 activation quantization with 1x128 per-token scales, the step
// that feeds the M-grouped GEMMs their FP8 activations (C ABI in
// include/moe_grouped_gemm_nt.h: quantize_fp8_1x128, swiglu_quant_fp8_1x128).
//
// Per row and 128-column group: amax = max |x|; scale s = amax / 448 (an all-zero group
// takes the caller's `sf_zero`; F32 scales are floored at 1e-30), codes = E4M3(x / s)
// computed as x * (1 / s) — the float32 arithmetic of the cast printed in the repro
// script of the DeepGEMM issue "Non-deterministic numerical problem of
// k_grouped_fp8_gemm_nt_contiguous", applied along K per token. UE8M0 scales are the
// smallest power of two not below amax / 448 (exact scaling, no code can overflow).
//
// The SwiGLU variant sits between an expert's gate/up GEMM (w13) and its down GEMM (w2)
// (the chain of the DeepGEMM issue "SM120 m_grouped_fp8 contiguous kernel: illegal memory
// access at CUDA graph replay", sections "Environment" and "What works"): x is
// silu(gate) * up in float32, gate the first I columns of the bf16 w13 output and up the
// last I, and x is quantized exactly as above.
//
// Layout: X bf16 [M][K] (K contiguous; [M][2K] for SwiGLU), Q E4M3 bytes [M][K],
// SF [K/128][M] (float32 or one byte per scale) — the activation-scale layout the GEMM
// entry points read.
//
// One workgroup handles 64 (row, 128-column group) units, 16 with SwiGLU (see
// quant_rows_1x128); the group maximum is a 16-lane butterfly. The kernel is HBM-bound (3 bytes per element; 5 for SwiGLU).

#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>

#include "act_math.h"
#include "moe_grouped_gemm_nt.h"

namespace {

using mgg::group_scale_1x128;
using mgg::silu_fixed;
using mgg::to_e4m3x4;

// (row, 128-column group) units per workgroup: 16 quarters x 4 steps. The SwiGLU variant,
// bound by its float32 exp and division rather than by memory, takes one step per wave
// (16 units): more, shorter workgroups measured 7-19 % faster there and 4 % slower for the
// plain cast.
template <bool SWIGLU>
struct QuantShape {
  static constexpr int kSteps = SWIGLU ? 1 : 4;
  static constexpr int kUnits = 16 * kSteps;
  static constexpr int kUnitsLog = SWIGLU ? 4 : 6;
};
constexpr int kThreadsQ = 256;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// One workgroup covers U = QuantShape::kUnits (row, 128-column group) units: GB = 2^gb_log
// groups side by side (GB = 4 for rows of at least 512 columns, fewer for narrower rows so
// no lane idles) times U / GB rows. Each 16-lane quarter of a wave takes one unit per step
// (8 elements per lane, one contiguous 256-byte run of the row), the quarters of a wave
// cover GB adjacent groups of 4 / GB consecutive rows, and each wave does kSteps steps. The
// U scales of the block are collected in LDS and written as GB runs of consecutive rows. With
// SWIGLU, X has 2K columns per row and each lane also loads the matching up-projection
// columns K + col.
template <bool UE8M0, bool SWIGLU>
__global__ __launch_bounds__(kThreadsQ) void quant_rows_1x128(const uint16_t* __restrict__ X,
                                                              uint8_t* __restrict__ Q,
                                                              void* __restrict__ SF, int M,
                                                              int K, float sf_zero,
                                                              int gb_log) {
  using QS = QuantShape<SWIGLU>;
  constexpr int ST = QS::kSteps;
  __shared__ uint32_t s_sf[QS::kUnits];  // [group][row] scale bits or codes
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane >> 4, l16 = lane & 15;
  const int rows_log = QS::kUnitsLog - gb_log;  // U / GB rows per block
  const int m0 = blockIdx.x << rows_log;
  const long ldx = SWIGLU ? 2L * K : (long)K;
  // X is read once and Q written once: both go through the non-temporal cache policy
  u32x4 w[ST], u[ST];
  int rl[ST], kb[ST];
#pragma unroll
  for (int r = 0; r < ST; ++r) {
    const int unit = (wave * ST + r) * 4 + grp;
    rl[r] = unit >> gb_log;
    kb[r] = (blockIdx.y << gb_log) + (unit & ((1 << gb_log) - 1));
    const int m = m0 + rl[r];
    const long col = (long)kb[r] * 128 + l16 * 8;
    w[r] = (u32x4){0u, 0u, 0u, 0u};
    u[r] = (u32x4){0u, 0u, 0u, 0u};
    if (m < M && kb[r] * 128 < K) {  // uniform per 16-lane quarter
      w[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(X + (long)m * ldx + col));
      if constexpr (SWIGLU) u[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(X + (long)m * ldx + K + col));
    }
  }
#pragma unroll
  for (int r = 0; r < ST; ++r) {
    const int m = m0 + rl[r];
    const long col = (long)kb[r] * 128 + l16 * 8;
    float v[8] = {bf16_lo(w[r].x), bf16_hi(w[r].x), bf16_lo(w[r].y), bf16_hi(w[r].y),
                  bf16_lo(w[r].z), bf16_hi(w[r].z), bf16_lo(w[r].w), bf16_hi(w[r].w)};
    if constexpr (SWIGLU) {
      const float up[8] = {bf16_lo(u[r].x), bf16_hi(u[r].x), bf16_lo(u[r].y), bf16_hi(u[r].y),
                           bf16_lo(u[r].z), bf16_hi(u[r].z), bf16_lo(u[r].w), bf16_hi(u[r].w)};
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = silu_fixed(v[i]) * up[i];
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 16));
    uint32_t sfbits;
    const float inv = group_scale_1x128<UE8M0>(amax, sf_zero, sfbits);
    u32x2 out;
    out.x = to_e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
    out.y = to_e4m3x4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
    if (m < M && kb[r] * 128 < K) __builtin_nontemporal_store(out, reinterpret_cast<u32x2*>(Q + (long)m * K + col));
    const int g = kb[r] - (blockIdx.y << gb_log);
    if (l16 == 0) s_sf[(g << rows_log) + rl[r]] = sfbits;
  }
  __syncthreads();
  if (threadIdx.x < QS::kUnits) {
    const int g = threadIdx.x >> rows_log, r = threadIdx.x & ((1 << rows_log) - 1);
    const int m = m0 + r, k2 = (blockIdx.y << gb_log) + g;
    if (m < M && k2 * 128 < K) {
      if constexpr (UE8M0)
        reinterpret_cast<uint8_t*>(SF)[(long)k2 * M + m] = (uint8_t)s_sf[threadIdx.x];
      else
        reinterpret_cast<uint32_t*>(SF)[(long)k2 * M + m] = s_sf[threadIdx.x];
    }
  }
}

}  // namespace

namespace {

mgg_status launch_quant(bool swiglu, int M, int K, const void* X, void* Q, void* SF,
                        mgg_sf_fmt sf, float sf_zero, hipStream_t stream, const char** err) {
  if (M < 1 || K < 128 || K % 128 != 0) {
    *err = swiglu ? "M must be positive and I a positive multiple of 128"
                  : "M must be positive and K a positive multiple of 128";
    return MGG_EINVAL;
  }
  if (!X || !Q || !SF) {
    *err = "null pointer";
    return MGG_EINVAL;
  }
  if ((uintptr_t)X % 16 || (uintptr_t)Q % 8 || (sf == MGG_SF_F32 && (uintptr_t)SF % 4)) {
    *err = "the bf16 input must be 16-byte, Q 8-byte and float32 scales 4-byte aligned";
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
  if (K / 128 > 65535 || (swiglu && K > INT_MAX / 2)) {
    *err = swiglu ? "I too large" : "K too large";
    return MGG_EUNSUPPORTED;
  }
  const int kgroups = K / 128;
  const int gb_log = kgroups >= 4 ? 2 : kgroups >= 2 ? 1 : 0;
  const int rows = (swiglu ? QuantShape<true>::kUnits : QuantShape<false>::kUnits) >> gb_log;
  const dim3 grid((unsigned)((M + rows - 1) / rows),
                  (unsigned)((kgroups + (1 << gb_log) - 1) >> gb_log));
  const bool ue = sf == MGG_SF_UE8M0;
  auto kern = swiglu ? (ue ? quant_rows_1x128<true, true> : quant_rows_1x128<false, true>)
                     : (ue ? quant_rows_1x128<true, false> : quant_rows_1x128<false, false>);
  hipLaunchKernelGGL(kern, grid, dim3(kThreadsQ), 0, stream, (const uint16_t*)X, (uint8_t*)Q,
                     SF, M, K, sf_zero, gb_log);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    *err = hipGetErrorString(e);
    return MGG_EHIP;
  }
  return MGG_OK;
}

}  // namespace

// Called by the public entry points in grouped_gemm.hip (which own the error text).
extern "C" __attribute__((visibility("hidden"))) mgg_status quantize_fp8_1x128_impl(
    int M, int K, const void* X, void* Q, void* SF, mgg_sf_fmt sf, float sf_zero,
    hipStream_t stream, const char** err) {
  return launch_quant(false, M, K, X, Q, SF, sf, sf_zero, stream, err);
}

extern "C" __attribute__((visibility("hidden"))) mgg_status swiglu_quant_fp8_1x128_impl(
    int M, int I, const void* H, void* Q, void* SF, mgg_sf_fmt sf, float sf_zero,
    hipStream_t stream, const char** err) {
  return launch_quant(true, M, I, H, Q, SF, sf, sf_zero, stream, err);
}
