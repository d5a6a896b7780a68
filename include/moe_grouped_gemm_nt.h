/*
 * moe_grouped_gemm_nt.h - C ABI of the MI355X (gfx950) grouped NT GEMM library for
 * mixture-of-experts layers.
 *
 * Three grouped products, each in BF16 or in FP8 E4M3 with fine-grained scales and
 * FP32 accumulation. "NT" means both operands are stored with K contiguous and the
 * product is D = A * B^T per expert.
 *
 *   grouped_gemm_masked      per-expert capacity, device-side valid-row counts; only
 *                            valid rows are written (DeepGEMM PR "Fix cross-expert
 *                            output overwrites in SM90 masked GEMM", sections
 *                            "Description" and "Reproduction and validation").
 *   grouped_gemm_contiguous  expert row segments concatenated, a device-side expert
 *                            index per row (DeepGEMM issue "SM120 m_grouped_fp8
 *                            contiguous kernel: illegal memory access at CUDA graph
 *                            replay", sections "Environment" and the analysis comment).
 *   grouped_gemm_kgrouped    weight-gradient form, D_e (+)= A_e * B_e^T over expert e's
 *                            token slice, with per-channel scales on both operands
 *                            (DeepGEMM issue "Non-deterministic numerical problem of
 *                            k_grouped_fp8_gemm_nt_contiguous", section "repro script").
 * The contiguous and K-grouped products also take their routing as per-expert prefix
 * sums (the "_psum" entry points), and quantize_fp8_1x128 produces FP8 activations with
 * their 1x128 scales.
 *
 * Common rules for every entry point:
 *  - Every pointer is caller-owned device memory; the caller allocates every output.
 *  - Sizes: operands and outputs may exceed 2 GiB. What must stay below 2 GiB is 128 rows of
 *    an activation, output or K-grouped operand, 256 weight rows (the fused SwiGLU call:
 *    one expert's 2I weight rows), and each scale and routing tensor; otherwise
 *    MGG_EUNSUPPORTED.
 *  - The call validates its host arguments first. On any violation it returns an error
 *    code and enqueues nothing.
 *  - Otherwise it enqueues kernels on `stream` and returns without synchronizing. It
 *    never allocates, frees, copies to or from the host, or reads device memory on the
 *    host, so it may be captured into a hipGraph. All routing (counts, row indices,
 *    per-expert K) is read from device memory by the kernels at run time, so a graph
 *    replay sees whatever values those buffers hold at replay time.
 *  - Results are bitwise identical from call to call on the same inputs, independent
 *    of `expected_m`, of other experts' counts and of launch shapes: each output
 *    element is produced by one lane, in ascending K order, with no atomics.
 *  - FP8 E4M3 is the OCP "E4M3FN" byte format (max 448, no infinities). Scales are
 *    either float32 (MGG_SF_F32) or one unsigned byte u per scale meaning 2^(u-127)
 *    (MGG_SF_UE8M0). A scale covers 128 consecutive K elements of one row (1x128) or
 *    a 128x128 block of a weight matrix.
 *  - FP8 x FP4 (MGG_FP8_FP4, the "fp8_fp4" kernel family the DeepGEMM issue "SM120
 *    m_grouped_fp8 contiguous kernel: illegal memory access at CUDA graph replay" names
 *    without describing it; the format reading is this library's): activations are FP8
 *    E4M3 with 1x128 UE8M0 scales; weights are FP4 E2M1 (OCP microscaling: 1 sign, 2
 *    exponent, 1 mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), two per byte with
 *    the even K element in the low nibble, so a weight row is K/2 bytes; each weight row
 *    has one UE8M0 scale per 32 consecutive K (MGG_SFB_BLOCK32), stored per expert as
 *    [K/128][N][4] bytes (byte j of entry [kb][n] scales K 128 kb + 32 j .. + 31). Only
 *    the M-grouped entry points take it (the K-grouped ones return MGG_EUNSUPPORTED),
 *    and only with MGG_SF_UE8M0 (else MGG_EUNSUPPORTED).
 *  - Accumulation is FP32; BF16 outputs are rounded to nearest even.
 *  - Inputs must not overlap outputs (except C == D in grouped_gemm_kgrouped).
 *  - Calls on one stream are ordered; calls that run concurrently on different streams
 *    must use disjoint outputs.
 */
#ifndef MOE_GROUPED_GEMM_NT_H
#define MOE_GROUPED_GEMM_NT_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MGG_OK = 0,
  MGG_EINVAL = 1,       /* a host argument is invalid; nothing enqueued */
  MGG_EUNSUPPORTED = 2, /* valid but outside what the library implements; nothing enqueued */
  MGG_EHIP = 3          /* the HIP runtime reported an error at launch */
} mgg_status;

typedef enum {
  MGG_BF16 = 0,      /* both operands bfloat16 */
  MGG_FP8_E4M3 = 1,  /* both operands FP8 E4M3 */
  MGG_FP8_FP4 = 2    /* FP8 E4M3 activations, FP4 E2M1 weights (M-grouped entry points) */
} mgg_dtype;
typedef enum { MGG_SF_F32 = 0, MGG_SF_UE8M0 = 1 } mgg_sf_fmt;
typedef enum {
  MGG_SFB_BLOCK128 = 0, /* one weight scale per 128x128 block */
  MGG_SFB_CHANNEL = 1,  /* one weight scale per weight row and 128-K group */
  MGG_SFB_BLOCK32 = 2   /* FP4 weights: one UE8M0 scale per weight row and 32-K block */
} mgg_sfb_gran;

/*
 * Masked M-grouped NT GEMM: for every expert g and valid row m < clamp(masked_m[g], 0,
 * cap), D[g, m, n] = sum_k A[g, m, k] * B[g, n, k] (dequantized for FP8).
 *
 *   dt          MGG_BF16, MGG_FP8_E4M3 (both operands) or MGG_FP8_FP4.
 *   G, cap      experts and rows per expert (capacity); 1 <= G <= 4096, cap >= 1.
 *   N, K        N >= 1 with N % 8 == 0; K >= 1 with K % 8 == 0 (BF16), K % 128 == 0 (FP8).
 *   A           [G][cap][K] elements (bf16 or e4m3 bytes); 16-byte aligned.
 *   SFA         FP8 only (else NULL): activation scales [G][K/128][cap], one per row and
 *               128-K group, rows contiguous within each group.
 *   B           [G][N][K] elements (FP4: [G][N][K/2] bytes); 16-byte aligned.
 *   SFB         FP8 only: BLOCK128 -> [G][ceil(N/128)][K/128]; CHANNEL -> [G][K/128][N];
 *               BLOCK32 (FP4 weights) -> [G][K/128][N][4].
 *   sf, gran    scale storage format and weight-scale granularity (ignored for BF16).
 *   D           bf16 [G][cap][N]; 16-byte aligned. Only valid rows are written: padding
 *               rows and every byte outside the valid rows keep their previous contents.
 *   masked_m    device int32 [G]; values outside [0, cap] are clamped (never a fault).
 *   expected_m  host hint of the typical valid rows per expert (<= 0: unknown). It picks
 *               a tile shape and never changes the result.
 */
mgg_status grouped_gemm_masked(mgg_dtype dt, int G, int cap, int N, int K,
                               const void* A, const void* SFA,
                               const void* B, const void* SFB,
                               mgg_sf_fmt sf, mgg_sfb_gran gran,
                               void* D, const int32_t* masked_m, int expected_m,
                               hipStream_t stream);

/*
 * Contiguous M-grouped NT GEMM: row r belongs to expert e = m_indices[r] when e lies in
 * [0, G); then D[r, n] = sum_k A[r, k] * B[e, n, k]. Rows with any other index are
 * padding and are not written.
 *
 *   M           total rows, M >= 1 and M <= 524288.
 *   A           [M][K] elements; SFA (FP8) [K/128][M].
 *   B, SFB      as in grouped_gemm_masked (per expert).
 *   D           bf16 [M][N].
 *   m_indices   device int32 [M]. Contract: every aligned block of 128 rows holds rows
 *               of at most one expert, valid rows first (segments padded with -1 to
 *               multiples of 128). The expert of a block is the index of its first row;
 *               a block whose first index is outside [0, G) is padding, and a row whose
 *               index differs from its block's expert is not written. Never a fault.
 */
mgg_status grouped_gemm_contiguous(mgg_dtype dt, int G, int M, int N, int K,
                                   const void* A, const void* SFA,
                                   const void* B, const void* SFB,
                                   mgg_sf_fmt sf, mgg_sfb_gran gran,
                                   void* D, const int32_t* m_indices, int expected_m,
                                   hipStream_t stream);

/*
 * M-grouped NT GEMM, contiguous rows in prefix-sum ("psum") layout: the routing is one
 * cumulative row end per expert instead of one expert index per row. The pages name this
 * mode (DeepGEMM issue "Non-deterministic numerical problem of
 * k_grouped_fp8_gemm_nt_contiguous", repro script: the use_psum_layout argument; DeepGEMM
 * issue "SM120 m_grouped_fp8 contiguous kernel: illegal memory access at CUDA graph
 * replay", verification comment: the psum mode of its graph-mutation test) without
 * describing it; the reading implemented here: expert e owns rows [start_e, end_e) with
 *   end_e   = clamp(psum[e], 0, M) raised to the largest end_j of any j < e,
 *   start_e = end_{e-1} (0 for e = 0),
 * so segments are consecutive, never overlap and need no alignment.
 * D[r, :] = A[r, :] . B[e]^T for r in [start_e, end_e); rows at or beyond end_{G-1} are
 * not written.
 *
 *   A           [M][K] (bf16 or e4m3 bytes), 16-byte aligned.
 *   SFA         FP8 only: [K/128][M].
 *   B, SFB      as for grouped_gemm_masked.
 *   D           bf16 [M][N], 16-byte aligned.
 *   psum        device int32 [G], read by the kernel on every launch (graph-replay safe).
 *   expected_m  rows per expert hint (<= 0: unknown); never changes results.
 * Errors: as grouped_gemm_masked.
 */
mgg_status grouped_gemm_contiguous_psum(mgg_dtype dt, int G, int M, int N, int K,
                                        const void* A, const void* SFA,
                                        const void* B, const void* SFB,
                                        mgg_sf_fmt sf, mgg_sfb_gran gran,
                                        void* D, const int32_t* psum, int expected_m,
                                        hipStream_t stream);

/*
 * K-grouped NT GEMM (weight gradient): expert e owns k_e = ks[e] consecutive tokens
 * starting at token p_e = sum_{j<e} max(ks[j], 0). Operand blocks are packed per
 * expert, tokens contiguous:
 *   A: expert e's [M][k_e] block starts at element M * p_e;
 *   B: expert e's [N][k_e] block starts at element N * p_e.
 * D[e, i, j] = (accumulate ? D[e, i, j] : 0) + sum_{t < k_e} A_e[i, t] * B_e[j, t].
 *
 *   K_total     size of the token axis of both buffers (elements per channel).
 *   SFA, SFB    FP8 only: per-channel scales [K_total/128][M] and [K_total/128][N];
 *               token t of expert e uses scale row (p_e + t) / 128.
 *   D           fp32 [G][M][N], 16-byte aligned.
 *   ks          device int32 [G]. Contract: k_e >= 0; k_e and p_e multiples of 128
 *               (FP8) or of 8 (BF16); p_e + k_e <= K_total. An expert outside the
 *               contract is skipped (its D_e is not written). k_e == 0 gives D_e = 0
 *               (accumulate == 0) or leaves D_e unchanged (accumulate == 1).
 *   accumulate  1: D += product (the caller's C aliases D); 0: D = product.
 *   FP8 scales must be MGG_SF_F32 or MGG_SF_UE8M0 and are per channel on both operands.
 */
mgg_status grouped_gemm_kgrouped(mgg_dtype dt, int G, int M, int N, int K_total,
                                 const void* A, const void* SFA,
                                 const void* B, const void* SFB,
                                 mgg_sf_fmt sf,
                                 float* D, const int32_t* ks, int accumulate,
                                 hipStream_t stream);

/*
 * K-grouped NT GEMM with the token counts in prefix-sum ("psum") layout (the
 * use_psum_layout argument of the K-grouped call in the repro script of the DeepGEMM issue
 * "Non-deterministic numerical problem of k_grouped_fp8_gemm_nt_contiguous", not
 * described there): psum[e] is the
 * cumulative token end of expert e, so k_e = psum[e] - psum[e-1] (psum[-1] = 0); then
 * exactly as grouped_gemm_kgrouped with ks[e] = k_e (a decreasing entry gives a negative
 * k_e: that expert is skipped).
 */
mgg_status grouped_gemm_kgrouped_psum(mgg_dtype dt, int G, int M, int N, int K_total,
                                      const void* A, const void* SFA,
                                      const void* B, const void* SFB,
                                      mgg_sf_fmt sf,
                                      float* D, const int32_t* psum, int accumulate,
                                      hipStream_t stream);

/*
 * FP8 E4M3 activation quantization with 1x128 per-token scales: the cast that produces
 * the FP8 activations and their scales for the M-grouped entry points. For each row m and
 * 128-column group kb, with float32 arithmetic throughout:
 *   amax = max |X[m, 128 kb .. 128 kb + 127]|,  s = amax / 448
 *   F32 scales:   s = sf_zero if s == 0; s = max(s, 1e-30); SF[kb, m] = s;
 *                 Q[m, k] = E4M3(X[m, k] * (1 / s))
 *   UE8M0 scales: u = smallest exponent code with 2^(u-127) >= (s == 0 ? sf_zero : s);
 *                 SF[kb, m] = u; Q[m, k] = E4M3(X[m, k] * 2^(127-u))
 * E4M3 conversion rounds to nearest, ties to even. This is the cast printed in the repro
 * script of the DeepGEMM issue "Non-deterministic numerical problem of
 * k_grouped_fp8_gemm_nt_contiguous" (there per channel over 128 tokens, with its sf_val
 * as sf_zero), applied per token over 128 columns; the UE8M0 rounding rule is not printed
 * on the pages (the reading taken: round the scale up to a power of two).
 *
 *   X    bf16 [M][K], 16-byte aligned; K a positive multiple of 128.
 *   Q    E4M3 bytes [M][K], 8-byte aligned (may not overlap X).
 *   SF   [K/128][M]: float32 (4-byte aligned) or one byte per scale (MGG_SF_UE8M0).
 *   sf_zero  positive finite scale for all-zero groups.
 * Errors: MGG_EINVAL for bad sizes, pointers, alignment, format or sf_zero.
 */
mgg_status quantize_fp8_1x128(int M, int K, const void* X, void* Q, void* SF, mgg_sf_fmt sf,
                              float sf_zero, hipStream_t stream);

/*
 * SwiGLU + FP8 re-quantization between an expert's gate/up GEMM (w13) and its down GEMM
 * (w2): the step between the two contiguous FP8 GEMMs of the serving chain in the
 * DeepGEMM issue "SM120 m_grouped_fp8 contiguous kernel: illegal memory access at CUDA
 * graph replay" (sections "Environment" and "What works"), whose activation the pages
 * leave unnamed (the reading taken: the gated unit silu(gate) * up). For each row m and
 * column i < I, in float32:
 *   x[m, i] = silu(H[m, i]) * H[m, I + i],  silu(g) = g / (1 + e^-g)
 * with e^y one fixed evaluation (t = y log2 e; n = nearest integer to t, ties to even;
 * degree-7 Taylor polynomial of 2^(t - n) in Horner form, every multiply and add rounded
 * separately; scaled by 2^n; t > 128 gives +inf, t < -150 gives 0), and x is then
 * quantized exactly as quantize_fp8_1x128 does with K = I.
 *
 *   H    bf16 [M][2I] (w13 output: gate columns first, then up), 16-byte aligned;
 *        I a positive multiple of 128.
 *   Q    E4M3 bytes [M][I], 8-byte aligned (may not overlap H).
 *   SF   [I/128][M]: float32 (4-byte aligned) or one byte per scale (MGG_SF_UE8M0).
 *   sf_zero  positive finite scale for all-zero groups.
 * Every row is processed (rows a contiguous GEMM skipped hold whatever H holds there).
 * Errors: MGG_EINVAL for bad sizes, pointers, alignment, format or sf_zero.
 */
mgg_status swiglu_quant_fp8_1x128(int M, int I, const void* H, void* Q, void* SF,
                                  mgg_sf_fmt sf, float sf_zero, hipStream_t stream);

/*
 * Contiguous FP8 GEMM with the SwiGLU + FP8 re-quantization fused into its epilogue: the
 * w13 GEMM of the expert chain in the DeepGEMM issue "SM120 m_grouped_fp8 contiguous
 * kernel: illegal memory access at CUDA graph replay" (sections "Environment" and "What
 * works") followed by the step swiglu_quant_fp8_1x128 performs, without the bf16
 * intermediate ever reaching memory. For each routed row r (expert e = m_indices[r], the
 * contiguous rule of grouped_gemm_contiguous) and output column i < I:
 *   h[r, c] = bf16(sum_k A[r, k] * B[e, c, k]) for c = i (gate) and c = I + i (up),
 *   Q[r, i], SFQ[i / 128, r] = the 1x128 quantization of silu(h[r, i]) * h[r, I + i]
 * exactly as swiglu_quant_fp8_1x128 computes it on the bf16 output of
 * grouped_gemm_contiguous (the codes and scales are bit-identical to running the two).
 *
 *   dt          MGG_FP8_E4M3 or MGG_FP8_FP4 (MGG_BF16: MGG_EUNSUPPORTED).
 *   M, I, K     rows (<= 524288), output columns per row (positive multiple of 128), K
 *               (positive multiple of 128).
 *   A, SFA      [M][K] codes, [K/128][M] scales, as in grouped_gemm_contiguous.
 *   B, SFB      the w13 weights in their usual layout [G][2I][K] (gate rows 0..I-1, up
 *               rows I..2I-1; FP4: [G][2I][K/2]) with their scales: FP8 BLOCK128 (float32
 *               or UE8M0) or CHANNEL with float32 scales; FP4 BLOCK32.
 *   Q           E4M3 bytes [M][I], 16-byte aligned.
 *   SFQ, sfq    [I/128][M] scales, float32 (4-byte aligned) or UE8M0 bytes.
 *   sf_zero     positive finite scale for all-zero groups.
 *   m_indices   as in grouped_gemm_contiguous; rows that are not routed keep their Q and
 *               SFQ contents.
 * Errors: as grouped_gemm_contiguous; MGG_EUNSUPPORTED for BF16 or FP8 CHANNEL weight
 * scales in UE8M0.
 */
mgg_status grouped_gemm_contiguous_swiglu_quant(mgg_dtype dt, int G, int M, int I, int K,
                                               const void* A, const void* SFA,
                                               const void* B, const void* SFB,
                                               mgg_sf_fmt sf, mgg_sfb_gran gran,
                                               void* Q, void* SFQ, mgg_sf_fmt sfq,
                                               float sf_zero, const int32_t* m_indices,
                                               hipStream_t stream);

/* Human-readable text for a status code (static storage). */
const char* mgg_status_string(mgg_status s);

/* Text of the most recent error on the calling thread ("" if none). */
const char* mgg_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_GROUPED_GEMM_NT_H */
