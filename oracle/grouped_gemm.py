"""Plain FP64 CPU oracle for the three grouped NT GEMMs of an MoE layer.

TEST INFRASTRUCTURE ONLY: this module is imported by the tests, by the smoke check and
by the CPU-baseline leg of the benchmark. The product path never imports it and shares
no code with it.

What is computed, and where it is defined:

* The masked M-grouped GEMM of the DeepGEMM PR "Fix cross-expert output overwrites in
  SM90 masked GEMM" (section "Reproduction and validation"): expert g owns a capacity
  of `cap` rows; only rows m < counts[g] are valid, and for them
  D[g, m, :] = A[g, m, :] . B[g]^T, the reference being an FP64 batched product rounded
  to bfloat16 and the comparison made over valid rows only. The same section states the
  FP8 rule: the reference uses the actually quantized inputs and their scales.
* The contiguous M-grouped GEMM of the DeepGEMM issue "SM120 m_grouped_fp8 contiguous
  kernel: illegal memory access at CUDA graph replay" (sections "Environment" and the
  analysis comment): rows of all experts are concatenated and a per-row expert index
  (`m_indices`) routes each row to its expert's weight; scales are 1x128 per token group
  on activations and 128x128 blocks on weights, possibly powers of two.
* The prefix-sum ("psum") routing of the contiguous and K-grouped GEMMs, named on the
  pages without a description (see psum_segments and kgrouped_ks_from_psum for the
  reading taken).
* The K-grouped weight-gradient GEMM of the DeepGEMM issue "Non-deterministic numerical
  problem of k_grouped_fp8_gemm_nt_contiguous" (section "repro script"): expert e owns
  k_e consecutive tokens; both operands are packed per expert as [channels][k_e] blocks
  (tokens contiguous) at offset channels * (sum of earlier k); scales are per channel and
  per 128 global tokens; D_e = C_e + A_e^T-style product over the expert's tokens, with
  C aliasing D (the script passes the zeroed output as both `d` and `c`).

* FP8 x FP4 ("fp8_fp4", the kernel family of the SM120 issue, named there but not
  described): activations are FP8 E4M3 with their 1x128 scales as above; weights are
  FP4 E2M1, two per byte, with one UE8M0 scale per 32 consecutive K of a weight row (the
  OCP microscaling block), stored per expert as [K/128][N][4] (byte j of a [kb][n] entry
  scales K elements 128 kb + 32 j .. + 31 of row n). The weight-scale granularity is
  called "block32".

FP8 dequantization: value = decode(code) * scale, exact in float64. The GEMM itself is
the plain definition sum_k Ahat[m, k] * Bhat[n, k], evaluated by numpy's float64 matmul
(a library primitive, no reordering beyond its own). Outputs stay float64; rounding to
bf16 (`formats.round_to_bf16`) is a separate, explicit step.

calc_diff(x, y) = 1 - 2 sum(x*y) / sum(x*x + y*y), in float64, the similarity measure the
PR's reproduction script applies to valid rows (the formula itself is not printed on the
pages; this is the plain reading used throughout, with 0 for two all-zero inputs).
"""

from __future__ import annotations

import numpy as np

from .formats import decode_bf16, decode_e2m1, decode_e4m3fn, decode_scale, decode_ue8m0, unpack_fp4

SCALE_K = 128  # K elements sharing one scale (recipe (1, 1, 128) of the K-grouped call)
MX_BLOCK = 32  # K elements sharing one FP4 weight scale


# --------------------------------------------------------------------------- helpers


def _decode_elems(dtype: str, codes) -> np.ndarray:
    if dtype == "bf16":
        return decode_bf16(codes)
    if dtype in ("fp8", "fp8_fp4"):  # activations of the FP8 x FP4 product are FP8
        return decode_e4m3fn(codes)
    raise ValueError(f"unknown dtype {dtype!r}")


def _expand_k(sf_rows_by_kb: np.ndarray, K: int) -> np.ndarray:
    """[rows, K/128] per-block scales -> [rows, K] per-element scales."""
    return np.repeat(sf_rows_by_kb, SCALE_K, axis=1)[:, :K]


def dequant_act_rows(dtype, codes_rows, sfa_kb_by_row=None, sf_fmt="f32"):
    """Activation rows [R, K] -> float64. FP8: each row's 1x128 groups carry one scale.

    `sfa_kb_by_row` is laid out [K/128, R] (rows contiguous within a K block), the
    "column-major" activation-scale layout.
    """
    vals = _decode_elems(dtype, codes_rows)
    if dtype == "bf16":
        return vals
    sf = decode_scale(sfa_kb_by_row, sf_fmt).T  # [R, K/128]
    return vals * _expand_k(sf, vals.shape[1])


def dequant_weight_rows(dtype, codes_rows, n_index, sfb=None, sfb_gran="block128",
                        sf_fmt="f32"):
    """Weight rows B[n, :] for n in `n_index` -> float64 [len(n_index), K].

    `codes_rows` holds the codes of those rows. FP8 scales of one expert:
      block128: sfb[ceil(N/128), K/128], one scale per 128x128 block;
      channel:  sfb[K/128, N], one scale per row n and 128-K group.
    FP4 ("fp8_fp4"): `codes_rows` are packed bytes [R, K/2]; scales (always UE8M0)
      block32:  sfb[K/128, N, 4], one scale per row n and 32-K block.
    """
    if dtype == "fp8_fp4":
        if sfb_gran != "block32":
            raise ValueError("FP4 weights take block32 scales")
        vals = decode_e2m1(unpack_fp4(codes_rows))
        n_index = np.asarray(n_index)
        sf = decode_ue8m0(np.asarray(sfb))  # [K/128, N, 4]
        per_row = sf[:, n_index, :].transpose(1, 0, 2).reshape(n_index.size, -1)  # [R, K/32]
        return vals * np.repeat(per_row, MX_BLOCK, axis=1)[:, :vals.shape[1]]
    vals = _decode_elems(dtype, codes_rows)
    if dtype == "bf16":
        return vals
    sf = decode_scale(sfb, sf_fmt)
    n_index = np.asarray(n_index)
    if sfb_gran == "block128":
        per_row = sf[n_index // SCALE_K, :]  # [R, K/128]
    elif sfb_gran == "channel":
        per_row = sf[:, n_index].T
    else:
        raise ValueError(f"unknown weight-scale granularity {sfb_gran!r}")
    return vals * _expand_k(per_row, vals.shape[1])


def gemm_nt_fp64(a_hat: np.ndarray, b_hat: np.ndarray) -> np.ndarray:
    """Plain NT product: out[m, n] = sum_k a_hat[m, k] * b_hat[n, k], float64."""
    return np.asarray(a_hat, np.float64) @ np.asarray(b_hat, np.float64).T


# --------------------------------------------------------------------------- variants


def valid_counts(counts, cap: int) -> np.ndarray:
    """Per-expert valid rows: counts clamped to [0, cap] (out-of-range counts are a
    caller error; the clamp is the reading adopted for them)."""
    return np.clip(np.asarray(counts, dtype=np.int64), 0, cap)


def grouped_gemm_masked(dtype, A, B, counts, SFA=None, SFB=None, sfb_gran="block128",
                        sf_fmt="f32", experts=None, rows=None, cols=None):
    """Masked M-grouped NT GEMM, float64 result.

    A[G, cap, K], B[G, N, K] codes; counts[G]. FP8 scales: SFA[G, K/128, cap];
    SFB[G, ceil(N/128), K/128] (block128) or SFB[G, K/128, N] (channel).

    Returns (ref, valid): ref[G, cap, N] float64 with NaN on invalid rows, and
    valid[G, cap] bool. `experts`, `rows` (per-expert row lists) and `cols` restrict the
    work to a sample; unsampled entries stay NaN.
    """
    A = np.asarray(A)
    B = np.asarray(B)
    G, cap, K = A.shape
    N = B.shape[1]
    c = valid_counts(counts, cap)
    valid = np.arange(cap)[None, :] < c[:, None]
    ref = np.full((G, cap, N), np.nan)
    cols = np.arange(N) if cols is None else np.asarray(cols)
    for g in (range(G) if experts is None else experts):
        m_rows = np.arange(c[g]) if rows is None else np.asarray(
            [m for m in rows[g] if m < c[g]], dtype=np.int64)
        if m_rows.size == 0:
            continue
        a_hat = dequant_act_rows(dtype, A[g][m_rows],
                                 None if SFA is None else np.asarray(SFA)[g][:, m_rows], sf_fmt)
        b_hat = dequant_weight_rows(dtype, B[g][cols], cols,
                                    None if SFB is None else np.asarray(SFB)[g], sfb_gran, sf_fmt)
        ref[g][np.ix_(m_rows, cols)] = gemm_nt_fp64(a_hat, b_hat)
    return ref, valid


def contiguous_row_expert(m_indices, G: int) -> np.ndarray:
    """Expert of each row, -1 for rows whose index is outside [0, G) (padding)."""
    idx = np.asarray(m_indices, dtype=np.int64)
    return np.where((idx >= 0) & (idx < G), idx, -1)


def grouped_gemm_contiguous(dtype, A, B, m_indices, SFA=None, SFB=None,
                            sfb_gran="block128", sf_fmt="f32", rows=None, cols=None):
    """Contiguous M-grouped NT GEMM, float64 result.

    A[M, K] codes; B[G, N, K] codes; m_indices[M]. FP8 scales: SFA[K/128, M];
    SFB per expert as in the masked variant. Row r belongs to expert m_indices[r] when
    that index lies in [0, G); other rows are padding and are not computed.

    Returns (ref[M, N] float64 with NaN on padding/unsampled rows, valid[M] bool).
    """
    A = np.asarray(A)
    B = np.asarray(B)
    M, K = A.shape
    G, N, _ = B.shape
    expert = contiguous_row_expert(m_indices, G)
    valid = expert >= 0
    ref = np.full((M, N), np.nan)
    cols = np.arange(N) if cols is None else np.asarray(cols)
    want = valid.copy()
    if rows is not None:
        sel = np.zeros(M, bool)
        sel[np.asarray(rows, dtype=np.int64)] = True
        want &= sel
    for g in np.unique(expert[want]):
        r = np.nonzero(want & (expert == g))[0]
        a_hat = dequant_act_rows(dtype, A[r], None if SFA is None else np.asarray(SFA)[:, r],
                                 sf_fmt)
        b_hat = dequant_weight_rows(dtype, B[g][cols], cols,
                                    None if SFB is None else np.asarray(SFB)[g], sfb_gran, sf_fmt)
        ref[np.ix_(r, cols)] = gemm_nt_fp64(a_hat, b_hat)
    return ref, valid


def psum_segments(psum, M: int):
    """Row segment [start_e, end_e) of each expert in the prefix-sum ("psum") routing of
    the contiguous GEMM. The pages name this mode (the use_psum_layout argument in the
    repro script of the K-grouped issue; the psum mode of the graph-mutation test in the
    SM120 issue's verification comment) without describing it. Reading: psum[e] is the
    cumulative end row of expert e; each end is clamped to [0, M] and raised to the
    largest earlier end, and expert e starts where expert e - 1 ends (row 0 for e = 0),
    so segments are consecutive and never overlap."""
    out = []
    end_prev = 0
    for v in np.asarray(psum, dtype=np.int64):
        end = max(end_prev, min(max(int(v), 0), M))
        out.append((end_prev, end))
        end_prev = end
    return out


def grouped_gemm_contiguous_psum(dtype, A, B, psum, SFA=None, SFB=None,
                                 sfb_gran="block128", sf_fmt="f32", cols=None):
    """Contiguous M-grouped NT GEMM with prefix-sum routing, float64 result.

    A[M, K] codes; B[G, N, K] codes; psum[G]. FP8 scales: SFA[K/128, M]; SFB per expert
    as in the masked variant. Rows of expert e's segment (psum_segments) are
    D[r, :] = A[r, :] . B[e]^T; rows outside every segment are not computed.

    Returns (ref[M, N] float64 with NaN outside the segments, valid[M] bool).
    """
    A = np.asarray(A)
    B = np.asarray(B)
    M, K = A.shape
    G, N, _ = B.shape
    ref = np.full((M, N), np.nan)
    valid = np.zeros(M, bool)
    cols = np.arange(N) if cols is None else np.asarray(cols)
    for e, (r0, r1) in enumerate(psum_segments(psum, M)):
        if r1 <= r0:
            continue
        valid[r0:r1] = True
        a_hat = dequant_act_rows(dtype, A[r0:r1],
                                 None if SFA is None else np.asarray(SFA)[:, r0:r1], sf_fmt)
        b_hat = dequant_weight_rows(dtype, B[e][cols], cols,
                                    None if SFB is None else np.asarray(SFB)[e], sfb_gran, sf_fmt)
        ref[np.ix_(np.arange(r0, r1), cols)] = gemm_nt_fp64(a_hat, b_hat)
    return ref, valid


def kgrouped_ks_from_psum(psum):
    """Per-expert token counts of the K-grouped call's prefix-sum routing (its
    use_psum_layout argument, not described on the pages): psum[e] is the cumulative
    token end of expert e, so k_e = psum[e] - psum[e - 1] with psum[-1] = 0; a
    decreasing entry gives a negative count, which is out of contract."""
    ps = np.asarray(psum, dtype=np.int64)
    return np.diff(np.concatenate([[0], ps]))


def kgrouped_layout(ks, K_total: int, granule: int):
    """Per-expert (offset p_e, length k_e, usable) of the packed K-grouped operands.

    p_e = sum_{j<e} max(ks[j], 0). An expert is usable when 0 <= k_e, both k_e and p_e
    are multiples of `granule` (128 for FP8, so that every 128-token scale group lies
    inside one expert; 8 for BF16) and p_e + k_e <= K_total. Unusable experts are out of
    contract and have no defined output.
    """
    ks = np.asarray(ks, dtype=np.int64)
    out = []
    p = 0
    for k in ks:
        usable = bool(k >= 0 and k % granule == 0 and p % granule == 0 and p + k <= K_total)
        out.append((p, int(k), usable))
        p += max(int(k), 0)
    return out


def grouped_gemm_kgrouped(dtype, A, B, ks, M: int, N: int, K_total: int, SFA=None,
                          SFB=None, sf_fmt="f32", C=None, experts=None, rows=None,
                          cols=None):
    """K-grouped NT GEMM (weight-gradient form), float64 result.

    A: flat codes; expert e's block [M][k_e] starts at element M * p_e.
    B: flat codes; expert e's block [N][k_e] starts at element N * p_e.
    FP8 scales: SFA[K_total/128, M], SFB[K_total/128, N]; token t of expert e uses scale
    row (p_e + t) // 128 (the scale groups are 128 global tokens).
    C: optional fp32 [G, M, N] added to the product (accumulation, C aliasing D).

    Returns (ref[G, M, N] float64, usable[G] bool); unusable experts are NaN.
    """
    A = np.asarray(A).reshape(-1)
    B = np.asarray(B).reshape(-1)
    G = len(ks)
    granule = 128 if dtype == "fp8" else 8
    layout = kgrouped_layout(ks, K_total, granule)
    ref = np.full((G, M, N), np.nan)
    usable = np.array([u for (_, _, u) in layout])
    rows_all = np.arange(M) if rows is None else np.asarray(rows)
    cols_all = np.arange(N) if cols is None else np.asarray(cols)
    for e in (range(G) if experts is None else experts):
        p, k, ok = layout[e]
        if not ok:
            continue
        if k == 0:
            prod = np.zeros((rows_all.size, cols_all.size))
        else:
            a_blk = A[M * p: M * (p + k)].reshape(M, k)[rows_all]
            b_blk = B[N * p: N * (p + k)].reshape(N, k)[cols_all]
            a_hat = _decode_elems(dtype, a_blk)
            b_hat = _decode_elems(dtype, b_blk)
            if dtype == "fp8":
                kb = (p + np.arange(k)) // SCALE_K  # scale row of each token
                sfa = decode_scale(SFA, sf_fmt)  # [K_total/128, M]
                sfb = decode_scale(SFB, sf_fmt)
                a_hat = a_hat * sfa[kb][:, rows_all].T
                b_hat = b_hat * sfb[kb][:, cols_all].T
            prod = gemm_nt_fp64(a_hat, b_hat)
        if C is not None:
            prod = prod + np.asarray(C, dtype=np.float64)[e][np.ix_(rows_all, cols_all)]
        ref[e][np.ix_(rows_all, cols_all)] = prod
    return ref, usable


# --------------------------------------------------------------------------- comparison


def calc_diff(x, y) -> float:
    """1 - 2 sum(xy) / sum(x^2 + y^2) in float64; 0 when both inputs are all zero."""
    x = np.asarray(x, dtype=np.float64).ravel()
    y = np.asarray(y, dtype=np.float64).ravel()
    denom = float(np.sum(x * x + y * y))
    if denom == 0.0:
        return 0.0
    return 1.0 - 2.0 * float(np.sum(x * y)) / denom
