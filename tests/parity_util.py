"""Helpers for the GPU parity tests: run the HIP path through the binding, run the
oracle on the same bytes, and compare.

Comparison rules (all from the pages' validation descriptions, the tolerance numbers
from the stated acceptance bar):
  * valid rows only; padding rows and other experts' rows must keep the sentinel bytes
    the output was filled with;
  * calc_diff against the FP64 reference rounded to bf16 (bf16 outputs) or unrounded
    (fp32 K-grouped outputs): < 1e-5 for BF16 inputs, < 1e-3 for FP8 inputs;
  * element by element: |gpu - ref| <= 2^-8 |ref| + 1.25 K 2^-24 S + 2^-6 T + tiny, where
    S = sum_k |a_k b_k| (the oracle run on sign-cleared codes) and T = sum over 128-K
    blocks of max|a| * max|b| within the block (dequantized, scales included). The first
    term is bf16 output rounding (zero for fp32 outputs), the second a first-order bound
    on FP32 accumulation over K products plus the per-128-K promotion roundings. The third
    (FP8 and FP8 x FP4 only) is the scaled MFMA's own sum of a block's 128 products,
    which measured on gfx950 aligns every product to the block's largest one and cuts it
    toward zero about 13 bits below (tests/test_gpu_mfma_block_error.py pins this): each
    product loses less than 2^-13 of the largest |product| <= max|a| max|b|, so a block
    sum is off by less than 128 * 2^-13 = 2^-6 of it.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from moe_grouped_gemm_nt_amd import synth

SENTINEL = synth.SENTINEL_BF16


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def np_codes(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


def abs_codes(codes: np.ndarray, dtype: str, weights: bool = False) -> np.ndarray:
    """Sign bits cleared: decodes to |value| for every element format (packed FP4 weight
    bytes carry two sign bits, bits 3 and 7)."""
    if dtype == "bf16":
        return codes & np.uint16(0x7FFF)
    if dtype == "fp8_fp4" and weights:
        return codes & np.uint8(0x77)
    return codes & np.uint8(0x7F)


def sentinel_like(shape, device) -> torch.Tensor:
    return torch.full(shape, SENTINEL - 65536, dtype=torch.int16, device=device).view(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return np_codes(t).astype(np.uint16)


def tol(dtype: str) -> float:
    return 1e-5 if dtype == "bf16" else 1e-3


# the scaled MFMA's block-sum error per unit of T (see the module docstring)
MFMA_ALIGN = {"bf16": 0.0, "fp8": 2.0 ** -6, "fp8_fp4": 2.0 ** -6}


def block_max_term(a_hat: np.ndarray, b_hat: np.ndarray) -> np.ndarray:
    """T[m, n] = sum over 128-K blocks of max_k |a_hat[m, k]| * max_k |b_hat[n, k]|."""
    a = np.abs(np.asarray(a_hat, np.float64))
    b = np.abs(np.asarray(b_hat, np.float64))
    K = a.shape[1]
    if K == 0:
        return np.zeros((a.shape[0], b.shape[0]))
    kb = -(-K // 128)
    pad = kb * 128 - K
    if pad:
        a = np.pad(a, ((0, 0), (0, pad)))
        b = np.pad(b, ((0, 0), (0, pad)))
    am = a.reshape(a.shape[0], kb, 128).max(axis=2)
    bm = b.reshape(b.shape[0], kb, 128).max(axis=2)
    return am @ bm.T


def elementwise_ok(gpu: np.ndarray, ref: np.ndarray, S: np.ndarray, K: int, rounded: bool,
                   dtype: str, T=None):
    if MFMA_ALIGN[dtype] and T is None:
        raise ValueError("FP8 comparisons need the block-max term T")
    bound = ((2.0 ** -8 * np.abs(ref) if rounded else 0.0) + 1.25 * K * 2.0 ** -24 * S
             + (MFMA_ALIGN[dtype] * T if MFMA_ALIGN[dtype] else 0.0) + 1e-30)
    err = np.abs(gpu - ref)
    bad = ~(err <= bound)
    return int(bad.sum()), float(np.max(err / bound)) if err.size else 0.0


# ----------------------------------------------------------------------------- masked


def run_masked(p: synth.Problem, expected_m=0, D=None):
    import moe_grouped_gemm_nt_amd as mgg
    if D is None:
        D = sentinel_like((p.G, p.cap, p.N), p.A.device)
    mgg.grouped_gemm_masked(p.A, p.B, D, p.counts, p.SFA, p.SFB, p.sfb_gran, expected_m)
    return D


def oracle_masked_expert(p: synth.Problem, g: int, rows=None, cols=None, host=None):
    """Oracle on expert g only (its slices copied to the host): (ref, S, valid_rows)."""
    h = host if host is not None else {}
    A = h.get("A", {}).get(g)
    if A is None:
        A = np_codes(p.A[g])[None]
    B = np_codes(p.B[g])[None]
    SFA = None if p.SFA is None else np_codes(p.SFA[g])[None]
    SFB = None if p.SFB is None else np_codes(p.SFB[g])[None]
    cnt = [int(p.meta["counts"][g])]
    rr = None if rows is None else {0: rows}
    ref, valid = oracle.grouped_gemm_masked(p.dtype, A, B, cnt, SFA, SFB, p.sfb_gran, p.sf_fmt,
                                            experts=[0], rows=rr, cols=cols)
    S, _ = oracle.grouped_gemm_masked(p.dtype, abs_codes(A, p.dtype), abs_codes(B, p.dtype, True), cnt,
                                      SFA, SFB, p.sfb_gran, p.sf_fmt, experts=[0], rows=rr,
                                      cols=cols)
    return ref[0], S[0], valid[0]


def masked_block_term(p: synth.Problem, g: int, rows, cols):
    """T of the element-wise bound for expert g's rows x cols (None for BF16)."""
    if not MFMA_ALIGN[p.dtype]:
        return None
    rows, cols = np.asarray(rows), np.asarray(cols)
    a_hat = oracle.dequant_act_rows(p.dtype, np_codes(p.A[g])[rows],
                                    np_codes(p.SFA[g])[:, rows], p.sf_fmt)
    b_hat = oracle.dequant_weight_rows(p.dtype, np_codes(p.B[g])[cols], cols,
                                       np_codes(p.SFB[g]), p.sfb_gran, p.sf_fmt)
    return block_max_term(a_hat, b_hat)


def check_masked(p: synth.Problem, D: torch.Tensor, experts=None, rows=None, cols=None,
                 check_sentinel=True):
    """Compares D with the oracle on the chosen experts/rows/cols. Returns a report."""
    Dh = bf16_bits(D)
    G = p.G
    experts = range(G) if experts is None else experts
    all_gpu, all_ref = [], []
    n_bad = 0
    worst = 0.0
    counts = np.clip(p.meta["counts"], 0, p.cap)
    for g in experts:
        rg = None if rows is None else rows[g]
        ref, S, valid = oracle_masked_expert(p, g, rg, cols)
        sel_rows = np.arange(counts[g]) if rg is None else np.array([m for m in rg if m < counts[g]], int)
        if sel_rows.size == 0:
            continue
        cc = np.arange(p.N) if cols is None else np.asarray(cols)
        gpu = oracle.decode_bf16(Dh[g][np.ix_(sel_rows, cc)])
        r = ref[np.ix_(sel_rows, cc)]
        s = S[np.ix_(sel_rows, cc)]
        T = masked_block_term(p, g, sel_rows, cc)
        nb, w = elementwise_ok(gpu, r, s, p.K, rounded=True, dtype=p.dtype, T=T)
        n_bad += nb
        worst = max(worst, w)
        all_gpu.append(gpu.ravel())
        all_ref.append(oracle.decode_bf16(oracle.round_to_bf16(r)).ravel())
    diff = oracle.calc_diff(np.concatenate(all_gpu), np.concatenate(all_ref)) if all_gpu else 0.0
    stray = 0
    if check_sentinel:
        invalid = np.arange(p.cap)[None, :] >= counts[:, None]
        stray = int((Dh[invalid] != SENTINEL).sum())
    return {"calc_diff": diff, "n_bad": n_bad, "worst": worst, "stray": stray}


def assert_report(rep, dtype):
    assert rep["stray"] == 0, f"{rep['stray']} output elements outside valid rows were written"
    assert rep["n_bad"] == 0, f"{rep['n_bad']} elements outside the error bound (worst ratio {rep['worst']:.3g})"
    assert rep["calc_diff"] < tol(dtype), f"calc_diff {rep['calc_diff']:.3e}"


# ----------------------------------------------------------------------------- contiguous


def run_contiguous(p: synth.Problem, expected_m=0, D=None):
    import moe_grouped_gemm_nt_amd as mgg
    if D is None:
        D = sentinel_like((p.M, p.N), p.A.device)
    mgg.grouped_gemm_contiguous(p.A, p.B, D, p.m_indices, p.SFA, p.SFB, p.sfb_gran, expected_m)
    return D


def cut_contiguous_rows(p: synth.Problem, M: int) -> synth.Problem:
    """The first M rows of a contiguous problem (M need not be a multiple of 128)."""
    idx = p.meta["m_indices"][:M]
    return synth.Problem("contiguous", p.dtype, p.G, p.N, p.K, p.A[:M].contiguous(), p.B,
                         None if p.SFA is None else p.SFA[:, :M].contiguous(), p.SFB,
                         p.sf_fmt, p.sfb_gran, M=M, m_indices=p.m_indices[:M].contiguous(),
                         meta={"m_indices": idx, "valid_rows": int((idx >= 0).sum())})


def check_contiguous(p: synth.Problem, D: torch.Tensor, rows=None, cols=None,
                     check_sentinel=True):
    Dh = bf16_bits(D)
    idx = p.meta["m_indices"]
    expert = oracle.contiguous_row_expert(idx, p.G)
    want = expert >= 0
    if rows is not None:
        sel = np.zeros(p.M, bool)
        sel[np.asarray(rows)] = True
        want &= sel
    cc = np.arange(p.N) if cols is None else np.asarray(cols)
    all_gpu, all_ref = [], []
    n_bad, worst = 0, 0.0
    for g in np.unique(expert[want]):
        r_idx = np.nonzero(want & (expert == g))[0]
        B = np_codes(p.B[int(g)])[None]
        SFB = None if p.SFB is None else np_codes(p.SFB[int(g)])[None]
        sub_idx = np.zeros(r_idx.size, np.int32)
        # only the rows under test leave the device (operands may be gigabytes)
        sel_t = torch.from_numpy(r_idx).to(p.A.device)
        A_r = np_codes(p.A.index_select(0, sel_t))
        sfa = None if p.SFA is None else np_codes(p.SFA.index_select(1, sel_t))
        ref, _ = oracle.grouped_gemm_contiguous(p.dtype, A_r, B, sub_idx, sfa, SFB,
                                                p.sfb_gran, p.sf_fmt, cols=cc)
        S, _ = oracle.grouped_gemm_contiguous(p.dtype, abs_codes(A_r, p.dtype),
                                              abs_codes(B, p.dtype, True), sub_idx, sfa, SFB,
                                              p.sfb_gran, p.sf_fmt, cols=cc)
        ref, S = ref[:, cc], S[:, cc]
        T = None
        if MFMA_ALIGN[p.dtype]:
            T = block_max_term(oracle.dequant_act_rows(p.dtype, A_r, sfa, p.sf_fmt),
                               oracle.dequant_weight_rows(p.dtype, B[0][cc], cc, SFB[0],
                                                          p.sfb_gran, p.sf_fmt))
        gpu = oracle.decode_bf16(Dh[np.ix_(r_idx, cc)])
        nb, w = elementwise_ok(gpu, ref, S, p.K, rounded=True, dtype=p.dtype, T=T)
        n_bad += nb
        worst = max(worst, w)
        all_gpu.append(gpu.ravel())
        all_ref.append(oracle.decode_bf16(oracle.round_to_bf16(ref)).ravel())
    diff = oracle.calc_diff(np.concatenate(all_gpu), np.concatenate(all_ref)) if all_gpu else 0.0
    stray = int((Dh[expert < 0] != SENTINEL).sum()) if check_sentinel else 0
    return {"calc_diff": diff, "n_bad": n_bad, "worst": worst, "stray": stray}


# ----------------------------------------------------------------------------- K-grouped


def run_kgrouped(p: synth.Problem, D=None, accumulate=True):
    import moe_grouped_gemm_nt_amd as mgg
    if D is None:
        D = torch.zeros((p.G, p.M, p.N), dtype=torch.float32, device=p.A.device)
    mgg.grouped_gemm_kgrouped(p.A, p.B, D, p.ks, p.M, p.N, p.SFA, p.SFB, accumulate)
    return D


def check_kgrouped(p: synth.Problem, D: torch.Tensor, C=None, experts=None, rows=None,
                   cols=None):
    """D (fp32, after the call) against C + product; C is the pre-call content (None: 0)."""
    Dh = D.detach().cpu().numpy()
    A, B = np_codes(p.A), np_codes(p.B)
    SFA = None if p.SFA is None else np_codes(p.SFA)
    SFB = None if p.SFB is None else np_codes(p.SFB)
    ks = list(p.meta["ks"])
    Cn = None if C is None else C.detach().cpu().numpy()
    ref, usable = oracle.grouped_gemm_kgrouped(p.dtype, A, B, ks, p.M, p.N, p.K_total, SFA, SFB,
                                               p.sf_fmt, C=Cn, experts=experts, rows=rows,
                                               cols=cols)
    S, _ = oracle.grouped_gemm_kgrouped(p.dtype, abs_codes(A, p.dtype), abs_codes(B, p.dtype), ks,
                                        p.M, p.N, p.K_total, SFA, SFB, p.sf_fmt,
                                        C=None if Cn is None else np.abs(Cn), experts=experts,
                                        rows=rows, cols=cols)
    rr = np.arange(p.M) if rows is None else np.asarray(rows)
    cc = np.arange(p.N) if cols is None else np.asarray(cols)
    all_gpu, all_ref = [], []
    n_bad, worst = 0, 0.0
    layout = oracle.kgrouped_layout(ks, p.K_total, 128 if p.dtype == "fp8" else 8)
    for e in (range(p.G) if experts is None else experts):
        if not usable[e]:
            continue
        gpu = Dh[e][np.ix_(rr, cc)].astype(np.float64)
        r = ref[e][np.ix_(rr, cc)]
        s = S[e][np.ix_(rr, cc)]
        T = None
        if MFMA_ALIGN[p.dtype]:
            pe, k, _ = layout[e]
            kb = (pe + np.arange(k)) // 128  # scale row of each of the expert's tokens
            a_hat = oracle.decode_e4m3fn(A[p.M * pe: p.M * (pe + k)].reshape(p.M, k)[rr]) * \
                oracle.decode_scale(SFA, p.sf_fmt)[kb][:, rr].T
            b_hat = oracle.decode_e4m3fn(B[p.N * pe: p.N * (pe + k)].reshape(p.N, k)[cc]) * \
                oracle.decode_scale(SFB, p.sf_fmt)[kb][:, cc].T
            T = block_max_term(a_hat, b_hat)
        nb, w = elementwise_ok(gpu, r, s, max(ks[e], 1) + 2, rounded=False,
                              dtype=p.dtype, T=T)
        n_bad += nb
        worst = max(worst, w)
        all_gpu.append(gpu.ravel())
        all_ref.append(r.ravel())
    diff = oracle.calc_diff(np.concatenate(all_gpu), np.concatenate(all_ref))
    return {"calc_diff": diff, "n_bad": n_bad, "worst": worst, "stray": 0, "ref": ref}


# ----------------------------------------------------------------------------- prefix sums


def run_psum(p: synth.Problem, expected_m=0, D=None, psum=None):
    import moe_grouped_gemm_nt_amd as mgg
    if D is None:
        D = sentinel_like((p.M, p.N), p.A.device)
    mgg.grouped_gemm_contiguous_psum(p.A, p.B, D, p.psum if psum is None else psum, p.SFA,
                                     p.SFB, p.sfb_gran, expected_m)
    return D


def check_psum(p: synth.Problem, D: torch.Tensor, psum=None, check_sentinel=True):
    """D against the prefix-sum oracle on every row of every segment; every row outside
    the segments must keep the sentinel."""
    Dh = bf16_bits(D)
    ps = p.meta["psum"] if psum is None else np.asarray(psum)
    A, B = np_codes(p.A), np_codes(p.B)
    SFA = None if p.SFA is None else np_codes(p.SFA)
    SFB = None if p.SFB is None else np_codes(p.SFB)
    ref, valid = oracle.grouped_gemm_contiguous_psum(p.dtype, A, B, ps, SFA, SFB, p.sfb_gran,
                                                     p.sf_fmt)
    S, _ = oracle.grouped_gemm_contiguous_psum(p.dtype, abs_codes(A, p.dtype),
                                               abs_codes(B, p.dtype, True), ps, SFA, SFB, p.sfb_gran,
                                               p.sf_fmt)
    T = None
    if MFMA_ALIGN[p.dtype]:
        T = np.zeros((p.M, p.N))
        for e, (r0, r1) in enumerate(oracle.psum_segments(ps, p.M)):
            if r1 > r0:
                rows = np.arange(r0, r1)
                T[r0:r1] = block_max_term(
                    oracle.dequant_act_rows(p.dtype, A[r0:r1], SFA[:, r0:r1], p.sf_fmt),
                    oracle.dequant_weight_rows(p.dtype, B[e], np.arange(p.N), SFB[e],
                                               p.sfb_gran, p.sf_fmt))
        T = T[valid]
    gpu = oracle.decode_bf16(Dh[valid])
    nb, w = elementwise_ok(gpu, ref[valid], S[valid], p.K, rounded=True, dtype=p.dtype, T=T)
    diff = oracle.calc_diff(gpu, oracle.decode_bf16(oracle.round_to_bf16(ref[valid])))
    stray = int((Dh[~valid] != SENTINEL).sum()) if check_sentinel else 0
    return {"calc_diff": diff, "n_bad": nb, "worst": w, "stray": stray}


# ----------------------------------------------------------------------------- SwiGLU


# Largest relative difference between the kernel's float32 h = silu(gate) * up (its fixed
# e^y evaluation: relative error below 1e-5, pinned against float64 exp) and the plain
# definition rounded once to float32: 1e-5 plus four float32 roundings (1 + e^-g, the
# division, the product with up, the final rounding of the float64 value), with margin.
SWIGLU_REL = 1.5e-5
# Where the two evaluations also differ in absolute terms: the fixed e^y saturates to
# +inf for -g > 88.7, so the kernel's silu is exactly 0 where the plain silu is below
# 2^-121. Groups whose largest plain value is below SWIGLU_TINY are compared by value
# (each dequantized code within 2^-99 of the plain value; no scale check, since a group
# the kernel sees as all zero takes the zero-group scale). Above it such elements round
# to code 0 on both sides (at most 2^-121 * 448 / 2^-100 < 2^-11 of a scale unit).
SWIGLU_TINY = 2.0 ** -100


def compare_swiglu_to_plain(h_codes, q, sf, fmt: str, sf_zero: float = 1.0):
    """Codes Q[M, I] and scales SF[I/128, M] of the SwiGLU + 1x128 step against the plain
    definition (float64 exp, rounded once to float32, then the 1x128 cast).

    Scales: float32 scales within SWIGLU_REL of the plain definition's; UE8M0 codes equal,
    or one apart where the plain definition's amax / 448 lies within SWIGLU_REL of the power
    of two between them ("scale flips"). Codes: with the scale the step chose, each code is
    the nearest E4M3 value (ties to even) of the plain value, or the other neighbour where
    the plain value lies within SWIGLU_REL of the midpoint between the two ("code flips").
    Returns counts of checked elements, mismatches and flips."""
    from oracle.quantize import encode_e4m3_rne
    _, sf_e, h = oracle.swiglu_quant_rows_1x128_exact(h_codes, fmt, sf_zero)
    M, I = h.shape
    G = I // 128
    hg = h.astype(np.float64).reshape(M, G, 128)
    amax = np.abs(hg).max(axis=2)
    tiny = amax < SWIGLU_TINY
    sf = np.asarray(sf)
    if fmt == "f32":
        sg = sf.T.astype(np.float64)
        se = np.asarray(sf_e).T.astype(np.float64)
        scale_bad = ~tiny & ~(np.abs(sg - se) <= SWIGLU_REL * se)
        scale_flip = np.zeros_like(scale_bad)
        sval = sg
    else:
        cg = sf.T.astype(np.int64)
        ce = np.asarray(sf_e).T.astype(np.int64)
        lower = np.ldexp(1.0, np.minimum(cg, ce) - 127)
        ratio = amax / 448.0
        near = np.abs(ratio - lower) <= SWIGLU_REL * lower
        scale_flip = ~tiny & (np.abs(cg - ce) == 1) & near
        scale_bad = ~tiny & (cg != ce) & ~scale_flip
        sval = np.ldexp(1.0, cg - 127)
    y = hg / sval[:, :, None]
    c0 = encode_e4m3_rne(y).reshape(M, G, 128)
    qg = np.asarray(q).reshape(M, G, 128)
    vg = oracle.decode_e4m3fn(qg)
    v0 = oracle.decode_e4m3fn(c0)
    same = vg == v0
    mg, m0 = qg & 0x7F, c0 & 0x7F
    adjacent = (np.abs(mg.astype(np.int64) - m0.astype(np.int64)) == 1) & \
        (((qg ^ c0) & 0x80 == 0) | (np.minimum(mg, m0) == 0))
    mid = 0.5 * (vg + v0)
    flip = ~same & adjacent & (np.abs(y - mid) <= SWIGLU_REL * np.abs(y) + 1e-300)
    code_bad = ~same & ~flip
    tiny_e = np.broadcast_to(tiny[:, :, None], code_bad.shape)
    by_value = np.abs(vg * sval[:, :, None] - hg) > 2.0 ** -99
    code_bad = np.where(tiny_e, by_value, code_bad)
    flip = flip & ~tiny_e
    return {"codes": int(qg.size), "code_bad": int(code_bad.sum()), "code_flips": int(flip.sum()),
            "groups": int(amax.size), "scale_bad": int(scale_bad.sum()),
            "scale_flips": int(scale_flip.sum()), "tiny_groups": int(tiny.sum())}


def assert_swiglu_plain(rep):
    assert rep["scale_bad"] == 0, f"{rep['scale_bad']} scales differ from the plain definition"
    assert rep["code_bad"] == 0, f"{rep['code_bad']} codes differ from the plain definition"
    # flips need the plain value within 1.5e-5 of a boundary: rare by construction
    assert rep["code_flips"] <= max(4, rep["codes"] // 1000), rep
    assert rep["scale_flips"] <= max(2, rep["groups"] // 1000), rep
