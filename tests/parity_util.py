"""Helpers for the GPU parity tests: run the HIP path through the binding, run the
oracle on the same bytes, and compare.

Comparison rules (all from the pages' validation descriptions, the tolerance numbers
from the stated acceptance bar):
  * valid rows only; padding rows and other experts' rows must keep the sentinel bytes
    the output was filled with;
  * calc_diff against the FP64 reference rounded to bf16 (bf16 outputs) or unrounded
    (fp32 K-grouped outputs): < 1e-5 for BF16 inputs, < 1e-3 for FP8 inputs;
  * element by element: |gpu - ref| <= 2^-8 |ref| + 1.25 K 2^-24 S [+ 2^-14 S for FP8]
    + tiny, where S = sum_k |a_k b_k| (the oracle run on sign-cleared codes). The first
    term is bf16 output rounding (zero for fp32 outputs), the second a first-order bound
    on FP32 accumulation over K products plus the per-128-K promotion roundings. The
    third covers the FP8 MFMA's own sum of 128 products, whose internal precision is
    not published: measured on gfx950 it errs by up to about 1.3e-5 of that block's
    sum of |products| (roughly 2^-16); 2^-14 of S keeps a 4x margin. With FP4 weights
    each 32-K block carries its own scale inside one instruction; a probe with block
    scales spread over 15 binades measured up to 1.0e-4 of the sum of |products|, so
    that dtype takes 2^-12 (2.4x margin over that extreme).
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


# error of the scaled MFMA's own sum of 128 products, relative to their sum of |products|
MFMA_BLOCK_REL = {"bf16": 0.0, "fp8": 2.0 ** -14, "fp8_fp4": 2.0 ** -12}


def elementwise_ok(gpu: np.ndarray, ref: np.ndarray, S: np.ndarray, K: int, rounded: bool,
                   dtype: str):
    bound = ((2.0 ** -8 * np.abs(ref) if rounded else 0.0) + 1.25 * K * 2.0 ** -24 * S
             + MFMA_BLOCK_REL[dtype] * S + 1e-30)
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
        nb, w = elementwise_ok(gpu, r, s, p.K, rounded=True, dtype=p.dtype)
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
        gpu = oracle.decode_bf16(Dh[np.ix_(r_idx, cc)])
        nb, w = elementwise_ok(gpu, ref, S, p.K, rounded=True, dtype=p.dtype)
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
                                               "f32", C=Cn, experts=experts, rows=rows, cols=cols)
    S, _ = oracle.grouped_gemm_kgrouped(p.dtype, abs_codes(A, p.dtype), abs_codes(B, p.dtype), ks,
                                        p.M, p.N, p.K_total, SFA, SFB, "f32",
                                        C=None if Cn is None else np.abs(Cn), experts=experts,
                                        rows=rows, cols=cols)
    rr = np.arange(p.M) if rows is None else np.asarray(rows)
    cc = np.arange(p.N) if cols is None else np.asarray(cols)
    all_gpu, all_ref = [], []
    n_bad, worst = 0, 0.0
    for e in (range(p.G) if experts is None else experts):
        if not usable[e]:
            continue
        gpu = Dh[e][np.ix_(rr, cc)].astype(np.float64)
        r = ref[e][np.ix_(rr, cc)]
        s = S[e][np.ix_(rr, cc)]
        nb, w = elementwise_ok(gpu, r, s, max(ks[e], 1) + 2, rounded=False,
                              dtype=p.dtype)
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
    gpu = oracle.decode_bf16(Dh[valid])
    nb, w = elementwise_ok(gpu, ref[valid], S[valid], p.K, rounded=True, dtype=p.dtype)
    diff = oracle.calc_diff(gpu, oracle.decode_bf16(oracle.round_to_bf16(ref[valid])))
    stray = int((Dh[~valid] != SENTINEL).sum()) if check_sentinel else 0
    return {"calc_diff": diff, "n_bad": nb, "worst": w, "stray": stray}
