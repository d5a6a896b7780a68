"""The GPU parity checkers themselves, on the CPU: a "GPU output" built from the oracle
(correct by construction) must pass, and the same output with one planted mistake must be
reported and make assert_report raise: a write into a padding row, into another expert's
capacity rows or outside every segment, one element moved just outside the element-wise
bound, and a NaN. A checker that missed any of these would make the GPU tests vacuous."""

import numpy as np
import pytest
import torch

import oracle
from moe_grouped_gemm_nt_amd import synth
from parity_util import (MFMA_ALIGN, SENTINEL, abs_codes, assert_report, block_max_term,
                         check_contiguous, check_kgrouped, check_masked, check_psum,
                         elementwise_ok, masked_block_term, np_codes)


def as_bf16_tensor(codes: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(codes.astype(np.uint16).view(np.int16)).view(torch.bfloat16)


def bf16_step(code, steps: int):
    """The bf16 code `steps` representable values above (away from zero) code."""
    return np.uint16(int(code) + steps)


def moved(ref_val: float, bound: float, factor: float) -> np.uint16:
    """bf16 code of ref + factor * bound (away from zero)."""
    v = ref_val + np.copysign(factor * bound, ref_val if ref_val != 0 else 1.0)
    return np.uint16(oracle.round_to_bf16(np.array([v]))[0])


def bound_at(dtype, ref_val, S_val, K, T_val=0.0):
    return 2.0 ** -8 * abs(ref_val) + 1.25 * K * 2.0 ** -24 * S_val + MFMA_ALIGN[dtype] * T_val


def must_fail(rep, dtype):
    with pytest.raises(AssertionError):
        assert_report(rep, dtype)


# ----------------------------------------------------------------------------- masked


@pytest.fixture(scope="module")
def masked_case():
    counts = [5, 0, 9, 1]
    p = synth.make_masked("fp8", 4, 12, 136, 256, counts, seed=7)
    ref, valid = oracle.grouped_gemm_masked("fp8", np_codes(p.A), np_codes(p.B), counts,
                                            np_codes(p.SFA), np_codes(p.SFB))
    codes = np.where(valid[..., None], oracle.round_to_bf16(np.where(valid[..., None], ref, 0)),
                     np.uint16(SENTINEL)).astype(np.uint16)
    return p, codes, valid


def test_masked_correct_output_passes(masked_case):
    p, codes, _ = masked_case
    rep = check_masked(p, as_bf16_tensor(codes))
    assert rep["stray"] == 0 and rep["n_bad"] == 0 and rep["calc_diff"] < 1e-12
    assert_report(rep, "fp8")


@pytest.mark.parametrize("where", ["padding_row", "empty_expert", "next_expert_capacity"])
def test_masked_stray_write_is_reported(masked_case, where):
    p, codes, _ = masked_case
    bad = codes.copy()
    g, m = {"padding_row": (0, 5), "empty_expert": (1, 0), "next_expert_capacity": (3, 11)}[where]
    bad[g, m, 17] = 0x3F80  # 1.0
    rep = check_masked(p, as_bf16_tensor(bad))
    assert rep["stray"] == 1
    must_fail(rep, "fp8")


def test_masked_element_outside_bound_is_reported(masked_case):
    """One element moved by 1.5 times its bound is reported; moved by half of it, not."""
    p, codes, valid = masked_case
    ref, _ = oracle.grouped_gemm_masked("fp8", np_codes(p.A), np_codes(p.B), p.meta["counts"],
                                        np_codes(p.SFA), np_codes(p.SFB))
    S, _ = oracle.grouped_gemm_masked("fp8", abs_codes(np_codes(p.A), "fp8"),
                                      abs_codes(np_codes(p.B), "fp8"), p.meta["counts"],
                                      np_codes(p.SFA), np_codes(p.SFB))
    for (g, m, n) in ((2, 4, 100), (0, 0, 3), (3, 0, 135)):
        T = masked_block_term(p, g, [m], [n])[0, 0]
        b = bound_at("fp8", ref[g, m, n], S[g, m, n], p.K, T)
        bad = codes.copy()
        bad[g, m, n] = moved(ref[g, m, n], b, 1.5)
        rep = check_masked(p, as_bf16_tensor(bad))
        assert rep["n_bad"] == 1 and rep["worst"] > 1.0, (g, m, n)
        must_fail(rep, "fp8")
        bad[g, m, n] = moved(ref[g, m, n], b, 0.5)
        assert check_masked(p, as_bf16_tensor(bad))["n_bad"] == 0, (g, m, n)


def test_masked_nan_is_reported(masked_case):
    p, codes, _ = masked_case
    bad = codes.copy()
    bad[0, 0, 0] = 0x7FC0
    rep = check_masked(p, as_bf16_tensor(bad))
    assert rep["n_bad"] == 1
    must_fail(rep, "fp8")


# ----------------------------------------------------------------------------- contiguous


def contiguous_output(p):
    idx = p.meta["m_indices"]
    ref, _ = oracle.grouped_gemm_contiguous(p.dtype, np_codes(p.A), np_codes(p.B), idx,
                                            np_codes(p.SFA), np_codes(p.SFB), p.sfb_gran, p.sf_fmt)
    routed = oracle.contiguous_row_expert(idx, p.G) >= 0
    return np.where(routed[:, None], oracle.round_to_bf16(np.where(routed[:, None], ref, 0)),
                    np.uint16(SENTINEL)).astype(np.uint16), routed


def test_contiguous_checker_reports_planted_mistakes():
    p = synth.make_contiguous("fp8", 3, 136, 256, [70, 0, 130], seed=8, sf_fmt="ue8m0",
                              M_max=512)
    codes, routed = contiguous_output(p)
    assert_report(check_contiguous(p, as_bf16_tensor(codes)), "fp8")
    pad_row = int(np.nonzero(~routed)[0][0])
    for plant in ("stray", "bound", "nan"):
        bad = codes.copy()
        if plant == "stray":
            bad[pad_row, 3] = 0x3F80
        elif plant == "bound":
            ref, _ = oracle.grouped_gemm_contiguous("fp8", np_codes(p.A)[5:6], np_codes(p.B),
                                                    [0], np_codes(p.SFA)[:, 5:6], np_codes(p.SFB),
                                                    p.sfb_gran, p.sf_fmt)
            S, _ = oracle.grouped_gemm_contiguous("fp8", abs_codes(np_codes(p.A)[5:6], "fp8"),
                                                  abs_codes(np_codes(p.B), "fp8"), [0],
                                                  np_codes(p.SFA)[:, 5:6], np_codes(p.SFB),
                                                  p.sfb_gran, p.sf_fmt)
            a_hat = oracle.dequant_act_rows("fp8", np_codes(p.A)[5:6], np_codes(p.SFA)[:, 5:6],
                                            p.sf_fmt)
            b_hat = oracle.dequant_weight_rows("fp8", np_codes(p.B)[0][[9]], [9],
                                               np_codes(p.SFB)[0], p.sfb_gran, p.sf_fmt)
            T = block_max_term(a_hat, b_hat)[0, 0]
            bad[5, 9] = moved(ref[0, 9], bound_at("fp8", ref[0, 9], S[0, 9], p.K, T), 1.5)
        else:
            bad[200, 1] = 0xFFC0
        rep = check_contiguous(p, as_bf16_tensor(bad))
        assert (rep["stray"] if plant == "stray" else rep["n_bad"]) == 1, plant
        must_fail(rep, "fp8")


def test_psum_checker_reports_planted_mistakes():
    p = synth.make_contiguous_psum("bf16", 3, 136, 64, [40, 3, 77], seed=9, tail=11)
    ref, valid = oracle.grouped_gemm_contiguous_psum("bf16", np_codes(p.A), np_codes(p.B),
                                                     p.meta["psum"])
    codes = np.where(valid[:, None], oracle.round_to_bf16(np.where(valid[:, None], ref, 0)),
                     np.uint16(SENTINEL)).astype(np.uint16)
    assert_report(check_psum(p, as_bf16_tensor(codes)), "bf16")
    bad = codes.copy()
    bad[p.M - 1, 0] = 0x3F80  # an unrouted tail row
    rep = check_psum(p, as_bf16_tensor(bad))
    assert rep["stray"] == 1
    must_fail(rep, "bf16")
    bad = codes.copy()
    # BF16 inputs: the bound is 2^-8 |ref| plus a tiny accumulation term, so three bf16
    # steps away from the correctly rounded value lies outside it
    bad[41, 7] = bf16_step(bad[41, 7], 3)
    rep = check_psum(p, as_bf16_tensor(bad))
    assert rep["n_bad"] == 1
    must_fail(rep, "bf16")


# ----------------------------------------------------------------------------- K-grouped


def test_kgrouped_checker_reports_planted_mistakes():
    p = synth.make_kgrouped("fp8", [128, 256], 64, 72, seed=10, std_a=1.0, std_b=1.0)
    ref, _ = oracle.grouped_gemm_kgrouped("fp8", np_codes(p.A), np_codes(p.B), [128, 256], 64, 72,
                                          p.K_total, np_codes(p.SFA), np_codes(p.SFB))
    D = torch.from_numpy(ref.astype(np.float32))
    assert_report(check_kgrouped(p, D), "fp8")
    S, _ = oracle.grouped_gemm_kgrouped("fp8", abs_codes(np_codes(p.A), "fp8"),
                                        abs_codes(np_codes(p.B), "fp8"), [128, 256], 64, 72,
                                        p.K_total, np_codes(p.SFA), np_codes(p.SFB))
    # expert 1 (tokens 128..383): its dequantized rows 3 and columns 4 give T[1, 3, 4]
    A = oracle.decode_e4m3fn(np_codes(p.A)[64 * 128: 64 * 384].reshape(64, 256)[3])
    B = oracle.decode_e4m3fn(np_codes(p.B)[72 * 128: 72 * 384].reshape(72, 256)[4])
    kb = (128 + np.arange(256)) // 128
    a_hat = A * np_codes(p.SFA)[kb, 3]
    b_hat = B * np_codes(p.SFB)[kb, 4]
    T = block_max_term(a_hat[None], b_hat[None])[0, 0]
    bound = 1.25 * (256 + 2) * 2.0 ** -24 * S[1, 3, 4] + MFMA_ALIGN["fp8"] * T
    bad = D.clone()
    bad[1, 3, 4] += float(3 * bound)
    rep = check_kgrouped(p, bad)
    assert rep["n_bad"] == 1
    must_fail(rep, "fp8")
    bad = D.clone()
    bad[0, 10, 10] = float("nan")
    must_fail(check_kgrouped(p, bad), "fp8")


def test_elementwise_bound_terms():
    """The bound's terms one by one: bf16 rounding (rounded outputs only), the FP32
    accumulation term and the FP8 block-sum term 2^-6 T (none for BF16)."""
    ref = np.array([1.0, 1.0, 1.0])
    S = np.array([1.0, 1.0, 1.0])
    T = np.array([1.0, 1.0, 1.0])
    half_ulp = 2.0 ** -8
    n, _ = elementwise_ok(ref + np.array([0.99 * half_ulp, 0, 0]), ref, S, 1, True, "bf16")
    assert n == 0
    n, _ = elementwise_ok(ref + np.array([0, 1.02 * half_ulp + 1e-7, 0]), ref, S, 1, True, "bf16")
    assert n == 1
    # unrounded (fp32) output: the bf16 term drops out
    n, _ = elementwise_ok(ref + np.array([0, 0, 1e-5]), ref, S, 1, False, "bf16")
    assert n == 1
    n, _ = elementwise_ok(ref + np.array([0, 0, 0.99 * 2.0 ** -6]), ref, S, 1, False, "fp8", T)
    assert n == 0
    n, _ = elementwise_ok(ref + np.array([0, 0, 1.01 * 2.0 ** -6]), ref, S, 1, False, "fp8_fp4", T)
    assert n == 1
    with pytest.raises(ValueError):
        elementwise_ok(ref, ref, S, 1, False, "fp8")


def test_block_max_term():
    a = np.zeros((2, 256))
    b = np.zeros((3, 256))
    a[0, 5], a[0, 200] = -4.0, 0.5   # block 0 max 4, block 1 max 0.5
    a[1, 130] = 2.0                  # block 1 only
    b[0, :] = 1.0
    b[1, 127] = -3.0                 # block 0 only
    b[2, 255] = 8.0                  # block 1 only
    T = block_max_term(a, b)
    assert T.tolist() == [[4.5, 12.0, 4.0], [2.0, 0.0, 16.0]]
    # a ragged K is padded with zeros
    assert block_max_term(a[:, :130], b[:, :130]).tolist() == [[4.0, 12.0, 0.0], [0.0, 0.0, 0.0]]
