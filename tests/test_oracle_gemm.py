"""Pins for the grouped-GEMM oracle, each against something other than the oracle:
exact rational brute force that indexes the raw layouts directly and decodes through
torch, integer-exact cases, one-hot weights, identities between the three variants,
the zero-channel exact zero and the printed reference norm of the K-grouped repro.
CPU only."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from moe_grouped_gemm_nt_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- independent helpers


def torch_decode(codes, dtype):
    """Element values through torch's own conversions (not the oracle's decoders)."""
    t = torch.as_tensor(np.ascontiguousarray(codes))
    if dtype == "fp8":
        return t.view(torch.float8_e4m3fn).double().numpy()
    return t.view(torch.int16).view(torch.bfloat16).double().numpy()


def np_codes(t: torch.Tensor):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def scale_value(sf, fmt):
    if fmt == "f32":
        return Fraction(float(sf))
    return Fraction(2) ** (int(sf) - 127)


def brute_masked(p, fmt):
    """Exact rationals, layouts indexed as the API defines them, loop by loop."""
    A = np_codes(p.A)
    B = np_codes(p.B)
    av = torch_decode(A, p.dtype)
    bv = torch_decode(B, p.dtype)
    SFA = None if p.SFA is None else p.SFA.numpy()
    SFB = None if p.SFB is None else p.SFB.numpy()
    counts = p.meta["counts"]
    out = {}
    for g in range(p.G):
        for m in range(min(max(int(counts[g]), 0), p.cap)):
            for n in range(p.N):
                acc = Fraction(0)
                for k in range(p.K):
                    a = Fraction(float(av[g, m, k]))
                    b = Fraction(float(bv[g, n, k]))
                    if p.dtype == "fp8":
                        a *= scale_value(SFA[g, k // 128, m], fmt)
                        if p.sfb_gran == "block128":
                            b *= scale_value(SFB[g, n // 128, k // 128], fmt)
                        else:
                            b *= scale_value(SFB[g, k // 128, n], fmt)
                    acc += a * b
                out[(g, m, n)] = acc
    return out


def run_masked_oracle(p):
    return oracle.grouped_gemm_masked(
        p.dtype, np_codes(p.A), np_codes(p.B), p.meta["counts"],
        None if p.SFA is None else p.SFA.numpy(), None if p.SFB is None else p.SFB.numpy(),
        p.sfb_gran, p.sf_fmt)


def rel_bound(p):
    """|fp64 - exact| <= K * 2^-52 * sum|terms|; the terms' magnitudes are bounded via
    the largest product, so a loose but safe per-element bound is used."""
    return p.K * 2.0 ** -52


# ---------------------------------------------------------------- masked


@pytest.mark.parametrize("dtype,fmt,gran", [
    ("bf16", "f32", "block128"),
    ("fp8", "f32", "block128"),
    ("fp8", "f32", "channel"),
    ("fp8", "ue8m0", "block128"),
    ("fp8", "ue8m0", "channel"),
])
def test_masked_bruteforce_exact(dtype, fmt, gran):
    p = synth.make_masked(dtype, G=3, cap=5, N=3, K=256, counts=[2, 0, 5], seed=1,
                          sf_fmt=fmt, sfb_gran=gran)
    ref, valid = run_masked_oracle(p)
    exact = brute_masked(p, fmt)
    assert valid.sum() == 7
    for (g, m, n), v in exact.items():
        x = ref[g, m, n]
        assert abs(Fraction(x) - v) <= Fraction(rel_bound(p)) * (abs(v) + 1e-300) * 64 + Fraction(1, 2 ** 200)
    assert np.isnan(ref[~valid]).all()


def test_masked_weight_blocks_span_n_boundary():
    """N=130 puts rows 128, 129 in the second 128-row weight-scale block."""
    p = synth.make_masked("fp8", G=1, cap=2, N=130, K=128, counts=[2], seed=3)
    ref, _ = run_masked_oracle(p)
    exact = brute_masked(p, "f32")
    for (g, m, n), v in exact.items():
        assert abs(ref[g, m, n] - float(v)) <= 1e-12 * abs(float(v)) + 1e-300


def test_masked_integer_exact():
    """Small-integer operands with power-of-two scales: every partial sum is an exact
    integer, so the oracle must equal an int64 matmul exactly."""
    rng = np.random.default_rng(5)
    G, cap, N, K = 2, 7, 9, 256
    a_int = rng.integers(-3, 4, (G, cap, K))
    b_int = rng.integers(-3, 4, (G, N, K))
    A = torch.tensor(a_int, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    B = torch.tensor(b_int, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    SFA = np.full((G, K // 128, cap), 0.5, np.float32)
    SFB = np.full((G, 1, K // 128), 4.0, np.float32)
    counts = [4, 7]
    ref, valid = oracle.grouped_gemm_masked("fp8", A, B, counts, SFA, SFB)
    want = np.einsum("gmk,gnk->gmn", a_int, b_int) * 2
    assert (ref[valid] == want[valid]).all()
    # bf16 operands, same integers
    Ab = torch.tensor(a_int, dtype=torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    Bb = torch.tensor(b_int, dtype=torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ref2, valid2 = oracle.grouped_gemm_masked("bf16", Ab, Bb, counts)
    assert (ref2[valid2] == want[valid2] / 2).all()


def test_masked_one_hot_weights_return_dequantized_activations():
    """B[g, n, k] = 1 iff k == n (scale 1): D[g, m, n] = A-hat[g, m, n]. Pins the
    activation scale layout [G][K/128][cap] and the row/column indexing."""
    G, cap, N, K = 2, 6, 256, 256
    p = synth.make_masked("fp8", G, cap, N, K, counts=[6, 3], seed=7)
    onehot = torch.zeros((N, K))
    onehot[torch.arange(N), torch.arange(N)] = 1.0
    B = onehot.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    B = np.stack([B] * G)
    SFB = np.ones((G, 2, 2), np.float32)
    ref, valid = oracle.grouped_gemm_masked("fp8", p.A.numpy(), B, [6, 3], p.SFA.numpy(), SFB)
    av = torch_decode(p.A.numpy(), "fp8")
    sfa = p.SFA.numpy()
    for g in range(G):
        for m in range(cap):
            if not valid[g, m]:
                continue
            want = av[g, m, :N] * np.repeat(sfa[g, :, m], 128)[:N]
            assert (ref[g, m] == want).all()


def test_masked_counts_clamped_and_all_empty():
    p = synth.make_masked("bf16", G=3, cap=4, N=2, K=8, counts=[0, 0, 0], seed=2)
    ref, valid = oracle.grouped_gemm_masked("bf16", np_codes(p.A), np_codes(p.B), [-5, 0, 99])
    assert valid.sum(axis=1).tolist() == [0, 0, 4]
    assert np.isnan(ref[0]).all() and not np.isnan(ref[2]).any()


def test_masked_sampled_matches_full():
    p = synth.make_masked("fp8", G=4, cap=40, N=300, K=384, counts=[40, 3, 0, 17], seed=9,
                          sfb_gran="block128")
    full, _ = run_masked_oracle(p)
    rows = {0: [0, 39], 1: [2], 3: [5, 16, 30]}
    cols = [0, 127, 128, 299]
    part, _ = oracle.grouped_gemm_masked(
        "fp8", p.A.numpy(), p.B.numpy(), p.meta["counts"], p.SFA.numpy(), p.SFB.numpy(),
        experts=[0, 1, 3], rows=rows, cols=cols)
    for g, ms in rows.items():
        for m in ms:
            if m < p.meta["counts"][g]:
                # BLAS may sum in another order for another shape: fp64 rounding only
                assert np.allclose(part[g, m, cols], full[g, m, cols], rtol=1e-12, atol=0)
    assert np.isnan(part[3, 30]).all()  # row 30 >= count 17 is never computed


# ---------------------------------------------------------------- contiguous


@pytest.mark.parametrize("dtype,fmt", [("bf16", "f32"), ("fp8", "f32"), ("fp8", "ue8m0")])
def test_contiguous_equals_masked_on_same_rows(dtype, fmt):
    """Concatenating the masked experts' valid rows (padded to 128 per expert) and
    routing them with m_indices gives the masked result row for row."""
    G, cap, N, K = 3, 130, 20, 256
    counts = [130, 0, 5]
    pm = synth.make_masked(dtype, G, cap, N, K, counts, seed=11, sf_fmt=fmt)
    ref_m, valid_m = run_masked_oracle(pm)
    idx, _ = synth.contiguous_indices(counts, 128)
    M = idx.size
    A = np.zeros((M, K), np_codes(pm.A).dtype)
    SFA = None
    if dtype == "fp8":
        SFA = np.zeros((K // 128, M), pm.SFA.numpy().dtype)
    row_of = []
    r0 = 0
    for g, c in enumerate(counts):
        for m in range(c):
            A[r0 + m] = np_codes(pm.A)[g, m]
            if SFA is not None:
                SFA[:, r0 + m] = pm.SFA.numpy()[g, :, m]
            row_of.append((r0 + m, g, m))
        r0 += (c + 127) // 128 * 128
    ref_c, valid_c = oracle.grouped_gemm_contiguous(
        dtype, A, np_codes(pm.B), idx, SFA, None if pm.SFB is None else pm.SFB.numpy(),
        "block128", fmt)
    assert valid_c.sum() == sum(counts)
    for r, g, m in row_of:
        assert (ref_c[r] == ref_m[g, m]).all()
    assert np.isnan(ref_c[~valid_c]).all()


def test_contiguous_out_of_range_indices_are_padding():
    p = synth.make_contiguous("bf16", G=2, N=4, K=16, seg_counts=[1, 1], seed=4, align=2)
    idx = np.array([0, -1, 1, 7], np.int32)
    ref, valid = oracle.grouped_gemm_contiguous("bf16", np_codes(p.A), np_codes(p.B), idx)
    assert valid.tolist() == [True, False, True, False]
    want = torch_decode(np_codes(p.A)[2], "bf16") @ torch_decode(np_codes(p.B)[1], "bf16").T
    assert np.allclose(ref[2], want, rtol=1e-14, atol=0)


# ---------------------------------------------------------------- K-grouped


def test_kgrouped_bruteforce_exact():
    ks = [128, 0, 256]
    M, N = 3, 2
    p = synth.make_kgrouped("fp8", ks, M, N, seed=5, std_a=1.0, std_b=1.0, sf_val=1.0)
    C = np.random.default_rng(1).standard_normal((3, M, N)).astype(np.float32)
    ref, usable = oracle.grouped_gemm_kgrouped("fp8", p.A.numpy(), p.B.numpy(), ks, M, N,
                                               p.K_total, p.SFA.numpy(), p.SFB.numpy(),
                                               C=C)
    assert usable.all()
    av = torch_decode(p.A.numpy(), "fp8")
    bv = torch_decode(p.B.numpy(), "fp8")
    sfa, sfb = p.SFA.numpy(), p.SFB.numpy()
    pe = 0
    for e, k in enumerate(ks):
        for i in range(M):
            for j in range(N):
                acc = Fraction(float(C[e, i, j]))
                for t in range(k):
                    a = Fraction(float(av[M * pe + i * k + t])) * Fraction(float(sfa[(pe + t) // 128, i]))
                    b = Fraction(float(bv[N * pe + j * k + t])) * Fraction(float(sfb[(pe + t) // 128, j]))
                    acc += a * b
                assert abs(Fraction(ref[e, i, j]) - acc) <= abs(acc) * Fraction(1, 2 ** 40) + Fraction(1, 2 ** 200)
        pe += k
    # k_e = 0 leaves exactly C
    assert (ref[1] == C[1]).all()


def test_kgrouped_equals_masked_per_expert():
    """Expert e of the K-grouped GEMM is a one-expert masked GEMM with K = k_e and
    per-channel weight scales."""
    ks = [256, 128]
    M, N = 5, 7
    p = synth.make_kgrouped("fp8", ks, M, N, seed=6, std_a=1.0, std_b=1.0)
    ref, _ = oracle.grouped_gemm_kgrouped("fp8", p.A.numpy(), p.B.numpy(), ks, M, N,
                                          p.K_total, p.SFA.numpy(), p.SFB.numpy())
    pe = 0
    for e, k in enumerate(ks):
        A = p.A.numpy()[M * pe: M * (pe + k)].reshape(1, M, k)
        B = p.B.numpy()[N * pe: N * (pe + k)].reshape(1, N, k)
        SFA = p.SFA.numpy()[pe // 128:(pe + k) // 128][None]
        SFB = p.SFB.numpy()[pe // 128:(pe + k) // 128][None]
        rm, _ = oracle.grouped_gemm_masked("fp8", A, B, [M], SFA, SFB, "channel")
        assert (rm[0] == ref[e]).all()
        pe += k


def test_kgrouped_contract_violations_unusable():
    lay = oracle.kgrouped_layout([128, 100, -3, 256], K_total=512, granule=128)
    # expert 3 starts at token 228, not a multiple of 128: unusable as well
    assert [u for (_, _, u) in lay] == [True, False, False, False]
    assert [p for (p, _, _) in lay] == [0, 128, 228, 228]
    lay = oracle.kgrouped_layout([128, -3, 256], K_total=512, granule=128)
    assert [u for (_, _, u) in lay] == [True, False, True]
    lay = oracle.kgrouped_layout([256, 256], K_total=384, granule=128)
    assert [u for (_, _, u) in lay] == [True, False]


@pytest.mark.parametrize("sf_val", [1.0, 1e-30])
def test_kgrouped_zero_channel_row_is_exact_zero(sf_val):
    """Channel 0 of grad_y is zero inside each 128-token expert, so row 0 of that
    expert's output is exactly zero whatever the zero-group scale is."""
    ks = [256, 128, 128, 256]
    p = synth.make_kgrouped("fp8", ks, 64, 48, seed=0, sf_val=sf_val)
    ref, _ = oracle.grouped_gemm_kgrouped("fp8", p.A.numpy(), p.B.numpy(), ks, 64, 48,
                                          p.K_total, p.SFA.numpy(), p.SFB.numpy())
    for e in (1, 2):
        assert (ref[e, 0] == 0).all()
    for e in (0, 3):
        assert (ref[e, 0] != 0).any()


@pytest.mark.slow
def test_kgrouped_repro_reference_norm_matches_printed_value():
    """The printed reference max norm of the K-grouped repro, 1.311e-03, is reproduced
    by the oracle on a fresh draw of the same recipe (to the printed 4 digits, which the
    draw-to-draw spread allows), and the closed form sigma_g*sigma_s*sqrt(k*M*N) agrees."""
    gold = json.load(open(os.path.join(GOLDEN, "kgrouped_repro.json")))
    ks, M, N = gold["ks"], gold["hidden_M"], gold["ffn_N"]
    closed = gold["grad_y_std"] * gold["act_std"] * np.sqrt(max(ks) * M * N)
    assert abs(closed - gold["printed_reference_max_norm"]) < 5e-7
    for sf_val in (1.0, 1e-30):
        p = synth.make_kgrouped("fp8", ks, M, N, seed=0, std_a=gold["grad_y_std"],
                                std_b=gold["act_std"], sf_val=sf_val)
        ref, _ = oracle.grouped_gemm_kgrouped("fp8", p.A.numpy(), p.B.numpy(), ks, M, N,
                                              p.K_total, p.SFA.numpy(), p.SFB.numpy())
        norms = np.sqrt((ref.reshape(len(ks), -1) ** 2).sum(axis=1))
        assert abs(norms.max() - gold["printed_reference_max_norm"]) / 1.311e-3 < 0.01
        # FP8 oracle vs the unquantized bf16 product: quantization noise only
        gy = p.meta["grad_y"].double().numpy()
        act = p.meta["act"].double().numpy()
        pe = 0
        for e, k in enumerate(ks):
            exact = gy[pe:pe + k].T @ act[pe:pe + k]
            assert oracle.calc_diff(ref[e], exact) < 2e-3
            thresh = max(100 * np.linalg.norm(exact), 1.0)
            assert norms[e] <= thresh
            pe += k


# ---------------------------------------------------------------- calc_diff


def test_calc_diff_closed_forms():
    x = np.array([1.0, -2.0, 3.0])
    assert oracle.calc_diff(x, x) == 0.0
    assert oracle.calc_diff(x, -x) == 2.0
    assert oracle.calc_diff(x, np.zeros(3)) == 1.0
    assert oracle.calc_diff(np.zeros(3), np.zeros(3)) == 0.0
    # y = x (1 + eps): 1 - 2(1+eps)/(1 + (1+eps)^2) = eps^2 / (2 + 2 eps + eps^2)
    eps = 1e-3
    want = eps ** 2 / (2 + 2 * eps + eps ** 2)
    assert abs(oracle.calc_diff(x, x * (1 + eps)) - want) < 1e-15


# ---------------------------------------------------------------- prefix-sum routing


def test_psum_segments_literal_cases():
    """The reading of the prefix-sum routing, case by case (hand-written expectations)."""
    assert oracle.psum_segments([3, 3, 10], 8) == [(0, 3), (3, 3), (3, 8)]
    # a decreasing end is raised to the running maximum: expert 1 is empty and expert 2
    # starts where expert 0 ended, so nothing overlaps
    assert oracle.psum_segments([10, 5, 20], 16) == [(0, 10), (10, 10), (10, 16)]
    assert oracle.psum_segments([-4, 2, 2], 5) == [(0, 0), (0, 2), (2, 2)]
    assert oracle.psum_segments([0, 0], 1) == [(0, 0), (0, 0)]


@pytest.mark.parametrize("dtype,fmt,gran", [
    ("bf16", "f32", "block128"),
    ("fp8", "f32", "block128"),
    ("fp8", "ue8m0", "channel"),
])
def test_contiguous_psum_equals_masked_per_segment(dtype, fmt, gran):
    """Each expert's segment, taken as a masked expert of capacity = its row count,
    gives the same rows through the masked oracle."""
    segs = [37, 0, 130, 1]
    p = synth.make_contiguous_psum(dtype, 4, 20, 256, segs, seed=8, sf_fmt=fmt,
                                   sfb_gran=gran, tail=5)
    A, B = np_codes(p.A), np_codes(p.B)
    SFA = None if p.SFA is None else p.SFA.numpy()
    SFB = None if p.SFB is None else p.SFB.numpy()
    ref, valid = oracle.grouped_gemm_contiguous_psum(dtype, A, B, p.meta["psum"], SFA, SFB,
                                                     gran, fmt)
    assert valid.sum() == sum(segs) and not valid[-5:].any()
    r0 = 0
    for e, c in enumerate(segs):
        if c:
            sfa_e = None if SFA is None else SFA[None, :, r0:r0 + c]
            ref_m, _ = oracle.grouped_gemm_masked(dtype, A[None, r0:r0 + c], B[e:e + 1], [c],
                                                  sfa_e, None if SFB is None else SFB[e:e + 1],
                                                  gran, fmt)
            assert (ref[r0:r0 + c] == ref_m[0]).all()
        r0 += c
    assert np.isnan(ref[~valid]).all()


def test_contiguous_psum_bruteforce_exact():
    """Exact rationals over the raw layouts (rows routed by the literal segments)."""
    p = synth.make_contiguous_psum("fp8", 2, 3, 256, [2, 3], seed=12, tail=1)
    A, B = np_codes(p.A), np_codes(p.B)
    av, bv = torch_decode(A, "fp8"), torch_decode(B, "fp8")
    SFA, SFB = p.SFA.numpy(), p.SFB.numpy()
    ref, valid = oracle.grouped_gemm_contiguous_psum("fp8", A, B, [2, 5], SFA, SFB)
    assert valid.tolist() == [True] * 5 + [False]
    for r, e in [(0, 0), (1, 0), (2, 1), (3, 1), (4, 1)]:
        for n in range(3):
            acc = Fraction(0)
            for k in range(256):
                acc += (Fraction(float(av[r, k])) * Fraction(float(SFA[k // 128, r])) *
                        Fraction(float(bv[e, n, k])) * Fraction(float(SFB[e, n // 128, k // 128])))
            assert abs(Fraction(ref[r, n]) - acc) <= abs(acc) * Fraction(1, 2 ** 40) + Fraction(1, 2 ** 200)


def test_kgrouped_ks_from_psum_literal():
    assert oracle.kgrouped_ks_from_psum([256, 384, 512, 768]).tolist() == [256, 128, 128, 256]
    assert oracle.kgrouped_ks_from_psum([128, 0, 128]).tolist() == [128, -128, 128]
