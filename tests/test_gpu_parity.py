"""GPU parity of the HIP path against the CPU oracle at sizes the oracle finishes in
seconds: several tiles, ragged tails in every dimension, every dtype / scale format /
weight-scale granularity / tile shape, boundary capacities, empty experts, sentinel
checks of every byte outside valid rows, and tile-shape independence of the bits."""

import json
import os

import numpy as np
import pytest
import torch

import oracle
from moe_grouped_gemm_nt_amd import synth
from parity_util import (SENTINEL, assert_report, bf16_bits, check_contiguous, check_kgrouped,
                         check_masked, check_psum, cut_contiguous_rows, run_contiguous,
                         run_kgrouped, run_masked, run_psum, say)

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
DEV = "cuda"


# ----------------------------------------------------------------------------- masked


def test_masked_bf16_pr_repro():
    """The PR's reproduction: seed 29, G=8, cap=32, N=K=256, the printed counts, 16 calls,
    calc_diff < 1e-5 on valid rows every time; nothing outside valid rows written."""
    gold = json.load(open(os.path.join(GOLDEN, "masked_repro.json")))
    say("masked bf16 repro", gold["counts"])
    p = synth.make_masked("bf16", gold["G"], gold["cap"], gold["N"], gold["K"], gold["counts"],
                          seed=gold["seed"], device=DEV)
    first = None
    for call in range(gold["calls"]):
        D = run_masked(p, gold["expected_m"])
        torch.cuda.synchronize()
        rep = check_masked(p, D)
        assert rep["calc_diff"] < gold["calc_diff_threshold"], (call, rep)
        assert_report(rep, "bf16")
        bits = bf16_bits(D)
        if first is None:
            first = bits
        assert (bits == first).all(), f"call {call} differs from call 0"


@pytest.mark.parametrize("dtype,sf_fmt,gran", [
    ("bf16", "f32", "block128"),
    ("fp8", "f32", "block128"),
    ("fp8", "f32", "channel"),
    ("fp8", "ue8m0", "block128"),
    ("fp8", "ue8m0", "channel"),
])
def test_masked_ragged_all_tiles(dtype, sf_fmt, gran):
    """G=5, cap=300 (not a tile multiple), N=520 (ragged last n tile), K=384 (3 slices);
    counts cover 0, 1, partial, full. Every tile shape gives the same bits."""
    G, cap, N, K = 5, 300, 520, 384
    counts = [0, 1, 77, 300, 129]
    say("masked ragged", dtype, sf_fmt, gran)
    p = synth.make_masked(dtype, G, cap, N, K, counts, seed=3, device=DEV, sf_fmt=sf_fmt,
                          sfb_gran=gran)
    outs = []
    for em in (16, 48, 200):  # picks the 32-, 64- and 128-row tiles
        say("  expected_m", em)
        D = run_masked(p, em)
        torch.cuda.synchronize()
        outs.append(bf16_bits(D))
    rep = check_masked(p, D)
    assert_report(rep, dtype)
    assert (outs[0] == outs[1]).all() and (outs[1] == outs[2]).all(), "tile shapes disagree"


def test_masked_bf16_k_tail():
    """BF16 with K=200: the last 128-byte slice is partly past the row end."""
    say("masked bf16 K tail")
    p = synth.make_masked("bf16", 3, 40, 64, 200, [40, 7, 33], seed=4, device=DEV)
    D = run_masked(p, 40)
    torch.cuda.synchronize()
    assert_report(check_masked(p, D), "bf16")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_masked_boundary_panel(dtype):
    """Capacities 1..257 (not tile-divisible among them), random counts including full
    and empty experts, a single-expert case and an all-empty case; other experts' rows
    and padding rows keep the sentinel."""
    gold = json.load(open(os.path.join(GOLDEN, "masked_boundary_panel.json")))
    rng = np.random.default_rng(gold["seed"])
    N, K = 64, 256
    for cap in gold["capacities"]:
        G = 4
        counts = rng.integers(0, cap + 1, size=G)
        counts[rng.integers(0, G)] = cap  # one full expert
        counts[rng.integers(0, G)] = max(cap - 1, 0)  # one nearly full
        say("boundary", dtype, "cap", cap, "counts", counts.tolist())
        p = synth.make_masked(dtype, G, cap, N, K, counts, seed=cap, device=DEV)
        for em in (0, cap):
            D = run_masked(p, em)
            torch.cuda.synchronize()
            assert_report(check_masked(p, D), dtype)
    say("boundary single expert", dtype)
    p = synth.make_masked(dtype, 1, 96, N, K, [95], seed=1, device=DEV)
    assert_report(check_masked(p, run_masked(p, 96)), dtype)
    say("boundary all empty", dtype)
    p = synth.make_masked(dtype, 6, 64, N, K, [0] * 6, seed=2, device=DEV)
    D = run_masked(p, 32)
    torch.cuda.synchronize()
    assert (bf16_bits(D) == SENTINEL).all()


def test_masked_out_of_range_counts_are_clamped():
    say("masked clamp")
    p = synth.make_masked("fp8", 3, 40, 64, 128, [40, 0, 7], seed=5, device=DEV)
    p.counts.copy_(torch.tensor([-3, 1000, 7], dtype=torch.int32))
    p.meta["counts"] = np.array([-3, 1000, 7])
    D = run_masked(p, 16)
    torch.cuda.synchronize()
    assert_report(check_masked(p, D), "fp8")


def test_masked_integer_exact_bitwise():
    """Operands in {-1, 0, 1} with power-of-two scales: every sum is a small integer,
    exact in FP32 and in bf16, so the GPU must equal the rounded oracle bit for bit."""
    say("masked integer exact")
    G, cap, N, K = 3, 70, 136, 256
    rng = np.random.default_rng(8)
    a = rng.integers(-1, 2, (G, cap, K)).astype(np.float32)
    b = rng.integers(-1, 2, (G, N, K)).astype(np.float32)
    A = torch.tensor(a).to(torch.float8_e4m3fn).view(torch.uint8).to(DEV)
    B = torch.tensor(b).to(torch.float8_e4m3fn).view(torch.uint8).to(DEV)
    SFA = torch.full((G, K // 128, cap), 0.5, device=DEV)
    SFB = torch.full((G, 2, K // 128), 2.0, device=DEV)
    counts = np.array([70, 3, 64], np.int32)
    p = synth.Problem("masked", "fp8", G, N, K, A, B, SFA, SFB, cap=cap,
                      counts=torch.tensor(counts, device=DEV), meta={"counts": counts})
    D = run_masked(p, 64)
    torch.cuda.synchronize()
    ref, valid = oracle.grouped_gemm_masked("fp8", A.cpu().numpy(), B.cpu().numpy(), counts,
                                            SFA.cpu().numpy(), SFB.cpu().numpy())
    want = oracle.round_to_bf16(np.where(valid[..., None], ref, 0))
    got = bf16_bits(D)
    assert (got[valid] == want[valid]).all()
    # the same integers as bf16 operands
    pb = synth.Problem("masked", "bf16", G, N, K, torch.tensor(a).to(torch.bfloat16).to(DEV),
                       torch.tensor(b).to(torch.bfloat16).to(DEV), cap=cap,
                       counts=torch.tensor(counts, device=DEV), meta={"counts": counts})
    D2 = run_masked(pb, 64)
    torch.cuda.synchronize()
    want2 = oracle.round_to_bf16(np.where(valid[..., None], ref, 0))  # same integers
    assert (bf16_bits(D2)[valid] == want2[valid]).all()


# ----------------------------------------------------------------------------- contiguous


@pytest.mark.parametrize("dtype,sf_fmt,gran", [
    ("bf16", "f32", "block128"),
    ("fp8", "f32", "block128"),
    ("fp8", "ue8m0", "block128"),
    ("fp8", "ue8m0", "channel"),
])
def test_contiguous_ragged(dtype, sf_fmt, gran):
    """Segments of 130, 0, 1, 127, 128 and 45 rows padded to 128, plus trailing padding
    blocks; N=264 (ragged); every tile shape gives the same bits; padding rows keep the
    sentinel."""
    segs = [130, 0, 1, 127, 128, 45]
    say("contiguous", dtype, sf_fmt, gran, segs)
    p = synth.make_contiguous(dtype, len(segs), 264, 256, segs, seed=6, device=DEV,
                              sf_fmt=sf_fmt, sfb_gran=gran, M_max=1152)
    outs = []
    for em in (8, 64, 128):
        say("  expected_m", em)
        D = run_contiguous(p, em)
        torch.cuda.synchronize()
        outs.append(bf16_bits(D))
    assert_report(check_contiguous(p, D), dtype)
    assert (outs[0] == outs[1]).all() and (outs[1] == outs[2]).all(), "tile shapes disagree"


@pytest.mark.parametrize("dtype,sf_fmt,gran", [
    ("bf16", "f32", "block128"),
    ("fp8", "f32", "block128"),
    ("fp8", "ue8m0", "channel"),
    ("fp8_fp4", "ue8m0", "block32"),
])
@pytest.mark.parametrize("M", [70, 326])
def test_contiguous_total_rows_not_a_block_multiple(dtype, sf_fmt, gran, M):
    """M = 70 (one partial block) and M = 326 (the last expert's block cut after its 70
    valid rows): the rows past M are not part of the operands; every tile shape gives the
    same bits and matches the oracle."""
    segs = [70] if M == 70 else [130, 70]
    say("contiguous rows", M, dtype, sf_fmt, gran)
    full = synth.make_contiguous(dtype, len(segs), 264, 384, segs, seed=8, device=DEV,
                                 sf_fmt=sf_fmt, sfb_gran=gran)
    p = cut_contiguous_rows(full, M)
    assert int(p.meta["m_indices"][-1]) == len(segs) - 1
    outs = []
    for em in (8, 64, 128):
        D = run_contiguous(p, em)
        torch.cuda.synchronize()
        outs.append(bf16_bits(D))
    assert_report(check_contiguous(p, D), dtype)
    assert all((o == outs[0]).all() for o in outs), "tile shapes disagree"


@pytest.mark.parametrize("dtype,sf_fmt,gran", [
    ("bf16", "f32", "block128"),
    ("fp8", "f32", "block128"),
    ("fp8", "ue8m0", "channel"),
    ("fp8_fp4", "ue8m0", "block32"),
])
def test_smallest_shapes(dtype, sf_fmt, gran):
    """The smallest sizes each entry point accepts: one expert, N = 8, K = 8 (BF16) or 128
    (FP8), one row (masked capacity 1, contiguous and prefix-sum M = 1), and a K-grouped
    call with M = 1, N = 8 and one group of tokens."""
    K = 8 if dtype == "bf16" else 128
    say("smallest", dtype, sf_fmt, gran)
    p = synth.make_masked(dtype, 1, 1, 8, K, [1], seed=9, device=DEV, sf_fmt=sf_fmt,
                          sfb_gran=gran)
    for em in (0, 1, 200):
        D = run_masked(p, em)
        torch.cuda.synchronize()
        assert_report(check_masked(p, D), dtype)
    p = cut_contiguous_rows(synth.make_contiguous(dtype, 1, 8, K, [1], seed=10, device=DEV,
                                                  sf_fmt=sf_fmt, sfb_gran=gran), 1)
    D = run_contiguous(p, 1)
    torch.cuda.synchronize()
    assert_report(check_contiguous(p, D), dtype)
    q = synth.make_contiguous_psum(dtype, 1, 8, K, [1], seed=11, device=DEV, sf_fmt=sf_fmt,
                                   sfb_gran=gran)
    assert q.M == 1
    D = run_psum(q, 1)
    torch.cuda.synchronize()
    assert_report(check_psum(q, D), dtype)
    if dtype == "fp8_fp4":
        return  # FP4 weights are M-grouped only
    ks = [8] if dtype == "bf16" else [128]
    r = synth.make_kgrouped(dtype, ks, 1, 8, seed=12, device=DEV, std_a=1.0,
                            zero_channel_k=-1, sf_fmt=sf_fmt)
    D = run_kgrouped(r, accumulate=False)
    torch.cuda.synchronize()
    assert_report(check_kgrouped(r, D), dtype)


def test_contiguous_matches_masked_bitwise():
    """The same expert rows through the masked and the contiguous entry points give
    identical bits (same engine, same K order)."""
    say("contiguous vs masked")
    G, cap, N, K = 3, 128, 256, 512
    counts = [128, 5, 77]
    pm = synth.make_masked("fp8", G, cap, N, K, counts, seed=12, device=DEV)
    Dm = bf16_bits(run_masked(pm, 128))
    idx, _ = synth.contiguous_indices(counts)
    A = torch.zeros((idx.size, K), dtype=torch.uint8, device=DEV)
    SFA = torch.zeros((K // 128, idx.size), device=DEV)
    r0 = 0
    rows = []
    for g, c in enumerate(counts):
        A[r0:r0 + c] = pm.A[g, :c]
        SFA[:, r0:r0 + c] = pm.SFA[g, :, :c]
        rows.append((r0, g, c))
        r0 += (c + 127) // 128 * 128
    pc = synth.Problem("contiguous", "fp8", G, N, K, A, pm.B, SFA, pm.SFB, M=idx.size,
                       m_indices=torch.tensor(idx, device=DEV),
                       meta={"m_indices": idx, "valid_rows": sum(counts)})
    Dc = bf16_bits(run_contiguous(pc, 64))
    for r0, g, c in rows:
        assert (Dc[r0:r0 + c] == Dm[g, :c]).all()


# ----------------------------------------------------------------------------- K-grouped


@pytest.mark.parametrize("sf_val", [1.0, 1e-4, 1e-8, 1e-30])
def test_kgrouped_fp8_repro_shape_small(sf_val):
    """The K-grouped repro's token split [256, 128, 128, 256] and zeroed channel at a
    reduced channel count (M=N=256): parity, exact zeros in row 0 of the 128-token
    experts, accumulation into a non-zero C."""
    ks = [256, 128, 128, 256]
    say("kgrouped fp8 small sf_val", sf_val)
    p = synth.make_kgrouped("fp8", ks, 256, 264, seed=0, sf_val=sf_val, device=DEV)
    C = torch.randn((4, 256, 264), device=DEV) * 1e-4
    D = C.clone()
    run_kgrouped(p, D, accumulate=True)
    torch.cuda.synchronize()
    rep = check_kgrouped(p, D, C=C)
    assert_report(rep, "fp8")
    D0 = run_kgrouped(p, None, accumulate=False)
    torch.cuda.synchronize()
    for e in (1, 2):
        assert (D0[e, 0] == 0).all(), "zero channel must give exact zeros"
    rep0 = check_kgrouped(p, D0)
    assert_report(rep0, "fp8")


def test_kgrouped_bf16_and_edge_ks():
    """BF16 with k_e = 0, a non-multiple-of-128 count (BF16 allows multiples of 8), and
    an out-of-contract expert that must be left untouched."""
    ks = [0, 200, 8, 64]
    say("kgrouped bf16", ks)
    p = synth.make_kgrouped("bf16", ks, 72, 136, seed=2, std_a=1.0, std_b=1.0, device=DEV,
                            K_total=288)
    C = torch.randn((4, 72, 136), device=DEV)
    D = C.clone()
    run_kgrouped(p, D, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(D[0], C[0]), "k_e = 0 with accumulation leaves D_e unchanged"
    assert_report(check_kgrouped(p, D, C=C), "bf16")
    # out of contract: k_1 = 13 (not a multiple of 8) -> expert 1 untouched, and every
    # later expert starts at an unaligned token offset -> untouched as well
    bad = torch.tensor([0, 13, 8, 64], dtype=torch.int32, device=DEV)
    D2 = C.clone()
    import moe_grouped_gemm_nt_amd as mgg
    mgg.grouped_gemm_kgrouped(p.A, p.B, D2, bad, 72, 136, accumulate=False)
    torch.cuda.synchronize()
    assert torch.equal(D2[1:], C[1:])
    assert (D2[0] == 0).all()


@pytest.mark.parametrize("sf_val", [1.0, 1e-30])
def test_kgrouped_ue8m0_scales(sf_val):
    """Power-of-two per-channel scales on both operands (the repro's zeroed channel
    included, so all-zero groups take the UE8M0 code of sf_val), with and without
    accumulation onto a random C: element-wise bound, calc_diff and exact zeros."""
    ks = [128, 384, 0, 256]
    say("kgrouped ue8m0", ks, sf_val)
    p = synth.make_kgrouped("fp8", ks, 192, 136, seed=9, std_a=1.0, std_b=1.0, device=DEV,
                            sf_val=sf_val, sf_fmt="ue8m0")
    assert p.SFA.dtype == torch.uint8
    D = run_kgrouped(p, None, accumulate=False)
    torch.cuda.synchronize()
    assert (D[0, 0] == 0).all(), "the zeroed channel gives exact zeros"
    assert_report(check_kgrouped(p, D), "fp8")
    C = torch.randn((p.G, p.M, p.N), device=DEV)
    D2 = C.clone()
    run_kgrouped(p, D2, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(D2[2], C[2]), "k_e = 0 with accumulation leaves D_e unchanged"
    assert_report(check_kgrouped(p, D2, C=C), "fp8")


# ----------------------------------------------------------------------------- prefix sums


@pytest.mark.parametrize("dtype,sf_fmt,gran", [
    ("bf16", "f32", "block128"),
    ("fp8", "f32", "block128"),
    ("fp8", "ue8m0", "channel"),
])
def test_psum_ragged_unaligned(dtype, sf_fmt, gran):
    """Prefix-sum routing: unaligned segments of 130, 0, 1, 127, 45 and 300 rows back to
    back, then 7 unrouted rows; N=264; every tile shape gives the same bits; rows outside
    the segments keep the sentinel."""
    segs = [130, 0, 1, 127, 45, 300]
    say("psum", dtype, sf_fmt, gran, segs)
    p = synth.make_contiguous_psum(dtype, len(segs), 264, 256, segs, seed=21, device=DEV,
                                   sf_fmt=sf_fmt, sfb_gran=gran, tail=7)
    outs = []
    for em in (8, 64, 256):
        say("  expected_m", em)
        D = run_psum(p, em)
        torch.cuda.synchronize()
        outs.append(bf16_bits(D))
    assert_report(check_psum(p, D), dtype)
    assert (outs[0] == outs[1]).all() and (outs[1] == outs[2]).all(), "tile shapes disagree"


def test_psum_routing_is_clamped():
    """Ends beyond M, negative and decreasing entries follow the stated reading (ends
    clamped to [0, M] and raised to the running maximum); nothing overlaps and nothing
    outside the resulting segments is written."""
    say("psum clamped")
    p = synth.make_contiguous_psum("fp8", 5, 136, 256, [40, 40, 40, 40, 40], seed=22,
                                   device=DEV)
    for ps in ([60, 30, -5, 150, 900], [0, 0, 0, 0, 0], [-1, 200, 10, 10, 200]):
        say("  psum", ps)
        t = torch.tensor(ps, dtype=torch.int32, device=DEV)
        D = run_psum(p, 64, psum=t)
        torch.cuda.synchronize()
        assert_report(check_psum(p, D, psum=ps), "fp8")


def test_psum_matches_contiguous_bitwise():
    """128-aligned segments routed by prefix sums and by per-row indices give the same
    bits."""
    say("psum vs m_indices")
    segs = [128, 256, 0, 128]
    p = synth.make_contiguous_psum("fp8", 4, 256, 512, segs, seed=23, device=DEV)
    idx = np.concatenate([np.full(c, e, np.int32) for e, c in enumerate(segs)])
    pc = synth.Problem("contiguous", "fp8", 4, 256, 512, p.A, p.B, p.SFA, p.SFB, M=p.M,
                       m_indices=torch.tensor(idx, device=DEV),
                       meta={"m_indices": idx, "valid_rows": int(sum(segs))})
    Dp = bf16_bits(run_psum(p, 128))
    Dc = bf16_bits(run_contiguous(pc, 128))
    assert (Dp == Dc).all()


@pytest.mark.parametrize("dtype", ["fp8", "bf16"])
def test_kgrouped_psum_matches_counts(dtype):
    """The K-grouped call with cumulative token ends gives the same bits as with counts,
    and matches the oracle."""
    import moe_grouped_gemm_nt_amd as mgg
    ks = [256, 128, 0, 128, 256]
    say("kgrouped psum", dtype, ks)
    p = synth.make_kgrouped(dtype, ks, 96, 200, seed=24, device=DEV)
    ps = torch.tensor(np.cumsum(ks).astype(np.int32), device=DEV)
    D1 = run_kgrouped(p, accumulate=False)
    D2 = torch.full_like(D1, 7.0)
    mgg.grouped_gemm_kgrouped(p.A, p.B, D2, ps, p.M, p.N, p.SFA, p.SFB, accumulate=False,
                              psum=True)
    torch.cuda.synchronize()
    assert torch.equal(D1, D2)
    assert_report(check_kgrouped(p, D2), dtype)


@pytest.mark.parametrize("mode", ["counts", "psum"])
def test_kgrouped_routing_beyond_int32(mode):
    """Routing values whose token prefix leaves the int32 range (K_total = 512).
    Counts [-128, 256, 2^31 - 128, 128]: expert 1 owns tokens 0 .. 255, expert 3 would
    start at token 2^31 + 128 (a 32-bit prefix wraps it to -2^31 + 128, a multiple of 128
    that passes the bounds test). Cumulative ends [256, 2^31 - 128, -2^31, -2^31 + 256]:
    expert 0 owns tokens 0 .. 255, expert 2's count is -(2^32 - 128) (+128 in 32-bit
    arithmetic, which would wrap expert 3's prefix to -2^31). Skipped experts keep D
    untouched; the usable one matches the oracle, which takes the exact counts."""
    import dataclasses
    import moe_grouped_gemm_nt_amd as mgg
    p = synth.make_kgrouped("fp8", [256, 128, 128], 64, 96, seed=31, std_a=1.0, std_b=1.0,
                            device=DEV)
    if mode == "counts":
        route = [-128, 256, 2 ** 31 - 128, 128]
        eff, want = route, [False, True, False, False]
    else:
        route = [256, 2 ** 31 - 128, -2 ** 31, -2 ** 31 + 256]
        eff = [route[0]] + [route[e] - route[e - 1] for e in range(1, 4)]
        want = [True, False, False, False]
    say("kgrouped routing beyond int32", mode, route)
    G = len(route)
    g = torch.Generator(device=DEV).manual_seed(31)
    C = torch.randn((G, p.M, p.N), device=DEV, generator=g)
    D = C.clone()
    mgg.grouped_gemm_kgrouped(p.A, p.B, D, torch.tensor(route, dtype=torch.int32, device=DEV),
                              p.M, p.N, p.SFA, p.SFB, accumulate=True, psum=(mode == "psum"))
    torch.cuda.synchronize()
    q = dataclasses.replace(p, G=G, meta=dict(p.meta, ks=np.asarray(eff, np.int64)))
    rep = check_kgrouped(q, D, C=C)
    usable = (~np.isnan(rep["ref"]).all(axis=(1, 2))).tolist()
    assert usable == want, usable
    for e in range(G):
        if not want[e]:
            assert torch.equal(D[e], C[e]), f"expert {e} must be left untouched"
    assert_report(rep, "fp8")


# ----------------------------------------------------------------------------- split last round
# 100 experts (or row blocks) of one 128-row tile each x 3 n-tiles of the 128 x 256 tile =
# 300 tiles: one full round of 256 workgroups and a last round of 44 tiles, which the
# scheduler splits along N (FP8: four pieces of 64 columns, BF16: two of 128). N = 520 makes
# the last n-tile ragged, so pieces of it start past N and must stay empty. Every output is
# checked against the oracle and bitwise against the 32-row tile, which does not split.


@pytest.mark.parametrize("variant", ["masked", "contiguous", "psum"])
@pytest.mark.parametrize("dtype,sf_fmt,gran", [
    ("fp8", "f32", "block128"),
    ("fp8", "f32", "channel"),  # contiguous: the four-wave 128 x 256 tile
    ("fp8", "ue8m0", "channel"),
    ("bf16", "f32", "block128"),
])
def test_split_last_round_ragged_n(variant, dtype, sf_fmt, gran):
    G, N, K = 100, 520, 256
    rng = np.random.default_rng(61)
    segs = rng.integers(1, 129, size=G)
    segs[[0, G - 1]] = [128, 1]
    say("split last round", variant, dtype, sf_fmt, gran)
    if variant == "masked":
        p = synth.make_masked(dtype, G, 128, N, K, segs, seed=61, device=DEV, sf_fmt=sf_fmt,
                              sfb_gran=gran)
        run, check = run_masked, check_masked
    elif variant == "contiguous":
        p = synth.make_contiguous(dtype, G, N, K, segs, seed=61, device=DEV, sf_fmt=sf_fmt,
                                  sfb_gran=gran, M_max=128 * G)
        run, check = run_contiguous, check_contiguous
    else:
        p = synth.make_contiguous_psum(dtype, G, N, K, segs, seed=61, device=DEV,
                                       sf_fmt=sf_fmt, sfb_gran=gran, tail=3)
        run, check = run_psum, check_psum
    outs = []
    for em in (16, 100):  # the 32-row tile, then the 128 x 256 tile
        say("  expected_m", em)
        D = run(p, em)
        torch.cuda.synchronize()
        outs.append(bf16_bits(D))
    assert_report(check(p, D), dtype)
    assert (outs[0] == outs[1]).all(), "the split tile disagrees with the 32-row tile"


# Masked calls whose expected rows pick the 32- or 64-row tile and whose weights reach
# 64 MB run that tile's streamed twin (weight copies with the streaming cache policy). The
# policy changes no value: every valid row against the oracle, every padding byte keeps
# its sentinel, and the 32-row and 64-row tiles give the same bits.
@pytest.mark.parametrize("dtype", ["fp8", "bf16"])
def test_masked_streamed_small_tiles(dtype):
    G, N, K = (8, 4096, 2048) if dtype == "fp8" else (4, 4096, 2048)  # 64 MiB of weights
    esz = 1 if dtype == "fp8" else 2
    assert G * N * K * esz >= 64 << 20
    rng = np.random.default_rng(71)
    counts = rng.integers(0, 65, size=G)
    counts[[0, G - 1]] = [64, 1]
    say("streamed small tiles", dtype, counts.tolist())
    p = synth.make_masked(dtype, G, 64, N, K, counts, seed=71, device=DEV)
    outs = []
    for em in (16, 48):  # the 32-row tile, then the 64-row tile (both streamed)
        say("  expected_m", em)
        D = run_masked(p, em)
        torch.cuda.synchronize()
        outs.append(bf16_bits(D))
    assert_report(check_masked(p, D), dtype)
    assert (outs[0] == outs[1]).all(), "the 32- and 64-row streamed tiles disagree"
