"""GPU parity of the FP8 x FP4 M-grouped products (FP8 E4M3 activations with 1x128
UE8M0 scales, FP4 E2M1 weights with one UE8M0 scale per 32 K of a weight row) against the
oracle: masked, contiguous and prefix-sum routing over ragged shapes and every tile
shape, weight scales spread over many binades, graph replays with new routing,
run-to-run determinism, and the contiguous configuration's shapes at full size."""

import numpy as np
import pytest
import torch

from moe_grouped_gemm_nt_amd import synth
from parity_util import (assert_report, bf16_bits, check_contiguous, check_masked, check_psum,
                         run_contiguous, run_masked, run_psum, say, sentinel_like)

pytestmark = pytest.mark.gpu
DEV = "cuda"
DT = "fp8_fp4"


def test_fp4_masked_ragged_all_tiles():
    """G=5, cap=300, N=520 (ragged last n tile for every tile width), K=384; counts 0, 1,
    partial, full. Every tile shape gives the same bits."""
    G, cap, N, K = 5, 300, 520, 384
    counts = [0, 1, 77, 300, 129]
    say("fp4 masked ragged")
    p = synth.make_masked(DT, G, cap, N, K, counts, seed=3, device=DEV, sf_fmt="ue8m0",
                          sfb_gran="block32")
    outs = []
    for em in (16, 48, 200):
        say("  expected_m", em)
        D = run_masked(p, em)
        torch.cuda.synchronize()
        outs.append(bf16_bits(D))
    assert_report(check_masked(p, D), DT)
    assert (outs[0] == outs[1]).all() and (outs[1] == outs[2]).all(), "tile shapes disagree"


def test_fp4_contiguous_ragged():
    segs = [130, 0, 1, 127, 128, 45]
    say("fp4 contiguous", segs)
    p = synth.make_contiguous(DT, len(segs), 264, 256, segs, seed=6, device=DEV,
                              sf_fmt="ue8m0", sfb_gran="block32", M_max=1152)
    outs = []
    for em in (8, 64, 128):
        say("  expected_m", em)
        D = run_contiguous(p, em)
        torch.cuda.synchronize()
        outs.append(bf16_bits(D))
    assert_report(check_contiguous(p, D), DT)
    assert (outs[0] == outs[1]).all() and (outs[1] == outs[2]).all(), "tile shapes disagree"


def test_fp4_psum_ragged():
    segs = [130, 0, 1, 127, 45, 300]
    say("fp4 psum", segs)
    p = synth.make_contiguous_psum(DT, len(segs), 264, 256, segs, seed=21, device=DEV,
                                   sf_fmt="ue8m0", sfb_gran="block32", tail=7)
    outs = []
    for em in (8, 64, 256):
        say("  expected_m", em)
        D = run_psum(p, em)
        torch.cuda.synchronize()
        outs.append(bf16_bits(D))
    assert_report(check_psum(p, D), DT)
    assert (outs[0] == outs[1]).all() and (outs[1] == outs[2]).all(), "tile shapes disagree"


def test_fp4_block_scales_spread_over_binades():
    """Weight scales of neighbouring 32-K blocks differ by up to 2^12 (random per block),
    so every lane of an MFMA carries a different scale."""
    G, cap, N, K = 3, 96, 256, 512
    say("fp4 spread scales")
    p = synth.make_masked(DT, G, cap, N, K, [96, 50, 3], seed=31, device=DEV, sf_fmt="ue8m0",
                          sfb_gran="block32")
    g = torch.Generator(device=DEV).manual_seed(31)
    shift = torch.randint(-6, 7, p.SFB.shape, device=DEV, generator=g, dtype=torch.int32)
    p.SFB.copy_((p.SFB.to(torch.int32) + shift).clamp(1, 254).to(torch.uint8))
    D = run_masked(p, 96)
    torch.cuda.synchronize()
    assert_report(check_masked(p, D), DT)


def test_fp4_determinism_and_graph_replay():
    """Ten eager calls are bitwise identical; one captured contiguous call replayed with
    new routing values (an all-empty phase included) matches the eager call and the
    oracle every time."""
    G, N, K, M_max = 8, 256, 256, 2048
    rng = np.random.default_rng(7)
    draws = [np.minimum(rng.poisson(60, G), 200) for _ in range(2)]
    draws += [np.zeros(G, int), np.minimum(rng.poisson(150, G), 200)]
    say("fp4 graph")
    p = synth.make_contiguous(DT, G, N, K, draws[0], seed=7, device=DEV, sf_fmt="ue8m0",
                              sfb_gran="block32", M_max=M_max)
    D = sentinel_like((M_max, N), DEV)
    first = bf16_bits(run_contiguous(p, 64, D))
    for _ in range(10):
        run_contiguous(p, 64, D)
        assert (bf16_bits(D) == first).all()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_contiguous(p, 64, D)
    fill = sentinel_like((M_max, N), DEV)
    for ph, segs in enumerate(draws):
        idx, _ = synth.contiguous_indices(segs, 128, M_max)
        say("  phase", ph, segs.tolist())
        p.m_indices.copy_(torch.from_numpy(idx))
        p.meta["m_indices"] = idx
        D.copy_(fill)
        g.replay()
        torch.cuda.synchronize()
        got = bf16_bits(D)
        eager = bf16_bits(run_contiguous(p, 64))
        torch.cuda.synchronize()
        assert (got == eager).all()
        assert_report(check_contiguous(p, D), DT)


@pytest.mark.parametrize("name", ["contig_fp4_w13", "contig_fp4_w2"])
def test_fp4_contiguous_g288_full(name):
    """The contiguous configuration's w13 / w2 shapes (288 experts) with FP4 weights, in
    the launch configuration the benchmark times: sampled rows, all columns."""
    say("cfg", name)
    p, opt = synth.make_workload(name, DEV)
    D = run_contiguous(p, opt["expected_m"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    idx = p.meta["m_indices"]
    valid_rows = np.nonzero(idx >= 0)[0]
    rows = np.sort(rng.choice(valid_rows, size=256, replace=False))
    assert_report(check_contiguous(p, D, rows=rows), DT)


def test_fp4_masked_g6_n4096_sampled():
    say("cfg masked_fp4_g6_n4096")
    p, opt = synth.make_workload("masked_fp4_g6_n4096", DEV)
    D = run_masked(p, opt["expected_m"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    rows = [np.sort(rng.choice(max(int(c), 1), size=min(64, max(int(c), 1)), replace=False))
            for c in p.meta["counts"]]
    assert_report(check_masked(p, D, rows=rows), DT)
