"""GPU parity at the library's documented maximum sizes: 4096 experts (every M-grouped
layout and the K-grouped one), the contiguous layout's 4096 row blocks (524288 rows, one
expert per block), an activation operand one row block short of 2 GiB (the largest byte
offsets a 32-bit buffer offset addresses), and expert counts whose scheduler tables push
the largest tiles out of LDS (the host then falls back to a smaller tile, which must give
the same bits). Oracle checks use sampled rows where the full output is large; every
padding row is checked to keep its sentinel."""

import numpy as np
import pytest
import torch

from moe_grouped_gemm_nt_amd import synth
from parity_util import (assert_report, bf16_bits, check_contiguous, check_kgrouped,
                         check_masked, check_psum, run_contiguous, run_kgrouped, run_masked,
                         run_psum, say, sentinel_like)

pytestmark = pytest.mark.gpu
DEV = "cuda"
MAX_EXPERTS = 4096
MAX_CONTIG_ROWS = 4096 * 128


def sample_rows(valid_rows, n, seed, must=()):
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(valid_rows, size=min(n, valid_rows.size), replace=False).tolist())
    pick |= {int(r) for r in must}
    return np.array(sorted(pick))


def test_contiguous_max_experts_and_rows():
    """4096 experts, each owning exactly one of the 4096 row blocks (1..128 valid rows),
    524288 rows in all; the 128 x 256 tile's scheduler table does not fit next to its
    pipeline, so the host falls back to 64-row tiles, and the 32-row tile gives the same
    bits."""
    rng = np.random.default_rng(11)
    segs = rng.integers(1, 129, size=MAX_EXPERTS)
    segs[[0, 1, MAX_EXPERTS - 1]] = [128, 1, 128]
    say("contiguous max experts/rows", int(segs.sum()))
    p = synth.make_contiguous("fp8", MAX_EXPERTS, 16, 128, segs, seed=11, device=DEV,
                              M_max=MAX_CONTIG_ROWS)
    assert p.M == MAX_CONTIG_ROWS
    outs = []
    for em in (113, 32):
        say("  expected_m", em)
        D = sentinel_like((p.M, p.N), DEV)
        run_contiguous(p, em, D)
        torch.cuda.synchronize()
        outs.append(bf16_bits(D))
    assert (outs[0] == outs[1]).all(), "tile shapes disagree"
    valid = np.nonzero(p.meta["m_indices"] >= 0)[0]
    rows = sample_rows(valid, 384, 1, must=(0, 128, MAX_CONTIG_ROWS - 128, valid[-1]))
    assert_report(check_contiguous(p, D, rows=rows), "fp8")


def test_contiguous_operand_just_under_2gib():
    """A is 524160 x 4096 FP8 bytes (4095 row blocks, 2 146 959 360 bytes < 2^31): the
    last expert's segment ends on the last row, so the largest activation byte offsets
    come within one row of 2^31. UE8M0 scales, 128 x 128 weight blocks."""
    M, K, N, G = 4095 * 128, 4096, 32, 8
    rng = np.random.default_rng(12)
    head = rng.integers(1, 40000, size=G - 1)
    padded = int(sum((s + 127) // 128 * 128 for s in head))
    segs = np.concatenate([head, [M - padded]])
    say("contiguous 2 GiB operand", segs.tolist())
    p = synth.make_contiguous("fp8", G, N, K, segs, seed=12, device=DEV, sf_fmt="ue8m0",
                              M_max=M)
    assert p.A.numel() == M * K and p.A.numel() < 2 ** 31
    assert p.meta["m_indices"][-1] == G - 1
    D = sentinel_like((M, N), DEV)
    run_contiguous(p, 113, D)
    torch.cuda.synchronize()
    valid = np.nonzero(p.meta["m_indices"] >= 0)[0]
    rows = sample_rows(valid, 256, 2, must=(valid[0], M - 3, M - 2, M - 1))
    assert_report(check_contiguous(p, D, rows=rows), "fp8")


@pytest.mark.parametrize("em", [24, 200])
def test_masked_max_experts(em):
    """4096 experts of capacity 40 (counts 0..40, the first empty, the last full); with
    expected M 200 the largest tile's scheduler table does not fit and the host falls
    back to the 64-row tile. Every row of 96 sampled experts against the oracle and the
    sentinel on every padding row of all 4096."""
    G, cap, N, K = MAX_EXPERTS, 40, 64, 256
    rng = np.random.default_rng(13)
    counts = rng.integers(0, cap + 1, size=G)
    counts[[0, G - 1]] = [0, cap]
    say("masked max experts, expected_m", em)
    p = synth.make_masked("fp8", G, cap, N, K, counts, seed=13, device=DEV)
    D = run_masked(p, em)
    torch.cuda.synchronize()
    experts = sorted(set(rng.choice(G, size=96, replace=False).tolist()) | {0, 1, G - 1})
    assert_report(check_masked(p, D, experts=experts), "fp8")


def test_psum_max_experts():
    """4096 back-to-back segments (many empty, ragged lengths) with a tail of rows past
    the last segment; every row checked."""
    G = MAX_EXPERTS
    rng = np.random.default_rng(14)
    segs = np.minimum(rng.poisson(6, size=G), 40)
    segs[rng.choice(G, size=400, replace=False)] = 0
    segs[G - 1] = 37
    say("psum max experts", int(segs.sum()))
    p = synth.make_contiguous_psum("fp8", G, 64, 128, segs, seed=14, device=DEV, tail=9)
    D = run_psum(p, 48)
    torch.cuda.synchronize()
    assert_report(check_psum(p, D), "fp8")


@pytest.mark.parametrize("dt", ["fp8", "bf16"])
def test_kgrouped_max_experts(dt):
    """4096 experts with 0, 1 or 2 token granules each, accumulating onto random C."""
    G = MAX_EXPERTS
    rng = np.random.default_rng(15)
    gran = 128 if dt == "fp8" else 8
    ks = [gran * int(k) for k in rng.integers(0, 3, size=G)]
    ks[0], ks[-1] = 0, 2 * gran
    say("kgrouped max experts", dt, sum(ks))
    p = synth.make_kgrouped(dt, ks, 32, 48, seed=15, device=DEV, std_a=1.0, std_b=1.0)
    g = torch.Generator(device=DEV).manual_seed(15)
    C = torch.randn((p.G, p.M, p.N), device=DEV, generator=g)
    D = C.clone()
    run_kgrouped(p, D, accumulate=True)
    torch.cuda.synchronize()
    assert_report(check_kgrouped(p, D, C=C), dt)
