"""GPU parity at the library's documented maximum sizes: 4096 experts (every M-grouped
layout and the K-grouped one), the contiguous layout's 4096 row blocks (524288 rows, one
expert per block), activation operands and outputs beyond 2 GiB in every layout (buffer
resources start at each tile's first row), and expert counts whose scheduler tables push
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


# ----------------------------------------------------------------------------- beyond 2 GiB
# Operand and output buffer resources start at each tile's first row, so tensors larger
# than 2 GiB are addressed with 32-bit offsets that never span more than one tile.


def test_contiguous_activations_beyond_2gib():
    """A = 524288 x 7168 FP8 bytes (3.76 GB, M K > 2^31), 8 experts with long segments, the
    last ending on the last row; sampled rows (every segment's first and last included)
    against the oracle and the sentinel on every padding row."""
    M, K, N, G = MAX_CONTIG_ROWS, 7168, 64, 8
    rng = np.random.default_rng(16)
    head = rng.integers(30000, 70000, size=G - 1)
    padded = int(sum((s + 127) // 128 * 128 for s in head))
    segs = np.concatenate([head, [M - padded]])
    say("contiguous A beyond 2 GiB", segs.tolist())
    p = synth.make_contiguous("fp8", G, N, K, segs, seed=16, device=DEV, M_max=M)
    assert p.A.numel() == M * K and p.A.numel() > 2 ** 31
    D = sentinel_like((M, N), DEV)
    run_contiguous(p, 113, D)
    torch.cuda.synchronize()
    idx = p.meta["m_indices"]
    valid = np.nonzero(idx >= 0)[0]
    starts = np.nonzero(np.diff(np.concatenate([[-2], idx])) != 0)[0]
    ends = np.nonzero(np.diff(np.concatenate([idx, [-2]])) != 0)[0]
    edges = [r for r in np.concatenate([starts, ends]) if idx[r] >= 0]
    rows = sample_rows(valid, 192, 3, must=edges + [M - 1])
    assert_report(check_contiguous(p, D, rows=rows), "fp8")


def test_contiguous_output_beyond_2gib():
    """D = 524288 x 2304 bf16 (2.4 GB, M N 2 > 2^31), BF16 operands with K = 64."""
    M, K, N, G = MAX_CONTIG_ROWS, 64, 2304, 4
    segs = np.array([150000, 1, 200000, M - 350208])
    say("contiguous D beyond 2 GiB", segs.tolist())
    p = synth.make_contiguous("bf16", G, N, K, segs, seed=17, device=DEV, M_max=M)
    D = sentinel_like((M, N), DEV)
    assert D.numel() * 2 > 2 ** 31
    run_contiguous(p, 128, D)
    torch.cuda.synchronize()
    valid = np.nonzero(p.meta["m_indices"] >= 0)[0]
    rows = sample_rows(valid, 128, 4, must=(0, 149999, 150016, 150144, valid[-1], M - 1))
    assert_report(check_contiguous(p, D, rows=rows), "bf16")


def test_psum_segment_beyond_2gib():
    """One prefix-sum segment of 300000 rows x K = 7168 (2.15 GB of activations), five
    unrouted tail rows; sampled rows against the oracle (through the per-row expert view of
    the same segments) and the sentinel on the tail."""
    G, K, N = 3, 7168, 64
    segs = [1000, 300000, 77]
    say("psum segment beyond 2 GiB", segs)
    p = synth.make_contiguous_psum("fp8", G, N, K, segs, seed=18, device=DEV, sf_fmt="ue8m0",
                                   tail=5)
    assert segs[1] * K > 2 ** 31
    D = sentinel_like((p.M, N), DEV)
    run_psum(p, 200, D)
    torch.cuda.synchronize()
    ends = np.cumsum(segs)
    idx = np.full(p.M, -1, np.int32)
    for e, (r0, r1) in enumerate(zip(np.concatenate([[0], ends[:-1]]), ends)):
        idx[r0:r1] = e
    rows = sample_rows(np.arange(ends[-1]), 160, 5,
                       must=(0, 999, 1000, 1001, 300999, 301000, ends[-1] - 1))
    view = synth.Problem("contiguous", "fp8", G, N, K, p.A, p.B, p.SFA, p.SFB, p.sf_fmt,
                         p.sfb_gran, M=p.M, meta={"m_indices": idx})
    assert_report(check_contiguous(view, D, rows=rows), "fp8")


def test_masked_expert_block_beyond_2gib():
    """One expert of capacity 131200 x K = 16384 FP8 (2.15 GB), all rows valid but the last."""
    G, cap, N, K = 1, 131200, 64, 16384
    counts = [cap - 1]
    say("masked expert block beyond 2 GiB")
    p = synth.make_masked("fp8", G, cap, N, K, counts, seed=19, device=DEV)
    assert cap * K > 2 ** 31
    D = run_masked(p, 4096)
    torch.cuda.synchronize()
    rows = {0: list(sample_rows(np.arange(cap - 1), 128, 6, must=(0, 1, cap - 3, cap - 2)))}
    assert_report(check_masked(p, D, experts=[0], rows=rows), "fp8")


def test_kgrouped_output_beyond_2gib():
    """K-grouped with M = N = 24576: the expert's fp32 output is 2.4 GB; sampled rows and
    columns (the first and last of each included) against the oracle."""
    M = N = 24576
    ks = [256]
    say("kgrouped D beyond 2 GiB")
    p = synth.make_kgrouped("fp8", ks, M, N, seed=20, device=DEV, std_a=1.0, std_b=1.0)
    D = torch.zeros((1, M, N), device=DEV)
    assert D.numel() * 4 > 2 ** 31
    run_kgrouped(p, D, accumulate=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([rng.choice(M, 48, replace=False), [0, 1, M - 2, M - 1]]))
    cols = np.unique(np.concatenate([rng.choice(N, 48, replace=False), [0, 1, N - 2, N - 1]]))
    assert_report(check_kgrouped(p, D, rows=rows, cols=cols), "fp8")
