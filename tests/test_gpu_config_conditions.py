"""The named configurations under the conditions the pages put them in, at full size:

* the G = 288 contiguous configuration (w13 N = 512, K = 4096 and w2 N = 4096, K = 256,
  UE8M0 scales) captured once into a hipGraph and replayed over routings redrawn from
  Poisson(113) per expert, an all-empty phase included, with the routing buffer rewritten
  in place between replays (the SM120 issue's failing case: a graph replayed after the
  batch changed; its verification comment's graph-mutation test): every replay equals the
  eager call bit for bit, sampled rows and every segment's first and last row match the
  oracle, and every padding row keeps the sentinel; the same for the fused w13 chain;
* the two large masked configurations (32 experts N = 6144 K = 7168, and 6 experts
  N = K = 4096), FP8 and BF16: every row and column of the largest and the smallest
  non-empty expert against the oracle (the PR's supplemental validation compares whole
  outputs with independent FP64 references);
* 1000 calls of the bench-shaped workloads, each into an output refilled with the
  sentinel, all bitwise equal to the first (the K-grouped issue's H200 check applied to
  every configuration)."""

import numpy as np
import pytest
import torch

import oracle
from moe_grouped_gemm_nt_amd import synth
from parity_util import (assert_report, assert_swiglu_plain, bf16_bits, check_contiguous,
                         check_masked, compare_swiglu_to_plain, np_codes, run_contiguous,
                         run_masked, say, sentinel_like)

pytestmark = pytest.mark.gpu
DEV = "cuda"
ROWS_PER_EXPERT_MAX = 256  # the fixed row budget of the G = 288 configuration


def redrawn_routings(G, lam, seeds):
    """Per-expert rows ~ Poisson(lam) for each seed, then an all-empty phase, then a
    draw with a few experts at the 129-row maximum (two 128-row blocks each)."""
    draws = [synth.contiguous_draw(G, lam, s, ROWS_PER_EXPERT_MAX) for s in seeds]
    draws.append(np.zeros(G, np.int32))
    big = synth.contiguous_draw(G, lam, 99, ROWS_PER_EXPERT_MAX)
    big[::37] = ROWS_PER_EXPERT_MAX - 127
    draws.append(big)
    return draws


def set_routing(p, segs):
    idx, valid = synth.contiguous_indices(segs, 128, p.M)
    p.m_indices.copy_(torch.from_numpy(idx))
    p.meta["m_indices"] = idx
    p.meta["valid_rows"] = valid
    p.meta["seg_counts"] = np.asarray(segs, np.int64)
    return idx


def boundary_and_sampled_rows(idx, n_random, seed):
    """Every segment's first and last row plus n_random random routed rows."""
    routed = np.nonzero(idx >= 0)[0]
    if routed.size == 0:
        return routed
    change = np.nonzero(np.diff(np.concatenate([[-2], idx, [-2]])) != 0)[0]
    firsts = change[:-1]
    lasts = change[1:] - 1
    ends = np.concatenate([firsts, lasts])
    ends = ends[(ends < idx.size) & (idx[np.clip(ends, 0, idx.size - 1)] >= 0)]
    rng = np.random.default_rng(seed)
    pick = rng.choice(routed, size=min(n_random, routed.size), replace=False)
    return np.unique(np.concatenate([ends, pick]))


@pytest.mark.parametrize("name", ["contig_fp8_w13", "contig_fp8_w2"])
def test_cfg4_graph_replay_redrawn_routing_full_size(name):
    say("cfg4 replay", name)
    p, opt = synth.make_workload(name, DEV)
    em = opt["expected_m"]
    D = sentinel_like((p.M, p.N), DEV)
    fill = sentinel_like((p.M, p.N), DEV)
    run_contiguous(p, em, D)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_contiguous(p, em, D)
    for ph, segs in enumerate(redrawn_routings(p.G, 113, seeds=(11, 12, 13, 14))):
        idx = set_routing(p, segs)
        say("  phase", ph, "valid rows", int((idx >= 0).sum()))
        D.copy_(fill)
        g.replay()
        torch.cuda.synchronize()
        got = bf16_bits(D)
        eager = bf16_bits(run_contiguous(p, em))
        torch.cuda.synchronize()
        assert (got == eager).all(), f"replay differs from eager in phase {ph}"
        rows = boundary_and_sampled_rows(idx, 96, seed=ph)
        rep = check_contiguous(p, D, rows=rows if rows.size else None)
        say("  ", {k: v for k, v in rep.items()})
        assert_report(rep, "fp8")


def test_cfg4_fused_chain_graph_replay_redrawn_routing_full_size():
    """w13 with the SwiGLU + UE8M0 re-quantization fused into its epilogue, then w2, in one
    graph at the full G = 288 shape, replayed over redrawn routings: each replay equals the
    eager chain bit for bit, the fused codes equal the separate steps' on every routed row
    and agree with the plain definition, and sampled w2 rows match the oracle run on the
    GPU's own codes."""
    import moe_grouped_gemm_nt_amd as mgg
    say("cfg4 fused chain replay")
    p, opt = synth.make_workload("contig_fp8_w13", DEV)
    em = opt["expected_m"]
    I, Hd = p.N // 2, p.K
    w2 = synth.make_contiguous("fp8", p.G, Hd, I, p.meta["seg_counts"], 3, DEV, sf_fmt="ue8m0",
                               M_max=p.M)
    Q = torch.zeros((p.M, I), dtype=torch.uint8, device=DEV)
    SF = torch.zeros((I // 128, p.M), dtype=torch.uint8, device=DEV)
    D = sentinel_like((p.M, Hd), DEV)
    fill = sentinel_like((p.M, Hd), DEV)

    def chain():
        mgg.grouped_gemm_contiguous_swiglu_quant(p.A, p.B, p.m_indices, p.SFA, p.SFB, Q, SF,
                                                 sfq_fmt="ue8m0")
        mgg.grouped_gemm_contiguous(Q, w2.B, D, p.m_indices, SF, w2.SFB, "block128", em)

    chain()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        chain()
    H = sentinel_like((p.M, p.N), DEV)
    for ph, segs in enumerate(redrawn_routings(p.G, 113, seeds=(21, 22, 23, 24))):
        idx = set_routing(p, segs)
        say("  phase", ph, "valid rows", int((idx >= 0).sum()))
        D.copy_(fill)
        g.replay()
        torch.cuda.synchronize()
        got_d, got_q, got_sf = bf16_bits(D), Q.clone(), SF.clone()
        D.copy_(fill)
        chain()
        torch.cuda.synchronize()
        assert (got_d == bf16_bits(D)).all(), f"replay differs from eager in phase {ph}"
        routed = torch.from_numpy(idx >= 0).to(DEV)
        if not bool(routed.any()):
            assert (got_d == synth.SENTINEL_BF16).all()
            continue
        assert torch.equal(got_q[routed], Q[routed]) and torch.equal(got_sf[:, routed], SF[:, routed])
        # the separate steps on the same routing: bf16 w13 output, then SwiGLU + quantization
        H.copy_(sentinel_like((p.M, p.N), DEV))
        mgg.grouped_gemm_contiguous(p.A, p.B, H, p.m_indices, p.SFA, p.SFB, "block128", em)
        Qs, SFs = mgg.swiglu_quant_fp8_1x128(H, sf_fmt="ue8m0")
        torch.cuda.synchronize()
        assert torch.equal(Q[routed], Qs[routed]) and torch.equal(SF[:, routed], SFs[:, routed])
        rows = idx >= 0
        rep = compare_swiglu_to_plain(np_codes(H)[rows], Q.cpu().numpy()[rows],
                                      SF.cpu().numpy()[:, rows], "ue8m0")
        say("  fused codes vs plain definition", rep)
        assert_swiglu_plain(rep)
        w2p = synth.Problem("contiguous", "fp8", p.G, Hd, I, Q, w2.B, SF, w2.SFB, "ue8m0",
                            "block128", M=p.M, m_indices=p.m_indices, meta=dict(p.meta))
        sample = boundary_and_sampled_rows(idx, 64, seed=100 + ph)
        assert_report(check_contiguous(w2p, D, rows=sample), "fp8")


@pytest.mark.parametrize("name", ["masked_fp8_g32_n6144", "masked_bf16_g32_n6144",
                                  "masked_fp8_g6_n4096", "masked_bf16_g6_n4096",
                                  "masked_fp8ch_g6_n4096"])
def test_cfg5_whole_experts(name):
    """Every row and column of the largest and the smallest non-empty expert, plus the
    sentinel on every byte outside the valid rows of all experts."""
    say("cfg5 whole experts", name)
    p, opt = synth.make_workload(name, DEV)
    D = run_masked(p, opt["expected_m"])
    torch.cuda.synchronize()
    counts = np.clip(p.meta["counts"], 0, p.cap)
    nonempty = np.nonzero(counts > 0)[0]
    experts = sorted({int(nonempty[np.argmax(counts[nonempty])]),
                      int(nonempty[np.argmin(counts[nonempty])])})
    say("  experts", experts, "rows", [int(counts[g]) for g in experts])
    rep = check_masked(p, D, experts=experts)
    say("  ", rep)
    assert_report(rep, p.dtype)


def _runner(name):
    p, opt = synth.make_workload(name, DEV)
    if p.variant == "masked":
        shape = (p.G, p.cap, p.N)
        return p, shape, lambda D: run_masked(p, opt["expected_m"], D)
    shape = (p.M, p.N)
    return p, shape, lambda D: run_contiguous(p, opt["expected_m"], D)


@pytest.mark.parametrize("name", ["masked_bf16_repro", "masked_fp8_g32_n1536", "contig_fp8_w13",
                                  "masked_fp8_g6_n4096", "masked_fp8ch_g6_n4096",
                                  "contig_fp8ch_w13"])
def test_1000_calls_bitwise(name):
    say("1000 calls", name)
    p, shape, run = _runner(name)
    fill = sentinel_like(shape, DEV)
    D = fill.clone()
    run(D)
    first = D.clone()
    bad = 0
    for it in range(1000):
        D.copy_(fill)
        run(D)
        if not torch.equal(D.view(torch.int16), first.view(torch.int16)):
            bad += 1
    torch.cuda.synchronize()
    assert bad == 0, f"{bad}/1000 calls differ from the first"
