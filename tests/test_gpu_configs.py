"""The pages' workloads at full size, in the launch configuration the benchmark times:
every valid row where the oracle finishes in seconds, sampled rows (all columns) of
sampled experts otherwise, plus the sentinel check of every byte outside valid rows."""

import numpy as np
import pytest
import torch

from moe_grouped_gemm_nt_amd import synth
from parity_util import (assert_report, check_contiguous, check_kgrouped, check_masked,
                         run_contiguous, run_kgrouped, run_masked, say)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_cfg_kgrouped_fp8_wgrad_full():
    """K-grouped FP8 wgrad, ks [256,128,128,256], M=N=2048, accumulating into a zeroed
    output exactly as the benchmark calls it; every output element checked."""
    for sf_val in (1.0, 1e-30):
        say("cfg kgrouped_fp8_wgrad sf_val", sf_val)
        p, opt = synth.make_workload("kgrouped_fp8_wgrad", DEV, sf_val=sf_val)
        D = torch.zeros((p.G, p.M, p.N), device=DEV)
        run_kgrouped(p, D, accumulate=opt["accumulate"])
        torch.cuda.synchronize()
        rep = check_kgrouped(p, D)
        assert_report(rep, "fp8")
        norms = torch.linalg.vector_norm(D.reshape(p.G, -1), dim=1).cpu().numpy()
        ref_norms = np.sqrt((rep["ref"].reshape(p.G, -1) ** 2).sum(axis=1))
        assert (norms <= np.maximum(100 * ref_norms, 1.0)).all()
        assert abs(norms.max() - 1.311e-3) / 1.311e-3 < 0.01


def test_cfg_masked_fp8_g32_n1536_full():
    say("cfg masked_fp8_g32_n1536")
    p, opt = synth.make_workload("masked_fp8_g32_n1536", DEV)
    D = run_masked(p, opt["expected_m"])
    torch.cuda.synchronize()
    assert_report(check_masked(p, D), "fp8")


@pytest.mark.parametrize("name", ["contig_fp8_w13", "contig_fp8_w2", "contig_fp8ch_w13"])
def test_cfg_contiguous_g288(name):
    say("cfg", name)
    p, opt = synth.make_workload(name, DEV)
    D = run_contiguous(p, opt["expected_m"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    idx = p.meta["m_indices"]
    valid_rows = np.nonzero(idx >= 0)[0]
    rows = np.sort(rng.choice(valid_rows, size=256, replace=False))
    # every row boundary of a few segments too
    starts = np.nonzero(np.diff(np.concatenate([[-1], idx])) != 0)[0]
    rows = np.unique(np.concatenate([rows, starts[:40], np.clip(starts[:40] - 1, 0, None)]))
    rows = rows[idx[rows] >= 0]
    assert_report(check_contiguous(p, D, rows=rows), "fp8")


@pytest.mark.parametrize("name", ["masked_fp8_g32_n6144", "masked_bf16_g32_n6144",
                                  "masked_fp8_g6_n4096", "masked_bf16_g6_n4096",
                                  "masked_fp8ch_g6_n4096"])
def test_cfg_masked_large(name):
    say("cfg", name)
    p, opt = synth.make_workload(name, DEV)
    D = run_masked(p, opt["expected_m"])
    torch.cuda.synchronize()
    counts = np.clip(p.meta["counts"], 0, p.cap)
    rng = np.random.default_rng(1)
    experts = sorted(rng.choice(p.G, size=min(4, p.G), replace=False).tolist())
    rows = {}
    for g in experts:
        c = int(counts[g])
        pick = set(rng.choice(c, size=min(6, c), replace=False).tolist()) if c else set()
        pick |= {0, max(c - 1, 0)}  # first and last valid row
        rows[g] = sorted(m for m in pick if m < c)
    say("  sampled", {g: r for g, r in rows.items()})
    rep = check_masked(p, D, experts=experts, rows=rows)
    assert_report(rep, p.dtype)
