"""Seeded random sweep of the GPU parity: many small problems with shapes, routing values,
element types, scale formats and tile choices drawn at random (ragged N and K, empty
experts, out-of-range routing values, BF16 K tails, accumulation onto random C), each
compared with the oracle element by element, by calc_diff and by the sentinel rule.

Each case prints its parameters before it runs, so a failure names its case."""

import numpy as np
import pytest
import torch

from moe_grouped_gemm_nt_amd import synth
from parity_util import (assert_report, check_contiguous, check_kgrouped, check_masked,
                         check_psum, run_contiguous, run_kgrouped, run_masked, run_psum, say)

pytestmark = pytest.mark.gpu
DEV = "cuda"

TYPES = [("bf16", "f32", "block128"), ("fp8", "f32", "block128"), ("fp8", "f32", "channel"),
         ("fp8", "ue8m0", "block128"), ("fp8", "ue8m0", "channel"),
         ("fp8_fp4", "ue8m0", "block32")]


def m_cases(n=72, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        variant = ["masked", "contiguous", "psum"][c % 3]
        dt, sf, gran = TYPES[rng.integers(len(TYPES))]
        G = int(rng.integers(1, 10))
        N = 8 * int(rng.integers(1, 49))
        # K up to 1024 bytes per row: contiguous calls with at most 512 take the tiles
        # with streamed weight copies, longer ones the plain tiles
        K = 128 * int(rng.integers(1, 9)) if dt != "bf16" else 8 * int(rng.integers(1, 65))
        em = int(rng.choice([0, 8, 48, 200]))
        out.append(dict(case=c, variant=variant, dt=dt, sf=sf, gran=gran, G=G, N=N, K=K,
                        em=em, seed=int(rng.integers(1 << 30))))
    return out


@pytest.mark.parametrize("cfg", m_cases(), ids=lambda c: f"m{c['case']}-{c['variant']}-{c['dt']}")
def test_random_m_grouped(cfg):
    say("random", cfg)
    rng = np.random.default_rng(cfg["seed"])
    dt, sf, gran, G, N, K, em = (cfg[k] for k in ("dt", "sf", "gran", "G", "N", "K", "em"))
    if cfg["variant"] == "masked":
        cap = int(rng.integers(1, 301))
        counts = rng.integers(-5, cap + 6, size=G)  # outside [0, cap] is clamped
        p = synth.make_masked(dt, G, cap, N, K, np.clip(counts, 0, cap), cfg["seed"], DEV,
                              sf_fmt=sf, sfb_gran=gran)
        p.counts.copy_(torch.tensor(counts, dtype=torch.int32))
        D = run_masked(p, em)
        torch.cuda.synchronize()
        assert_report(check_masked(p, D), dt)
    elif cfg["variant"] == "contiguous":
        segs = rng.integers(0, 201, size=G)
        padded = int(sum((s + 127) // 128 * 128 for s in segs))
        M_max = max(128, padded + 128 * int(rng.integers(0, 3)))
        p = synth.make_contiguous(dt, G, N, K, segs, cfg["seed"], DEV, sf_fmt=sf, sfb_gran=gran,
                                  M_max=M_max)
        D = run_contiguous(p, em)
        torch.cuda.synchronize()
        assert_report(check_contiguous(p, D), dt)
    else:
        segs = rng.integers(0, 201, size=G)
        tail = int(rng.integers(0, 41))
        if int(segs.sum()) + tail == 0:
            tail = 1
        p = synth.make_contiguous_psum(dt, G, N, K, segs, cfg["seed"], DEV, sf_fmt=sf,
                                       sfb_gran=gran, tail=tail)
        D = run_psum(p, em)
        torch.cuda.synchronize()
        assert_report(check_psum(p, D), dt)


def k_cases(n=16, seed=77):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        dt = "fp8" if c % 2 == 0 else "bf16"
        G = int(rng.integers(1, 6))
        gran = 128 if dt == "fp8" else 8
        ks = [gran * int(rng.integers(0, 5 if dt == "fp8" else 60)) for _ in range(G)]
        out.append(dict(case=c, dt=dt, ks=ks, M=8 * int(rng.integers(1, 41)),
                        N=8 * int(rng.integers(1, 41)), acc=int(rng.integers(0, 2)),
                        seed=int(rng.integers(1 << 30)),
                        sf="ue8m0" if dt == "fp8" and (c // 2) % 2 else "f32"))
    return out


@pytest.mark.parametrize("cfg", k_cases(), ids=lambda c: f"k{c['case']}-{c['dt']}-{c['sf']}")
def test_random_k_grouped(cfg):
    say("random", cfg)
    if sum(cfg["ks"]) == 0:
        cfg = dict(cfg, ks=[128 if cfg["dt"] == "fp8" else 8] + cfg["ks"][1:])
    p = synth.make_kgrouped(cfg["dt"], cfg["ks"], cfg["M"], cfg["N"], cfg["seed"], DEV,
                            std_a=1.0, std_b=1.0, sf_fmt=cfg["sf"])
    g = torch.Generator(device=DEV).manual_seed(cfg["seed"])
    C = torch.randn((p.G, p.M, p.N), device=DEV, generator=g)
    D = C.clone()
    run_kgrouped(p, D, accumulate=bool(cfg["acc"]))
    torch.cuda.synchronize()
    assert_report(check_kgrouped(p, D, C=C if cfg["acc"] else None), cfg["dt"])
