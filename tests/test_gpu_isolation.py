"""Bytes that no valid output depends on cannot change a valid output.

A masked expert's rows at or past its count, their activation scales, the weights and
weight scales of experts with no rows, a contiguous or prefix-sum call's unrouted rows and
a K-grouped call's unrouted tokens are filled with NaN bit patterns (bf16 0x7FC0, E4M3
0x7F, float32 NaN, UE8M0 0xFF; packed FP4 weights, which have no NaN, get the byte 0x7F)
after a clean call. The call is then repeated on a fresh output: every byte of it must
equal the clean call's bytes, so valid rows are bit-identical and nothing is written
outside them. The rows of
one expert are independent of each other in D = A B^T, so a NaN reaching a valid row can
only come from a read across rows, experts or tiles; a control poisons one valid row and
requires exactly that output row to change.
"""

import numpy as np
import pytest
import torch

from moe_grouped_gemm_nt_amd import synth
from parity_util import bf16_bits, run_contiguous, run_kgrouped, run_masked, run_psum, say

pytestmark = pytest.mark.gpu
DEV = "cuda"

TYPES = [("bf16", "f32", "block128"), ("fp8", "f32", "block128"), ("fp8", "f32", "channel"),
         ("fp8", "ue8m0", "block128"), ("fp8", "ue8m0", "channel"),
         ("fp8_fp4", "ue8m0", "block32")]


def poison_rows(t: torch.Tensor):
    """Fill a slice of operand codes in place: bf16 NaN, E4M3 NaN (packed FP4 weights,
    which have no NaN, get 0x7F: the values 6 and -6)."""
    if t.dtype == torch.bfloat16:
        t.view(torch.int16).fill_(0x7FC0)
    else:
        t.fill_(0x7F)


def poison_scales(t: torch.Tensor):
    if t.dtype == torch.float32:
        t.fill_(float("nan"))
    else:
        t.fill_(0xFF)  # UE8M0 NaN


@pytest.mark.parametrize("dtype,sf_fmt,gran", TYPES)
def test_masked_poison_outside_valid_rows(dtype, sf_fmt, gran):
    G, cap, N, K = 6, 200, 392, 512
    counts = [0, 1, 64, 130, 200, 0]
    say("masked poison", dtype, sf_fmt, gran)
    p = synth.make_masked(dtype, G, cap, N, K, counts, seed=41, device=DEV, sf_fmt=sf_fmt,
                          sfb_gran=gran)
    for em in (0, 24, 60, 150):
        clean = bf16_bits(run_masked(p, em))
        q = synth.make_masked(dtype, G, cap, N, K, counts, seed=41, device=DEV, sf_fmt=sf_fmt,
                              sfb_gran=gran)
        for g, c in enumerate(counts):
            poison_rows(q.A[g, c:])
            if q.SFA is not None:
                poison_scales(q.SFA[g, :, c:])
            if c == 0:
                poison_rows(q.B[g])
                if q.SFB is not None:
                    poison_scales(q.SFB[g])
        torch.cuda.synchronize()
        dirty = bf16_bits(run_masked(q, em))
        torch.cuda.synchronize()
        diff = int((clean != dirty).sum())
        assert diff == 0, f"expected_m={em}: {diff} output bytes changed by poisoned inputs"
    # control: a poisoned valid row (expert 3, row 5) reaches its own output row and no other
    poison_rows(q.A[3, 5:6])
    torch.cuda.synchronize()
    hit = bf16_bits(run_masked(q, 0))
    torch.cuda.synchronize()
    changed = np.argwhere((hit != dirty).any(axis=2)).tolist()
    assert changed == [[3, 5]], changed


@pytest.mark.parametrize("dtype,sf_fmt,gran", TYPES)
@pytest.mark.parametrize("variant", ["contiguous", "psum"])
def test_unrouted_rows_poison(variant, dtype, sf_fmt, gran):
    G, N, K = 5, 264, 384
    segs = [0, 70, 129, 3, 0]
    say(variant, "poison", dtype, sf_fmt, gran)

    def make():
        if variant == "contiguous":
            return synth.make_contiguous(dtype, G, N, K, segs, seed=43, device=DEV,
                                         sf_fmt=sf_fmt, sfb_gran=gran, M_max=640)
        return synth.make_contiguous_psum(dtype, G, N, K, segs, seed=43, device=DEV,
                                          sf_fmt=sf_fmt, sfb_gran=gran, tail=37)

    run = run_contiguous if variant == "contiguous" else run_psum
    p = make()
    if variant == "contiguous":
        unrouted = (p.m_indices < 0) | (p.m_indices >= G)
    else:
        unrouted = torch.ones(p.M, dtype=torch.bool, device=DEV)
        unrouted[:int(np.sum(segs))] = False
    assert bool(unrouted.any()) and not bool(unrouted.all())
    for em in (0, 48, 150):
        clean = bf16_bits(run(p, em))
        q = make()
        rows = unrouted.nonzero().flatten()
        if q.A.dtype == torch.bfloat16:
            q.A.view(torch.int16)[rows] = 0x7FC0
        else:
            q.A[rows] = 0x7F
        if q.SFA is not None:
            q.SFA[:, rows] = float("nan") if q.SFA.dtype == torch.float32 else 0xFF
        for g, c in enumerate(segs):
            if c == 0:
                poison_rows(q.B[g])
                if q.SFB is not None:
                    poison_scales(q.SFB[g])
        torch.cuda.synchronize()
        dirty = bf16_bits(run(q, em))
        torch.cuda.synchronize()
        diff = int((clean != dirty).sum())
        assert diff == 0, f"expected_m={em}: {diff} output bytes changed by poisoned inputs"


@pytest.mark.parametrize("dtype,sf_fmt", [("bf16", "f32"), ("fp8", "f32"), ("fp8", "ue8m0")])
@pytest.mark.parametrize("accumulate", [True, False])
def test_kgrouped_unrouted_tokens_poison(dtype, sf_fmt, accumulate):
    """The K-grouped call's token axis past the last expert (unrouted tokens of the packed
    operands and their scale groups) does not reach any output."""
    ks, M, N, K_total = [128, 0, 256, 384], 192, 264, 1024
    T = sum(ks)
    say("kgrouped poison", dtype, sf_fmt, accumulate)

    def make():
        return synth.make_kgrouped(dtype, ks, M, N, seed=47, device=DEV, std_a=1.0,
                                   K_total=K_total, sf_fmt=sf_fmt)

    def run(q):
        D = torch.full((q.G, M, N), 0.25, dtype=torch.float32, device=DEV)
        run_kgrouped(q, D, accumulate)
        torch.cuda.synchronize()
        return D.view(torch.int32).cpu().numpy()

    clean = run(make())
    q = make()
    poison_rows(q.A[T * M:])
    poison_rows(q.B[T * N:])
    if q.SFA is not None:
        poison_scales(q.SFA[T // 128:])
        poison_scales(q.SFB[T // 128:])
    dirty = run(q)
    diff = int((clean != dirty).sum())
    assert diff == 0, f"{diff} output words changed by poisoned unrouted tokens"
