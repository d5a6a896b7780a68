"""Calls on two HIP streams at once, and from two host threads at once, give the same bits
as the same calls made one after the other on one stream (each call reads its routing on
the device and writes only its own output, and the host's launch cache is shared under a
lock). Streams are created at the default priority."""

import threading

import pytest
import torch

from moe_grouped_gemm_nt_amd import synth
from parity_util import bf16_bits, run_contiguous, run_masked, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def problems():
    pm = synth.make_masked("fp8", 6, 300, 776, 512, [0, 1, 77, 300, 129, 256], seed=61,
                           device=DEV)
    pc = synth.make_contiguous("bf16", 5, 520, 256, [130, 0, 1, 127, 64], seed=62,
                               device=DEV, M_max=768)
    return pm, pc


def test_two_streams_concurrently():
    pm, pc = problems()
    say("two streams")
    ref_m = bf16_bits(run_masked(pm, 64))
    ref_c = bf16_bits(run_contiguous(pc, 128))
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(10):
        with torch.cuda.stream(s1):
            Dm = run_masked(pm, 64)
        with torch.cuda.stream(s2):
            Dc = run_contiguous(pc, 128)
        outs.append((Dm, Dc))
    torch.cuda.synchronize()
    for Dm, Dc in outs:
        assert (bf16_bits(Dm) == ref_m).all()
        assert (bf16_bits(Dc) == ref_c).all()


def test_two_host_threads():
    pm, pc = problems()
    say("two host threads")
    ref_m = bf16_bits(run_masked(pm, 200))
    ref_c = bf16_bits(run_contiguous(pc, 8))
    torch.cuda.synchronize()
    results, errors = {}, []

    def worker(key, fn):
        try:
            s = torch.cuda.Stream()
            outs = []
            with torch.cuda.stream(s):
                for _ in range(10):
                    outs.append(fn())
            s.synchronize()
            results[key] = [bf16_bits(D) for D in outs]
        except Exception as e:  # reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=("m", lambda: run_masked(pm, 200))),
               threading.Thread(target=worker, args=("c", lambda: run_contiguous(pc, 8)))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    assert all((b == ref_m).all() for b in results["m"])
    assert all((b == ref_c).all() for b in results["c"])
