"""GPU parity of the FP8 1x128 activation quantization against the CPU oracle: codes
and scales must match bit for bit (the float32 decisions are the same on both sides),
on ragged row counts, all-zero groups, values landing exactly on rounding midpoints,
both scale formats, the full hidden size of the large configs, and graph replays."""

import numpy as np
import pytest
import torch

import oracle
from parity_util import np_codes, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def quantize(X, fmt, z=1.0):
    import moe_grouped_gemm_nt_amd as mgg
    Q, SF = mgg.quantize_fp8_1x128(X, sf_fmt=fmt, sf_zero=z)
    torch.cuda.synchronize()
    return Q, SF


def check(X, Q, SF, fmt, z=1.0):
    q_ref, sf_ref = oracle.quantize_rows_1x128(np_codes(X), fmt, z)
    q = Q.cpu().numpy()
    sf = SF.cpu().numpy()
    bad_q = int((q != q_ref).sum())
    if fmt == "f32":
        bad_s = int((sf.view(np.uint32) != sf_ref.astype(np.float32).view(np.uint32)).sum())
    else:
        bad_s = int((sf != sf_ref).sum())
    assert bad_q == 0 and bad_s == 0, f"{bad_q} codes and {bad_s} scales differ"


def draw(M, K, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    x = torch.randn((M, K), device=DEV, generator=g)
    # row magnitudes over many binades, a few all-zero groups and a tiny-valued row
    x *= torch.exp2(torch.randint(-20, 12, (M, 1), device=DEV, generator=g).float())
    x[min(3, M - 1), 128:256] = 0
    x[min(7, M - 1)] *= 2.0 ** -110
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("fmt,z", [("f32", 1.0), ("f32", 1e-30), ("ue8m0", 1.0), ("ue8m0", 1e-4)])
def test_quantize_ragged_rows(fmt, z):
    say("quantize ragged", fmt, z)
    X = draw(1000, 1024, 1)
    Q, SF = quantize(X, fmt, z)
    check(X, Q, SF, fmt, z)


@pytest.mark.parametrize("K", [128, 256, 384, 640])
def test_quantize_narrow_rows_few_rows(K):
    """Rows of one to five 128-column groups (several rows share a wave) and 1 to 17 rows
    (a partly filled last wave), both scale formats."""
    for M in (1, 2, 3, 5, 17):
        say("quantize narrow", M, K)
        X = draw(M, K, 100 + M)
        for fmt in ("f32", "ue8m0"):
            Q, SF = quantize(X, fmt)
            check(X, Q, SF, fmt)


def test_quantize_midpoints_round_to_even():
    """Groups whose maximum is 448 (scale exactly 1): every other value is a midpoint
    between adjacent E4M3 values that bf16 represents exactly."""
    vals = oracle.decode_e4m3fn(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2
    bf = torch.tensor(mids, dtype=torch.float64).to(torch.bfloat16).double().numpy()
    mids = mids[bf == mids]  # the midpoints bf16 holds exactly
    row = np.concatenate([mids, -mids])
    X = np.zeros((16, 512), np.float32)
    for r in range(16):
        vals_r = np.resize(np.roll(row, r), 4 * 127)
        for kb in range(4):  # 448 opens every 128-column group: scale exactly 1
            X[r, 128 * kb] = 448.0
            X[r, 128 * kb + 1:128 * (kb + 1)] = vals_r[127 * kb:127 * (kb + 1)]
    say("quantize midpoints", mids.size)
    Xt = torch.tensor(X, device=DEV).to(torch.bfloat16)
    for fmt in ("f32", "ue8m0"):
        Q, SF = quantize(Xt, fmt)
        check(Xt, Q, SF, fmt)


def test_quantize_hidden_7168_full():
    """4096 tokens x 7168 (the large configs' hidden size), both formats, every output."""
    say("quantize 4096x7168")
    X = draw(4096, 7168, 2)
    for fmt in ("f32", "ue8m0"):
        Q, SF = quantize(X, fmt)
        check(X, Q, SF, fmt)


def test_quantize_graph_replay():
    """A captured quantization replayed over new input values in the same buffer matches
    the eager call and the oracle each time."""
    import moe_grouped_gemm_nt_amd as mgg
    say("quantize graph")
    X = draw(300, 768, 3)
    Q = torch.empty((300, 768), dtype=torch.uint8, device=DEV)
    SF = torch.empty((6, 300), dtype=torch.float32, device=DEV)
    mgg.quantize_fp8_1x128(X, Q, SF)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mgg.quantize_fp8_1x128(X, Q, SF)
    for seed in (4, 5, 6):
        X.copy_(draw(300, 768, seed))
        Q.zero_()
        g.replay()
        torch.cuda.synchronize()
        check(X, Q, SF, "f32")
        Qe, SFe = quantize(X, "f32")
        assert torch.equal(Q, Qe) and torch.equal(SF, SFe)
