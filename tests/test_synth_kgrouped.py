"""The K-grouped input generator against the oracle's own definitions (CPU only): the
packed operand bytes are read back through `oracle.kgrouped_layout` (expert e's block
[channels][k_e] at element channels * p_e), and the codes and scales equal the oracle's
1x128 cast applied per channel over 128 tokens, for both scale formats and the zero-group
scale values of the repro script."""

import numpy as np
import pytest
import torch

import oracle
from moe_grouped_gemm_nt_amd import synth


def bf16_codes(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("ks,M,N,sf_val,fmt,K_total", [
    ([256, 128, 128, 256], 256, 384, 1.0, "f32", None),
    ([256, 128, 128, 256], 256, 384, 1e-30, "f32", None),
    ([128, 0, 384], 128, 256, 1e-4, "ue8m0", None),
    ([128, 256], 128, 128, 1e-8, "ue8m0", 640),
    ([0, 256, 0], 64, 128, 1.0, "f32", 384),
])
def test_kgrouped_generator_matches_oracle_layout_and_cast(ks, M, N, sf_val, fmt, K_total):
    p = synth.make_kgrouped("fp8", ks, M, N, seed=11, sf_val=sf_val, sf_fmt=fmt,
                            K_total=K_total)
    gy, act = p.meta["grad_y"], p.meta["act"]
    T = sum(ks)
    assert p.sf_fmt == fmt and p.K_total == (T if K_total is None else K_total)
    A, B = p.A.numpy(), p.B.numpy()
    for channels, raw, packed, sf in ((M, gy, A, p.SFA.numpy()), (N, act, B, p.SFB.numpy())):
        # the oracle's cast, per channel (one row of raw^T) over 128 consecutive tokens
        if T:
            q_ref, sf_ref = oracle.quantize_rows_1x128(bf16_codes(raw.t()), fmt, sf_val)
        else:
            q_ref, sf_ref = np.zeros((channels, 0), np.uint8), np.zeros((0, channels))
        if fmt == "f32":
            assert (sf[:T // 128].view(np.uint32) == sf_ref.astype(np.float32).view(np.uint32)).all()
        else:
            assert (sf[:T // 128] == sf_ref).all()
        # unrouted tail tokens: zero codes, unit scales
        assert (packed[channels * T:] == 0).all()
        assert (sf[T // 128:] == (1.0 if fmt == "f32" else 127)).all()
        for e, (pe, k, usable) in enumerate(oracle.kgrouped_layout(ks, p.K_total, 128)):
            assert usable
            block = packed[channels * pe: channels * (pe + k)].reshape(channels, k)
            assert (block == q_ref[:, pe:pe + k]).all(), f"expert {e}"


def test_zero_channel_only_in_the_128_token_experts():
    ks = [256, 128, 384, 128]
    p = synth.make_kgrouped("fp8", ks, 128, 128, seed=2)
    gy = p.meta["grad_y"].float()
    starts = np.concatenate([[0], np.cumsum(ks)])
    for e, k in enumerate(ks):
        col = gy[starts[e]:starts[e + 1], 0]
        if k == 128:
            assert (col == 0).all()
            # the group's scale is the zero-group value and its codes are zero
            assert float(p.SFA[starts[e] // 128, 0]) == 1.0
        else:
            assert (col != 0).any()


def test_bf16_packing_matches_oracle_layout():
    ks = [128, 8, 0, 64]
    p = synth.make_kgrouped("bf16", ks, 32, 48, seed=3)
    for channels, raw, packed in ((32, p.meta["grad_y"], p.A), (48, p.meta["act"], p.B)):
        codes = bf16_codes(packed)
        ref = bf16_codes(raw)
        for pe, k, usable in oracle.kgrouped_layout(ks, sum(ks), 8):
            assert usable
            block = codes[channels * pe: channels * (pe + k)].reshape(channels, k)
            assert (block == ref[pe:pe + k].T).all()
