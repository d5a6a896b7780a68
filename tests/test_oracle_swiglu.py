"""Pins for the SwiGLU + re-quantization oracle against things other than itself:
float64 exp and torch's silu, special values, the exact cases where silu(x) = x, and
the plain quantization of exactly representable products. CPU only."""

import numpy as np
import torch

import oracle


def bf16_codes(x):
    return torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(
        np.uint16)


def test_exp_against_float64():
    y = np.linspace(-87, 88, 400001).astype(np.float32)
    rel = np.abs(oracle.exp_f32(y) / np.exp(y.astype(np.float64)) - 1)
    assert rel.max() < 1e-5
    assert oracle.exp_f32(np.float32(0.0)) == 1.0


def test_silu_special_values_and_torch():
    s = oracle.silu_f32(np.array([0.0, 17.0, 20.0, 300.0, -100.0, -1e30], np.float32))
    assert s[0] == 0 and s[1] == 17.0 and s[2] == 20.0 and s[3] == 300.0
    assert s[4] == 0 and np.signbit(s[4]) and s[5] == 0
    x = np.linspace(-40, 40, 100001).astype(np.float32)
    ref = torch.nn.functional.silu(torch.tensor(x, dtype=torch.float64)).numpy()
    err = np.abs(oracle.silu_f32(x) - ref)
    assert (err <= 2e-5 * np.abs(ref) + 1e-30).all()


def test_swiglu_with_saturated_gate_is_plain_quantization():
    """gate = 32: e^-32 < 2^-24, so silu(32) = 32 exactly and h = 32 * up exactly;
    the result must equal quantizing the bf16 row 32 * up directly."""
    rng = np.random.default_rng(3)
    up = torch.tensor(rng.standard_normal((8, 256)), dtype=torch.bfloat16).float().numpy()
    H = np.concatenate([np.full((8, 256), 32.0, np.float32), up], axis=1)
    for fmt in ("f32", "ue8m0"):
        q, sf = oracle.swiglu_quant_rows_1x128(bf16_codes(H), fmt)
        q2, sf2 = oracle.quantize_rows_1x128(bf16_codes(32.0 * up), fmt)
        assert (q == q2).all() and (sf == sf2).all()


def test_swiglu_values_against_torch():
    rng = np.random.default_rng(4)
    H = torch.tensor(rng.standard_normal((16, 512)) * 3, dtype=torch.bfloat16)
    h = oracle.swiglu_values(H.view(torch.int16).numpy().view(np.uint16))
    Hd = H.double()
    ref = (torch.nn.functional.silu(Hd[:, :256]) * Hd[:, 256:]).numpy()
    assert (np.abs(h - ref) <= 3e-5 * np.abs(ref) + 1e-30).all()
