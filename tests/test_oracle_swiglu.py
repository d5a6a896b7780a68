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


# ----------------------------------------------------------------------------- plain definition


def test_silu_exact_against_torch_and_closed_forms():
    x = np.linspace(-700, 700, 200001)
    ref = torch.nn.functional.silu(torch.tensor(x, dtype=torch.float64)).numpy()
    got = oracle.silu_exact(x)
    assert np.allclose(got, ref, rtol=1e-15, atol=0)  # a few ulps: x·sigmoid(x) vs x/(1+e^-x)
    # silu(ln 3) = ln 3 / (1 + 1/3) = 0.75 ln 3;  silu(-ln 3) = -ln 3 / 4
    assert abs(oracle.silu_exact(np.log(3.0)) - 0.75 * np.log(3.0)) < 1e-15
    assert abs(oracle.silu_exact(-np.log(3.0)) + 0.25 * np.log(3.0)) < 1e-15
    assert oracle.silu_exact(0.0) == 0.0
    s = oracle.silu_exact(np.array([-800.0, -1e300]))
    assert (s == 0).all() and np.signbit(s).all()


def test_swiglu_exact_saturated_gate_is_plain_quantization():
    """gate = 32: e^-32 < 2^-24, so the float32 rounding of silu(32) is 32 and h = 32 * up
    exactly; the plain-definition path must equal quantizing bf16(32 * up) directly."""
    rng = np.random.default_rng(5)
    up = torch.tensor(rng.standard_normal((8, 256)), dtype=torch.bfloat16).float().numpy()
    H = np.concatenate([np.full((8, 256), 32.0, np.float32), up], axis=1)
    for fmt in ("f32", "ue8m0"):
        q, sf, h = oracle.swiglu_quant_rows_1x128_exact(bf16_codes(H), fmt)
        q2, sf2 = oracle.quantize_rows_1x128(bf16_codes(32.0 * up), fmt)
        assert (q == q2).all() and (sf == sf2).all()
        assert (h == (32.0 * up).astype(np.float32)).all()


def test_fixed_evaluation_agrees_with_plain_definition():
    """The mirror path (fixed e^y) against the plain definition through the comparison the
    GPU tests use: no mismatch beyond rounding-boundary flips, and few of those."""
    from parity_util import assert_swiglu_plain, compare_swiglu_to_plain
    rng = np.random.default_rng(6)
    gate = rng.standard_normal((512, 384)) * 4
    up = rng.standard_normal((512, 384)) * np.exp2(rng.integers(-20, 12, (512, 1)))
    gate[7] *= 40
    gate[9, :128] = -200.0
    up[11, 128:256] = 0.0
    H = bf16_codes(np.concatenate([gate, up], axis=1))
    for fmt in ("f32", "ue8m0"):
        for z in (1.0, 1e-30):
            q, sf = oracle.swiglu_quant_rows_1x128(H, fmt, z)
            rep = compare_swiglu_to_plain(H, q, sf, fmt, z)
            assert_swiglu_plain(rep)


def test_plain_comparison_reports_planted_mistakes():
    """The comparison itself: a code two steps off, a code one step off away from any
    boundary, and a scale off by 1e-4 are each reported."""
    from parity_util import compare_swiglu_to_plain
    rng = np.random.default_rng(7)
    H = bf16_codes(rng.standard_normal((64, 512)) * 2)
    for fmt in ("f32", "ue8m0"):
        q, sf = oracle.swiglu_quant_rows_1x128(H, fmt)
        base = compare_swiglu_to_plain(H, q, sf, fmt)
        assert base["code_bad"] == 0 and base["scale_bad"] == 0
        bad = q.copy()
        i = np.nonzero((bad & 0x7F) > 8)[0][:1], np.nonzero((bad[np.nonzero((bad & 0x7F) > 8)[0][0]] & 0x7F) > 8)[0][:1]
        bad[i] = bad[i] - 2
        assert compare_swiglu_to_plain(H, bad, sf, fmt)["code_bad"] == 1
        bad = q.copy()
        bad[3, 5] = bad[3, 5] ^ 1
        rep = compare_swiglu_to_plain(H, bad, sf, fmt)
        assert rep["code_bad"] + rep["code_flips"] == 1 and rep["code_bad"] == 1
        badsf = sf.copy()
        if fmt == "f32":
            badsf[1, 2] = np.float32(badsf[1, 2] * (1 + 1e-4))
        else:
            badsf[1, 2] = badsf[1, 2] + 1
        assert compare_swiglu_to_plain(H, q, badsf, fmt)["scale_bad"] == 1
