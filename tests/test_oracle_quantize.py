"""Pins for the FP8 activation-quantization oracle, each against something other than
the oracle: torch's own float32 -> float8_e4m3fn conversion (random values and every
rounding midpoint), literal power-of-two scale codes, groups whose codes follow in
closed form, and the round-trip error bound of the format. CPU only."""

import numpy as np
import pytest
import torch

import oracle


def torch_e4m3(y):
    return torch.from_numpy(np.asarray(y, np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def bf16_codes(x):
    return torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(
        np.uint16)


def test_encode_matches_torch_on_random_values():
    rng = np.random.default_rng(1)
    y = np.concatenate([rng.standard_normal(200000) * s for s in (1e-3, 0.1, 10, 100)])
    y = y[np.abs(y) < 460].astype(np.float32)  # torch gives NaN from 464 up; no cast input gets there
    assert (oracle.encode_e4m3_rne(y) == torch_e4m3(y)).all()


def test_encode_midpoints_round_to_even():
    """Every midpoint between adjacent positive E4M3 values (exactly representable in
    float32), and one float32 step either side of it."""
    vals = oracle.decode_e4m3fn(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    assert ((vals[:-1] + vals[1:]) / 2 == mids.astype(np.float64)).all()
    for y in (mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))):
        ys = np.concatenate([y, -y]).astype(np.float32)
        assert (oracle.encode_e4m3_rne(ys) == torch_e4m3(ys)).all()
    # ties go to the even code
    codes = oracle.encode_e4m3_rne(mids)
    assert (codes % 2 == 0).all()


def test_ue8m0_code_literals():
    c = oracle.ue8m0_code_at_least(np.array([1.0, 0.75, 1.0000001, 2.0 ** -5, 3.0, 2.0 ** -100],
                                            np.float32))
    assert c.tolist() == [127, 127, 128, 122, 129, 27]


def test_quantize_group_at_full_range_is_identity_scaled():
    """A group whose maximum is exactly 448 gets scale 1 and codes = the bf16 values'
    nearest E4M3 values; a group scaled by 2^-3 gets scale 2^-3 and the same codes."""
    codes = np.concatenate([np.arange(0, 0x7F), [0x7E]]).astype(np.uint8)  # 128 codes
    vals = oracle.decode_e4m3fn(codes).astype(np.float32)
    vals[1::2] *= -1  # both signs
    row = np.concatenate([vals, vals / 8]).astype(np.float32)[None]
    q, sf = oracle.quantize_rows_1x128(bf16_codes(row), "f32")
    assert sf.shape == (2, 1) and sf[0, 0] == 1.0 and sf[1, 0] == np.float32(0.125)
    want = torch_e4m3(torch.tensor(row).to(torch.bfloat16).float().numpy()[:, :128])
    assert (q[:, :128] == want).all() and (q[:, 128:] == want).all()


def test_quantize_zero_group_takes_sf_zero():
    x = np.zeros((2, 256), np.float32)
    x[1, 130] = -3.0
    for fmt, z, want in [("f32", 1.0, 1.0), ("f32", 1e-30, 1e-30), ("ue8m0", 1.0, 127),
                         ("ue8m0", 0.3, 126)]:
        q, sf = oracle.quantize_rows_1x128(bf16_codes(x), fmt, z)
        assert (q[0] == 0).all()
        if fmt == "f32":
            assert sf[0, 0] == np.float32(want) and sf[1, 0] == np.float32(want)
        else:
            assert sf[0, 0] == want and sf[1, 0] == want
    q, sf = oracle.quantize_rows_1x128(bf16_codes(x), "f32", 1.0)
    assert sf[1, 1] == np.float32(3.0) / np.float32(448.0)
    assert oracle.decode_e4m3fn(q[1, 130]) == -448.0


@pytest.mark.parametrize("fmt", ["f32", "ue8m0"])
def test_quantize_roundtrip_bound(fmt):
    """|dequant - x| <= half an E4M3 step of |x|'s binade times the scale (2^-4 relative
    for normals, plus the subnormal step 2^-10 * scale), and no code exceeds 448."""
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((64, 512)) * np.exp(rng.uniform(-8, 4, (64, 1)))).astype(np.float32)
    xc = bf16_codes(x)
    xb = oracle.decode_bf16(xc)
    q, sf = oracle.quantize_rows_1x128(xc, fmt)
    s = oracle.decode_scale(sf, fmt).T  # [M, K/128]
    deq = oracle.decode_e4m3fn(q) * np.repeat(s, 128, axis=1)
    err = np.abs(deq - xb)
    bound = np.abs(xb) * 2.0 ** -4 + np.repeat(s, 128, axis=1) * 2.0 ** -10 * 1.0001
    assert (err <= bound).all()
    assert (np.abs(oracle.decode_e4m3fn(q)) <= 448).all()
