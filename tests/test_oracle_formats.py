"""Pins for the oracle's number formats: spec values, full-code comparisons against
torch's own conversions, rounding ties. CPU only."""

import math

import numpy as np
import pytest
import torch

from oracle import decode_bf16, decode_e4m3fn, decode_ue8m0, round_to_bf16


# E4M3FN values fixed by the format definition (sign, 4-bit exponent bias 7, 3-bit
# mantissa, no infinities, S.1111.111 is NaN).
E4M3_SPEC = {
    0x00: 0.0,
    0x01: 2.0 ** -9,  # smallest subnormal
    0x07: 7 * 2.0 ** -9,  # largest subnormal
    0x08: 2.0 ** -6,  # smallest normal
    0x38: 1.0,
    0x39: 1.125,
    0x40: 2.0,
    0x7E: 448.0,  # largest finite
    0x80: -0.0,
    0xB8: -1.0,
    0xFE: -448.0,
}


def test_e4m3_spec_values():
    for code, val in E4M3_SPEC.items():
        got = decode_e4m3fn(np.array([code], np.uint8))[0]
        assert got == val and math.copysign(1, got) == math.copysign(1, val), hex(code)
    assert np.isnan(decode_e4m3fn(np.array([0x7F, 0xFF], np.uint8))).all()


def test_e4m3_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = decode_e4m3fn(codes)
    theirs = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().double().numpy()
    nan = np.isnan(theirs)
    assert (np.isnan(ours) == nan).all()
    assert (ours[~nan] == theirs[~nan]).all()
    # sign symmetry and monotonicity of the positive codes
    assert (ours[0x80:0xFF] == -ours[0:0x7F]).all()
    assert (np.diff(ours[0:0x7F]) > 0).all()


def test_e4m3_roundtrip_finite_codes():
    """Every finite code's value converts back to the same code."""
    codes = np.arange(256, dtype=np.uint8)
    vals = decode_e4m3fn(codes)
    finite = ~np.isnan(vals) & (codes != 0x80)
    back = torch.from_numpy(vals[finite].astype(np.float32)).to(torch.float8_e4m3fn)
    assert (back.view(torch.uint8).numpy() == codes[finite]).all()
    assert finite.sum() == 253  # 254 finite codes, -0 excluded


def test_bf16_decode_matches_torch():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    ours = decode_bf16(bits)
    theirs = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    nan = np.isnan(theirs)
    assert (np.isnan(ours) == nan).all()
    assert (ours[~nan] == theirs[~nan]).all()


def test_ue8m0_spec():
    got = decode_ue8m0(np.array([127, 0, 254, 128, 126, 255], np.uint8))
    assert got[0] == 1.0 and got[1] == 2.0 ** -127 and got[2] == 2.0 ** 127
    assert got[3] == 2.0 and got[4] == 0.5 and np.isnan(got[5])


def test_round_to_bf16_ties_and_specials():
    one = 1.0
    cases = {
        one: 0x3F80,
        one + 2.0 ** -8: 0x3F80,  # tie, even stays
        one + 3 * 2.0 ** -8: 0x3F82,  # tie, rounds up to even
        one + 2.0 ** -8 + 2.0 ** -30: 0x3F81,  # just above the tie
        -one: 0xBF80,
        0.0: 0x0000,
        2.0 ** -133: 0x0001,  # smallest subnormal
        2.0 ** -134: 0x0000,  # tie at half the smallest subnormal -> even (zero)
        3 * 2.0 ** -134: 0x0002,
        (2 - 2.0 ** -7) * 2.0 ** 127: 0x7F7F,  # largest finite
        (2 - 2.0 ** -8) * 2.0 ** 127: 0x7F80,  # rounds to infinity
    }
    xs = np.array(list(cases.keys()))
    got = round_to_bf16(xs)
    for x, want, g in zip(xs, cases.values(), got):
        assert int(g) == want, (x, hex(int(g)), hex(want))
    sp = round_to_bf16(np.array([np.inf, -np.inf, np.nan]))
    assert list(sp) == [0x7F80, 0xFF80, 0x7FC0]


def test_round_to_bf16_matches_torch_on_float32_inputs():
    """torch rounds float32 -> bf16 to nearest even; on float32-representable inputs
    the one-step float64 rounding must agree bit for bit."""
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000) * 10.0 ** rng.integers(-40, 38, 100000),
        rng.standard_normal(1000) * 1e-40,  # bf16 subnormals
    ]).astype(np.float32)
    ours = round_to_bf16(x.astype(np.float64))
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (ours == theirs).all()


def test_round_to_bf16_is_one_step_not_two():
    """A float64 value just above a bf16 tie must round up, even though rounding it to
    float32 first would land exactly on the tie and round to even (down)."""
    x = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert int(round_to_bf16(np.array([x]))[0]) == 0x3F81
    assert int(torch.tensor(np.float32(x)).to(torch.bfloat16).view(torch.int16)) == 0x3F80


@pytest.mark.parametrize("fmt", ["f32", "ue8m0"])
def test_decode_scale_types(fmt):
    from oracle import decode_scale
    if fmt == "f32":
        s = decode_scale(np.array([0.5, 3.0], np.float32), fmt)
        assert list(s) == [0.5, 3.0]
        with pytest.raises(TypeError):
            decode_scale(np.array([1.0]), fmt)
    else:
        assert list(decode_scale(np.array([127, 130], np.uint8), fmt)) == [1.0, 8.0]
