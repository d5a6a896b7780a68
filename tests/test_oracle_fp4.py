"""Pins of the FP8 x FP4 oracle: the E2M1 value table, the nibble packing, exact-rational
brute force over raw bytes, one-hot weights, and the route through the FP8 oracle when
the four 32-K block scales of each 128-K group agree. CPU only."""

from fractions import Fraction

import numpy as np
import pytest

import oracle

# E2M1 magnitudes of codes 0..7 (OCP microscaling formats' FP4 table)
E2M1_MAG = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
# the same magnitudes as E4M3 codes, derived by hand from the E4M3 fields
# (0.5 = 2^-1 -> exponent field 6; 1.5 = 1.100b; 6 = 1.1b * 2^2)
E2M1_AS_E4M3 = [0x00, 0x30, 0x38, 0x3C, 0x40, 0x44, 0x48, 0x4C]


def test_e2m1_table():
    v = oracle.decode_e2m1(np.arange(16, dtype=np.uint8))
    assert list(v[:8]) == E2M1_MAG
    assert list(v[8:]) == [-x for x in E2M1_MAG]
    assert np.signbit(v[8]) and not np.signbit(v[0])
    with pytest.raises(ValueError):
        oracle.decode_e2m1(np.array([16], np.uint8))


def test_unpack_fp4_low_nibble_first():
    c = oracle.unpack_fp4(np.array([[0x21, 0xF0, 0x9A]], np.uint8))
    assert c.tolist() == [[1, 2, 0, 15, 10, 9]]


def test_e2m1_codes_are_exact_e4m3_values():
    e4 = oracle.decode_e4m3fn(np.array(E2M1_AS_E4M3, np.uint8))
    assert list(e4) == E2M1_MAG


def _frac_e4m3(c):
    s, e, m = c >> 7, (c >> 3) & 15, c & 7
    v = Fraction(m, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -v if s else v


def _frac_e2m1(c):
    v = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
         Fraction(4), Fraction(6)][c & 7]
    return -v if c & 8 else v


def _draw(rng, G, cap, N, K):
    A = rng.integers(0, 256, (G, cap, K), dtype=np.uint8)
    A[(A & 0x7F) == 0x7F] = 0x38  # no NaN codes
    B = rng.integers(0, 256, (G, N, K // 2), dtype=np.uint8)
    SFA = rng.integers(118, 136, (G, K // 128, cap), dtype=np.uint8)
    SFB = rng.integers(118, 136, (G, K // 128, N, 4), dtype=np.uint8)
    return A, B, SFA, SFB


def test_masked_fp8_fp4_brute_force_exact():
    """Every valid output against a sum of exact rationals built from the raw bytes: the
    activation scale of (row, 128-K group) and the weight scale of (row, 32-K block)."""
    rng = np.random.default_rng(8)
    G, cap, N, K = 2, 3, 5, 256
    A, B, SFA, SFB = _draw(rng, G, cap, N, K)
    counts = np.array([3, 2])
    ref, valid = oracle.grouped_gemm_masked("fp8_fp4", A, B, counts, SFA, SFB, "block32", "ue8m0")
    for g in range(G):
        for m in range(counts[g]):
            for n in range(N):
                tot = Fraction(0)
                for k in range(K):
                    byte = int(B[g, n, k // 2])
                    code = (byte >> 4) if k & 1 else (byte & 15)
                    sa = Fraction(2) ** (int(SFA[g, k // 128, m]) - 127)
                    sb = Fraction(2) ** (int(SFB[g, k // 128, n, (k // 32) % 4]) - 127)
                    tot += _frac_e4m3(int(A[g, m, k])) * sa * _frac_e2m1(code) * sb
                assert abs(ref[g, m, n] - float(tot)) <= 1e-12 * max(1.0, abs(float(tot)))
    assert not valid[1, 2] and np.isnan(ref[1, 2]).all()


def test_one_hot_fp4_weights_return_scaled_activations():
    """Weight row n holds 1.0 (code 2) at K = 3n + 1 and zeros elsewhere: D[m, n] is the
    dequantized activation at that K times the weight scale of its 32-K block."""
    rng = np.random.default_rng(9)
    G, cap, N, K = 1, 4, 40, 256
    A, _, SFA, SFB = _draw(rng, G, cap, N, K)
    codes = np.zeros((G, N, K), np.uint8)
    for n in range(N):
        codes[0, n, 3 * n + 1] = 2
    B = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    ref, _ = oracle.grouped_gemm_masked("fp8_fp4", A, B, [cap], SFA, SFB, "block32", "ue8m0")
    a_hat = oracle.dequant_act_rows("fp8", A[0], SFA[0], "ue8m0")
    for n in range(N):
        k = 3 * n + 1
        sb = 2.0 ** (int(SFB[0, k // 128, n, (k // 32) % 4]) - 127)
        assert np.array_equal(ref[0, :, n], a_hat[:, k] * sb)


def test_fp4_equals_fp8_channel_route_when_block_scales_agree():
    """With the four 32-K block scales of every (row, 128-K group) equal, FP4 weights
    re-encoded as E4M3 codes (hand-derived table) with per-channel scales give the same
    float64 result through the FP8 oracle, for the masked and contiguous variants."""
    rng = np.random.default_rng(10)
    G, cap, N, K = 3, 6, 7, 384
    A, B, SFA, SFB = _draw(rng, G, cap, N, K)
    SFB[...] = SFB[..., :1]
    codes = oracle.unpack_fp4(B)
    table = np.array(E2M1_AS_E4M3 + [c | 0x80 for c in E2M1_AS_E4M3], np.uint8)
    B8 = table[codes]
    SFB_ch = SFB[..., 0]  # [G, K/128, N]
    counts = [6, 0, 4]
    r4, _ = oracle.grouped_gemm_masked("fp8_fp4", A, B, counts, SFA, SFB, "block32", "ue8m0")
    r8, _ = oracle.grouped_gemm_masked("fp8", A, B8, counts, SFA, SFB_ch, "channel", "ue8m0")
    assert np.array_equal(np.isnan(r4), np.isnan(r8))
    assert np.array_equal(np.nan_to_num(r4), np.nan_to_num(r8))
    idx = np.array([0] * 5 + [-1] * 3 + [2] * 4, np.int32)
    Ac = A.reshape(-1, K)[: idx.size]
    SFAc = SFA.transpose(1, 0, 2).reshape(K // 128, -1)[:, : idx.size]
    c4, _ = oracle.grouped_gemm_contiguous("fp8_fp4", Ac, B, idx, SFAc, SFB, "block32", "ue8m0")
    c8, _ = oracle.grouped_gemm_contiguous("fp8", Ac, B8, idx, SFAc, SFB_ch, "channel", "ue8m0")
    assert np.array_equal(np.nan_to_num(c4), np.nan_to_num(c8))
