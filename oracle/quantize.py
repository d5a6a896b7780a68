"""Plain CPU oracle of the FP8 activation quantization that precedes the grouped GEMM.

TEST INFRASTRUCTURE ONLY (imported by the tests, the smoke check and the benchmark's
CPU-baseline leg; the product path never imports it and shares no code with it).

What is computed, and where it is defined. The DeepGEMM issue "Non-deterministic
numerical problem of k_grouped_fp8_gemm_nt_contiguous" prints, in its repro script, the
cast its operands go through: values are grouped 128 at a time, each group's scale is
its absolute maximum divided by 448 (the largest E4M3 value), an all-zero group takes a
caller-chosen scale instead, scales are floored at 1e-30, and the codes are the values
times the reciprocal of the scale, converted to E4M3. The arithmetic is float32 (the
bf16 input is widened, the maximum, the division by 448, the reciprocal and the product
are float32 operations). That script groups along tokens, per channel; the activations
of the M-grouped products take the same cast per token, along K (1x128 groups: the
"1x128 act" scales of the PR "Fix cross-expert output overwrites in SM90 masked GEMM"
and of the SM120 issue), which is what `quantize_rows_1x128` computes.

UE8M0 scales (one byte u meaning 2^(u-127)) are named on the pages without a rounding
rule. Reading: the scale is the smallest power of two not below amax / 448, so no code
overflows; the codes are then the values times that power's reciprocal (an exact
float32 scaling).

The float32 -> E4M3 conversion is round to nearest, ties to even, written from the
format's value table (saturating at 448, a value no input of this cast can exceed by a
rounding step).
"""

from __future__ import annotations

import numpy as np

from .formats import decode_bf16, decode_e4m3fn

GROUP = 128
E4M3_MAX = 448.0

# the 127 non-negative finite E4M3 values, in code order (codes 0x00 .. 0x7E)
_POS_VALUES = decode_e4m3fn(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)


def encode_e4m3_rne(y) -> np.ndarray:
    """float32 values -> E4M3 codes, round to nearest, ties to even code; |y| above 448
    saturates to 448. NaN inputs give the NaN code 0x7F (sign kept)."""
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y.astype(np.float64))
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, E4M3_MAX))
    # neighbours in the value table: lo <= a <= hi
    hi = np.searchsorted(_POS_VALUES, a, side="left")
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.where(_POS_VALUES[hi] > a, hi - 1, hi)
    lo = np.maximum(lo, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0) & (hi != lo))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(nan, np.uint8(0x7F), code)
    sign = np.signbit(y).astype(np.uint8) << 7
    return (code | sign).astype(np.uint8)


def ue8m0_code_at_least(s) -> np.ndarray:
    """Smallest u with 2^(u-127) >= s, for positive normal float32 s, from its bits."""
    s = np.asarray(s, dtype=np.float32)
    bits = s.view(np.uint32)
    exp = ((bits >> 23) & 0xFF).astype(np.int64)
    frac = bits & 0x7FFFFF
    return (exp + (frac != 0)).astype(np.uint8)


def quantize_rows_1x128(x_codes, sf_fmt: str = "f32", sf_zero: float = 1.0):
    """bf16 rows X[M, K] (raw uint16 codes, K a multiple of 128) -> (Q[M, K] E4M3 codes,
    SF[K/128, M]). SF is float32 (sf_fmt "f32") or UE8M0 bytes (sf_fmt "ue8m0"); an
    all-zero group takes the scale `sf_zero` (for UE8M0, the smallest power of two not
    below it)."""
    return quantize_values_1x128(decode_bf16(np.asarray(x_codes)).astype(np.float32), sf_fmt,
                                 sf_zero)


def quantize_values_1x128(x, sf_fmt: str = "f32", sf_zero: float = 1.0):
    """The same cast on float32 values X[M, K]."""
    x = np.asarray(x, dtype=np.float32)
    M, K = x.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    xg = x.reshape(M, K // GROUP, GROUP)
    amax = np.max(np.abs(xg), axis=2)  # float32, exact
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    if sf_fmt == "f32":
        s = np.where(s == 0, np.float32(sf_zero), s).astype(np.float32)
        s = np.maximum(s, np.float32(1e-30))
        inv = (np.float32(1.0) / s).astype(np.float32)
        sf_out = s
    elif sf_fmt == "ue8m0":
        zero = s == 0
        code = ue8m0_code_at_least(np.where(zero, np.float32(sf_zero), s))
        inv = np.ldexp(np.float32(1.0), 127 - code.astype(np.int64)).astype(np.float32)
        sf_out = code
    else:
        raise ValueError(f"unknown scale format {sf_fmt!r}")
    y = (xg * inv[:, :, None]).astype(np.float32)
    q = encode_e4m3_rne(y).reshape(M, K)
    return q, np.ascontiguousarray(sf_out.T)
