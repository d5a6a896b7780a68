"""Number formats used by the grouped NT GEMM oracle: decoders and bf16 rounding.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import this module.

Every decoder is written out from the public format definitions and produces exact
float64 values, so products of a decoded FP8 code and an fp32 scale are exact too.

* E4M3FN ("float8_e4m3fn", the FP8 element type of the per-channel cast script on the
  DeepGEMM issue "Non-deterministic numerical problem of k_grouped_fp8_gemm_nt_contiguous",
  section "repro script"): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no
  infinities, a single NaN mantissa pattern (exponent 15 with mantissa 7), largest finite
  magnitude 448 (the divisor the same script uses for its scales).
* bfloat16: the upper 16 bits of an IEEE binary32.
* UE8M0: an unsigned 8-bit biased exponent, value 2^(u-127), code 255 is NaN (the
  power-of-two "2^k" scales named in the environment section of the DeepGEMM issue
  "SM120 m_grouped_fp8 contiguous kernel: illegal memory access at CUDA graph replay").
* E2M1 (FP4, the element type of the "fp8_fp4" kernel family that issue names, from the
  OCP microscaling formats): 1 sign bit, 2 exponent bits with bias 1, 1 mantissa bit, no
  infinities or NaN; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6. Two codes per byte; the
  pages do not state the packing, and the reading taken is the even element in the low
  nibble.
"""

from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0


def _e4m3_value(code: int) -> float:
    """Exact value of one E4M3FN byte, from the field definitions."""
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return math.nan
    if exp == 0:  # subnormal: 0.mmm * 2^(1-7)
        return sign * (man / 8.0) * 2.0 ** -6
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


_E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)


def decode_e4m3fn(codes) -> np.ndarray:
    """uint8 E4M3FN codes (any shape) -> float64 values."""
    codes = np.asarray(codes)
    if codes.dtype != np.uint8:
        raise TypeError(f"E4M3 codes must be uint8, got {codes.dtype}")
    return _E4M3_TABLE[codes]


def _e2m1_value(code: int) -> float:
    """Exact value of one E2M1 code (0..15), from the field definitions."""
    sign = -1.0 if (code >> 3) & 1 else 1.0
    exp = (code >> 1) & 0x3
    man = code & 0x1
    if exp == 0:  # subnormal: 0.m * 2^(1-1)
        return sign * (man / 2.0)
    return sign * (1.0 + man / 2.0) * 2.0 ** (exp - 1)


_E2M1_TABLE = np.array([_e2m1_value(c) for c in range(16)], dtype=np.float64)


def decode_e2m1(codes) -> np.ndarray:
    """E2M1 codes 0..15 (uint8, any shape) -> float64 values."""
    codes = np.asarray(codes)
    if codes.dtype != np.uint8:
        raise TypeError(f"E2M1 codes must be uint8, got {codes.dtype}")
    if (codes > 15).any():
        raise ValueError("E2M1 codes are 4-bit")
    return _E2M1_TABLE[codes]


def unpack_fp4(packed) -> np.ndarray:
    """Packed FP4 bytes [..., K/2] -> codes [..., K]: element 2i is the low nibble of
    byte i, element 2i + 1 the high nibble."""
    packed = np.asarray(packed)
    if packed.dtype != np.uint8:
        raise TypeError(f"packed FP4 must be uint8, got {packed.dtype}")
    out = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), np.uint8)
    out[..., 0::2] = packed & 0x0F
    out[..., 1::2] = packed >> 4
    return out


def decode_bf16(bits) -> np.ndarray:
    """uint16 bfloat16 bit patterns -> float64 values (exact)."""
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        raise TypeError(f"bf16 bits must be uint16, got {bits.dtype}")
    as_f32 = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns stay NaN
        return as_f32.astype(np.float64)


def decode_ue8m0(codes) -> np.ndarray:
    """uint8 UE8M0 codes -> float64 values 2^(u-127); 255 is NaN."""
    codes = np.asarray(codes)
    if codes.dtype != np.uint8:
        raise TypeError(f"UE8M0 codes must be uint8, got {codes.dtype}")
    out = np.ldexp(1.0, codes.astype(np.int64) - 127)
    return np.where(codes == 255, np.nan, out)


def decode_scale(sf, fmt: str) -> np.ndarray:
    """Scale tensor in either storage format -> float64."""
    if fmt == "f32":
        sf = np.asarray(sf)
        if sf.dtype != np.float32:
            raise TypeError(f"f32 scales must be float32, got {sf.dtype}")
        return sf.astype(np.float64)
    if fmt == "ue8m0":
        return decode_ue8m0(sf)
    raise ValueError(f"unknown scale format {fmt!r}")


def round_to_bf16(x) -> np.ndarray:
    """float64 -> uint16 bfloat16 bits, round to nearest, ties to even, in one step.

    bfloat16 keeps 8 significant bits and binary32's exponent range: normal numbers
    down to 2^-126, subnormals in steps of 2^-133, overflow to infinity at or beyond
    2^128 after rounding. The value is rounded on its own quantum (a power of two), so
    x / quantum is exact and numpy's half-to-even rounding gives the tie rule.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    finite = np.isfinite(x)
    xf = np.where(finite, x, 0.0)
    _, e = np.frexp(xf)  # xf = m * 2^e with 0.5 <= |m| < 1
    # Quantum of an 8-bit significand whose leading bit has weight 2^(e-1),
    # floored at the subnormal step 2^-133.
    q_exp = np.maximum(e - 8, -133)
    q = np.ldexp(1.0, q_exp)
    r = np.round(xf / q) * q
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, xf), r)
    bits = (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    out[...] = bits
    # Non-finite inputs: infinities keep their sign, NaN becomes the canonical quiet NaN.
    inf_bits = np.where(x > 0, np.uint16(0x7F80), np.uint16(0xFF80))
    out = np.where(np.isinf(x), inf_bits, out)
    out = np.where(np.isnan(x), np.uint16(0x7FC0), out)
    return out.astype(np.uint16)
