"""Plain CPU oracle of the SwiGLU + FP8 re-quantization step between the two expert
GEMMs (w13 -> SwiGLU -> w2) of the contiguous configuration's serving model.

TEST INFRASTRUCTURE ONLY (imported by the tests, the smoke check and the benchmark's
CPU-baseline leg; the product path never imports it and shares no code with it).

The pages place the contiguous FP8 GEMM between an MLP's gate/up projection (w13) and
its down projection (w2) (DeepGEMM issue "SM120 m_grouped_fp8 contiguous kernel:
illegal memory access at CUDA graph replay", sections "Environment" and "What works")
without spelling out the activation in between. Reading: the usual gated unit of that
model family, h = silu(gate) * up with gate = the first I columns of the w13 output and
up = the last I, silu(x) = x / (1 + e^-x), in float32; h is then quantized like the
activations (1x128 per-token scales, `quantize.quantize_values_1x128`).

So that the GPU kernel and this oracle take every float32 decision identically (the
quantized codes are integers and are compared bit for bit), e^y is not a library call
but one fixed evaluation, done the same way on both sides: Cody-Waite style range
reduction to 2^r with |r| <= 1/2 and the degree-7 Taylor polynomial of 2^r = e^(r ln 2)
in Horner form, every operation a separately rounded float32 multiply or add (no fused
multiply-add), then an exact scaling by 2^n. Its relative error stays below 1e-5 over
the range that matters for silu (dominated by the rounding of y log2(e) for large |y|),
far below what the bf16/FP8 formats around it resolve.
"""

from __future__ import annotations

import numpy as np

from .quantize import quantize_values_1x128
from .formats import decode_bf16

LN2 = 0.6931471805599453
LOG2E_F32 = np.float32(1.4426950408889634)


def _taylor_coeffs():
    """float32 of (ln 2)^k / k!, k = 0..7, each computed in float64 as c_k = c_(k-1) ln2/k."""
    c = [1.0]
    for k in range(1, 8):
        c.append(c[-1] * LN2 / k)
    return [np.float32(v) for v in c]


_C = _taylor_coeffs()


def exp_f32(y) -> np.ndarray:
    """e^y for float32 y by the fixed evaluation described above (float32 throughout)."""
    y = np.asarray(y, dtype=np.float32)
    t = (y * LOG2E_F32).astype(np.float32)
    big, small = t > np.float32(128.0), t < np.float32(-150.0)
    t = np.clip(t, np.float32(-150.0), np.float32(128.0))
    n = np.rint(t).astype(np.float32)  # ties to even
    r = (t - n).astype(np.float32)  # exact
    p = np.full_like(r, _C[7])
    for k in range(6, -1, -1):
        p = ((p * r).astype(np.float32) + _C[k]).astype(np.float32)
    with np.errstate(over="ignore"):
        out = np.ldexp(p, n.astype(np.int32)).astype(np.float32)
    out = np.where(big, np.float32(np.inf), out)
    out = np.where(small, np.float32(0.0), out)
    return out.astype(np.float32)


def silu_f32(x) -> np.ndarray:
    """x / (1 + e^-x) in float32 (one rounding per operation)."""
    x = np.asarray(x, dtype=np.float32)
    d = (np.float32(1.0) + exp_f32(-x)).astype(np.float32)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        return (x / d).astype(np.float32)


def swiglu_values(h_codes) -> np.ndarray:
    """bf16 w13 output H[M, 2I] (raw codes) -> float32 h[M, I] = silu(gate) * up."""
    h = decode_bf16(np.asarray(h_codes)).astype(np.float32)
    I2 = h.shape[1]
    if I2 % 2:
        raise ValueError("the w13 output has an even number of columns")
    gate, up = h[:, : I2 // 2], h[:, I2 // 2:]
    return (silu_f32(gate) * up).astype(np.float32)


def swiglu_quant_rows_1x128(h_codes, sf_fmt: str = "f32", sf_zero: float = 1.0):
    """bf16 H[M, 2I] -> (Q[M, I] E4M3 codes, SF[I/128, M]) of silu(gate) * up."""
    return quantize_values_1x128(swiglu_values(h_codes), sf_fmt, sf_zero)


# --------------------------------------------------------------------------- plain definition
#
# The same step from the plain definition, independent of the fixed e^y evaluation above:
# silu(g) = g / (1 + e^-g) and h = silu(gate) * up evaluated in float64 with the library's
# exp, then rounded once to float32 (the type the reading fixes for h), then the 1x128
# cast. The codes of the fixed evaluation can differ from these only where the two h values
# (relative difference below the fixed evaluation's error, 1e-5, plus a few float32
# roundings) fall on opposite sides of an E4M3 rounding boundary, or move a group's scale
# by as much.


def silu_exact(x) -> np.ndarray:
    """x / (1 + e^-x) in float64 (e^-x overflowing to inf gives -0 for very negative x)."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def swiglu_values_exact(h_codes) -> np.ndarray:
    """bf16 w13 output H[M, 2I] (raw codes) -> float64 h[M, I] = silu(gate) * up."""
    h = decode_bf16(np.asarray(h_codes)).astype(np.float64)
    I2 = h.shape[1]
    if I2 % 2:
        raise ValueError("the w13 output has an even number of columns")
    return silu_exact(h[:, : I2 // 2]) * h[:, I2 // 2:]


def swiglu_quant_rows_1x128_exact(h_codes, sf_fmt: str = "f32", sf_zero: float = 1.0):
    """bf16 H[M, 2I] -> (Q[M, I], SF[I/128, M], h[M, I] float32): the 1x128 cast of the
    plain-definition values, each rounded once to float32."""
    h32 = swiglu_values_exact(h_codes).astype(np.float32)
    q, sf = quantize_values_1x128(h32, sf_fmt, sf_zero)
    return q, sf, h32
