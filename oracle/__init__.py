"""CPU FP64 oracle for grouped NT GEMM (masked / contiguous / K-grouped, BF16 and FP8).

TEST INFRASTRUCTURE ONLY. Only the tests, the package smoke check and the benchmark's
CPU-baseline leg may import or run anything in this directory. The product library
(the HIP kernels behind the C ABI and their Python binding) never imports it, and the
two share no code: the oracle has its own decoders, its own bf16 rounding and its own
layout arithmetic, written from the format definitions and the pages' descriptions.

Parity status of each function (what pins it lives in tests/test_oracle_*.py):
  decode_e4m3fn, decode_bf16, decode_ue8m0, round_to_bf16  pinned (spec values, torch)
  grouped_gemm_masked / _contiguous / _kgrouped               pinned (brute force with
      exact rationals, integer-exact cases, one-hot weights, cross-variant identities,
      the zero-channel exact zero, the printed reference norm of the K-grouped repro)
  grouped_gemm_contiguous_psum, psum_segments,
  kgrouped_ks_from_psum                                       pinned (literal segment
      cases, equality with the masked oracle per segment, exact-rational brute force)
  calc_diff                                                   pinned (closed forms)
  encode_e4m3_rne, ue8m0_code_at_least, quantize_rows_1x128   pinned (torch's float32 ->
      float8_e4m3fn conversion on random values and every rounding midpoint, literal
      power-of-two cases, closed-form groups, round-trip error bound)
  exp_f32, silu_f32, swiglu_values, swiglu_quant_rows_1x128   pinned (float64 exp and
      torch's silu within a few ulps, special values, exact cases where silu(x) = x,
      equality with the plain quantization of exactly representable products); these
      mirror the kernel's fixed e^y evaluation so codes can be compared bit for bit
  silu_exact, swiglu_values_exact,
  swiglu_quant_rows_1x128_exact                               pinned (torch's float64
      silu, closed-form values, the saturated-gate identity, and agreement with the
      fixed evaluation up to rounding-boundary flips); the plain definition (float64 exp)
      that the GPU codes are also compared against
  decode_e2m1, unpack_fp4, the "fp8_fp4" dtype of the M-grouped products   pinned
      (the format's value table, literal nibble cases, exact-rational brute force over
      raw bytes, one-hot weights, equality with the FP8 channel-scale product when the
      four block scales of each 128-K group agree)
"""

from .formats import (  # noqa: F401
    E4M3_MAX,
    decode_bf16,
    decode_e2m1,
    decode_e4m3fn,
    decode_scale,
    decode_ue8m0,
    round_to_bf16,
    unpack_fp4,
)
from .quantize import (  # noqa: F401
    encode_e4m3_rne,
    quantize_rows_1x128,
    quantize_values_1x128,
    ue8m0_code_at_least,
)
from .swiglu import (  # noqa: F401
    exp_f32,
    silu_exact,
    silu_f32,
    swiglu_quant_rows_1x128,
    swiglu_quant_rows_1x128_exact,
    swiglu_values,
    swiglu_values_exact,
)
from .grouped_gemm import (  # noqa: F401
    MX_BLOCK,
    SCALE_K,
    calc_diff,
    contiguous_row_expert,
    dequant_act_rows,
    dequant_weight_rows,
    gemm_nt_fp64,
    grouped_gemm_contiguous,
    grouped_gemm_contiguous_psum,
    grouped_gemm_kgrouped,
    grouped_gemm_masked,
    kgrouped_layout,
    kgrouped_ks_from_psum,
    psum_segments,
    valid_counts,
)
