"""Grouped NT GEMM for mixture-of-experts layers on MI355X (gfx950).

Thin Python binding of the C ABI in include/moe_grouped_gemm_nt.h. It only marshals
arguments: it derives sizes from tensor shapes, passes raw device pointers and the
current HIP stream, and raises on a non-OK status. All computation happens in the HIP
kernels of libmoe_grouped_gemm_nt.so; there is no fallback of any kind, and calling an
entry point without the built library raises.

Entry points (same names as the C functions):
    grouped_gemm_masked(A, B, D, masked_m, SFA=None, SFB=None, sfb_gran=None,
                        expected_m=0)
    grouped_gemm_contiguous(A, B, D, m_indices, SFA=None, SFB=None, sfb_gran=None,
                            expected_m=0)
    grouped_gemm_contiguous_psum(A, B, D, psum, SFA=None, SFB=None, sfb_gran=None,
                                 expected_m=0)
    grouped_gemm_kgrouped(A, B, D, ks, M, N, SFA=None, SFB=None, accumulate=True,
                          psum=False)   (psum=True calls grouped_gemm_kgrouped_psum)
    quantize_fp8_1x128(X, Q=None, SF=None, sf_fmt="f32", sf_zero=1.0) -> (Q, SF)
    swiglu_quant_fp8_1x128(H, Q=None, SF=None, sf_fmt="f32", sf_zero=1.0) -> (Q, SF)
    grouped_gemm_contiguous_swiglu_quant(A, B, m_indices, SFA, SFB, Q=None, SFQ=None,
                                         sfq_fmt="ue8m0", sf_zero=1.0, sfb_gran=None)
                                         -> (Q, SFQ)

Element types: bfloat16 tensors select BF16; uint8 (or float8_e4m3fn) tensors select
FP8 E4M3; FP8 activations with weights of K/2 bytes per row (uint8 or float4_e2m1fn_x2)
select FP8 x FP4 (E2M1 weights, two per byte, 1x32 UE8M0 weight scales "block32").
Scale tensors: float32 selects FP32 scales, uint8 selects UE8M0 scales. `sfb_gran`
defaults to "block128" (FP8) or "block32" (FP4 weights).
"""

from __future__ import annotations

import ctypes
import os

__all__ = [
    "grouped_gemm_masked",
    "grouped_gemm_contiguous",
    "grouped_gemm_contiguous_psum",
    "grouped_gemm_kgrouped",
    "quantize_fp8_1x128",
    "swiglu_quant_fp8_1x128",
    "grouped_gemm_contiguous_swiglu_quant",
    "library_path",
    "load_library",
    "MggError",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libmoe_grouped_gemm_nt.so"
_lib = None

MGG_BF16, MGG_FP8_E4M3, MGG_FP8_FP4 = 0, 1, 2
MGG_SF_F32, MGG_SF_UE8M0 = 0, 1
MGG_SFB_BLOCK128, MGG_SFB_CHANNEL, MGG_SFB_BLOCK32 = 0, 1, 2
_GRAN = {"block128": MGG_SFB_BLOCK128, "channel": MGG_SFB_CHANNEL, "block32": MGG_SFB_BLOCK32}


class MggError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"status {status}: {message}")
        self.status = status


def library_path() -> str:
    return os.path.join(_PKG, _LIB_NAME)


def load_library() -> ctypes.CDLL:
    """Load the built HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m moe_grouped_gemm_nt_amd.build` "
            "(there is no non-HIP implementation)")
    lib = ctypes.CDLL(path)
    vp, i32, st = ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p
    lib.grouped_gemm_masked.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, i32, i32,
                                        vp, vp, i32, st]
    lib.grouped_gemm_contiguous.argtypes = list(lib.grouped_gemm_masked.argtypes)
    lib.grouped_gemm_contiguous_psum.argtypes = list(lib.grouped_gemm_masked.argtypes)
    lib.grouped_gemm_kgrouped.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, i32, vp,
                                          vp, i32, st]
    lib.grouped_gemm_kgrouped_psum.argtypes = list(lib.grouped_gemm_kgrouped.argtypes)
    lib.quantize_fp8_1x128.argtypes = [i32, i32, vp, vp, vp, i32, ctypes.c_float, st]
    lib.swiglu_quant_fp8_1x128.argtypes = list(lib.quantize_fp8_1x128.argtypes)
    lib.grouped_gemm_contiguous_swiglu_quant.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp,
                                                         vp, i32, i32, vp, vp, i32,
                                                         ctypes.c_float, vp, st]
    for f in (lib.grouped_gemm_masked, lib.grouped_gemm_contiguous,
              lib.grouped_gemm_contiguous_psum, lib.grouped_gemm_kgrouped,
              lib.grouped_gemm_kgrouped_psum, lib.quantize_fp8_1x128,
              lib.swiglu_quant_fp8_1x128, lib.grouped_gemm_contiguous_swiglu_quant):
        f.restype = ctypes.c_int
    lib.mgg_status_string.argtypes = [ctypes.c_int]
    lib.mgg_status_string.restype = ctypes.c_char_p
    lib.mgg_last_error.argtypes = []
    lib.mgg_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        lib = load_library()
        msg = lib.mgg_last_error().decode() or lib.mgg_status_string(status).decode()
        raise MggError(status, msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _elem_dtype(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return MGG_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return MGG_FP8_E4M3
    raise TypeError(f"operands must be bfloat16 or FP8 bytes, got {t.dtype}")


def _m_operands(A, B, K):
    """Element type of an M-grouped call from the operand tensors: bf16 x bf16, FP8 x
    FP8 (B [G, N, K] bytes) or FP8 x FP4 (B [G, N, K/2] packed bytes, or torch's packed
    float4 type); returns (dtype code, default weight-scale granularity)."""
    import torch
    dt = _elem_dtype(A)
    fp4_t = getattr(torch, "float4_e2m1fn_x2", None)
    if dt == MGG_FP8_E4M3 and B.dim() == 3 and 2 * B.shape[2] == K and \
            B.dtype in (torch.uint8, fp4_t):
        return MGG_FP8_FP4, "block32"
    _require(B.dim() == 3 and B.shape[2] == K, "B must be [G, N, K] (FP4 weights: [G, N, K/2])")
    _require(_elem_dtype(B) == dt, "A and B must have the same element type")
    return dt, "block128"


def _sf_fmt(sf) -> int:
    import torch
    if sf is None:
        return MGG_SF_F32
    if sf.dtype == torch.float32:
        return MGG_SF_F32
    if sf.dtype == torch.uint8:
        return MGG_SF_UE8M0
    raise TypeError(f"scales must be float32 or uint8 (UE8M0), got {sf.dtype}")


def _require(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _check_scales(dt: int, SFA, SFB, sfa_shape, sfb_shapes, gran: str):
    """Scale tensors against the layouts of include/moe_grouped_gemm_nt.h: none for BF16;
    for FP8 both present, of one storage type (float32, or uint8 UE8M0) and of exactly the
    shape the layout and weight-scale granularity fix (`sfb_shapes` maps granularity ->
    shape). The kernels size their reads from the problem shape, not from the tensors, so
    a scale tensor of another type or shape would be read out of bounds or misread."""
    import torch
    if dt == MGG_BF16:
        _require(SFA is None and SFB is None, "BF16 operands take no scale tensors")
        return
    _require(SFA is not None and SFB is not None, "FP8 operands need SFA and SFB")
    _require(SFA.dtype in (torch.float32, torch.uint8),
             f"scales must be float32 or uint8 (UE8M0), got {SFA.dtype}")
    _require(SFB.dtype == SFA.dtype, f"SFA ({SFA.dtype}) and SFB ({SFB.dtype}) must have the "
                                     "same storage type")
    if dt == MGG_FP8_FP4:
        _require(SFA.dtype == torch.uint8, "FP8 x FP4 products take UE8M0 (uint8) scales")
    _require(gran in sfb_shapes, f"weight-scale granularity {gran!r} does not fit these operands "
                                 f"(expected one of {sorted(sfb_shapes)})")
    _require(tuple(SFA.shape) == tuple(sfa_shape),
             f"SFA must be {list(sfa_shape)}, got {list(SFA.shape)}")
    want = tuple(sfb_shapes[gran])
    _require(tuple(SFB.shape) == want,
             f"SFB ({gran}) must be {list(want)}, got {list(SFB.shape)}")


def _m_sfb_shapes(dt: int, G: int, N: int, K: int) -> dict:
    """Weight-scale shapes of an M-grouped call per granularity."""
    if dt == MGG_FP8_FP4:
        return {"block32": (G, K // 128, N, 4)}
    return {"block128": (G, -(-N // 128), K // 128), "channel": (G, K // 128, N)}


def _same_device(*ts):
    devs = {t.device for t in ts if t is not None}
    _require(len(devs) == 1 and next(iter(devs)).type == "cuda",
             "all tensors must be on the same GPU")


def _contig(*ts):
    for t in ts:
        if t is not None:
            _require(t.is_contiguous(), "tensors must be contiguous")


def grouped_gemm_masked(A, B, D, masked_m, SFA=None, SFB=None, sfb_gran=None,
                        expected_m=0):
    """D[g, m, :] = A[g, m, :] @ B[g].T for m < masked_m[g]; A[G, cap, K], B[G, N, K],
    D bf16 [G, cap, N], masked_m int32 [G] on the device."""
    import torch
    G, cap, K = A.shape
    N = B.shape[1]
    dt, gran = _m_operands(A, B, K)
    _require(B.shape[0] == G, "B must hold G experts")
    _require(tuple(D.shape) == (G, cap, N) and D.dtype == torch.bfloat16, "D must be bf16 [G, cap, N]")
    _require(masked_m.dtype == torch.int32 and masked_m.numel() == G, "masked_m must be int32 [G]")
    sfb_gran = sfb_gran or gran
    _check_scales(dt, SFA, SFB, (G, K // 128, cap), _m_sfb_shapes(dt, G, N, K), sfb_gran)
    lib = load_library()
    _same_device(A, B, D, masked_m, SFA, SFB)
    _contig(A, B, D, masked_m, SFA, SFB)
    with torch.cuda.device(A.device):
        _check(lib.grouped_gemm_masked(dt, G, cap, N, K, _ptr(A), _ptr(SFA), _ptr(B), _ptr(SFB),
                                       _sf_fmt(SFA), _GRAN[sfb_gran], _ptr(D), _ptr(masked_m),
                                       int(expected_m), _stream(A.device)))
    return D


def grouped_gemm_contiguous(A, B, D, m_indices, SFA=None, SFB=None, sfb_gran=None,
                            expected_m=0):
    """D[r, :] = A[r, :] @ B[m_indices[r]].T for rows with a valid expert index;
    A[M, K], B[G, N, K], D bf16 [M, N], m_indices int32 [M] on the device."""
    import torch
    M, K = A.shape
    G, N, _ = B.shape
    dt, gran = _m_operands(A, B, K)
    _require(tuple(D.shape) == (M, N) and D.dtype == torch.bfloat16, "D must be bf16 [M, N]")
    _require(m_indices.dtype == torch.int32 and m_indices.numel() == M, "m_indices must be int32 [M]")
    sfb_gran = sfb_gran or gran
    _check_scales(dt, SFA, SFB, (K // 128, M), _m_sfb_shapes(dt, G, N, K), sfb_gran)
    lib = load_library()
    _same_device(A, B, D, m_indices, SFA, SFB)
    _contig(A, B, D, m_indices, SFA, SFB)
    with torch.cuda.device(A.device):
        _check(lib.grouped_gemm_contiguous(dt, G, M, N, K, _ptr(A), _ptr(SFA), _ptr(B), _ptr(SFB),
                                           _sf_fmt(SFA), _GRAN[sfb_gran], _ptr(D),
                                           _ptr(m_indices), int(expected_m), _stream(A.device)))
    return D


def grouped_gemm_contiguous_psum(A, B, D, psum, SFA=None, SFB=None, sfb_gran=None,
                                 expected_m=0):
    """D[r, :] = A[r, :] @ B[e].T for r in expert e's row segment [psum[e-1], psum[e])
    (ends clamped to [0, M] and made non-decreasing); A[M, K], B[G, N, K], D bf16 [M, N],
    psum int32 [G] on the device."""
    import torch
    M, K = A.shape
    G, N, _ = B.shape
    dt, gran = _m_operands(A, B, K)
    _require(tuple(D.shape) == (M, N) and D.dtype == torch.bfloat16, "D must be bf16 [M, N]")
    _require(psum.dtype == torch.int32 and psum.numel() == G, "psum must be int32 [G]")
    sfb_gran = sfb_gran or gran
    _check_scales(dt, SFA, SFB, (K // 128, M), _m_sfb_shapes(dt, G, N, K), sfb_gran)
    lib = load_library()
    _same_device(A, B, D, psum, SFA, SFB)
    _contig(A, B, D, psum, SFA, SFB)
    with torch.cuda.device(A.device):
        _check(lib.grouped_gemm_contiguous_psum(dt, G, M, N, K, _ptr(A), _ptr(SFA), _ptr(B),
                                                _ptr(SFB), _sf_fmt(SFA), _GRAN[sfb_gran],
                                                _ptr(D), _ptr(psum), int(expected_m),
                                                _stream(A.device)))
    return D


def grouped_gemm_contiguous_swiglu_quant(A, B, m_indices, SFA, SFB, Q=None, SFQ=None,
                                         sfq_fmt="ue8m0", sf_zero=1.0, sfb_gran=None):
    """The contiguous FP8 GEMM with the SwiGLU + 1x128 re-quantization in its epilogue:
    A[M, K] FP8 codes, B[G, 2I, K] (FP4: [G, 2I, K/2]) w13 weights (gate rows, then up
    rows) -> (Q uint8 [M, I] E4M3 codes, SFQ [I/128, M] float32 or uint8 UE8M0); Q and SFQ
    are allocated when not given; rows that are not routed keep their contents."""
    import torch
    M, K = A.shape
    G, N2, _ = B.shape
    dt, gran = _m_operands(A, B, K)
    _require(N2 % 2 == 0, "B must hold 2I rows")
    I = N2 // 2
    sfb_gran = sfb_gran or gran
    _require(dt != MGG_BF16, "the fused SwiGLU epilogue takes FP8 activations")
    _check_scales(dt, SFA, SFB, (K // 128, M), _m_sfb_shapes(dt, G, N2, K), sfb_gran)
    lib = load_library()
    if Q is None:
        Q = torch.empty((M, I), dtype=torch.uint8, device=A.device)
    if SFQ is None:
        SFQ = torch.empty((I // 128, M), device=A.device,
                          dtype=torch.float32 if sfq_fmt == "f32" else torch.uint8)
    _same_device(A, B, m_indices, SFA, SFB, Q, SFQ)
    _contig(A, B, m_indices, SFA, SFB, Q, SFQ)
    _require(tuple(Q.shape) == (M, I) and Q.dtype in (torch.uint8, torch.float8_e4m3fn),
             "Q must be uint8 [M, I]")
    _require(tuple(SFQ.shape) == (I // 128, M), "SFQ must be [I/128, M]")
    fmt = {"f32": MGG_SF_F32, "ue8m0": MGG_SF_UE8M0}[sfq_fmt]
    _require((SFQ.dtype == torch.float32) == (fmt == MGG_SF_F32), "SFQ dtype must match sfq_fmt")
    _require(m_indices.dtype == torch.int32 and m_indices.numel() == M,
             "m_indices must be int32 [M]")
    with torch.cuda.device(A.device):
        _check(lib.grouped_gemm_contiguous_swiglu_quant(
            dt, G, M, I, K, _ptr(A), _ptr(SFA), _ptr(B), _ptr(SFB), _sf_fmt(SFA),
            _GRAN[sfb_gran], _ptr(Q), _ptr(SFQ), fmt, float(sf_zero), _ptr(m_indices),
            _stream(A.device)))
    return Q, SFQ


def grouped_gemm_kgrouped(A, B, D, ks, M, N, SFA=None, SFB=None, accumulate=True,
                          psum=False):
    """D[e] (+)= A_e @ B_e.T over expert e's ks[e] tokens; A, B flat packed buffers
    (expert blocks [M][k_e] / [N][k_e]), D fp32 [G, M, N], ks int32 [G] on the device.
    With psum=True, ks holds cumulative token ends (k_e = ks[e] - ks[e-1])."""
    import torch
    G = ks.numel()
    _require(A.numel() % M == 0 and B.numel() % N == 0, "packed buffers must hold whole channels")
    K_total = A.numel() // M
    _require(B.numel() // N == K_total, "A and B must cover the same token axis")
    _require(tuple(D.shape) == (G, M, N) and D.dtype == torch.float32, "D must be fp32 [G, M, N]")
    _require(ks.dtype == torch.int32, "ks must be int32")
    dt = _elem_dtype(A)
    _require(_elem_dtype(B) == dt, "A and B must have the same element type")
    _check_scales(dt, SFA, SFB, (K_total // 128, M), {"channel": (K_total // 128, N)},
                  "channel")
    lib = load_library()
    _same_device(A, B, D, ks, SFA, SFB)
    _contig(A, B, D, ks, SFA, SFB)
    with torch.cuda.device(A.device):
        fn = lib.grouped_gemm_kgrouped_psum if psum else lib.grouped_gemm_kgrouped
        _check(fn(dt, G, M, N, K_total, _ptr(A), _ptr(SFA), _ptr(B), _ptr(SFB), _sf_fmt(SFA),
                  _ptr(D), _ptr(ks), 1 if accumulate else 0, _stream(A.device)))
    return D


def quantize_fp8_1x128(X, Q=None, SF=None, sf_fmt="f32", sf_zero=1.0):
    """bf16 X[M, K] -> (Q uint8 [M, K] E4M3 codes, SF [K/128, M] float32 or uint8 UE8M0),
    1x128 per-token scales; Q and SF are allocated when not given."""
    return _quant(False, X, Q, SF, sf_fmt, sf_zero)


def swiglu_quant_fp8_1x128(H, Q=None, SF=None, sf_fmt="f32", sf_zero=1.0):
    """bf16 w13 output H[M, 2I] (gate columns, then up) -> (Q uint8 [M, I] E4M3 codes of
    silu(gate) * up, SF [I/128, M]); Q and SF are allocated when not given."""
    return _quant(True, H, Q, SF, sf_fmt, sf_zero)


def _quant(swiglu, X, Q, SF, sf_fmt, sf_zero):
    import torch
    lib = load_library()
    name = "H" if swiglu else "X"
    _require(X.dtype == torch.bfloat16 and X.dim() == 2,
             f"{name} must be bf16 [M, {'2I' if swiglu else 'K'}]")
    M, K = X.shape
    if swiglu:
        _require(K % 2 == 0, "H must have an even number of columns")
        K //= 2
    if Q is None:
        Q = torch.empty((M, K), dtype=torch.uint8, device=X.device)
    if SF is None:
        SF = torch.empty((K // 128, M), device=X.device,
                         dtype=torch.float32 if sf_fmt == "f32" else torch.uint8)
    _same_device(X, Q, SF)
    _contig(X, Q, SF)
    _require(tuple(Q.shape) == (M, K) and Q.dtype in (torch.uint8, torch.float8_e4m3fn),
             "Q must be uint8 [M, %s]" % ("I" if swiglu else "K"))
    _require(tuple(SF.shape) == (K // 128, M),
             "SF must be [%s/128, M]" % ("I" if swiglu else "K"))
    fmt = {"f32": MGG_SF_F32, "ue8m0": MGG_SF_UE8M0}[sf_fmt]
    _require((SF.dtype == torch.float32) == (fmt == MGG_SF_F32), "SF dtype must match sf_fmt")
    fn = lib.swiglu_quant_fp8_1x128 if swiglu else lib.quantize_fp8_1x128
    with torch.cuda.device(X.device):
        _check(fn(M, K, _ptr(X), _ptr(Q), _ptr(SF), fmt, float(sf_zero), _stream(X.device)))
    return Q, SF
