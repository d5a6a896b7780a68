"""The C-ABI library: it loads, exports every function include/*.h declares, and rejects
invalid host arguments before touching the GPU (these calls enqueue nothing, so they
run without a GPU). CPU only."""

import ctypes
import glob
import os
import re

import pytest

import moe_grouped_gemm_nt_amd as mgg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

EINVAL, EUNSUPPORTED = 1, 2


def declared_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                            text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mgg.library_path()):
        pytest.fail("library not built: run `python -m moe_grouped_gemm_nt_amd.build`")
    return mgg.load_library()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for f in ("grouped_gemm_masked", "grouped_gemm_contiguous", "grouped_gemm_contiguous_psum",
              "grouped_gemm_kgrouped", "grouped_gemm_kgrouped_psum", "quantize_fp8_1x128",
              "swiglu_quant_fp8_1x128", "grouped_gemm_contiguous_swiglu_quant",
              "mgg_status_string", "mgg_last_error"):
        assert f in names
    assert len(names) == 10, names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    assert lib.mgg_status_string(0) == b"ok"
    assert lib.mgg_status_string(1) == b"invalid argument"
    assert lib.mgg_status_string(3) == b"HIP runtime error"


# Fake, never-dereferenced device addresses: every call below fails host validation.
P = ctypes.c_void_p(1 << 20)
MIS = ctypes.c_void_p((1 << 20) + 8)  # 8-byte aligned only
NUL = None


def masked(lib, dt=1, G=2, cap=4, N=16, K=128, A=P, SFA=P, B=P, SFB=P, sf=0, gran=0, D=P,
           cnt=P, em=0):
    return lib.grouped_gemm_masked(dt, G, cap, N, K, A, SFA, B, SFB, sf, gran, D, cnt, em, None)


def contig(lib, dt=1, G=2, M=256, N=16, K=128, A=P, SFA=P, B=P, SFB=P, sf=0, gran=0, D=P,
           idx=P, em=0):
    return lib.grouped_gemm_contiguous(dt, G, M, N, K, A, SFA, B, SFB, sf, gran, D, idx, em, None)


def kgrp(lib, dt=1, G=2, M=16, N=16, KT=256, A=P, SFA=P, B=P, SFB=P, sf=0, D=P, ks=P, acc=1):
    return lib.grouped_gemm_kgrouped(dt, G, M, N, KT, A, SFA, B, SFB, sf, D, ks, acc, None)


def psum_contig(lib, dt=1, G=2, M=256, N=16, K=128, A=P, SFA=P, B=P, SFB=P, sf=0, gran=0, D=P,
                ps=P, em=0):
    return lib.grouped_gemm_contiguous_psum(dt, G, M, N, K, A, SFA, B, SFB, sf, gran, D, ps, em,
                                            None)


def kgrp_psum(lib, dt=1, G=2, M=16, N=16, KT=256, A=P, SFA=P, B=P, SFB=P, sf=0, D=P, ps=P,
              acc=1):
    return lib.grouped_gemm_kgrouped_psum(dt, G, M, N, KT, A, SFA, B, SFB, sf, D, ps, acc, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=7), EINVAL),
    (dict(G=0), EINVAL),
    (dict(G=4097), EINVAL),
    (dict(cap=0), EINVAL),
    (dict(N=12), EINVAL),
    (dict(N=0), EINVAL),
    (dict(K=64), EINVAL),  # FP8 needs K % 128 == 0
    (dict(dt=0, K=12), EINVAL),  # BF16 needs K % 8 == 0
    (dict(A=NUL), EINVAL),
    (dict(B=NUL), EINVAL),
    (dict(D=NUL), EINVAL),
    (dict(cnt=NUL), EINVAL),
    (dict(SFA=NUL), EINVAL),
    (dict(SFB=NUL), EINVAL),
    (dict(A=MIS), EINVAL),
    (dict(D=MIS), EINVAL),
    (dict(sf=5), EINVAL),
    (dict(gran=9), EINVAL),
])
def test_masked_rejects(lib, kw, code):
    assert masked(lib, **kw) == code
    assert lib.mgg_last_error() != b""


@pytest.mark.parametrize("kw,code", [
    (dict(dt=2, sf=0, gran=2), EUNSUPPORTED),  # FP8 x FP4 needs UE8M0 scales
    (dict(dt=2, sf=1, gran=0), EINVAL),  # FP4 weights take 32-K block scales
    (dict(dt=2, sf=1, gran=1), EINVAL),
    (dict(dt=1, sf=1, gran=2), EINVAL),  # 32-K block scales go with FP4 weights only
    (dict(dt=2, sf=1, gran=2, K=64), EINVAL),
    (dict(dt=2, sf=1, gran=2, SFB=NUL), EINVAL),
    (dict(dt=3), EINVAL),
])
def test_fp4_rejects(lib, kw, code):
    assert masked(lib, **kw) == code
    assert contig(lib, **kw) == code
    assert psum_contig(lib, **kw) == code


def fused(lib, dt=1, G=2, M=256, I=128, K=128, A=P, SFA=P, B=P, SFB=P, sf=1, gran=0, Q=P,
          SFQ=P, sfq=1, z=1.0, idx=P):
    return lib.grouped_gemm_contiguous_swiglu_quant(dt, G, M, I, K, A, SFA, B, SFB, sf, gran, Q,
                                                    SFQ, sfq, ctypes.c_float(z), idx, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=0), EUNSUPPORTED),
    (dict(dt=3), EINVAL),
    (dict(I=0), EINVAL),
    (dict(I=192), EINVAL),
    (dict(K=64), EINVAL),
    (dict(G=0), EINVAL),
    (dict(M=0), EINVAL),
    (dict(M=524289), EUNSUPPORTED),
    (dict(Q=NUL), EINVAL),
    (dict(Q=MIS), EINVAL),
    (dict(SFQ=NUL), EINVAL),
    (dict(sfq=0, SFQ=ctypes.c_void_p((1 << 20) + 2)), EINVAL),
    (dict(sfq=4), EINVAL),
    (dict(z=0.0), EINVAL),
    (dict(z=float("nan")), EINVAL),
    (dict(idx=NUL), EINVAL),
    (dict(sf=1, gran=1), EUNSUPPORTED),  # byte-run channel scales are not gathered
    (dict(dt=2, sf=1, gran=0), EINVAL),  # FP4 weights take 32-K block scales
    (dict(dt=2, sf=0, gran=2), EUNSUPPORTED),
])
def test_fused_swiglu_rejects(lib, kw, code):
    assert fused(lib, **kw) == code
    assert lib.mgg_last_error() != b""


def test_fp4_kgrouped_unsupported(lib):
    assert kgrp(lib, dt=2, sf=1) == EUNSUPPORTED
    assert kgrp_psum(lib, dt=2, sf=1) == EUNSUPPORTED


@pytest.mark.parametrize("kw,code", [
    (dict(M=0), EINVAL),
    (dict(M=524289), EUNSUPPORTED),
    (dict(G=0), EINVAL),
    (dict(idx=NUL), EINVAL),
    (dict(K=100), EINVAL),
    (dict(B=MIS), EINVAL),
])
def test_contiguous_rejects(lib, kw, code):
    assert contig(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(acc=2), EINVAL),
    (dict(KT=-128), EINVAL),
    (dict(KT=200), EINVAL),  # FP8 token axis must be a multiple of 128
    (dict(G=0), EINVAL),
    (dict(M=0), EINVAL),
    (dict(N=4), EINVAL),
    (dict(ks=NUL), EINVAL),
    (dict(SFB=NUL), EINVAL),
])
def test_kgrouped_rejects(lib, kw, code):
    assert kgrp(lib, **kw) == code


def test_binding_raises_with_message_on_bad_input():
    import torch
    A = torch.zeros((2, 4, 128), dtype=torch.uint8)
    with pytest.raises(ValueError):  # CPU tensors are refused before the C call
        mgg.grouped_gemm_masked(A, A, torch.zeros((2, 4, 4), dtype=torch.bfloat16),
                                torch.zeros(2, dtype=torch.int32))


def test_product_path_does_not_import_the_oracle():
    """The package and its sources never reference the oracle."""
    pkg = os.path.join(ROOT, "moe_grouped_gemm_nt_amd")
    for path in glob.glob(os.path.join(pkg, "**", "*"), recursive=True):
        if os.path.isfile(path) and path.endswith((".py", ".hip", ".h", ".cpp")):
            text = open(path).read()
            assert "import oracle" not in text and "from oracle" not in text, path
            assert "oracle/" not in text, path


@pytest.mark.parametrize("kw,code", [
    (dict(dt=7), EINVAL),
    (dict(G=0), EINVAL),
    (dict(G=4097), EINVAL),
    (dict(M=0), EINVAL),
    (dict(N=12), EINVAL),
    (dict(K=100), EINVAL),
    (dict(dt=0, K=12), EINVAL),
    (dict(A=NUL), EINVAL),
    (dict(ps=NUL), EINVAL),
    (dict(SFA=NUL), EINVAL),
    (dict(A=MIS), EINVAL),
    (dict(ps=ctypes.c_void_p((1 << 20) + 2)), EINVAL),
    (dict(sf=5), EINVAL),
    (dict(gran=9), EINVAL),
])
def test_contiguous_psum_rejects(lib, kw, code):
    assert psum_contig(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(dt=7), EINVAL),
    (dict(G=0), EINVAL),
    (dict(M=0), EINVAL),
    (dict(KT=-1), EINVAL),
    (dict(KT=200), EINVAL),
    (dict(ps=NUL), EINVAL),
    (dict(acc=2), EINVAL),
    (dict(D=MIS), EINVAL),
])
def test_kgrouped_psum_rejects(lib, kw, code):
    assert kgrp_psum(lib, **kw) == code


def quant(lib, M=64, K=256, X=P, Q=P, SF=P, sf=0, z=1.0):
    return lib.quantize_fp8_1x128(M, K, X, Q, SF, sf, ctypes.c_float(z), None)


@pytest.mark.parametrize("kw,code", [
    (dict(M=0), EINVAL),
    (dict(K=0), EINVAL),
    (dict(K=200), EINVAL),
    (dict(X=NUL), EINVAL),
    (dict(Q=NUL), EINVAL),
    (dict(SF=NUL), EINVAL),
    (dict(X=MIS), EINVAL),
    (dict(Q=ctypes.c_void_p((1 << 20) + 4)), EINVAL),
    (dict(SF=ctypes.c_void_p((1 << 20) + 2)), EINVAL),
    (dict(sf=3), EINVAL),
    (dict(z=0.0), EINVAL),
    (dict(z=-1.0), EINVAL),
    (dict(z=float("inf")), EINVAL),
    (dict(z=float("nan")), EINVAL),
    (dict(K=128 * 65536), EUNSUPPORTED),
])
def test_quantize_rejects(lib, kw, code):
    assert quant(lib, **kw) == code
    assert lib.mgg_last_error() != b""


def swiglu_quant(lib, M=64, I=256, H=P, Q=P, SF=P, sf=0, z=1.0):
    return lib.swiglu_quant_fp8_1x128(M, I, H, Q, SF, sf, ctypes.c_float(z), None)


@pytest.mark.parametrize("kw,code", [
    (dict(M=0), EINVAL),
    (dict(M=-3), EINVAL),
    (dict(I=0), EINVAL),
    (dict(I=192), EINVAL),
    (dict(H=NUL), EINVAL),
    (dict(Q=NUL), EINVAL),
    (dict(SF=NUL), EINVAL),
    (dict(H=MIS), EINVAL),
    (dict(Q=ctypes.c_void_p((1 << 20) + 4)), EINVAL),
    (dict(SF=ctypes.c_void_p((1 << 20) + 2)), EINVAL),
    (dict(sf=2), EINVAL),
    (dict(z=0.0), EINVAL),
    (dict(z=float("inf")), EINVAL),
    (dict(I=128 * 65536), EUNSUPPORTED),
])
def test_swiglu_quantize_rejects(lib, kw, code):
    assert swiglu_quant(lib, **kw) == code
    assert lib.mgg_last_error() != b""
