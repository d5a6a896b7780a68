"""The Python binding refuses scale tensors that do not match the layouts of
include/moe_grouped_gemm_nt.h before anything reaches the library (CPU only: the checks
run ahead of the device check, so CPU tensors exercise them; a call that passes them stops
at the device check instead).

The kernels size their scale reads from the problem shape, so a scale tensor of another
storage type, granularity or orientation would be read out of bounds or misread."""

import re

import pytest
import torch

import moe_grouped_gemm_nt_amd as mgg
from moe_grouped_gemm_nt_amd import synth

DEVICE_MSG = "same GPU"


def expect(fn, pattern):
    with pytest.raises(ValueError) as ei:
        fn()
    assert re.search(pattern, str(ei.value)), str(ei.value)


def reaches_device_check(fn):
    """The arguments pass every host-side check: the call stops at the device check."""
    expect(fn, DEVICE_MSG)


@pytest.fixture(scope="module")
def masked():
    return synth.make_masked("fp8", 2, 8, 256, 256, [3, 8], seed=1)


def test_masked_well_formed_reaches_device_check(masked):
    p = masked
    D = torch.zeros((2, 8, 256), dtype=torch.bfloat16)
    reaches_device_check(lambda: mgg.grouped_gemm_masked(p.A, p.B, D, p.counts, p.SFA, p.SFB))


@pytest.mark.parametrize("case", ["sfb_ue8m0", "sfa_transposed", "sfb_channel_shape",
                                  "gran_channel", "sfa_missing", "sfa_f64", "gran_block32",
                                  "sfb_one_expert"])
def test_masked_scale_mismatches(masked, case):
    p = masked
    D = torch.zeros((2, 8, 256), dtype=torch.bfloat16)
    SFA, SFB, gran, pat = p.SFA, p.SFB, None, None
    if case == "sfb_ue8m0":
        SFB, pat = torch.zeros(p.SFB.shape, dtype=torch.uint8), "same storage type"
    elif case == "sfa_transposed":
        SFA, pat = p.SFA.transpose(1, 2).contiguous(), r"SFA must be \[2, 2, 8\]"
    elif case == "sfb_channel_shape":
        SFB, pat = torch.ones((2, 2, 256)), r"SFB \(block128\) must be \[2, 2, 2\]"
    elif case == "gran_channel":
        gran, pat = "channel", r"SFB \(channel\) must be \[2, 2, 256\]"
    elif case == "sfa_missing":
        SFA, pat = None, "need SFA and SFB"
    elif case == "sfa_f64":
        SFA, SFB = p.SFA.double(), p.SFB.double()
        pat = "float32 or uint8"
    elif case == "gran_block32":
        gran, pat = "block32", "granularity 'block32'"
    elif case == "sfb_one_expert":
        SFB, pat = p.SFB[:1].contiguous(), r"SFB \(block128\) must be"
    expect(lambda: mgg.grouped_gemm_masked(p.A, p.B, D, p.counts, SFA, SFB, gran), pat)


def test_bf16_takes_no_scales():
    p = synth.make_masked("bf16", 2, 8, 256, 256, [3, 8], seed=1)
    D = torch.zeros((2, 8, 256), dtype=torch.bfloat16)
    expect(lambda: mgg.grouped_gemm_masked(p.A, p.B, D, p.counts, torch.ones(2, 2, 8),
                                           torch.ones(2, 2, 2)), "no scale tensors")
    reaches_device_check(lambda: mgg.grouped_gemm_masked(p.A, p.B, D, p.counts))


@pytest.mark.parametrize("entry", ["contiguous", "psum"])
def test_contiguous_scale_layouts(entry):
    p = synth.make_contiguous("fp8", 3, 256, 384, [100, 0, 60], seed=2, M_max=384,
                              sf_fmt="ue8m0")
    D = torch.zeros((p.M, 256), dtype=torch.bfloat16)
    route = p.m_indices if entry == "contiguous" else torch.tensor([100, 100, 160],
                                                                    dtype=torch.int32)
    fn = mgg.grouped_gemm_contiguous if entry == "contiguous" else mgg.grouped_gemm_contiguous_psum
    reaches_device_check(lambda: fn(p.A, p.B, D, route, p.SFA, p.SFB))
    expect(lambda: fn(p.A, p.B, D, route, p.SFA.t().contiguous(), p.SFB),
           r"SFA must be \[3, 384\]")
    expect(lambda: fn(p.A, p.B, D, route, p.SFA.float(), p.SFB), "same storage type")
    expect(lambda: fn(p.A, p.B, D, route, p.SFA, torch.zeros((3, 3, 256), dtype=torch.uint8),
                      "block128"), r"SFB \(block128\) must be \[3, 2, 3\]")


def test_fp4_weight_scales():
    p = synth.make_contiguous("fp8_fp4", 2, 128, 256, [64, 64], seed=3, M_max=256,
                              sf_fmt="ue8m0", sfb_gran="block32")
    D = torch.zeros((p.M, 128), dtype=torch.bfloat16)
    reaches_device_check(lambda: mgg.grouped_gemm_contiguous(p.A, p.B, D, p.m_indices, p.SFA,
                                                             p.SFB))
    expect(lambda: mgg.grouped_gemm_contiguous(p.A, p.B, D, p.m_indices, p.SFA, p.SFB,
                                               "block128"), "granularity 'block128'")
    expect(lambda: mgg.grouped_gemm_contiguous(p.A, p.B, D, p.m_indices, p.SFA.float(),
                                               p.SFB.float()), "UE8M0")
    expect(lambda: mgg.grouped_gemm_contiguous(p.A, p.B, D, p.m_indices, p.SFA,
                                               p.SFB[:, :, :, :2].contiguous()),
           r"SFB \(block32\) must be \[2, 2, 128, 4\]")


def test_kgrouped_scale_layouts():
    p = synth.make_kgrouped("fp8", [128, 256], 128, 256, seed=4)
    D = torch.zeros((2, 128, 256))
    reaches_device_check(lambda: mgg.grouped_gemm_kgrouped(p.A, p.B, D, p.ks, 128, 256, p.SFA,
                                                           p.SFB))
    expect(lambda: mgg.grouped_gemm_kgrouped(p.A, p.B, D, p.ks, 128, 256,
                                             p.SFA.t().contiguous(), p.SFB),
           r"SFA must be \[3, 128\]")
    expect(lambda: mgg.grouped_gemm_kgrouped(p.A, p.B, D, p.ks, 128, 256, p.SFA,
                                             p.SFA), r"SFB \(channel\) must be \[3, 256\]")
    expect(lambda: mgg.grouped_gemm_kgrouped(p.A, p.B, D, p.ks, 128, 256, p.SFA, None),
           "need SFA and SFB")


def test_fused_swiglu_weight_scales():
    p = synth.make_contiguous("fp8", 2, 512, 256, [64, 64], seed=5, M_max=256,
                              sf_fmt="ue8m0")
    Q = torch.zeros((p.M, 256), dtype=torch.uint8)
    SFQ = torch.zeros((2, p.M), dtype=torch.uint8)
    reaches_device_check(lambda: mgg.grouped_gemm_contiguous_swiglu_quant(
        p.A, p.B, p.m_indices, p.SFA, p.SFB, Q, SFQ))
    expect(lambda: mgg.grouped_gemm_contiguous_swiglu_quant(
        p.A, p.B, p.m_indices, p.SFA, p.SFB[:, :2].contiguous(), Q, SFQ),
        r"SFB \(block128\) must be \[2, 4, 2\]")
    bf = synth.make_contiguous("bf16", 2, 512, 256, [64, 64], seed=5, M_max=256)
    expect(lambda: mgg.grouped_gemm_contiguous_swiglu_quant(
        bf.A, bf.B, bf.m_indices, None, None, Q, SFQ), "takes FP8 activations")
