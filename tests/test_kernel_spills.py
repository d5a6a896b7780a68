"""No register spill inside the MFMA slice loop of any shipped kernel.

The eight-wave FP8 tile with float32 scales runs three waves per SIMD and so has 168
VGPRs per wave; it is compiled right at that limit and spills a few registers. Spills in
its set-up, per-tile decode or epilogue cost little, but a spill that the compiler places
in a basic block that issues MFMAs puts a scratch round trip into every 128-K slice: a
change to unrelated scheduler code once moved one there and slowed the 6-expert FP8 shape
by a quarter. This test compiles the library's device code for gfx950 to assembly, with
the flags of the shipped build, and fails if any basic block that contains an MFMA also
touches scratch memory."""

import os
import re
import subprocess

import pytest

from moe_grouped_gemm_nt_amd import build as mgg_build

try:
    HIPCC = mgg_build.hipcc()
except RuntimeError:
    HIPCC = None


def kernel_blocks(asm):
    """{kernel symbol: [(block label, [instruction lines])]} of every kernel in `asm`."""
    out = {}
    name, blocks = None, None
    for line in asm.splitlines():
        m = re.match(r"^(_Z\S+):\s*;\s*@", line)
        if m:
            name, blocks = m.group(1), [("entry", [])]
            out[name] = blocks
            continue
        if name is None:
            continue
        if line.startswith(".Lfunc_end"):
            name = None
            continue
        if re.match(r"^\.LBB\d+_\d+:", line):
            blocks.append((line.split(":")[0], []))
        else:
            blocks[-1][1].append(line)
    return out


@pytest.mark.skipif(HIPCC is None, reason="needs hipcc")
def test_no_spill_in_mfma_blocks(tmp_path):
    flags = [f for f in mgg_build.compile_flags() if f not in ("-fPIC", "-shared")]
    bad, n_mfma_blocks, n_kernels = [], 0, 0
    for src in mgg_build.SOURCES:
        out = tmp_path / (os.path.basename(src) + ".s")
        subprocess.run([HIPCC, *flags, "--cuda-device-only", "-S",
                        os.path.join(mgg_build.PKG, src), "-o", str(out)],
                       check=True, capture_output=True, text=True, timeout=600)
        for kern, blocks in kernel_blocks(out.read_text()).items():
            n_kernels += 1
            for label, lines in blocks:
                if not any("v_mfma" in x for x in lines):
                    continue
                n_mfma_blocks += 1
                if any("scratch_" in x for x in lines):
                    bad.append(f"{kern} {label}")
    assert n_kernels > 30 and n_mfma_blocks > 30, (n_kernels, n_mfma_blocks)
    assert not bad, "scratch access in MFMA blocks:\n" + "\n".join(bad)


def test_block_parser_finds_planted_spill():
    """The parser on a hand-written fragment: a scratch access next to an MFMA is found,
    one in another block of the same kernel is not."""
    asm = "\n".join([
        "_ZN3mgg1kE:  ; @_ZN3mgg1kE",
        "  scratch_store_dword off, v1, off",
        ".LBB0_1:",
        "  v_mfma_f32_16x16x128_f8f6f4 v[0:3], v[4:11], v[12:19], 0",
        "  scratch_load_dword v2, off, off",
        ".LBB0_2:",
        "  v_mfma_f32_16x16x128_f8f6f4 v[0:3], v[4:11], v[12:19], 0",
        ".Lfunc_end0:",
    ])
    blocks = kernel_blocks(asm)["_ZN3mgg1kE"]
    flagged = [lab for lab, lines in blocks
               if any("v_mfma" in x for x in lines) and any("scratch_" in x for x in lines)]
    assert flagged == [".LBB0_1"]
