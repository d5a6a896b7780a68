"""Ahead-of-time build of the HIP library for gfx950 (MI355X).

`python -m moe_grouped_gemm_nt_amd.build` compiles csrc/*.hip into
moe_grouped_gemm_nt_amd/libmoe_grouped_gemm_nt.so with hipcc. No JIT and no runtime
compilation: the library that ships next to this file is the one that runs.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB_NAME = "libmoe_grouped_gemm_nt.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["csrc/grouped_gemm.hip", "csrc/quantize.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def compile_flags(extra=()):
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-shared",
        # Packed-FP32 VALU instructions stay off: the compiler would otherwise form them
        # from ordinary float code.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
        "-I", os.path.join(PKG, "csrc"),
        *extra,
    ]


def build(verbose: bool = True, extra=()) -> str:
    """Compile the library in place; returns its path. Always recompiles."""
    srcs = [os.path.join(PKG, s) for s in SOURCES]
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *compile_flags(extra), *srcs, "-o", tmp]
    if verbose:
        print("[build]", " ".join(cmd), flush=True)
    res = subprocess.run(cmd, cwd=PKG, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print("[build] wrote", LIB_PATH, flush=True)
    return LIB_PATH


if __name__ == "__main__":
    build()
