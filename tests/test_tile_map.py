"""The scheduler's tile mapping compiled for the host and checked exhaustively.

`moe_grouped_gemm_nt_amd/csrc/tile_map.h` holds the integer functions the kernel decodes
its tiles with (XCD-aware first tile, the last round split along N, expert lookup over
the tile prefix, contiguous and K-grouped tile orders). `tests/tile_map_check.cpp` builds
them with the host compiler and, for thousands of seeded layouts, checks by brute force
that every output (expert, m-tile, column) of a masked, prefix-sum or contiguous layout
is covered exactly once, no tile starts past its expert's rows, the K-grouped order is a
bijection with the intended 8 x 4 footprint, and the first-tile order is a permutation.

The negative control compiles copies of the header with one planted mistake each, on the
CPU, and requires the check to fail on every one."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "moe_grouped_gemm_nt_amd", "csrc")
CHECK = os.path.join(ROOT, "tests", "tile_map_check.cpp")
HIP_INC = "/opt/rocm/include"

needs_gxx = pytest.mark.skipif(
    shutil.which("g++") is None or not os.path.isdir(HIP_INC),
    reason="needs g++ and the HIP headers")


def build_and_run(tmp_path, header_dir):
    exe = tmp_path / "tile_map_check"
    subprocess.run(["g++", "-std=c++17", "-O1", "-D__HIP_PLATFORM_AMD__", "-I" + HIP_INC,
                    "-I" + str(header_dir), CHECK, "-o", str(exe)],
                   check=True, capture_output=True, text=True, timeout=120)
    return subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)


@needs_gxx
def test_tile_map_covers_every_output_once(tmp_path):
    r = build_and_run(tmp_path, CSRC)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr


# (text in tile_map.h, planted replacement): each breaks one property the check covers
MUTATIONS = [
    ("(long)(b % xcds) * per + b / xcds", "(long)(b % xcds) * per + b / (xcds + 1)"),
    ("r.total = base + last * pieces;", "r.total = base + last * pieces - 1;"),
    ("if (4 * last <= grid && bn / 4 >= wtn)", "if (4 * last <= grid)"),
    ("const int b = a + width < N ? a + width : N;", "const int b = a + width;"),
    ("if (prefix[mid] <= t) lo = mid;", "if (prefix[mid] < t) lo = mid;"),
    ("*nt = local / mt_g;\n  *mt = local % mt_g;", "*nt = local % mt_g;\n  *mt = local / mt_g;"),
    ("*sub = (int)(rest % sub_per_block);", "*sub = (int)(rest % (sub_per_block + 1));"),
    ("*mt = m_first + in_g % gsz;", "*mt = m_first + in_g % group_m;"),
    ("*nt = in_g / gsz;", "*nt = in_g / group_m;"),
]


@needs_gxx
@pytest.mark.parametrize("i", range(len(MUTATIONS)))
def test_tile_map_check_catches_planted_mistake(tmp_path, i):
    old, new = MUTATIONS[i]
    src = open(os.path.join(CSRC, "tile_map.h")).read()
    assert src.count(old) == 1, f"mutation {i} no longer matches tile_map.h"
    hdr = tmp_path / "hdr"
    hdr.mkdir()
    (hdr / "tile_map.h").write_text(src.replace(old, new))
    r = build_and_run(tmp_path, hdr)
    assert r.returncode == 1 and "FAIL" in r.stdout, f"mutation {i} not caught: {r.stdout}"
