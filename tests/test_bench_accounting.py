"""CPU tests of the benchmark's host logic: the algorithmic bytes behind the roofline
and the split into input and output bytes that sizes the rotated input copies. Each
expected value is recomputed here from the problem's shapes and routing, element by
element, independently of bench.py's formulas; the refusal of more than one GPU;
and the rule that HBM counter readings are reported only for the kernel sources they were
taken on."""

import numpy as np
import pytest

import bench
from moe_grouped_gemm_nt_amd import synth


def _expected(p, accumulate=True):
    """(input bytes, output bytes) a perfect kernel moves: every operand element feeding a
    valid output once, every scale once, valid outputs written once (+ read once when
    accumulating)."""
    esz = 2 if p.dtype == "bf16" else 1
    wsz = 0.5 if p.dtype == "fp8_fp4" else esz
    sf = 4 if p.sf_fmt == "f32" else 1
    if p.variant == "kgrouped":
        T = int(np.sum(p.meta["ks"]))
        inp = p.M * T * esz + p.N * T * esz
        if p.dtype != "bf16":
            inp += (T // 128) * (p.M + p.N) * sf
        return inp, p.G * p.M * p.N * 4 * (2 if accumulate else 1)
    if p.variant == "masked":
        counts = np.clip(p.meta["counts"], 0, p.cap)
        experts_used = [g for g in range(p.G) if counts[g] > 0]
        rows = int(counts.sum())
    else:
        idx = p.meta["m_indices"]
        experts_used = sorted(set(int(e) for e in idx if e >= 0))
        rows = int((idx >= 0).sum())
    kb = p.K // 128
    inp = 0
    for _ in range(rows):  # activation row and its scales
        inp += p.K * esz + (kb * sf if p.dtype != "bf16" else 0)
    for _ in experts_used:  # each used expert's weights and weight scales, once
        inp += int(p.N * p.K * wsz)
        if p.dtype != "bf16":
            per = {"block128": -(-p.N // 128) * kb, "channel": p.N * kb,
                   "block32": p.N * kb * 4}[p.sfb_gran]
            inp += per * sf
    return inp, rows * p.N * 2


CASES = [
    ("masked", dict(dtype="bf16", G=4, cap=40, N=64, K=256, counts=[0, 40, 7, 100])),
    ("masked", dict(dtype="fp8", G=3, cap=33, N=136, K=384, counts=[33, 0, 5])),
    ("masked", dict(dtype="fp8", G=3, cap=33, N=136, K=384, counts=[1, 2, 3],
                    sf_fmt="ue8m0", sfb_gran="channel")),
    ("masked", dict(dtype="fp8_fp4", G=2, cap=16, N=128, K=256, counts=[16, 9],
                    sf_fmt="ue8m0", sfb_gran="block32")),
    ("contiguous", dict(dtype="fp8", G=4, N=200, K=256, seg_counts=[130, 0, 1, 127],
                        sf_fmt="ue8m0")),
    ("contiguous", dict(dtype="bf16", G=3, N=64, K=128, seg_counts=[5, 128, 0])),
    ("kgrouped", dict(dtype="fp8", ks=[256, 128, 0, 128], M=64, N=96)),
    ("kgrouped", dict(dtype="bf16", ks=[8, 24], M=32, N=16)),
]


@pytest.mark.parametrize("kind,kw", CASES)
@pytest.mark.parametrize("accumulate", [True, False])
def test_algorithmic_bytes_split(kind, kw, accumulate):
    kw = dict(kw)
    if kind == "masked":
        p = synth.make_masked(kw.pop("dtype"), kw.pop("G"), kw.pop("cap"), kw.pop("N"),
                              kw.pop("K"), kw.pop("counts"), seed=1, **kw)
    elif kind == "contiguous":
        p = synth.make_contiguous(kw.pop("dtype"), kw.pop("G"), kw.pop("N"), kw.pop("K"),
                                  kw.pop("seg_counts"), seed=2, **kw)
    else:
        p = synth.make_kgrouped(kw.pop("dtype"), kw.pop("ks"), kw.pop("M"), kw.pop("N"),
                                seed=3)
    opt = {"accumulate": accumulate, "expected_m": 0}
    exp_in, exp_out = _expected(p, accumulate)
    assert bench.algorithmic_output_bytes(p, opt) == exp_out
    assert bench.algorithmic_bytes(p, opt) == exp_in + exp_out


def test_rotated_input_copies():
    """Default copies: one cycle reads at least four times the Infinity Cache and one copy
    fewer would not; the 8 GiB allocation cap and an explicit request take precedence."""
    mall = bench.MALL_BYTES
    for in_read in (1, 3_200_000, 102_000_000, 126_000_000, 737_000_000, 1_600_000_000):
        n = bench.rotated_input_copies(in_read, in_read)
        assert n * in_read >= 4 * mall
        assert n == 1 or (n - 1) * in_read < 4 * mall
    # a 3.2 MB read from a 6 GB allocation (mostly unread capacity rows): capped at one copy
    assert bench.rotated_input_copies(3_200_000, 6 << 30) == 1
    assert bench.rotated_input_copies(3_200_000, 1 << 30) == 8
    assert bench.rotated_input_copies(102_000_000, 377_000_000, requested=1) == 1
    assert bench.rotated_input_copies(102_000_000, 377_000_000, requested=3) == 3


def test_more_than_one_gpu_is_refused():
    """`--gpus N` above 1 ends with a message and a non-zero status, before any GPU work."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_code_only_ignores_comments_and_blank_lines():
    a = "int f(int x) {  // twice\n\n  return 2 * x; /* doubled\n over lines */\n}\n"
    b = "int f(int x) {\n  return 2 * x;\n}"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(b) != bench._code_only(b.replace("2 *", "3 *"))


def _traffic_file(root, workload, digest, fetch, write):
    (root / "profiles").mkdir(exist_ok=True)
    (root / "profiles" / f"{workload}_hbm_traffic.md").write_text(
        f"# counters\n\n- kernel-source-sha256: {digest}\n"
        f"- fetch_bytes_per_launch: {fetch}\n- write_bytes_per_launch: {write}\n")


@pytest.mark.parametrize("workload", ["kgrouped_fp8_wgrad", "quant_fp8_1x128_6144x7168"])
def test_traffic_only_for_the_current_kernel_sources(tmp_path, monkeypatch, workload):
    """Counter readings are reported only while the kernel's sources hash to the digest
    stored with them; a stale or missing reading gives None (JSON null)."""
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic(workload) is None
    current = bench.kernel_source_digest(bench.kernel_name(workload))
    _traffic_file(tmp_path, workload, current, 1000, 234)
    assert bench.measured_traffic(workload) == 1234
    _traffic_file(tmp_path, workload, "0" * 64, 1000, 234)
    assert bench.measured_traffic(workload) is None
    # the two kernels are built from different sources, so their digests differ
    assert bench.kernel_source_digest(bench.KERNEL_NAME) != \
        bench.kernel_source_digest(bench.QUANT_KERNEL_NAME)


def test_host_cpu_model_is_named():
    """The oracle baseline names the host CPU it ran on."""
    name = bench.host_cpu_model()
    assert isinstance(name, str) and name


def _counter_csv(directory, dispatches):
    """A rocprofv3-style counter_collection.csv: dispatches = {id: {counter: [values]}};
    a counter with several values is written as several rows (summed per dispatch)."""
    import csv
    directory.mkdir(parents=True)
    kname = "void mgg::grouped_gemm_kernel<mgg::Tile<128, 256, 2, 4, 3, false, false>, 0, 1, 0, 0, false>(mgg::Params)"
    with open(directory / "w_counter_collection.csv", "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for d, cs in dispatches.items():
            for name, vals in cs.items():
                for v in vals:
                    wr.writerow([d, kname, name, v])


def test_counter_summary_arithmetic(tmp_path, monkeypatch):
    """The counter summary sums a dispatch's rows, takes medians over dispatches, and
    derives the clock, L2 hit rate and tile count from them and from the workload."""
    import argparse
    w = "masked_fp8_g6_n4096"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / f"{w}_kernel_trace.md").write_text(
        "| `void mgg::grouped_gemm_kernel<mgg::Tile<128, 256, 2, 4, 3, false, false>, 0, 1, 0, 0, "
        "false>(mgg::Params)` | 7050 | 100000 | 90000 | 110000 | 1000 |\n")
    names = [n for p in bench.COUNTER_PASSES for n in p.split()]
    base = {n: 10.0 for n in names}
    base.update({"GRBM_GUI_ACTIVE": 8 * 220000.0, "TCC_HIT_sum": 3.0, "TCC_MISS_sum": 1.0,
                 "SQ_WAVES": 3072.0, "SQ_INSTS_MFMA": 816 * 32 * 128.0})
    for i, p in enumerate(bench.COUNTER_PASSES, 1):
        disp = {}
        for d, scale in ((1, 0.5), (2, 1.0), (3, 3.0)):  # median dispatch: scale 1
            disp[d] = {n: ([base[n] * scale / 2] * 2 if n == "TCC_HIT_sum" else [base[n] * scale])
                       for n in p.split()}
        _counter_csv(tmp_path / f"cnt_{i}", disp)
    args = argparse.Namespace(workload=w, summarize_counters=str(tmp_path / "cnt"),
                              summarize_mfma_busy=None)
    bench.summarize_counters(args)
    text = (tmp_path / "profiles" / f"{w}_counters.md").read_text()
    assert "shader clock ~2.20 GHz" in text          # 220k cycles over 100 us
    assert "L2 hit rate 75.0 %" in text              # 3 / (3 + 1), the hit rows summed
    assert "816 tiles of 128 x 256" in text          # the workload's counts
    assert "100.0 % of 816 tiles x 32 slices x 128 MFMAs" in text
    assert "8 MFMA, 4 copy" in text
    assert bench.kernel_source_digest(bench.KERNEL_NAME) in text
