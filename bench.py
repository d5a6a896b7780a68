"""Benchmark of the grouped NT GEMM hot path on one MI355X.

One step = one grouped-GEMM call over one batch of synthetic inputs already resident in
HBM: the group scheduler, operand and scale staging, MFMA main loop, FP8 scale promotion
and the row-masked epilogue all run inside it. The default workload is the largest
masked configuration of the performance table in the DeepGEMM PR "Fix cross-expert
output overwrites in SM90 masked GEMM": 32 experts of capacity 4096, N = 6144, K = 7168,
valid rows ~ Poisson(192) per expert, FP8 E4M3 with 1x128 activation and 128x128 weight
float32 scales, bf16 output. --workload picks any other named workload, among them
`contig_fp8_w13_redraw` / `contig_fp8_w2_redraw`: the 288-expert contiguous GEMMs of the
DeepGEMM issue "SM120 m_grouped_fp8 contiguous kernel: illegal memory access at CUDA graph
replay" with the routing redrawn for every captured call (each call reads its own
pre-uploaded expert-index draw).

Timing: `--warmup` untimed steps, then exactly `--steps` steps captured into one hipGraph;
the graph is replayed `--samples` times (default 7), each replay between HIP events
recorded on the launch stream and bracketed by device synchronization, and the median
replay gives the time per step (the pages' method: the median of 7 event-timed samples
of graph-captured calls). Outputs rotate over enough buffers that their footprint exceeds
the 256 MB Infinity Cache, and so do copies of the inputs (the bytes each step reads,
times the copies, exceed four times the cache), so each step reads its operands from HBM
and writes its output there.

Prints one JSON line with the metric, the roofline of the kernel and the CPU oracle's
throughput on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

HBM_PEAK_GBS = 8000.0
# dense MFMA peaks; an FP8 x FP4 product is priced at the FP8 rate (the faster FP4 rate
# needs FP4 on both operands)
MFMA_PEAK_TFLOPS = {"bf16": 2516.6, "fp8": 5033.2, "fp8_fp4": 5033.2}
MALL_BYTES = 256 << 20
ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "moe_grouped_gemm_nt_amd", "csrc")


KERNEL_NAME = "grouped_gemm_kernel"
QUANT_KERNEL_NAME = "quant_rows_1x128"
# the sources each kernel is compiled from (the public header only declares entry points)
KERNEL_SOURCES = {
    KERNEL_NAME: ("gemm_engine.h", "grouped_gemm_kernel.h", "tile_map.h", "grouped_gemm.hip",
                  "act_math.h"),
    QUANT_KERNEL_NAME: ("quantize.hip", "act_math.h"),
}


def kernel_name(workload: str) -> str:
    return QUANT_KERNEL_NAME if workload in QUANT_WORKLOADS else KERNEL_NAME


def _code_only(text: str) -> str:
    """C++ source without comments and blank lines (edits to comments leave the kernel,
    and so its counter readings, unchanged)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_source_digest(kernel: str = KERNEL_NAME) -> str:
    """SHA-256 over the code (comments stripped) of the sources a kernel is built from, so
    that HBM counter readings taken on one version of the kernel are never reported for
    another."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        h.update(name.encode())
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per launch from the calibrated FETCH_SIZE / WRITE_SIZE readings stored in
    profiles/<workload>_hbm_traffic.md, or None when there are none for the current
    kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            m = re.match(r"^\s*-\s*([a-z_0-9-]+):\s*(\S+)", line)
            if m:
                fields[m.group(1)] = m.group(2)
    if fields.get("kernel-source-sha256") != kernel_source_digest(kernel_name(workload)):
        return None
    try:
        return int(fields["fetch_bytes_per_launch"]) + int(fields["write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--samples", type=int, default=7,
                    help="replays of the captured graph of `steps` calls; the median is reported")
    ap.add_argument("--workload", default="masked_fp8_g32_n6144")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--rotate-inputs", type=int, default=0,
                    help="input copies rotated over the steps (default: enough that the bytes "
                         "read per cycle exceed four times the Infinity Cache; 1 keeps the "
                         "inputs warm)")
    ap.add_argument("--rotate", type=int, default=0,
                    help="output buffers to rotate over (0: enough to exceed the MALL)")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="(no GPU) write profiles/<workload>_kernel_trace.md from the csv "
                         "output of `rocprofv3 --kernel-trace --stats` of this script")
    ap.add_argument("--summarize-counters", metavar="PREFIX",
                    help="(no GPU) write profiles/<workload>_counters.md from the csv output of "
                         "the four `rocprofv3 --pmc` passes in PREFIX_1 .. PREFIX_4 (counter "
                         "lists in COUNTER_PASSES)")
    ap.add_argument("--summarize-mfma-busy", metavar="PREFIX",
                    help="(no GPU) write profiles/grouped_gemm_kernel_mfma_busy_and_clock.md from "
                         "the csv output of one `rocprofv3 --pmc` run per workload in "
                         "PREFIX<workload> (counters in MFMA_BUSY_COUNTERS)")
    ap.add_argument("--summarize-traffic", nargs=4,
                    metavar=("COPY_FETCH", "COPY_WRITE", "FETCH", "WRITE"),
                    help="(no GPU) write profiles/<workload>_hbm_traffic.md from the csv "
                         "output of four `rocprofv3 --pmc` runs: FETCH_SIZE and WRITE_SIZE of "
                         "--workload copy_calibration, then of the workload")
    return ap.parse_args()


def rotated_input_copies(in_read: int, in_alloc: int, requested: int = 0) -> int:
    """Input copies to rotate over the timed steps: `requested` when positive, else enough
    that one cycle reads more than four times the Infinity Cache (in_read bytes per step);
    never more than 8 GiB of copies (in_alloc bytes each) and at least one."""
    n = requested if requested > 0 else -(-4 * MALL_BYTES // max(1, in_read))
    return max(1, min(n, (8 << 30) // max(1, in_alloc)))


def algorithmic_output_bytes(p, opt) -> int:
    """The output part of algorithmic_bytes: valid output rows written once (and read once
    more when accumulating)."""
    import numpy as np
    if p.variant == "kgrouped":
        return p.G * p.M * p.N * 4 * (2 if opt.get("accumulate", True) else 1)
    if p.variant == "masked":
        rows = int(np.clip(p.meta["counts"], 0, p.cap).sum())
    else:
        rows = int((p.meta["m_indices"] >= 0).sum())
    return rows * p.N * 2


def algorithmic_bytes(p, opt) -> int:
    """Bytes a perfect kernel must move per call: every operand byte that feeds a valid
    output once, every scale once, valid output rows written once (read once more when
    accumulating)."""
    import numpy as np
    esz = 2 if p.dtype == "bf16" else 1
    wsz = 0.5 if p.dtype == "fp8_fp4" else esz  # weight bytes per element
    sf = 4 if p.sf_fmt == "f32" else 1
    if p.variant == "kgrouped":
        T = int(np.sum(p.meta["ks"]))
        b = (p.M + p.N) * T * esz
        if p.dtype == "fp8":
            b += (T // 128) * (p.M + p.N) * sf
        out = p.G * p.M * p.N * 4
        return b + out * (2 if opt.get("accumulate", True) else 1)
    if p.variant == "masked":
        c = np.clip(p.meta["counts"], 0, p.cap)
        rows, experts = int(c.sum()), int((c > 0).sum())
    else:
        idx = p.meta["m_indices"]
        rows = int((idx >= 0).sum())
        experts = len(set(idx[idx >= 0].tolist()))
    b = rows * p.K * esz + int(experts * p.N * p.K * wsz) + rows * p.N * 2
    if p.dtype != "bf16":
        kb = p.K // 128
        b += rows * kb * sf
        wscales = {"block128": ((p.N + 127) // 128) * kb, "channel": p.N * kb,
                   "block32": p.N * kb * 4}[p.sfb_gran]
        b += experts * wscales * sf
    return b


def main():
    args = parse()
    if args.summarize_counters or args.summarize_mfma_busy:
        summarize_counters(args)
        return
    if args.summarize_trace or args.summarize_traffic:
        summarize(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the grouped GEMM shards by expert across GPUs with no exchange inside the "
              "kernel; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import moe_grouped_gemm_nt_amd as mgg
    from moe_grouped_gemm_nt_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload == "copy_calibration":
        copy_calibration(dev, args)
        return
    if args.workload in QUANT_WORKLOADS:
        quant_bench(dev, args)
        return
    if args.workload == "contig_fp8_chain":
        chain_bench(dev, args)
        return
    mgg.load_library()
    redraw = args.workload in REDRAW_WORKLOADS
    base = REDRAW_WORKLOADS[args.workload] if redraw else args.workload
    p, opt = synth.make_workload(base, dev)
    routes = None
    if redraw:
        # one routing draw per captured call (at most REDRAW_MAX distinct draws, cycled),
        # uploaded before capture; the counters of each call follow its own draw
        w = synth.WORKLOADS[base]
        nr = max(1, min(args.steps, REDRAW_MAX))
        segs = [synth.contiguous_draw(p.G, w["lam"], w["seed"] + 1000 + r, w["rows_per_expert_max"])
                for r in range(nr)]
        idx = [synth.contiguous_indices(sg, synth.GROUP, p.M)[0] for sg in segs]
        routes = [torch.from_numpy(x).to(dev) for x in idx]
        per_call_flops = [2.0 * int((x >= 0).sum()) * p.N * p.K for x in idx]
        per_call_bytes = []
        for x in idx:
            p.meta["m_indices"] = x
            per_call_bytes.append(algorithmic_bytes(p, opt))
        p.meta["m_indices"] = idx[0]
        flops = float(np.mean([per_call_flops[i % nr] for i in range(args.steps)]))
        abytes = int(np.mean([per_call_bytes[i % nr] for i in range(args.steps)]))
    else:
        flops = p.valid_flops()
        abytes = algorithmic_bytes(p, opt)

    # Output buffers, rotated so their footprint exceeds the Infinity Cache.
    if p.variant == "kgrouped":
        out_shape, out_dtype = (p.G, p.M, p.N), torch.float32
    elif p.variant == "masked":
        out_shape, out_dtype = (p.G, p.cap, p.N), torch.bfloat16
    else:
        out_shape, out_dtype = (p.M, p.N), torch.bfloat16
    out_bytes = int(np.prod(out_shape)) * (4 if out_dtype == torch.float32 else 2)
    nrot = args.rotate if args.rotate > 0 else max(1, min(8, -(-2 * MALL_BYTES // out_bytes)))
    outs = [torch.zeros(out_shape, dtype=out_dtype, device=dev) for _ in range(nrot)]

    # Input copies (same values, other addresses), rotated so that the operand and scale
    # bytes the steps read over one cycle exceed four times the Infinity Cache: each step
    # reads its inputs from HBM, as one layer of a model does between the other layers'
    # calls, instead of from the cache the previous identical step filled (with a cycle
    # only a little larger than the cache, a policy that keeps the oldest lines would still
    # serve part of every step from it).
    in_read = abytes - algorithmic_output_bytes(p, opt)
    tensors = [t for t in (p.A, p.B, p.SFA, p.SFB) if t is not None]
    in_alloc = sum(t.numel() * t.element_size() for t in tensors)
    nin = rotated_input_copies(in_read, in_alloc, args.rotate_inputs)
    ins = [(p.A, p.B, p.SFA, p.SFB)]
    for _ in range(nin - 1):
        ins.append(tuple(None if t is None else t.clone() for t in (p.A, p.B, p.SFA, p.SFB)))

    def step(i):
        D = outs[i % nrot]
        A, B, SFA, SFB = ins[i % nin]
        if p.variant == "kgrouped":
            mgg.grouped_gemm_kgrouped(A, B, D, p.ks, p.M, p.N, SFA, SFB,
                                      opt.get("accumulate", True))
        elif p.variant == "masked":
            mgg.grouped_gemm_masked(A, B, D, p.counts, SFA, SFB, p.sfb_gran,
                                    opt["expected_m"])
        else:
            route = p.m_indices if routes is None else routes[i % len(routes)]
            mgg.grouped_gemm_contiguous(A, B, D, route, SFA, SFB, p.sfb_gran,
                                        opt["expected_m"])

    stream = torch.cuda.Stream(dev)
    stream.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i)
    torch.cuda.synchronize(dev)
    print(f"[bench] {args.workload}: warmup {args.warmup} done; capturing {args.steps} steps",
          file=sys.stderr, flush=True)
    samples, wall = _timed_graph_samples(dev, stream, args.steps, step, args.samples)
    ms_total = float(np.median(samples))
    ms_step = ms_total / args.steps
    tflops = flops / (ms_step * 1e-3) / 1e12
    print(f"[bench] {args.samples} replays of {args.steps} steps: median {ms_total:.3f} ms on the "
          f"stream (min {min(samples):.3f}, max {max(samples):.3f}); {wall * 1e3:.3f} ms wall "
          "for all replays", file=sys.stderr, flush=True)

    ai = flops / abytes
    ridge = MFMA_PEAK_TFLOPS[p.dtype] * 1e12 / (HBM_PEAK_GBS * 1e9)
    gbs = abytes / (ms_step * 1e-3) / 1e9
    if ai < ridge:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 1),
                "peak": MFMA_PEAK_TFLOPS[p.dtype], "unit": "TFLOP/s",
                "frac": round(tflops / MFMA_PEAK_TFLOPS[p.dtype], 4)}
    roof["traffic"] = measured_traffic(args.workload)
    roof["algorithmic_bytes_per_launch"] = abytes
    roof["avg_launch_us"] = round(ms_step * 1e3, 3)
    if roof["bound"] == "hbm":
        roof["mfma_frac"] = round(tflops / MFMA_PEAK_TFLOPS[p.dtype], 4)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(p, opt, p.valid_flops(), args.cpu_seconds)

    cfg = {"workload": args.workload, "variant": p.variant, "dtype": p.dtype, "G": p.G,
           "N": p.N, "K": p.K, "valid_gflop": round(flops / 1e9, 4),
           "rotating_output_buffers": nrot, "rotating_input_copies": nin,
           "timing": f"median of {args.samples} replays of one hipGraph of `steps` calls"}
    if p.variant == "kgrouped":
        cfg.update(M=p.M, ks=[int(k) for k in p.meta["ks"]],
                   accumulate=bool(opt.get("accumulate", True)), scales="f32 per channel 1x128")
    elif p.variant == "masked":
        cfg.update(cap=p.cap, expected_m=opt["expected_m"],
                   valid_rows=int(np.clip(p.meta["counts"], 0, p.cap).sum()),
                   scales=f"{p.sf_fmt} 1x128 act / {p.sfb_gran} weight" if p.dtype != "bf16" else None)
    else:
        cfg.update(M=p.M, expected_m=opt["expected_m"], valid_rows=int(p.meta["valid_rows"]),
                   scales=f"{p.sf_fmt} 1x128 act / {p.sfb_gran} weight")
        if redraw:
            cfg.update(routing_draws=len(routes),
                       valid_rows=int(round(flops / (2.0 * p.N * p.K))),
                       routing="Poisson(113) rows per expert redrawn for every captured call")
    line = {
        "metric": "grouped FP8/BF16 GEMM TFLOPS (valid rows) + % of gfx950 MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "mfma_peak_frac": round(tflops / MFMA_PEAK_TFLOPS[p.dtype], 4),
        "dtype": p.dtype,
        "data": "synthetic",
        "config": cfg,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


# the 288-expert contiguous GEMMs with a new routing draw per captured call
REDRAW_WORKLOADS = {"contig_fp8_w13_redraw": "contig_fp8_w13",
                    "contig_fp8_w2_redraw": "contig_fp8_w2"}
REDRAW_MAX = 1000  # distinct draws uploaded (295 KB each at 73728 rows)


QUANT_WORKLOADS = {
    # bf16 activations -> FP8 E4M3 codes + 1x128 scales: the expected tokens of the
    # 32-expert N=6144 configuration (32 x 192) at its hidden size 7168
    "quant_fp8_1x128_6144x7168": (6144, 7168, "f32", False),
    "quant_fp8_1x128_ue8m0_6144x7168": (6144, 7168, "ue8m0", False),
    # SwiGLU + re-quantization of the contiguous configuration's w13 output: 288 experts x
    # 256-row budget = 73728 rows, 2I = 512 columns in, I = 256 out, UE8M0 scales
    "swiglu_quant_fp8_ue8m0_73728x256": (73728, 256, "ue8m0", True),
    # the same step for 4096 tokens at I = 2048
    "swiglu_quant_fp8_4096x2048": (4096, 2048, "f32", True),
}


def _timed_graph(dev, stream, steps, fn, samples=7):
    """`steps` calls of fn(i) captured in one hipGraph; the median of `samples` replays,
    in ms per call."""
    import numpy as np
    out, _ = _timed_graph_samples(dev, stream, steps, fn, samples)
    return float(np.median(out)) / steps


def _timed_graph_samples(dev, stream, steps, fn, samples):
    """`steps` calls of fn(i) captured in one hipGraph, replayed `samples` times, each
    replay between events recorded on the launch stream with device synchronization
    before and after; returns (ms per replay for each sample, wall seconds of all)."""
    import torch
    torch.cuda.synchronize(dev)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for i in range(steps):
            fn(i)
    torch.cuda.synchronize(dev)
    out = []
    wall0 = time.perf_counter()
    for _ in range(max(1, samples)):
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize(dev)
        with torch.cuda.stream(stream):
            t0.record(stream)
            graph.replay()
            t1.record(stream)
        torch.cuda.synchronize(dev)
        out.append(t0.elapsed_time(t1))
    return out, time.perf_counter() - wall0


def quant_bench(dev, args):
    """FP8 1x128 activation quantization (plain, or SwiGLU + quantization): `steps` calls
    in one hipGraph, inputs rotated over enough buffers to exceed the Infinity Cache; HBM
    roofline on the algorithmic bytes (bf16 in, codes out, one scale per 128 codes)."""
    import torch
    import moe_grouped_gemm_nt_amd as mgg
    mgg.load_library()
    M, K, fmt, swiglu = QUANT_WORKLOADS[args.workload]
    sf_b = 4 if fmt == "f32" else 1
    in_cols = 2 * K if swiglu else K
    abytes = M * in_cols * 2 + M * K + (K // 128) * M * sf_b
    nrot = max(1, min(8, -(-2 * MALL_BYTES // abytes)))
    g = torch.Generator(device=dev).manual_seed(0)
    Xs = [torch.randn((M, in_cols), device=dev, generator=g).to(torch.bfloat16)
          for _ in range(nrot)]
    Qs = [torch.empty((M, K), dtype=torch.uint8, device=dev) for _ in range(nrot)]
    SFs = [torch.empty((K // 128, M), device=dev,
                       dtype=torch.float32 if fmt == "f32" else torch.uint8) for _ in range(nrot)]
    fn = mgg.swiglu_quant_fp8_1x128 if swiglu else mgg.quantize_fp8_1x128

    def step(i):
        fn(Xs[i % nrot], Qs[i % nrot], SFs[i % nrot], fmt)

    stream = torch.cuda.Stream(dev)
    stream.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i)
    ms_step = _timed_graph(dev, stream, args.steps, step, args.samples)
    gbs = abytes / (ms_step * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        import numpy as np
        import oracle
        rows = 256
        x = Xs[0][:rows].cpu().view(torch.int16).numpy().view(np.uint16)
        ofn = oracle.swiglu_quant_rows_1x128 if swiglu else oracle.quantize_rows_1x128
        passes, t = 0, 0.0
        w0 = time.perf_counter()
        while t < args.cpu_seconds and passes < 10000:
            ofn(x, fmt)
            passes += 1
            t = time.perf_counter() - w0
        cpu = {"value": round(rows * abytes / M * passes / t / 1e9, 4), "unit": "GB/s",
               "cores": 1, "kind": "oracle",
               "sample": f"{rows} rows x {in_cols} per pass; {passes} passes in {t:.1f} s",
               "cpu": host_cpu_model()}
    what = "SwiGLU + FP8 1x128 re-quantization" if swiglu else "FP8 1x128 activation quantization"
    line = {
        "metric": f"{what} throughput (algorithmic bytes)",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16->e4m3", "data": "synthetic",
        "config": {"workload": args.workload, "M": M, ("I" if swiglu else "K"): K,
                   "scales": fmt, "rotating_buffers": nrot,
                   "timing": f"median of {args.samples} replays of one hipGraph of `steps` calls"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(args.workload),
                     "algorithmic_bytes_per_launch": abytes,
                     "avg_launch_us": round(ms_step * 1e3, 3)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def chain_bench(dev, args):
    """The expert chain of the contiguous configuration on one routing draw: FP8 tokens
    [73728, 4096] -> w13 contiguous GEMM (288 experts, N = 512) -> SwiGLU + 1x128 UE8M0
    re-quantization -> w2 contiguous GEMM (N = 4096, K = 256). The timed value is the
    chain with the SwiGLU step fused into the w13 epilogue; the three separate launches
    and their sum are timed too (each line in its own hipGraph of `steps` calls)."""
    import numpy as np
    import torch
    import moe_grouped_gemm_nt_amd as mgg
    from moe_grouped_gemm_nt_amd import synth
    mgg.load_library()
    p, opt = synth.make_workload("contig_fp8_w13", dev)
    em = opt["expected_m"]
    I, Hd = p.N // 2, p.K
    w2 = synth.make_contiguous("fp8", p.G, Hd, I, p.meta["seg_counts"], 3, dev, sf_fmt=p.sf_fmt,
                               M_max=p.M)
    B2, SFB2 = w2.B, w2.SFB
    del w2
    H = torch.empty((p.M, 2 * I), dtype=torch.bfloat16, device=dev)
    Q = torch.empty((p.M, I), dtype=torch.uint8, device=dev)
    SF = torch.empty((I // 128, p.M), dtype=torch.uint8, device=dev)
    D = torch.empty((p.M, Hd), dtype=torch.bfloat16, device=dev)

    def k13(i):
        mgg.grouped_gemm_contiguous(p.A, p.B, H, p.m_indices, p.SFA, p.SFB, p.sfb_gran, em)

    def kact(i):
        mgg.swiglu_quant_fp8_1x128(H, Q, SF, sf_fmt=p.sf_fmt)

    def k2(i):
        mgg.grouped_gemm_contiguous(Q, B2, D, p.m_indices, SF, SFB2, p.sfb_gran, em)

    def chain(i):
        k13(i)
        kact(i)
        k2(i)

    def k13f(i):  # w13 with the SwiGLU + quantization in its epilogue
        mgg.grouped_gemm_contiguous_swiglu_quant(p.A, p.B, p.m_indices, p.SFA, p.SFB, Q, SF,
                                                 sfq_fmt=p.sf_fmt)

    def fused(i):
        k13f(i)
        k2(i)

    stream = torch.cuda.Stream(dev)
    stream.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            chain(i)
    ms = {name: _timed_graph(dev, stream, args.steps, fn, args.samples)
          for name, fn in (("fused_chain", fused), ("chain", chain), ("w13", k13),
                           ("swiglu_quant", kact), ("w2", k2), ("w13_swiglu_fused", k13f))}
    valid = int(p.meta["valid_rows"])
    flops = {"w13": 2.0 * valid * p.N * p.K, "w2": 2.0 * valid * Hd * I}
    flops["w13_swiglu_fused"] = flops["w13"]
    total = flops["w13"] + flops["w2"]
    tflops = total / (ms["fused_chain"] * 1e-3) / 1e12
    # dominant launch of the timed (fused) chain; MFMA roofline on its valid FLOPs
    dom = max(("w13_swiglu_fused", "w2"), key=lambda k: ms[k])
    dt = flops[dom] / (ms[dom] * 1e-3) / 1e12
    peak = MFMA_PEAK_TFLOPS["fp8"]
    line = {
        "metric": "MoE expert chain (w13 GEMM + SwiGLU + FP8 quant fused -> w2 GEMM) TFLOPS "
                  "(valid rows, both GEMMs)",
        "value": round(tflops, 2), "unit": "TFLOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms["fused_chain"], 6),
        "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8", "data": "synthetic",
        "config": {"workload": "contig_fp8_chain", "G": p.G, "M": p.M, "hidden": Hd,
                   "intermediate": I, "valid_rows": valid, "expected_m": em,
                   "scales": p.sf_fmt, "per_launch_us": {k: round(v * 1e3, 3)
                                                         for k, v in ms.items()},
                   "timing": f"median of {args.samples} replays of one hipGraph of `steps` "
                             "calls per line"},
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": round(dt, 1), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(dt / peak, 4), "traffic": None,
                     "avg_launch_us": round(ms[dom] * 1e3, 3)},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def copy_calibration(dev, args):
    """A plain device-to-device copy of 256 MiB, for scaling the HBM byte counters: the
    copy reads and writes exactly 256 MiB per launch."""
    import torch
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(max(args.warmup, 1)):
        dst.copy_(src)
    torch.cuda.synchronize(dev)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize(dev)
    ms = t0.elapsed_time(t1) / args.steps
    print(json.dumps({"workload": "copy_calibration", "bytes_read": n, "bytes_written": n,
                      "ms_per_copy": round(ms, 5), "GBps_read_plus_write": round(2 * n / ms / 1e6, 1)}),
          flush=True)


COPY_KERNEL_NAME = "__amd_rocclr_copyBuffer"
COPY_BYTES = 256 << 20


def _csv_rows(directory, suffix):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True)):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _counter_median(directory, kernel_sub):
    import statistics
    vals = [float(r["Counter_Value"]) for r in _csv_rows(directory, "counter_collection.csv")
            if kernel_sub in r["Kernel_Name"]]
    if not vals:
        raise SystemExit(f"no {kernel_sub} dispatches in {directory}")
    return statistics.median(vals), len(vals)


# Counter passes behind profiles/<workload>_counters.md (each within one run's limits of
# the hardware's counter blocks), and the one-run counter set of the MFMA-busy table.
COUNTER_PASSES = [
    "SQ_WAVES SQ_BUSY_CYCLES SQ_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES "
    "SQ_INSTS_MFMA SQ_ACTIVE_INST_VALU SQ_INSTS_VALU_FMA_F32 GRBM_GUI_ACTIVE GRBM_COUNT",
    "SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_WAIT_INST_LDS SQ_ACTIVE_INST_LDS "
    "SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_LDS_DATA_FIFO_FULL",
    "TCC_HIT_sum TCC_MISS_sum TCC_EA0_RDREQ_sum TCC_EA0_RDREQ_LEVEL_sum",
    "TCP_TCC_READ_REQ_LATENCY_sum TCP_TCC_READ_REQ_sum TCP_PENDING_STALL_CYCLES_sum "
    "TCP_TCR_TCP_STALL_CYCLES_sum TA_BUFFER_READ_LDS_WAVEFRONTS_sum TA_TA_BUSY_sum",
]
MFMA_BUSY_COUNTERS = "SQ_CYCLES SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA SQ_WAVES GRBM_GUI_ACTIVE"
MFMA_BUSY_WORKLOADS = ["masked_fp8_g6_n4096", "masked_bf16_g6_n4096", "masked_fp8_g32_n6144",
                       "masked_bf16_g32_n6144", "contig_fp8_w13", "contig_fp8_w2"]
N_CUS, N_XCDS, N_SIMDS, N_L2_CHANNELS = 256, 8, 1024, 128


def _dispatch_medians(directory):
    """{counter: median over the dispatches of the GEMM kernel} (each dispatch summed over
    the rows rocprofv3 writes for it), and the kernel name."""
    import statistics
    by, name = {}, None
    for r in _csv_rows(directory, "counter_collection.csv"):
        if KERNEL_NAME not in r["Kernel_Name"]:
            continue
        name = r["Kernel_Name"]
        d = by.setdefault(r["Counter_Name"], {})
        d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not by:
        raise SystemExit(f"no {KERNEL_NAME} dispatches in {directory}")
    return {k: statistics.median(v.values()) for k, v in by.items()}, name


def _trace_average_us(workload):
    """Average launch time of the GEMM kernel in profiles/<workload>_kernel_trace.md."""
    path = os.path.join(ROOT, "profiles", f"{workload}_kernel_trace.md")
    m = re.search(r"grouped_gemm_kernel<[^|]*\| (\d+) \| (\d+) \|", open(path).read())
    if not m:
        raise SystemExit(f"no kernel average in {path}")
    return int(m.group(2)) / 1000.0


def summarize_counters(args):
    """The counter summaries under profiles/ (medians over the dispatches; readings derived
    from the chip's 256 CUs, 8 XCDs, 1024 SIMDs and 128 L2 channels)."""
    from moe_grouped_gemm_nt_amd import synth
    out_dir = os.path.join(ROOT, "profiles")
    dig = kernel_source_digest(KERNEL_NAME)
    cd = "`cd /tmp && export TMPDIR=/tmp` first, then back to the root"
    run = ("timeout -s KILL 150 rocprofv3 --kernel-include-regex grouped_gemm_kernel --pmc {c} "
           "-d {d} -o w --output-format csv -- python -u bench.py --workload {w} --steps 20 "
           "--warmup 2 --no-cpu-baseline")
    if args.summarize_counters:
        w, pre = args.workload, args.summarize_counters
        c, kname = {}, None
        for i in range(1, len(COUNTER_PASSES) + 1):
            v, kname = _dispatch_medians(f"{pre}_{i}")
            c.update(v)
        tm = re.search(r"Tile<(\d+), (\d+), (\d+), (\d+), (\d+)", kname)
        bm, bn, wm, wn = (int(tm.group(k)) for k in (1, 2, 3, 4))
        cfg = synth.WORKLOADS[w]
        slices = cfg["K"] * (2 if cfg["dtype"] == "bf16" else 1) // 128
        mfma_per_slice = (bm // 16) * (bn // 16) if cfg["dtype"] != "bf16" else (bm // 32) * (bn // 32) * 4
        nmw = wm * wn
        if cfg["variant"] != "masked":
            raise SystemExit("counter summaries are written for masked workloads")
        counts = synth.poisson_counts(cfg["G"], cfg["lam"], cfg["cap"], cfg["seed"])
        tiles = int(sum((int(n) + bm - 1) // bm for n in counts)) * ((cfg["N"] + bn - 1) // bn)
        mfma_per_wave = mfma_per_slice // nmw  # per MFMA wave per slice
        wave_slices = c["SQ_INSTS_MFMA"] / mfma_per_wave  # wave-slices that issued MFMAs
        dur = _trace_average_us(w)
        cyc = c["GRBM_GUI_ACTIVE"] / N_XCDS
        ghz = cyc / (dur * 1e3)
        rows = []

        def r(name, val, reading):
            rows.append(f"| {name} | {val} | {reading} |")
        wpg = int(round(c["SQ_WAVES"] / N_CUS))
        r("SQ_WAVES", f"{c['SQ_WAVES']:.0f}", f"{N_CUS} workgroups x {wpg} waves ({nmw} MFMA, {wpg - nmw} copy)")
        r("GRBM_GUI_ACTIVE", f"{c['GRBM_GUI_ACTIVE']:.4g}", f"/ {N_XCDS} XCDs = {cyc / 1e3:.0f}k cycles over the {dur:.1f} us launch (trace average): shader clock ~{ghz:.2f} GHz (an estimate: counted launches can run a few percent longer)")
        r("SQ_BUSY_CYCLES / SQ_CYCLES", f"{c['SQ_BUSY_CYCLES']:.4g} / {c['SQ_CYCLES']:.4g}", f"{100 * c['SQ_BUSY_CYCLES'] / c['SQ_CYCLES']:.1f} % of the launch has work on the shader engines")
        full = tiles * slices * mfma_per_slice
        r("SQ_INSTS_MFMA", f"{c['SQ_INSTS_MFMA']:.4g}", f"{100 * c['SQ_INSTS_MFMA'] / full:.1f} % of {tiles} tiles x {slices} slices x {mfma_per_slice} MFMAs ({full}): waves whose rows are all padding issue none; the whole chip is counted")
        mb = c["SQ_VALU_MFMA_BUSY_CYCLES"] / N_SIMDS
        r("SQ_VALU_MFMA_BUSY_CYCLES", f"{c['SQ_VALU_MFMA_BUSY_CYCLES']:.4g}", f"= SQ_INSTS_MFMA x 32; / {N_SIMDS} SIMDs = {mb / 1e3:.0f}k cycles: the MFMA pipe is busy {100 * mb / cyc:.0f} % of the launch")
        ce = c["SQ_VALU_MFMA_COEXEC_CYCLES"] / N_SIMDS
        r("SQ_VALU_MFMA_COEXEC_CYCLES", f"{c['SQ_VALU_MFMA_COEXEC_CYCLES']:.4g}", f"/ {N_SIMDS} = {ce / 1e3:.0f}k cycles: VALU work runs beside the MFMA pipe for {100 * ce / mb:.0f} % of its busy cycles")
        r("SQ_INSTS_VALU_FMA_F32", f"{c['SQ_INSTS_VALU_FMA_F32']:.4g}", f"the float32 promotion, one FMA per output element per slice: 4 per 16x16 MFMA ({4 * c['SQ_INSTS_MFMA']:.4g})")
        r("SQ_ACTIVE_INST_VALU", f"{c['SQ_ACTIVE_INST_VALU']:.4g}", "")
        per = c["SQ_INSTS_LDS"] / wave_slices
        r("SQ_INSTS_LDS", f"{c['SQ_INSTS_LDS']:.4g}", f"fragment and scale reads: {per:.1f} per MFMA wave per slice that issues MFMAs, the epilogue included ({bm // wm} x {bn // wn} outputs per wave)")
        r("SQ_LDS_BANK_CONFLICT / SQ_LDS_DATA_FIFO_FULL", f"{c['SQ_LDS_BANK_CONFLICT']:.0f} / {c['SQ_LDS_DATA_FIFO_FULL']:.0f}", "LDS bank conflicts and LDS data-path backups")
        r("SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES", f"{c['SQ_WAIT_INST_LDS']:.4g} / {c['SQ_WAVE_CYCLES']:.4g}", f"{100 * c['SQ_WAIT_INST_LDS'] / c['SQ_WAVE_CYCLES']:.1f} % of wave-cycles wait on LDS data")
        r("SQ_WAIT_ANY / SQ_WAVE_CYCLES", f"{c['SQ_WAIT_ANY']:.4g} / {c['SQ_WAVE_CYCLES']:.4g}", f"{100 * c['SQ_WAIT_ANY'] / c['SQ_WAVE_CYCLES']:.0f} % of wave-cycles wait on something (barriers, memory counters)")
        hr = c["TCC_HIT_sum"] / (c["TCC_HIT_sum"] + c["TCC_MISS_sum"])
        r("TCC_HIT_sum / TCC_MISS_sum", f"{c['TCC_HIT_sum']:.4g} / {c['TCC_MISS_sum']:.4g}", f"L2 hit rate {100 * hr:.1f} %")
        ea = c["TCC_EA0_RDREQ_sum"]
        r("TCC_EA0_RDREQ_sum", f"{ea:.4g}", f"x 128 B = {ea * 128 / 1e6:.0f} MB read past L2 (Infinity Cache or HBM)")
        lvl = c["TCC_EA0_RDREQ_LEVEL_sum"]
        r("TCC_EA0_RDREQ_LEVEL_sum", f"{lvl:.4g}", f"/ requests: {lvl / ea:.0f} cycles per read past L2; / cycles: {lvl / cyc / 1e3:.1f}k reads in flight on average, {lvl / cyc / N_L2_CHANNELS:.0f} per L2 channel")
        tr = c["TCP_TCC_READ_REQ_sum"]
        r("TCP_TCC_READ_REQ_sum", f"{tr:.4g}", f"x 128 B = {tr * 128 / 1e9:.2f} GB from L2 into the CUs (the operand slices copied into LDS)")
        lat = c["TCP_TCC_READ_REQ_LATENCY_sum"]
        r("TCP_TCC_READ_REQ_LATENCY_sum", f"{lat:.4g}", f"{lat / tr:.0f} cycles per L1->L2 read on average; {lat / cyc / N_CUS:.0f} reads in flight per CU on average")
        ps = c["TCP_PENDING_STALL_CYCLES_sum"] / N_CUS / cyc
        r("TCP_PENDING_STALL_CYCLES_sum", f"{c['TCP_PENDING_STALL_CYCLES_sum']:.4g}", f"/ {N_CUS} CUs: the L1 cannot take a new request for lack of a pending-request slot {100 * ps:.0f} % of the cycles")
        r("TCP_TCR_TCP_STALL_CYCLES_sum", f"{c['TCP_TCR_TCP_STALL_CYCLES_sum']:.4g}", f"/ {N_CUS}: the return path from L2 stalls {100 * c['TCP_TCR_TCP_STALL_CYCLES_sum'] / N_CUS / cyc:.1f} % of the cycles")
        r("TA_TA_BUSY_sum", f"{c['TA_TA_BUSY_sum']:.4g}", f"/ {N_CUS}: texture address unit busy {100 * c['TA_TA_BUSY_sum'] / N_CUS / cyc:.0f} %")
        r("TA_BUFFER_READ_LDS_WAVEFRONTS_sum", f"{c['TA_BUFFER_READ_LDS_WAVEFRONTS_sum']:.4g}", f"direct global->LDS copy instructions: {c['TA_BUFFER_READ_LDS_WAVEFRONTS_sum'] / (tiles * slices):.0f} per tile slice")
        rows_txt = (f"per-expert rows {[int(n) for n in counts]}" if cfg["G"] <= 8
                    else f"{int(counts.sum())} valid rows in all")
        desc = (f"{cfg['G']} experts, capacity {cfg['cap']}, N = {cfg['N']}, K = {cfg['K']}, "
                f"{rows_txt}, {cfg['dtype']} "
                f"({cfg.get('sf_fmt', 'f32')} scales, {cfg.get('sfb_gran', 'block128')} weight scales): "
                f"{tiles} tiles of {bm} x {bn} computed by {nmw} MFMA waves of {bm // wm} x {bn // wn}, "
                f"{slices} slices each ({tiles / N_CUS:.2f} rounds of {N_CUS} workgroups)")
        lines = [f"# grouped_gemm_kernel: SQ / L2 / L1 counters, workload {w}", "",
                 f"The workload: {desc}.", "",
                 f"Commands (repository root, one MI355X, {cd}), one pass per run:", ""]
        for i, cs in enumerate(COUNTER_PASSES, 1):
            lines.append("    " + run.format(c=cs, d=f"{pre}_{i}", w=w))
        lines += ["", f"Summarised with `python bench.py --workload {w} --summarize-counters {pre}`: "
                  "medians over the dispatches of `grouped_gemm_kernel` in each run (20 steps x 7 "
                  "samples + 2 warmup); counters summed over the XCDs, shader engines and L2 "
                  "channels of the dispatch:", "",
                  "| Counter | Median | Reading |", "|---|---|---|"] + rows + \
                 ["", f"kernel-source-sha256 of the profiled build: {dig}", ""]
        path = os.path.join(out_dir, f"{w}_counters.md")
        with open(path, "w") as f:
            f.write("\n".join(lines))
        print(f"wrote {path}")
    if args.summarize_mfma_busy:
        pre = args.summarize_mfma_busy
        rows = []
        for w in MFMA_BUSY_WORKLOADS:
            c, _ = _dispatch_medians(f"{pre}{w}")
            d = _trace_average_us(w)
            cyc = c["GRBM_GUI_ACTIVE"] / N_XCDS
            rows.append(f"| {w} | {d:.1f} | {c['SQ_CYCLES']:.4g} | {c['SQ_INSTS_MFMA']:.4g} | "
                        f"{c['SQ_VALU_MFMA_BUSY_CYCLES']:.4g} | {cyc / (d * 1e3):.2f} | "
                        f"{100 * c['SQ_VALU_MFMA_BUSY_CYCLES'] / N_SIMDS / cyc:.1f} % | "
                        f"{100 * c['SQ_BUSY_CYCLES'] / c['SQ_CYCLES']:.0f} % |")
        lines = ["# grouped_gemm_kernel: MFMA issue and shader clock, six GEMM workloads", "",
                 f"Commands (repository root, one MI355X, {cd}), one run per workload `W` in "
                 f"{', '.join(MFMA_BUSY_WORKLOADS)}:", "",
                 "    " + run.format(c=MFMA_BUSY_COUNTERS, d=f"{pre}W", w="W"), "",
                 f"Summarised with `python bench.py --summarize-mfma-busy {pre}`: medians over the "
                 "dispatches of each run. `SQ_VALU_MFMA_BUSY_CYCLES` equals `SQ_INSTS_MFMA` x 32 in "
                 "every run (the nominal issue time of a 16x16x128 FP8 or 32x32x16 BF16 MFMA), so "
                 "\"MFMA busy\" below is the nominal MFMA time over the elapsed cycles of the "
                 "dispatch; the elapsed cycles are `GRBM_GUI_ACTIVE` / 8 XCDs and the clock is "
                 "those cycles over the kernel-trace average duration "
                 "(`profiles/<W>_kernel_trace.md`).", "",
                 "| Workload | Duration (us) | SQ_CYCLES | SQ_INSTS_MFMA | SQ_VALU_MFMA_BUSY_CYCLES | "
                 "Clock (GHz) | MFMA busy at that clock | SQ busy |",
                 "|---|---|---|---|---|---|---|---|"] + rows + ["",
                 "The clock column is an estimate: the counted launches run under the profiler and "
                 "can last a few percent longer than the traced ones, which is why the HBM-bound "
                 "shapes can come out slightly above the 2.4 GHz maximum. The MFMA counts include "
                 "the padding rows that the tiles compute.", "",
                 f"kernel-source-sha256 of the profiled build: {dig}", ""]
        path = os.path.join(out_dir, "grouped_gemm_kernel_mfma_busy_and_clock.md")
        with open(path, "w") as f:
            f.write("\n".join(lines))
        print(f"wrote {path}")


def summarize(args):
    """Turn rocprofv3 csv output into the short summaries kept under profiles/."""
    out_dir = os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    w = args.workload
    kn = kernel_name(w)
    if args.summarize_trace:
        d = args.summarize_trace
        stats = [r for r in _csv_rows(d, "kernel_stats.csv") if kn in r["Name"]]
        trace = [r for r in _csv_rows(d, "kernel_trace.csv") if kn in r["Kernel_Name"]]
        if not stats:
            raise SystemExit(f"no {kn} in {d}")
        lines = [f"# {kn}: kernel trace, workload {w}", "",
                 "Command (repository root, one MI355X):", "",
                 f"    rocprofv3 --kernel-trace --stats -d {d} -o {w} --output-format csv "
                 f"-- python -u bench.py --workload {w} --no-cpu-baseline", "",
                 "Kernel statistics (`*_kernel_stats.csv`):", "",
                 "| Kernel | Calls | Average (ns) | Min (ns) | Max (ns) | StdDev (ns) |",
                 "|---|---|---|---|---|---|"]
        for r in stats:
            lines.append(f"| `{r['Name']}` | {r['Calls']} | {float(r['AverageNs']):.0f} | "
                         f"{r['MinNs']} | {r['MaxNs']} | {float(r['StdDev']):.0f} |")
        if trace:
            t = trace[-1]
            gx = int(t.get("Grid_Size_X") or t.get("Grid_Size") or 0)
            wx = int(t.get("Workgroup_Size_X") or t.get("Workgroup_Size") or 1)
            lines += ["", f"Launch shape (`*_kernel_trace.csv`): {gx // wx} workgroups of {wx} "
                      f"lanes; VGPR {t.get('VGPR_Count')}, AGPR {t.get('Accum_VGPR_Count')}, "
                      f"SGPR {t.get('SGPR_Count')} (LDS is allocated dynamically, so the trace "
                      f"lists {t.get('LDS_Block_Size')} B of static LDS)."]
        lines += ["", f"kernel-source-sha256 of the profiled build: {kernel_source_digest(kn)}", ""]
        path = os.path.join(out_dir, f"{w}_kernel_trace.md")
        with open(path, "w") as f:
            f.write("\n".join(lines))
        print(f"wrote {path}")
    if args.summarize_traffic:
        cf, cw, kf, kw = args.summarize_traffic
        copy_f, _ = _counter_median(cf, COPY_KERNEL_NAME)
        copy_w, _ = _counter_median(cw, COPY_KERNEL_NAME)
        ker_f, nf = _counter_median(kf, kn)
        ker_w, nw = _counter_median(kw, kn)
        fac_f = COPY_BYTES / (copy_f * 1024.0)
        fac_w = COPY_BYTES / (copy_w * 1024.0)
        fetch = int(round(ker_f * 1024.0 * fac_f))
        write = int(round(ker_w * 1024.0 * fac_w))
        # counters are collected only for the kernel of interest (--kernel-include-regex), so
        # the many small kernels that generate the inputs run unprofiled
        cmd = ("timeout -s KILL 150 rocprofv3 --kernel-include-regex {rx} --pmc {c} -d {d} "
               "-o w --output-format csv -- python -u bench.py --workload {w} --steps {s} "
               "--warmup 2{x}")
        lines = [f"# {kn}: HBM traffic, workload {w}", "",
                 "Commands (repository root, one MI355X, `export TMPDIR=/tmp` first), one "
                 "counter per run:", ""]
        for c, d, ww, rx, s, x in [("FETCH_SIZE", cf, "copy_calibration", "copy", 10, ""),
                                   ("WRITE_SIZE", cw, "copy_calibration", "copy", 10, ""),
                                   ("FETCH_SIZE", kf, w, kn, 20, " --no-cpu-baseline"),
                                   ("WRITE_SIZE", kw, w, kn, 20, " --no-cpu-baseline")]:
            lines.append("    " + cmd.format(c=c, d=d, rx=rx, w=ww, s=s, x=x))
        lines += ["", "Calibration: the copy reads and writes exactly "
                  f"{COPY_BYTES} B per launch; its median FETCH_SIZE is {copy_f:.1f} KiB and "
                  f"WRITE_SIZE {copy_w:.1f} KiB, so the counters are scaled by "
                  f"{fac_f:.4f} (fetch) and {fac_w:.4f} (write).", "",
                  f"Kernel medians: FETCH_SIZE {ker_f:.1f} KiB over {nf} dispatches, "
                  f"WRITE_SIZE {ker_w:.1f} KiB over {nw} dispatches.", "",
                  "Values read by bench.py (bytes per launch, after scaling):", "",
                  f"- kernel-source-sha256: {kernel_source_digest(kn)}",
                  f"- fetch_bytes_per_launch: {fetch}",
                  f"- write_bytes_per_launch: {write}", ""]
        path = os.path.join(out_dir, f"{w}_hbm_traffic.md")
        with open(path, "w") as f:
            f.write("\n".join(lines))
        print(f"wrote {path}")


def host_cpu_model() -> str:
    """The host CPU's model name (first entry of /proc/cpuinfo), for the baseline record."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(p, opt, flops, target_s):
    """The oracle, as it stands, on the host cores: a bounded sample of the same workload
    (whole experts, or a subset of experts for the large masked shapes)."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1

    def codes(t):
        t = t.detach().cpu().contiguous()
        import torch
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16)
        return t.numpy()

    if p.variant == "kgrouped":
        A, B = codes(p.A), codes(p.B)
        SFA = None if p.SFA is None else codes(p.SFA)
        SFB = None if p.SFB is None else codes(p.SFB)
        ks = list(p.meta["ks"])
        run = lambda: oracle.grouped_gemm_kgrouped(p.dtype, A, B, ks, p.M, p.N, p.K_total, SFA,
                                                   SFB, "f32")
        unit_flops = flops
        sample = "the whole workload (all experts) per pass"
    elif p.variant == "masked":
        c = np.clip(p.meta["counts"], 0, p.cap)
        gs = [g for g in range(p.G) if c[g] > 0][:2]
        A = codes(p.A[gs[0]:gs[-1] + 1])
        B = codes(p.B[gs[0]:gs[-1] + 1])
        SFA = None if p.SFA is None else codes(p.SFA[gs[0]:gs[-1] + 1])
        SFB = None if p.SFB is None else codes(p.SFB[gs[0]:gs[-1] + 1])
        cc = c[gs[0]:gs[-1] + 1]
        run = lambda: oracle.grouped_gemm_masked(p.dtype, A, B, cc, SFA, SFB, p.sfb_gran, p.sf_fmt)
        unit_flops = float(2 * int(cc.sum()) * p.N * p.K)
        sample = f"experts {gs[0]}..{gs[-1]} of {p.G} per pass"
    else:
        idx = p.meta["m_indices"]
        rows = np.nonzero(idx >= 0)[0][:2048]
        A = codes(p.A)[rows]
        SFA = None if p.SFA is None else codes(p.SFA)[:, rows]
        B = codes(p.B)
        SFB = None if p.SFB is None else codes(p.SFB)
        sub = idx[rows]
        run = lambda: oracle.grouped_gemm_contiguous(p.dtype, A, B, sub, SFA, SFB, p.sfb_gran,
                                                     p.sf_fmt)
        unit_flops = float(2 * rows.size * p.N * p.K)
        sample = f"the first {rows.size} valid rows per pass"
    passes, t = 0, 0.0
    t0 = time.perf_counter()
    while True:
        run()
        passes += 1
        t = time.perf_counter() - t0
        if t >= target_s or passes >= 10000:
            break
    return {"value": round(unit_flops * passes / t / 1e12, 6), "unit": "TFLOPS",
            "cores": int(threads), "kind": "oracle",
            "sample": f"{sample}; {passes} passes in {t:.1f} s (FP64 numpy/BLAS)",
            "cpu": host_cpu_model()}


if __name__ == "__main__":
    main()
