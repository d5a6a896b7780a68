"""Seeded synthetic inputs for the grouped NT GEMMs: random operands, per-expert row
counts, FP8 quantization with fine-grained scales, K-grouped packing.

This module produces inputs only. It holds none of the GEMM's arithmetic, and both the
HIP path (through the tests and the benchmark) and the CPU oracle consume the bytes it
makes. It uses torch for random numbers and elementwise work, on CPU for small cases and
on the GPU for full-size workloads (the bytes, not the device, are what both sides see).

Recipes, each from the DeepGEMM pages the workloads come from:

* Per-channel 1x128 cast of the K-grouped repro (issue "Non-deterministic numerical
  problem of k_grouped_fp8_gemm_nt_contiguous", section "repro script"): for each channel
  and each group of 128 consecutive tokens, scale = amax / 448; a zero amax takes a
  caller-chosen value (`sf_val`); scales are floored at 1e-30; codes are
  x * (1 / scale) converted to E4M3 (round to nearest even). Codes are clamped to +-448
  before conversion so an fp32 product that lands a hair above 448 cannot become NaN.
* The same cast's k-major packing: expert e's tokens, transposed to [channels][k_e], laid
  end to end.
* 1x128 per-token-group activation scales and 128x128 block weight scales (the "1d2d"
  FP8 masked path named in PR "Fix cross-expert output overwrites in SM90 masked GEMM",
  and the "blockwise-FP8" MoE of the SM120 graph-replay issue), stored with rows
  contiguous inside each K block.
* Power-of-two (UE8M0) scales, "2^k" in the SM120 issue's environment section. The
  rounding rule is not printed there; the reading taken is the smallest power of two not
  below amax / 448 (so no code saturates), and 2^0 for a zero amax.
* FP4 weights for the FP8 x FP4 products (the "fp8_fp4" kernel family the SM120 issue
  names): E2M1 codes, two per byte with the even K element in the low nibble, one UE8M0
  scale per weight row and 32-K block, the smallest power of two not below amax / 6 (6
  being the largest E2M1 magnitude), codes = round-to-nearest-even of x / scale on the
  E2M1 grid; scales stored [K/128][N][4].
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

FP8_MAX = 448.0
FP4_MAX = 6.0
_E2M1_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)
GROUP = 128  # elements per scale along K (and rows per weight block)
SENTINEL_BF16 = 0xDEAD  # bit pattern pre-filled into outputs to detect stray writes


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def randn(shape, seed: int, device="cpu", std: float = 1.0, gen=None) -> torch.Tensor:
    """N(0, std^2) values rounded once to bf16."""
    g = gen if gen is not None else _gen(seed, device)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return (x * std).to(torch.bfloat16)


def poisson_counts(G: int, lam: float, cap: int, seed: int) -> np.ndarray:
    """Per-expert row counts ~ Poisson(lam), clipped to [0, cap], int32."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.clip(rng.poisson(lam, size=G), 0, cap).astype(np.int32)


# --------------------------------------------------------------------------- scales


def _scale_from_amax(amax: torch.Tensor, sf_fmt: str, zero_sf: float = 1.0):
    """Group maxima (float32) -> (the scale each group's codes stand for, as float32; the
    scale in its storage format). The ratio amax / 448 is the float32 scale; a group with
    nothing in it (ratio 0) stands for `zero_sf` instead. F32 storage keeps that value,
    never below 1e-30; UE8M0 storage keeps the exponent of the smallest power of two that
    is not below it (frexp writes r = f * 2^e with f in [0.5, 1), so that power is 2^e, or
    2^(e-1) when r is itself a power of two)."""
    ratio = amax / FP8_MAX
    ratio = ratio.masked_fill(ratio == 0, zero_sf)
    if sf_fmt == "f32":
        scale = torch.clamp(ratio, min=1e-30)
        return scale, scale.contiguous()
    if sf_fmt == "ue8m0":
        frac, e = torch.frexp(ratio)
        e = e - (frac == 0.5).to(e.dtype)
        code = torch.clamp(e + 127, 0, 254)
        return torch.ldexp(torch.ones_like(ratio), code - 127), code.to(torch.uint8).contiguous()
    raise ValueError(f"unknown scale format {sf_fmt!r}")


def _to_e4m3(x: torch.Tensor) -> torch.Tensor:
    return x.clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn).view(torch.uint8)


def quant_rows_1x128(x: torch.Tensor, sf_fmt: str = "f32", zero_sf: float = 1.0):
    """Activation rows x[R, K] -> (codes uint8 [R, K], scales [K/128, R]).

    One scale per row per 128-element K group; the scale tensor is stored with rows
    contiguous inside each K group. K must be a multiple of 128. An all-zero group
    takes `zero_sf`.
    """
    R, K = x.shape
    assert K % GROUP == 0, "FP8 activations need K % 128 == 0"
    xv = x.float().reshape(R, K // GROUP, GROUP)
    amax = xv.abs().amax(dim=2)  # [R, K/128]
    sf, sf_store = _scale_from_amax(amax, sf_fmt, zero_sf)
    codes = _to_e4m3(xv * (1.0 / sf).unsqueeze(2)).view(R, K)
    return codes.contiguous(), sf_store.t().contiguous()


def quant_weight_128x128(w: torch.Tensor, sf_fmt: str = "f32"):
    """Weight w[N, K] -> (codes uint8 [N, K], scales [ceil(N/128), K/128])."""
    N, K = w.shape
    assert K % GROUP == 0, "FP8 weights need K % 128 == 0"
    nb = (N + GROUP - 1) // GROUP
    wp = torch.zeros((nb * GROUP, K), dtype=torch.float32, device=w.device)
    wp[:N] = w.float()
    wv = wp.view(nb, GROUP, K // GROUP, GROUP)
    amax = wv.abs().amax(dim=(1, 3))  # [nb, K/128]
    sf, sf_store = _scale_from_amax(amax, sf_fmt)
    codes = _to_e4m3(wv * (1.0 / sf)[:, None, :, None]).view(nb * GROUP, K)[:N]
    return codes.contiguous(), sf_store


def quant_weight_channel(w: torch.Tensor, sf_fmt: str = "f32"):
    """Weight w[N, K] with one scale per row and 128-K group -> (codes, scales [K/128, N])."""
    codes, sf = quant_rows_1x128(w, sf_fmt)
    return codes, sf


def _to_e2m1(y: torch.Tensor) -> torch.Tensor:
    """float32 values with |y| <= 6 -> E2M1 codes 0..15 (nearest grid point, ties to the
    even code), as uint8."""
    grid = torch.tensor(_E2M1_GRID, dtype=torch.float32, device=y.device)
    a = y.abs().clamp(max=FP4_MAX)
    hi = torch.bucketize(a, grid, right=False).clamp(max=len(_E2M1_GRID) - 1)  # grid[hi] >= a
    lo = (hi - 1).clamp(min=0)
    d_lo, d_hi = a - grid[lo], grid[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = torch.where(pick_hi, hi, lo)
    code = code | (torch.signbit(y).to(code.dtype) << 3)
    return code.to(torch.uint8)


def quant_weight_fp4_block32(w: torch.Tensor):
    """Weight w[N, K] -> (packed E2M1 bytes [N, K/2], UE8M0 scales [K/128, N, 4])."""
    N, K = w.shape
    assert K % GROUP == 0, "FP4 weights need K % 128 == 0"
    wv = w.float().view(N, K // 32, 32)
    ratio = wv.abs().amax(dim=2) / FP4_MAX  # [N, K/32]
    mant, exp = torch.frexp(ratio)
    e = torch.where(mant == 0.5, exp - 1, exp)
    e = torch.where(ratio == 0, torch.zeros_like(e), e)
    code = (e + 127).clamp(0, 254)
    sf = torch.ldexp(torch.ones_like(ratio), code - 127)
    c = _to_e2m1(wv / sf.unsqueeze(2)).view(N, K)
    packed = (c[:, 0::2] | (c[:, 1::2] << 4)).contiguous()
    scales = code.to(torch.uint8).view(N, K // GROUP, 4).permute(1, 0, 2).contiguous()
    return packed, scales


def quant_tokens_per_channel(x: torch.Tensor, sf_val: float = 1.0, sf_fmt: str = "f32"):
    """The K-grouped operands' cast: x[T, C] (tokens x channels) -> (codes [T, C], scales
    [T/128, C]). A channel's group of 128 consecutive tokens is one row group of x^T, so
    this is the 1x128 cast of the transposed operand; an all-zero group takes sf_val."""
    codes_ct, sf = quant_rows_1x128(x.t(), sf_fmt, zero_sf=sf_val)
    return codes_ct.t().contiguous(), sf


def pack_kmajor(x: torch.Tensor, ks) -> torch.Tensor:
    """Tokens-by-channels x[T, C] -> the K-grouped packed layout: x split into the experts'
    token ranges (k_e tokens each, in order), each range stored channel-major [C][k_e],
    the ranges one after another in a flat buffer."""
    parts = torch.split(x, [int(k) for k in ks], dim=0)
    if not parts:
        return x.new_empty(0)
    return torch.cat([part.t().reshape(-1) for part in parts])


# --------------------------------------------------------------------------- problems


@dataclass
class Problem:
    """One grouped-GEMM call's inputs. Tensors live on `device`; codes are uint8 (FP8)
    or bfloat16 (BF16); `meta` holds the host-side description of the draw."""

    variant: str
    dtype: str
    G: int
    N: int
    K: int
    A: torch.Tensor
    B: torch.Tensor
    SFA: torch.Tensor | None = None
    SFB: torch.Tensor | None = None
    sf_fmt: str = "f32"
    sfb_gran: str = "block128"
    cap: int = 0  # masked
    M: int = 0  # contiguous / K-grouped
    counts: torch.Tensor | None = None  # masked, int32 [G]
    m_indices: torch.Tensor | None = None  # contiguous, int32 [M]
    ks: torch.Tensor | None = None  # K-grouped, int32 [G]
    psum: torch.Tensor | None = None  # prefix-sum routing, int32 [G]
    K_total: int = 0
    meta: dict = field(default_factory=dict)

    def valid_flops(self) -> float:
        """2 * (valid rows) * N * K summed over experts (the throughput numerator)."""
        if self.variant == "masked":
            c = np.clip(self.meta["counts"], 0, self.cap)
            return float(2 * int(c.sum()) * self.N * self.K)
        if self.variant in ("contiguous", "psum"):
            return float(2 * int(self.meta["valid_rows"]) * self.N * self.K)
        return float(2 * self.M * self.N * int(np.sum(self.meta["ks"])))


def _weights(dtype, G, N, K, gen, device, sf_fmt, sfb_gran, std=1.0):
    """Per-expert weights B[G, N, K] and their scales, generated expert by expert."""
    if dtype == "fp8_fp4":
        assert sfb_gran == "block32"
        B = torch.empty((G, N, K // 2), dtype=torch.uint8, device=device)
        SFB = torch.empty((G, K // GROUP, N, 4), dtype=torch.uint8, device=device)
        for g in range(G):
            B[g], SFB[g] = quant_weight_fp4_block32(randn((N, K), 0, device, std, gen=gen))
        return B, SFB
    if dtype == "bf16":
        B = torch.empty((G, N, K), dtype=torch.bfloat16, device=device)
        for g in range(G):
            B[g] = randn((N, K), 0, device, std, gen=gen)
        return B, None
    B = torch.empty((G, N, K), dtype=torch.uint8, device=device)
    nb = (N + GROUP - 1) // GROUP
    if sfb_gran == "block128":
        shape = (G, nb, K // GROUP)
    else:
        shape = (G, K // GROUP, N)
    sf_dtype = torch.float32 if sf_fmt == "f32" else torch.uint8
    SFB = torch.empty(shape, dtype=sf_dtype, device=device)
    for g in range(G):
        w = randn((N, K), 0, device, std, gen=gen)
        if sfb_gran == "block128":
            B[g], SFB[g] = quant_weight_128x128(w, sf_fmt)
        else:
            B[g], SFB[g] = quant_weight_channel(w, sf_fmt)
    return B, SFB


def make_masked(dtype: str, G: int, cap: int, N: int, K: int, counts, seed: int,
                device="cpu", sf_fmt="f32", sfb_gran="block128", std_a=1.0,
                std_b=1.0) -> Problem:
    """Masked problem: A[G, cap, K] (all rows drawn, padding included), B[G, N, K]."""
    counts = np.asarray(counts, dtype=np.int32)
    gen = _gen(seed, device)
    if dtype == "bf16":
        A = randn((G, cap, K), 0, device, std_a, gen=gen)
        SFA = None
    else:
        A = torch.empty((G, cap, K), dtype=torch.uint8, device=device)
        sf_dtype = torch.float32 if sf_fmt == "f32" else torch.uint8
        SFA = torch.empty((G, K // GROUP, cap), dtype=sf_dtype, device=device)
        for g in range(G):
            A[g], SFA[g] = quant_rows_1x128(randn((cap, K), 0, device, std_a, gen=gen), sf_fmt)
    B, SFB = _weights(dtype, G, N, K, gen, device, sf_fmt, sfb_gran, std_b)
    return Problem("masked", dtype, G, N, K, A, B, SFA, SFB, sf_fmt, sfb_gran, cap=cap,
                   counts=torch.tensor(counts, dtype=torch.int32, device=device),
                   meta={"counts": counts, "seed": seed})


def contiguous_indices(seg_counts, align: int = GROUP, M_max: int | None = None):
    """Row-to-expert index for concatenated expert segments, each padded with -1 to a
    multiple of `align`; then -1 up to M_max rows. Returns (int32 array, valid rows)."""
    parts = []
    for g, c in enumerate(seg_counts):
        c = int(c)
        padded = (c + align - 1) // align * align
        seg = np.full(padded, -1, dtype=np.int32)
        seg[:c] = g
        parts.append(seg)
    idx = np.concatenate(parts) if parts else np.zeros(0, np.int32)
    if M_max is not None:
        assert idx.size <= M_max, "segments exceed the row budget"
        idx = np.concatenate([idx, np.full(M_max - idx.size, -1, np.int32)])
    return idx, int(np.sum(seg_counts))


def make_contiguous(dtype: str, G: int, N: int, K: int, seg_counts, seed: int,
                    device="cpu", sf_fmt="f32", sfb_gran="block128", M_max=None,
                    align=GROUP, std_a=1.0, std_b=1.0) -> Problem:
    """Contiguous problem: A[M, K] with per-expert segments padded to `align` rows."""
    idx, valid_rows = contiguous_indices(seg_counts, align, M_max)
    M = idx.size
    gen = _gen(seed, device)
    a = randn((M, K), 0, device, std_a, gen=gen)
    if dtype == "bf16":
        A, SFA = a, None
    else:
        A, SFA = quant_rows_1x128(a, sf_fmt)
    B, SFB = _weights(dtype, G, N, K, gen, device, sf_fmt, sfb_gran, std_b)
    return Problem("contiguous", dtype, G, N, K, A, B, SFA, SFB, sf_fmt, sfb_gran, M=M,
                   m_indices=torch.tensor(idx, dtype=torch.int32, device=device),
                   meta={"seg_counts": np.asarray(seg_counts, np.int64),
                         "m_indices": idx, "valid_rows": valid_rows, "seed": seed})


def make_contiguous_psum(dtype: str, G: int, N: int, K: int, seg_counts, seed: int,
                         device="cpu", sf_fmt="f32", sfb_gran="block128", tail=0,
                         std_a=1.0, std_b=1.0) -> Problem:
    """Prefix-sum routed contiguous problem: expert segments back to back with no
    alignment, then `tail` unrouted rows; psum[e] = rows of experts 0..e."""
    seg = np.asarray(seg_counts, np.int64)
    psum = np.cumsum(seg).astype(np.int32)
    M = int(seg.sum()) + int(tail)
    gen = _gen(seed, device)
    a = randn((M, K), 0, device, std_a, gen=gen)
    if dtype == "bf16":
        A, SFA = a, None
    else:
        A, SFA = quant_rows_1x128(a, sf_fmt)
    B, SFB = _weights(dtype, G, N, K, gen, device, sf_fmt, sfb_gran, std_b)
    return Problem("psum", dtype, G, N, K, A, B, SFA, SFB, sf_fmt, sfb_gran, M=M,
                   psum=torch.tensor(psum, dtype=torch.int32, device=device),
                   meta={"seg_counts": seg, "psum": psum, "valid_rows": int(seg.sum()),
                         "seed": seed})


def make_kgrouped(dtype: str, ks, M: int, N: int, seed: int, device="cpu",
                  std_a=1e-7, std_b=0.4, sf_val=1.0, zero_channel_k=128,
                  K_total: int | None = None, sf_fmt: str = "f32") -> Problem:
    """K-grouped problem after the repro recipe: grad_y[T, M] ~ N(0,1)*std_a,
    act[T, N] ~ N(0,1)*std_b, channel 0 of grad_y zeroed on the tokens of every expert
    that has exactly `zero_channel_k` of them; both cast per channel per 128 tokens (float32
    or UE8M0 scales) and packed k-major. A = packed grad_y (rows = M channels), B = packed
    act (rows = N channels). K_total > sum(ks) appends unrouted zero tokens."""
    ks = [int(k) for k in ks]
    T = sum(ks)
    K_total = T if K_total is None else K_total
    gen = _gen(seed, device)
    gy = randn((T, M), 0, device, std_a, gen=gen)
    act = randn((T, N), 0, device, std_b, gen=gen)
    if T:
        counts = torch.tensor(ks, device=device)
        token_in_small_expert = torch.repeat_interleave(counts == zero_channel_k, counts)
        gy[:, 0] = gy[:, 0].masked_fill(token_in_small_expert, 0)
    pad = K_total - T
    if dtype == "bf16":
        A = pack_kmajor(gy, ks)
        B = pack_kmajor(act, ks)
        SFA = SFB = None
    else:
        qa, SFA = quant_tokens_per_channel(gy, sf_val, sf_fmt)
        qb, SFB = quant_tokens_per_channel(act, sf_val, sf_fmt)
        A = pack_kmajor(qa, ks)
        B = pack_kmajor(qb, ks)
        if pad:
            unit = torch.ones(()) if sf_fmt == "f32" else torch.tensor(127, dtype=torch.uint8)
            SFA = torch.cat([SFA, unit.to(device).expand(pad // GROUP, M).to(SFA.dtype)])
            SFB = torch.cat([SFB, unit.to(device).expand(pad // GROUP, N).to(SFB.dtype)])
    if pad:
        A = torch.cat([A, torch.zeros(pad * M, dtype=A.dtype, device=device)])
        B = torch.cat([B, torch.zeros(pad * N, dtype=B.dtype, device=device)])
    return Problem("kgrouped", dtype, len(ks), N, K_total, A, B, SFA, SFB, sf_fmt,
                   "channel", M=M, K_total=K_total,
                   ks=torch.tensor(ks, dtype=torch.int32, device=device),
                   meta={"ks": np.asarray(ks, np.int64), "seed": seed, "sf_val": sf_val,
                         "grad_y": gy, "act": act})


# --------------------------------------------------------------------------- workloads
#
# The grouped-GEMM shapes the DeepGEMM pages run or quote, with synthetic values:
#   masked_bf16_repro      PR "Fix cross-expert output overwrites": its reproduction script
#   kgrouped_fp8_wgrad     issue "Non-deterministic numerical problem of
#                          k_grouped_fp8_gemm_nt_contiguous": its repro script
#   masked_fp8_g32_n1536   PR's latency table, row G=32 cap=4096 N=1536 K=2048 expected M 20
#   contig_fp8_w13/_w2     SM120 issue's environment: G=288, per-rank w13 N=512/K=4096 and
#                          w2 N=4096/K=256, power-of-two scales, expected M per group 113
#   masked_*_g32_n6144     PR's latency table, row G=32 cap=4096 N=6144 K=7168 expected M 192
#   masked_*_g6_n4096      PR's latency table, row G=6 cap=4096 N=K=4096 expected M 1024
# Per-expert valid rows are drawn ~Poisson(expected M), clipped to the capacity (the
# pages give only the expected value; the Poisson shape is an assumption).

WORKLOADS = {
    "masked_bf16_repro": dict(variant="masked", dtype="bf16", G=8, cap=32, N=256, K=256,
                              counts=[0, 1, 16, 31, 32, 1, 32, 32], expected_m=32, seed=29),
    "kgrouped_fp8_wgrad": dict(variant="kgrouped", dtype="fp8", ks=[256, 128, 128, 256],
                               M=2048, N=2048, seed=0, sf_val=1.0, accumulate=True),
    "masked_fp8_g32_n1536": dict(variant="masked", dtype="fp8", G=32, cap=4096, N=1536,
                                 K=2048, lam=20, expected_m=20, seed=1),
    "contig_fp8_w13": dict(variant="contiguous", dtype="fp8", G=288, N=512, K=4096, lam=113,
                           expected_m=113, seed=2, sf_fmt="ue8m0", rows_per_expert_max=256),
    "contig_fp8_w2": dict(variant="contiguous", dtype="fp8", G=288, N=4096, K=256, lam=113,
                          expected_m=113, seed=3, sf_fmt="ue8m0", rows_per_expert_max=256),
    # the w13 shape with float32 scales and per-channel weight scales
    "contig_fp8ch_w13": dict(variant="contiguous", dtype="fp8", G=288, N=512, K=4096,
                             lam=113, expected_m=113, seed=2, sfb_gran="channel",
                             rows_per_expert_max=256),
    "masked_fp8_g32_n6144": dict(variant="masked", dtype="fp8", G=32, cap=4096, N=6144,
                                 K=7168, lam=192, expected_m=192, seed=4),
    "masked_bf16_g32_n6144": dict(variant="masked", dtype="bf16", G=32, cap=4096, N=6144,
                                  K=7168, lam=192, expected_m=192, seed=4),
    "masked_fp8_g6_n4096": dict(variant="masked", dtype="fp8", G=6, cap=4096, N=4096,
                                K=4096, lam=1024, expected_m=1024, seed=5),
    # the same shape with float32 per-channel weight scales (1 x 128 along K per weight row)
    "masked_fp8ch_g6_n4096": dict(variant="masked", dtype="fp8", G=6, cap=4096, N=4096,
                                  K=4096, lam=1024, expected_m=1024, seed=5,
                                  sfb_gran="channel"),
    # FP8 activations x FP4 weights (1x32 UE8M0 weight scales) on the same shapes
    "contig_fp4_w13": dict(variant="contiguous", dtype="fp8_fp4", G=288, N=512, K=4096,
                           lam=113, expected_m=113, seed=2, sf_fmt="ue8m0",
                           sfb_gran="block32", rows_per_expert_max=256),
    "contig_fp4_w2": dict(variant="contiguous", dtype="fp8_fp4", G=288, N=4096, K=256,
                          lam=113, expected_m=113, seed=3, sf_fmt="ue8m0",
                          sfb_gran="block32", rows_per_expert_max=256),
    "masked_fp4_g6_n4096": dict(variant="masked", dtype="fp8_fp4", G=6, cap=4096, N=4096,
                                K=4096, lam=1024, expected_m=1024, seed=5, sf_fmt="ue8m0",
                                sfb_gran="block32"),
    "masked_bf16_g6_n4096": dict(variant="masked", dtype="bf16", G=6, cap=4096, N=4096,
                                 K=4096, lam=1024, expected_m=1024, seed=5),
}


def contiguous_draw(G: int, lam: float, seed: int, rows_max: int):
    """Per-expert rows ~ Poisson(lam), at most rows_max - 127 so every padded segment fits
    in rows_max rows (the fixed row budget M = G * rows_max)."""
    return poisson_counts(G, lam, rows_max - GROUP + 1, seed)


def make_workload(name: str, device="cuda", **override) -> tuple[Problem, dict]:
    """Problem for a named workload plus the call options (expected_m, accumulate)."""
    w = dict(WORKLOADS[name])
    w.update(override)
    v = w["variant"]
    if v == "masked":
        counts = w.get("counts")
        if counts is None:
            counts = poisson_counts(w["G"], w["lam"], w["cap"], w["seed"])
        p = make_masked(w["dtype"], w["G"], w["cap"], w["N"], w["K"], counts, w["seed"], device,
                        sf_fmt=w.get("sf_fmt", "f32"), sfb_gran=w.get("sfb_gran", "block128"))
        return p, {"expected_m": w["expected_m"]}
    if v == "contiguous":
        segs = contiguous_draw(w["G"], w["lam"], w["seed"], w["rows_per_expert_max"])
        p = make_contiguous(w["dtype"], w["G"], w["N"], w["K"], segs, w["seed"], device,
                            sf_fmt=w.get("sf_fmt", "f32"), sfb_gran=w.get("sfb_gran", "block128"),
                            M_max=w["G"] * w["rows_per_expert_max"])
        return p, {"expected_m": w["expected_m"]}
    p = make_kgrouped(w["dtype"], w["ks"], w["M"], w["N"], w["seed"], device,
                      sf_val=w.get("sf_val", 1.0))
    return p, {"accumulate": w.get("accumulate", True)}
