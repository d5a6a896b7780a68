"""GPU parity of the SwiGLU + FP8 re-quantization step, alone and inside the expert
chain (w13 contiguous GEMM -> SwiGLU + quantization -> w2 contiguous GEMM).

Two references. The plain definition (silu(g) = g / (1 + e^-g) with float64 exp, rounded
once to float32, then the 1x128 cast): codes and scales must agree up to the rounding-
boundary flips that the fixed e^y evaluation's 1e-5 relative error can cause
(parity_util.compare_swiglu_to_plain). And, as a regression check, the oracle's mirror
of the kernel's fixed e^y evaluation, which must match bit for bit. The chain is checked
stage by stage (each stage against the oracle run on the GPU's own input to it) and end
to end against the oracle chain, then captured in one graph and replayed with new
routing values."""

import numpy as np
import pytest
import torch

import oracle
from moe_grouped_gemm_nt_amd import synth
from parity_util import (assert_report, assert_swiglu_plain, bf16_bits, check_contiguous,
                         compare_swiglu_to_plain, cut_contiguous_rows, np_codes, say,
                         sentinel_like)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def swiglu_quant(H, fmt, z=1.0):
    import moe_grouped_gemm_nt_amd as mgg
    Q, SF = mgg.swiglu_quant_fp8_1x128(H, sf_fmt=fmt, sf_zero=z)
    torch.cuda.synchronize()
    return Q, SF


def check(H, Q, SF, fmt, z=1.0, rows=None):
    """Against the plain definition (up to rounding-boundary flips), then bit for bit
    against the mirror of the kernel's fixed e^y evaluation."""
    codes = np_codes(H)
    q = Q.cpu().numpy()
    sf = SF.cpu().numpy()
    if rows is not None:
        codes, q, sf = codes[rows], q[rows], sf[:, rows]
    rep = compare_swiglu_to_plain(codes, q, sf, fmt, z)
    say("  plain definition:", rep)
    assert_swiglu_plain(rep)
    q_ref, sf_ref = oracle.swiglu_quant_rows_1x128(codes, fmt, z)
    bad_q = int((q != q_ref).sum())
    if fmt == "f32":
        bad_s = int((sf.view(np.uint32) != sf_ref.astype(np.float32).view(np.uint32)).sum())
    else:
        bad_s = int((sf != sf_ref).sum())
    assert bad_q == 0 and bad_s == 0, f"{bad_q} codes and {bad_s} scales differ"


def draw_h(M, I, seed):
    """bf16 [M, 2I]: gates over the range where silu bends and saturates, up values whose
    row magnitudes span many binades, saturating rows both ways and a zeroed group."""
    g = torch.Generator(device=DEV).manual_seed(seed)
    gate = torch.randn((M, I), device=DEV, generator=g) * 4
    up = torch.randn((M, I), device=DEV, generator=g)
    up *= torch.exp2(torch.randint(-20, 12, (M, 1), device=DEV, generator=g).float())
    gate[min(5, M - 1)] *= 40  # e^-x over- and underflows
    gate[min(9, M - 1), :128] = -200.0  # silu = -0 -> an all-zero group
    up[min(11, M - 1), 128:256 if I >= 256 else 128] = 0.0
    return torch.cat([gate, up], dim=1).to(torch.bfloat16).contiguous()


@pytest.mark.parametrize("fmt,z", [("f32", 1.0), ("f32", 1e-30), ("ue8m0", 1.0),
                                   ("ue8m0", 1e-4)])
def test_swiglu_ragged_rows(fmt, z):
    say("swiglu ragged", fmt, z)
    H = draw_h(1000, 640, 1)
    Q, SF = swiglu_quant(H, fmt, z)
    check(H, Q, SF, fmt, z)


@pytest.mark.parametrize("I", [128, 256, 384])
def test_swiglu_narrow_rows_few_rows(I):
    """One to three 128-column output groups per row and 1 to 17 rows, both formats."""
    for M in (1, 2, 3, 5, 17):
        say("swiglu narrow", M, I)
        H = draw_h(M, I, 200 + M)
        for fmt in ("f32", "ue8m0"):
            Q, SF = swiglu_quant(H, fmt)
            check(H, Q, SF, fmt)


def test_swiglu_every_bf16_gate():
    """Every finite bf16 gate value with |g| < 2^9 (the exponent range where e^-g goes
    from 1 through subnormal to overflow), up = 1 or -3, in groups of 128."""
    codes = np.arange(0, 0x7F80, dtype=np.uint32)
    vals = oracle.decode_bf16(codes.astype(np.uint16))
    codes = codes[np.abs(vals) < 512.0]
    codes = np.concatenate([codes, codes | 0x8000]).astype(np.uint16)
    pad = (-codes.size) % 128
    codes = np.concatenate([codes, np.zeros(pad, np.uint16)])
    gate = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).reshape(-1, 128)
    for upv in (1.0, -3.0):
        say("swiglu every gate, up", upv, gate.shape)
        H = torch.cat([gate, torch.full_like(gate, upv)], dim=1).to(DEV)
        for fmt in ("f32", "ue8m0"):
            Q, SF = swiglu_quant(H, fmt)
            check(H, Q, SF, fmt)


@pytest.mark.parametrize("M,I", [(73728, 256), (4096, 2048)])
def test_swiglu_full_sizes(M, I):
    """The contiguous config's w13 output (288 experts x 256 rows, 2I = 512) and a
    4096-token batch at I = 2048: every output, both formats."""
    say("swiglu full", M, I)
    H = draw_h(M, I, 2)
    for fmt in ("f32", "ue8m0"):
        Q, SF = swiglu_quant(H, fmt)
        check(H, Q, SF, fmt)


def test_swiglu_graph_replay():
    import moe_grouped_gemm_nt_amd as mgg
    say("swiglu graph")
    H = draw_h(300, 384, 3)
    Q = torch.empty((300, 384), dtype=torch.uint8, device=DEV)
    SF = torch.empty((3, 300), dtype=torch.uint8, device=DEV)
    mgg.swiglu_quant_fp8_1x128(H, Q, SF, sf_fmt="ue8m0")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mgg.swiglu_quant_fp8_1x128(H, Q, SF, sf_fmt="ue8m0")
    for seed in (4, 5, 6):
        H.copy_(draw_h(300, 384, seed))
        Q.zero_()
        g.replay()
        torch.cuda.synchronize()
        check(H, Q, SF, "ue8m0")
        Qe, SFe = swiglu_quant(H, "ue8m0")
        assert torch.equal(Q, Qe) and torch.equal(SF, SFe)


# ----------------------------------------------------------------------------- chain


class Chain:
    """w13 [G, 2I, Hd] and w2 [G, Hd, I] FP8 expert weights, FP8 tokens A [M, Hd] routed by
    m_indices, and the buffers of the three steps."""

    def __init__(self, G, Hd, I, M, segs, fmt, seed):
        self.G, self.Hd, self.I, self.M, self.fmt = G, Hd, I, M, fmt
        self.p13 = synth.make_contiguous("fp8", G, 2 * I, Hd, segs, seed, DEV, sf_fmt=fmt,
                                         M_max=M, std_b=0.05)
        w2 = synth.make_contiguous("fp8", G, Hd, I, segs, seed + 1, DEV, sf_fmt=fmt, M_max=M,
                                   std_b=0.05)
        self.B2, self.SFB2 = w2.B, w2.SFB
        self.H = sentinel_like((M, 2 * I), DEV)
        self.Q = torch.zeros((M, I), dtype=torch.uint8, device=DEV)
        sfd = torch.float32 if fmt == "f32" else torch.uint8
        self.SF = torch.zeros((I // 128, M), dtype=sfd, device=DEV)
        self.D = sentinel_like((M, Hd), DEV)

    def run(self, expected_m=64):
        import moe_grouped_gemm_nt_amd as mgg
        p = self.p13
        mgg.grouped_gemm_contiguous(p.A, p.B, self.H, p.m_indices, p.SFA, p.SFB, p.sfb_gran,
                                    expected_m)
        mgg.swiglu_quant_fp8_1x128(self.H, self.Q, self.SF, sf_fmt=self.fmt)
        mgg.grouped_gemm_contiguous(self.Q, self.B2, self.D, p.m_indices, self.SF, self.SFB2,
                                    p.sfb_gran, expected_m)

    def set_routing(self, segs):
        idx, valid = synth.contiguous_indices(segs, 128, self.M)
        self.p13.m_indices.copy_(torch.from_numpy(idx))
        self.p13.meta["m_indices"] = idx
        self.p13.meta["valid_rows"] = valid

    def w2_problem(self):
        p = self.p13
        return synth.Problem("contiguous", "fp8", self.G, self.Hd, self.I, self.Q, self.B2,
                             self.SF, self.SFB2, self.fmt, p.sfb_gran, M=self.M,
                             m_indices=p.m_indices, meta=dict(p.meta))

    def check_stages(self):
        """Each stage against the oracle on the GPU's own input to that stage."""
        valid = np.nonzero(self.p13.meta["m_indices"] >= 0)[0]
        assert_report(check_contiguous(self.p13, self.H), "fp8")
        if valid.size:
            check(self.H, self.Q, self.SF, self.fmt, rows=valid)
        assert_report(check_contiguous(self.w2_problem(), self.D), "fp8")

    def oracle_end_to_end(self):
        """The whole chain in the oracle: float64 w13 rounded to bf16 (the GEMM's output
        type), SwiGLU + quantization, float64 w2."""
        p = self.p13
        idx = p.meta["m_indices"]
        valid = np.nonzero(idx >= 0)[0]
        h, _ = oracle.grouped_gemm_contiguous("fp8", np_codes(p.A), np_codes(p.B), idx,
                                              np_codes(p.SFA), np_codes(p.SFB), p.sfb_gran,
                                              self.fmt)
        hb = oracle.round_to_bf16(h[valid])
        q, sf = oracle.swiglu_quant_rows_1x128(hb, self.fmt)
        d, _ = oracle.grouped_gemm_contiguous("fp8", q, np_codes(self.B2), idx[valid], sf,
                                              np_codes(self.SFB2), p.sfb_gran, self.fmt)
        return valid, d


@pytest.mark.parametrize("fmt", ["ue8m0", "f32"])
def test_chain_stages_and_end_to_end(fmt):
    G, Hd, I, M = 6, 1024, 256, 1536
    segs = np.array([130, 0, 77, 255, 1, 200])
    say("chain", fmt, segs.tolist())
    c = Chain(G, Hd, I, M, segs, fmt, seed=40)
    c.run()
    torch.cuda.synchronize()
    c.check_stages()
    valid, ref = c.oracle_end_to_end()
    gpu = oracle.decode_bf16(bf16_bits(c.D)[valid])
    diff = oracle.calc_diff(gpu, oracle.decode_bf16(oracle.round_to_bf16(ref)))
    say("  end-to-end calc_diff", diff)
    assert diff < 1e-3


def test_chain_graph_replay_changing_routing():
    """The three steps captured in one graph, replayed with new routing values in the same
    index buffer (an all-empty phase included): every replay equals the eager chain bit
    for bit and passes the stage checks."""
    G, Hd, I, M = 8, 512, 256, 2048
    rng = np.random.default_rng(41)
    draws = [np.minimum(rng.poisson(90, G), 128) for _ in range(2)]
    draws += [np.zeros(G, int), np.minimum(rng.poisson(120, G), 128)]
    say("chain graph")
    c = Chain(G, Hd, I, M, draws[0], "ue8m0", seed=41)
    c.run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        c.run()
    fill, fill_h = sentinel_like((M, Hd), DEV), sentinel_like((M, 2 * I), DEV)
    for ph, segs in enumerate(draws):
        say("  phase", ph, segs.tolist())
        c.set_routing(segs)
        c.D.copy_(fill)
        c.H.copy_(fill_h)  # rows no longer routed must hold the sentinel again
        g.replay()
        torch.cuda.synchronize()
        got = bf16_bits(c.D)
        c.D.copy_(fill)
        c.H.copy_(fill_h)
        c.run()
        torch.cuda.synchronize()
        assert (got == bf16_bits(c.D)).all(), f"replay differs from eager in phase {ph}"
        c.check_stages()


# ----------------------------------------------------------------------------- fused


FUSED_TYPES = [("fp8", "ue8m0", "block128"), ("fp8", "f32", "block128"),
               ("fp8", "f32", "channel"), ("fp8_fp4", "ue8m0", "block32")]


def fused_vs_separate(p, sfq, z=1.0):
    """The fused entry point and the two separate steps on the same problem; returns
    (Qf, SFf, Qs, SFs, valid rows, H). Outputs start from fill patterns so that rows the
    fused call must not touch can be checked."""
    import moe_grouped_gemm_nt_amd as mgg
    I = p.N // 2
    H = sentinel_like((p.M, p.N), DEV)
    mgg.grouped_gemm_contiguous(p.A, p.B, H, p.m_indices, p.SFA, p.SFB, p.sfb_gran, 128)
    Qs, SFs = mgg.swiglu_quant_fp8_1x128(H, sf_fmt=sfq, sf_zero=z)
    Qf = torch.full((p.M, I), 0xAB, dtype=torch.uint8, device=DEV)
    sfd = torch.float32 if sfq == "f32" else torch.uint8
    SFf = torch.full((I // 128, p.M), 77, dtype=sfd, device=DEV)
    mgg.grouped_gemm_contiguous_swiglu_quant(p.A, p.B, p.m_indices, p.SFA, p.SFB, Qf, SFf,
                                             sfq_fmt=sfq, sf_zero=z, sfb_gran=p.sfb_gran)
    torch.cuda.synchronize()
    valid = torch.from_numpy(p.meta["m_indices"] >= 0).to(DEV)
    return Qf, SFf, Qs, SFs, valid, H


def assert_fused_plain(H, Qf, SFf, valid, sfq, z=1.0):
    """The fused epilogue's codes against the plain definition applied to the bf16 w13
    output (the fused tile rounds its accumulators to bf16 first, as the separate GEMM
    stores them)."""
    rows = valid.cpu().numpy()
    rep = compare_swiglu_to_plain(np_codes(H)[rows], Qf.cpu().numpy()[rows],
                                  SFf.cpu().numpy()[:, rows], sfq, z)
    say("  fused vs plain definition:", rep)
    assert_swiglu_plain(rep)


def assert_fused_equal(Qf, SFf, Qs, SFs, valid):
    assert torch.equal(Qf[valid], Qs[valid]), "codes differ from the separate steps"
    assert torch.equal(SFf[:, valid].view(torch.uint8), SFs[:, valid].view(torch.uint8)), \
        "scales differ from the separate steps"
    assert (Qf[~valid] == 0xAB).all(), "rows that are not routed were written"
    assert (SFf[:, ~valid] == 77).all(), "scales of rows that are not routed were written"


@pytest.mark.parametrize("dt,sf,gran", FUSED_TYPES)
@pytest.mark.parametrize("sfq", ["ue8m0", "f32"])
def test_fused_swiglu_matches_separate_steps(dt, sf, gran, sfq):
    """Ragged segments, I = 384 (three output groups, so gate and up blocks are gathered
    from different places), K = 512: bit-identical to GEMM -> SwiGLU + quantization."""
    segs = [130, 0, 1, 127, 128, 45]
    say("fused", dt, sf, gran, sfq, segs)
    p = synth.make_contiguous(dt, len(segs), 768, 512, segs, seed=50, device=DEV, sf_fmt=sf,
                              sfb_gran=gran, M_max=1152, std_b=0.05)
    Qf, SFf, Qs, SFs, valid, H = fused_vs_separate(p, sfq, z=1e-4)
    assert_fused_equal(Qf, SFf, Qs, SFs, valid)
    assert_fused_plain(H, Qf, SFf, valid, sfq, z=1e-4)


@pytest.mark.parametrize("M", [70, 326])
def test_fused_swiglu_total_rows_not_a_block_multiple(M):
    """M = 70 and M = 326 (the last block cut after its expert's 70 rows): bit-identical
    to GEMM -> SwiGLU + quantization on the same rows."""
    segs = [70] if M == 70 else [130, 70]
    say("fused rows", M)
    full = synth.make_contiguous("fp8", len(segs), 768, 512, segs, seed=53, device=DEV,
                                 sf_fmt="f32", sfb_gran="block128", std_b=0.05)
    p = cut_contiguous_rows(full, M)
    Qf, SFf, Qs, SFs, valid, H = fused_vs_separate(p, "ue8m0", z=1e-4)
    assert_fused_equal(Qf, SFf, Qs, SFs, valid)
    assert_fused_plain(H, Qf, SFf, valid, "ue8m0", z=1e-4)


def test_fused_swiglu_full_w13_shape():
    """The contiguous configuration's w13 (288 experts, I = 256, K = 4096, UE8M0): every
    routed row bit-identical to the separate steps."""
    say("fused full w13")
    p, _ = synth.make_workload("contig_fp8_w13", DEV)
    Qf, SFf, Qs, SFs, valid, H = fused_vs_separate(p, "ue8m0")
    assert_fused_equal(Qf, SFf, Qs, SFs, valid)
    assert_fused_plain(H, Qf, SFf, valid, "ue8m0")


# Row blocks at which the three-stage fused tile's scheduler table (4 bytes per 128-row
# block, after three 50 176 .. 51 200-byte pipeline stages) still fits in 160 KB of LDS:
# float32 scales with 128 x 128 weight blocks 3136, with per-channel weight scales 2560.
# One block more and the host falls back to the two-stage tile; 4096 blocks (524288 rows)
# is the contiguous layout's maximum.
@pytest.mark.parametrize("gran,blocks", [("block128", 3136), ("block128", 3137),
                                         ("channel", 2560), ("channel", 2561),
                                         ("block128", 4096)])
def test_fused_swiglu_row_block_limits(gran, blocks):
    """Either side of the fused tile's LDS limit and at the layout's maximum rows: every
    routed row bit-identical to the separate steps, untouched rows keep their fill."""
    M = blocks * 128
    rng = np.random.default_rng(blocks)
    segs = rng.integers(0, 129, size=blocks - 1)
    segs[-1] = 128
    say("fused row blocks", gran, blocks)
    p = synth.make_contiguous("fp8", int(segs.size), 256, 256, segs, seed=52, device=DEV,
                              sf_fmt="f32", sfb_gran=gran, M_max=M, std_b=0.05)
    assert p.M == M
    Qf, SFf, Qs, SFs, valid, H = fused_vs_separate(p, "f32")
    assert_fused_equal(Qf, SFf, Qs, SFs, valid)


def test_fused_chain_graph_replay_changing_routing():
    """Fused w13 + w2 captured in one graph and replayed with new routing values: every
    replay equals the eager chain and the separate steps, and the oracle chain within the
    FP8 bar."""
    import moe_grouped_gemm_nt_amd as mgg
    G, Hd, I, M = 8, 512, 256, 2048
    rng = np.random.default_rng(51)
    draws = [np.minimum(rng.poisson(90, G), 128) for _ in range(2)]
    draws += [np.zeros(G, int), np.minimum(rng.poisson(120, G), 128)]
    say("fused chain graph")
    c = Chain(G, Hd, I, M, draws[0], "ue8m0", seed=51)
    p = c.p13

    def run():
        mgg.grouped_gemm_contiguous_swiglu_quant(p.A, p.B, p.m_indices, p.SFA, p.SFB, c.Q, c.SF,
                                                 sfq_fmt="ue8m0")
        mgg.grouped_gemm_contiguous(c.Q, c.B2, c.D, p.m_indices, c.SF, c.SFB2, p.sfb_gran, 64)

    run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    fill = sentinel_like((M, Hd), DEV)
    for ph, segs in enumerate(draws):
        say("  phase", ph, segs.tolist())
        c.set_routing(segs)
        c.D.copy_(fill)
        g.replay()
        torch.cuda.synchronize()
        got = bf16_bits(c.D)
        c.D.copy_(fill)
        run()
        torch.cuda.synchronize()
        assert (got == bf16_bits(c.D)).all(), f"replay differs from eager in phase {ph}"
        valid = np.nonzero(p.meta["m_indices"] >= 0)[0]
        if valid.size:
            vv, ref = c.oracle_end_to_end()
            gpu = oracle.decode_bf16(bf16_bits(c.D)[vv])
            diff = oracle.calc_diff(gpu, oracle.decode_bf16(oracle.round_to_bf16(ref)))
            say("  end-to-end calc_diff", diff)
            assert diff < 1e-3
