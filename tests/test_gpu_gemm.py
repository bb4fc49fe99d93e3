"""GPU parity of the block-scaled GEMM (all epilogues, both formats, both
schedules, both scale layouts) against the oracle's binary64 reference of the
dequantized operands, under |gpu - ref| <= 2^-7 |ref| + 1e-6 L1.  Operands are
quantized by the oracle on the CPU and uploaded, so the oracle never consumes
anything the device produced."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_add_amd as lb
from block_scaled_fp4_add_amd import synth

from . import checkers
from .gpu_util import banner, dev_bf16, dev_f32, dev_u8, host_f64, host_u8

pytestmark = pytest.mark.gpu

EPI_FN = {
    0: lambda *a, bias, res, **k: lb.lowbit_gemm_bf16(*a, **k),
    1: lambda *a, bias, res, **k: lb.lowbit_gemm_bias_bf16(*a, bias, **k),
    2: lambda *a, bias, res, **k: lb.lowbit_gemm_residual_bf16(*a, res, **k),
    3: lambda *a, bias, res, **k: lb.lowbit_gemm_bias_residual_bf16(*a, bias, res, **k),
    4: lambda *a, bias, res, **k: lb.lowbit_gemm_bias_gelu_bf16(*a, bias, **k),
}


def operands(orc, M, N, K, fmt, la, lb_, seed, outliers=False):
    A = synth.activation(M, K, seed, outliers=outliers)
    W = synth.weight(N, K, seed)
    a, sfa = orc.quantize(synth.bits(A), fmt, la)
    b, sfb = orc.quantize(synth.bits(W), fmt, lb_)
    return a, sfa, b, sfb


def split_workspace(M, N, K, fmt, variant):
    """A workspace of the size the split-K schedule asks for, filled with NaN
    bytes (its contents need no initialisation), or None."""
    n = lb.lowbit_gemm_workspace_bytes(M, N, K, fmt, variant)
    return torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda") if n else None


def run_gemm(orc, M, N, K, fmt, la, lb_, epi, variant, seed, alpha=1.0, sample=None, outliers=False,
             workspace=False, l1_coef=1e-6):
    """fmt may be lb.MXFP8_MMA: MXFP8 operands (the oracle's MXFP8) contracted on
    the scaled FP8 MFMA, compared under its own l1_coef."""
    banner(f"gemm M={M} N={N} K={K} fmt={fmt} la={la} lb={lb_} epi={epi} variant={variant} seed={seed}"
           f" workspace={workspace}")
    ofmt = lb.MXFP8 if fmt == lb.MXFP8_MMA else fmt     # the oracle's format
    a, sfa, b, sfb = operands(orc, M, N, K, ofmt, la, lb_, seed, outliers)
    bias = synth.bias(N, seed)
    res = synth.residual(M, N, seed)
    ws = split_workspace(M, N, K, fmt, variant) if (workspace or variant == 2) else None
    out = EPI_FN[epi](dev_u8(a), dev_u8(b), dev_u8(sfa), dev_u8(sfb), bias=dev_bf16(bias), res=dev_bf16(res),
                      fmt=fmt, sfa_layout=la, sfb_layout=lb_, alpha=alpha, variant=variant, workspace=ws)
    torch.cuda.synchronize()
    got = host_f64(out)
    assert np.all(np.isfinite(got))
    kw = dict(alpha=alpha, epi=epi, bias=synth.bits(bias), residual=synth.bits(res))
    if sample is None:
        ref, l1 = orc.gemm(a, b, sfa, sfb, M, N, K, ofmt, la, lb_, **kw)
        ok, worst = checkers.gemm_within_tolerance(got, ref, l1, l1_coef)
    else:
        im, jn = sample
        ref, l1 = orc.gemm_entries(a, b, sfa, sfb, M, N, K, ofmt, la, lb_, im, jn, **kw)
        ok, worst = checkers.gemm_within_tolerance(got[im, jn], ref, l1, l1_coef)
    banner(f"  worst err/tol = {worst:.3g}, violations = {int((~ok).sum())}")
    assert ok.all(), f"{int((~ok).sum())} elements out of tolerance (worst ratio {worst})"


# small shapes, compared in full; they span several tiles and ragged tails,
# and (the last three) give the decode schedule's waves odd superstep counts
# (K / 256 = 9, 17, 18 over 8, 8 and 4 waves); the two with N > 8192 put
# more than 256 workgroups on the decode schedule.  NVFP4 runs 1, 3 and 4
# M-tiles with 8 single-buffered waves (M = 1, 3, 65-128 below), 2 M-tiles
# double-buffered.
SHAPES = [(8, 128, 256), (1, 32, 32), (1, 200, 1056), (1, 17, 4096), (5, 40, 96), (33, 70, 320), (128, 256, 512), (130, 200, 768),
          (41, 4608, 1536), (200, 96, 1056), (3, 96, 2304), (40, 64, 4352), (100, 48, 4608),
          (1, 8224, 544), (2, 9000, 1056), (70, 200, 2560), (96, 136, 1568)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("variant", [0, 1])
def test_gemm_plain(orc, M, N, K, fmt, variant):
    if K % (16 if fmt == 0 else 32):
        pytest.skip("K not a multiple of the block")
    if variant == 0 and M > 128:
        pytest.skip("decode schedule holds at most 128 rows")
    run_gemm(orc, M, N, K, fmt, 0, 1, 0, variant, seed=M + N + K, alpha=0.5)


@pytest.mark.parametrize("epi", [1, 2, 3, 4])
@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("variant", [0, 1])
def test_gemm_epilogues(orc, epi, fmt, variant):
    M = 33 if variant == 0 else 150
    run_gemm(orc, M, 264, 512, fmt, 1, 1, epi, variant, seed=epi * 10 + fmt)


@pytest.mark.parametrize("la,lb_", [(0, 0), (0, 1), (1, 0), (1, 1)])
@pytest.mark.parametrize("fmt", [0, 1])
def test_gemm_layouts(orc, la, lb_, fmt):
    run_gemm(orc, 65, 96, 544, fmt, la, lb_, 0, -1, seed=la * 2 + lb_)
    run_gemm(orc, 20, 96, 544, fmt, la, lb_, 0, -1, seed=la * 2 + lb_ + 7)


# NVFP4 prefill with K % 64 == 0 runs the 128 x 384 schedule that converts the
# activation fragments once per workgroup: full and half final stages
# (K % 128 == 0 and 64), M and N off the tile sizes, every scale layout pair,
# more than one tile in each direction
NV_PREFILL_SHAPES = [(129, 400, 512), (300, 1000, 576), (257, 770, 1088), (128, 384, 128), (5, 48, 64)]


@pytest.mark.parametrize("M,N,K", NV_PREFILL_SHAPES)
@pytest.mark.parametrize("la,lb_", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_gemm_nvfp4_prefill_schedule(orc, M, N, K, la, lb_):
    assert K % 64 == 0
    run_gemm(orc, M, N, K, 0, la, lb_, 0, 1, seed=M + N + K + 3 * la + lb_, alpha=0.5, outliers=True)


@pytest.mark.parametrize("epi", [1, 2, 3, 4])
def test_gemm_nvfp4_prefill_schedule_epilogues(orc, epi):
    run_gemm(orc, 200, 800, 576, 0, 0, 1, epi, 1, seed=epi + 40, outliers=True)


def test_gemm_tiny_mxfp4_workload(orc):
    c = synth.TINY_MXFP4
    run_gemm(orc, c["M"], c["N"], c["H"], orc.MXFP4, 0, 0, 0, -1, seed=c["seed"])


@pytest.mark.parametrize("shape", synth.MXFP4_DECODE["shapes"])
def test_gemm_mxfp4_decode_shapes_full(orc, shape):
    """The decode-shaped MXFP4 workloads at full size, every output checked."""
    M, N, K = shape
    run_gemm(orc, M, N, K, orc.MXFP4, 1, 1, 0, -1, seed=synth.MXFP4_DECODE["seed"])


@pytest.mark.timeout(900)
@pytest.mark.parametrize("shape", synth.MXFP4_PREFILL["shapes"])
def test_gemm_mxfp4_prefill_shapes_full(orc, shape):
    """The prefill workloads (bias + residual epilogue) at full size, in the
    schedule the benchmark times, every output checked against the oracle
    (about 4.8e11 multiply-adds each on the host)."""
    M, N, K = shape
    run_gemm(orc, M, N, K, orc.MXFP4, 1, 1, 3, -1, seed=synth.MXFP4_PREFILL["seed"], outliers=True)


# NVFP4 with K % 32 == 16: packed rows of 8 mod 16 bytes, whose last block
# half-fills a 16-byte chunk.  The decode schedule takes them at any M (128-row
# slices above 128 rows); an explicit prefill request is refused.
HALF_K_SHAPES = [(1, 64, 48), (40, 96, 80), (128, 200, 1552), (130, 72, 80), (300, 160, 1552), (3, 4100, 1552)]


@pytest.mark.parametrize("M,N,K", HALF_K_SHAPES)
@pytest.mark.parametrize("la,lb_", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_gemm_nvfp4_half_chunk_k(orc, M, N, K, la, lb_):
    assert K % 32 == 16
    for variant in (-1, 0):
        run_gemm(orc, M, N, K, 0, la, lb_, 0, variant, seed=M + N + K + la, alpha=0.75)
    assert lb.lowbit_gemm_pick_variant(M, N, K, 0, -1) == 0
    assert lb.lowbit_gemm_pick_variant(M, N, K, 0, 1) == -1


@pytest.mark.parametrize("epi", [1, 2, 3, 4])
def test_gemm_nvfp4_half_chunk_k_epilogues(orc, epi):
    for M in (33, 260):
        run_gemm(orc, M, 136, 1552, 0, 1, 1, epi, -1, seed=epi + M)


@pytest.mark.parametrize("M", [5, 200])
@pytest.mark.parametrize("out_layout", [0, 1])
def test_gemm_nvfp4_half_chunk_k_gelu_fp4(orc, M, out_layout):
    run_gelu_fp4(orc, M, 176, 1552, 0, -1, out_layout, seed=M + 1552)


def test_gemm_nvfp4_half_chunk_k_prefill_refused(orc):
    a, sfa, b, sfb = operands(orc, 256, 64, 48, 0, 0, 0, 3)
    with pytest.raises(lb.LowbitError) as e:
        lb.lowbit_gemm_bf16(dev_u8(a), dev_u8(b), dev_u8(sfa), dev_u8(sfb), fmt=0, variant=1)
    assert e.value.status == 3


def test_gemm_special_values(orc):
    """All-ones operands with unit scales give alpha * K exactly; zero operands give 0."""
    M, N, K = 40, 64, 512
    for fmt, unit in ((1, 127), (0, 0x38)):
        for variant in (0, 1):
            a = np.full((M, K // 2), 0x22, np.uint8)
            b = np.full((N, K // 2), 0x22, np.uint8)
            sfa = np.full(orc.sf_bytes(M, K, fmt, 0), unit, np.uint8)
            sfb = np.full(orc.sf_bytes(N, K, fmt, 0), unit, np.uint8)
            out = lb.lowbit_gemm_bf16(dev_u8(a), dev_u8(b), dev_u8(sfa), dev_u8(sfb), fmt=fmt, alpha=0.25,
                                      variant=variant)
            torch.cuda.synchronize()
            assert np.all(host_f64(out) == 0.25 * K)
            out = lb.lowbit_gemm_bf16(dev_u8(np.zeros_like(a)), dev_u8(b), dev_u8(sfa), dev_u8(sfb), fmt=fmt,
                                      variant=variant)
            torch.cuda.synchronize()
            assert np.all(host_f64(out) == 0.0)


def test_gemm_empty_and_errors(orc):
    a = torch.zeros((0, 64), dtype=torch.uint8, device="cuda")
    b = torch.zeros((32, 64), dtype=torch.uint8, device="cuda")
    s = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    out = lb.lowbit_gemm_bf16(a, b, s, s, fmt=1)
    assert out.shape == (0, 32)
    a = torch.zeros((200, 64), dtype=torch.uint8, device="cuda")
    with pytest.raises(lb.LowbitError) as e:
        lb.lowbit_gemm_bf16(a, b, s, s, fmt=1, variant=0)   # decode schedule cannot hold 200 rows
    assert e.value.status == 3


# --- FP4-output epilogue ---------------------------------------------------------------------

def run_gelu_fp4(orc, M, N, K, fmt, variant, out_layout, seed, gs_out=1.0):
    banner(f"gelu_fp4 M={M} N={N} K={K} fmt={fmt} variant={variant} out_layout={out_layout}")
    ws = split_workspace(M, N, K, fmt, variant) if variant == 2 else None
    a, sfa, b, sfb = operands(orc, M, N, K, fmt, 0, 1, seed)
    bias = synth.bias(N, seed)
    alpha = 1.0
    ref = orc.gemm_gelu_fp4(a, b, sfa, sfb, M, N, K, fmt, 0, 1, alpha, synth.bits(bias), gs_out,
                            out_layout, diag=True)
    p, s = lb.lowbit_gemm_bias_gelu_fp4(dev_u8(a), dev_u8(b), dev_u8(sfa), dev_u8(sfb), dev_bf16(bias),
                                        fmt=fmt, sfa_layout=0, sfb_layout=1, alpha=alpha,
                                        out_global_scale=dev_f32(gs_out), out_layout=out_layout,
                                        variant=variant, workspace=ws)
    torch.cuda.synchronize()
    code_extra, scale_extra = checkers.fp4_out_windows(ref, gs_out, M, N)
    rep = checkers.compare_quantized(orc, orc.NVFP4, gs_out, host_u8(p), host_u8(s), ref["packed"],
                                     ref["sf"], ref["y"], ref["v"], ref["spre"], M, N, out_layout,
                                     code_extra=code_extra, scale_extra=scale_extra)
    banner(f"  report {dict(rep)}")
    assert rep.ok(), rep
    if out_layout == 1:
        assert checkers.tiled_padding_is_zero(orc, host_u8(s), M, N // 16, 0)


@pytest.mark.parametrize("M,N,K", [(1, 64, 256), (33, 272, 512), (130, 176, 320), (1, 8256, 256), (96, 272, 512),
                                   (128, 160, 1024)])
@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("out_layout", [0, 1])
def test_gemm_gelu_fp4(orc, M, N, K, fmt, out_layout):
    for variant in (0, 1):
        if variant == 0 and M > 128:
            continue
        run_gelu_fp4(orc, M, N, K, fmt, variant, out_layout, seed=M + N)


# --- split-K (decode schedule with K also split across workgroups) ---------------------------

SPLITK_SHAPES = [(1, 32, 512), (5, 40, 768), (33, 70, 2048), (64, 96, 4352), (100, 48, 4608), (128, 264, 1536),
                 (17, 1000, 3072), (3, 96, 17408)]


@pytest.mark.parametrize("M,N,K", SPLITK_SHAPES)
@pytest.mark.parametrize("fmt", [0, 1])
def test_gemm_splitk_plain(orc, M, N, K, fmt):
    run_gemm(orc, M, N, K, fmt, 0, 1, 0, 2, seed=M + N + K + 5, alpha=0.5)


@pytest.mark.parametrize("epi", [1, 2, 3, 4])
@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("la,lb_", [(0, 0), (1, 1)])
def test_gemm_splitk_epilogues(orc, epi, fmt, la, lb_):
    run_gemm(orc, 97, 264, 2304, fmt, la, lb_, epi, 2, seed=epi * 10 + fmt + la)


@pytest.mark.parametrize("M,N,K", [(1, 64, 1024), (96, 272, 2560), (128, 160, 4096)])
@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("out_layout", [0, 1])
def test_gemm_splitk_gelu_fp4(orc, M, N, K, fmt, out_layout):
    run_gelu_fp4(orc, M, N, K, fmt, 2, out_layout, seed=M + N + 3)


# Above 128 rows NVFP4 with K % 64 == 0 splits the 128 x 384 schedule along
# K: ragged M (129: a one-row second M-tile) and N, a last stage of half
# length (4160 = 32.5 stages of 128), every layout pair and epilogue;
# explicit, and automatic with the workspace offered (all but the 16-stage
# shape have few tiles and K enough for the automatic choice to split)
PREFILL_SPLIT_SHAPES = [(300, 770, 4096), (600, 1000, 2048), (129, 96, 8192), (257, 400, 4160)]


@pytest.mark.parametrize("M,N,K", PREFILL_SPLIT_SHAPES)
@pytest.mark.parametrize("la,lb_", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_gemm_nvfp4_prefill_splitk(orc, M, N, K, la, lb_):
    run_gemm(orc, M, N, K, 0, la, lb_, 0, 2, seed=M + N + K + la, alpha=0.5, outliers=True)
    auto = lb.lowbit_gemm_workspace_bytes(M, N, K, 0, -1)
    assert (auto > 0) == (K >= 4096)
    if auto:
        run_gemm(orc, M, N, K, 0, la, lb_, 0, -1, seed=M + N + K + lb_ + 7, workspace=True)


@pytest.mark.parametrize("epi", [1, 2, 3, 4])
def test_gemm_nvfp4_prefill_splitk_epilogues(orc, epi):
    run_gemm(orc, 300, 400, 4096, 0, 1, 1, epi, 2, seed=epi + 40, outliers=True)


@pytest.mark.parametrize("out_layout", [0, 1])
def test_gemm_nvfp4_prefill_splitk_gelu_fp4(orc, out_layout):
    run_gelu_fp4(orc, 300, 400, 4096, 0, 2, out_layout, seed=301)


@pytest.mark.parametrize("M,N,K", [(40, 96, 1552), (128, 200, 4112), (3, 64, 2064)])
def test_gemm_splitk_nvfp4_half_chunk_k(orc, M, N, K):
    assert K % 32 == 16
    run_gemm(orc, M, N, K, 0, 1, 1, 3, 2, seed=M + K)


@pytest.mark.parametrize("shape", synth.MXFP4_DECODE["shapes"])
def test_gemm_splitk_mxfp4_decode_shapes_full(orc, shape):
    """The decode workloads with a workspace offered (the automatic choice
    splits K where its plan says so) and with split-K forced, every output
    checked."""
    M, N, K = shape
    run_gemm(orc, M, N, K, orc.MXFP4, 1, 1, 0, -1, seed=synth.MXFP4_DECODE["seed"], workspace=True)
    run_gemm(orc, M, N, K, orc.MXFP4, 1, 1, 0, 2, seed=synth.MXFP4_DECODE["seed"])


def test_gemm_splitk_repeatable(orc):
    """The partials are summed in split order: two launches give identical
    bits whatever the workspace held before."""
    M, N, K = 41, 1536, 6144
    a, sfa, b, sfb = operands(orc, M, N, K, 1, 1, 1, 17)
    args = (dev_u8(a), dev_u8(b), dev_u8(sfa), dev_u8(sfb))
    ws = split_workspace(M, N, K, 1, 2)
    o1 = lb.lowbit_gemm_bf16(*args, fmt=1, sfa_layout=1, sfb_layout=1, variant=2, workspace=ws)
    ws.fill_(0x7F)
    o2 = lb.lowbit_gemm_bf16(*args, fmt=1, sfa_layout=1, sfb_layout=1, variant=2, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_gemm_splitk_errors(orc):
    a, sfa, b, sfb = operands(orc, 8, 64, 1024, 1, 0, 0, 1)
    args = (dev_u8(a), dev_u8(b), dev_u8(sfa), dev_u8(sfb))
    with pytest.raises(lb.LowbitError) as e:
        lb.lowbit_gemm_bf16(*args, fmt=1, variant=2)                      # no workspace
    assert e.value.status == 1
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(lb.LowbitError) as e:
        lb.lowbit_gemm_bf16(*args, fmt=1, variant=2, workspace=small)     # too small
    assert e.value.status == 1
