"""lowbit_gemm_bf16_noalloc, the GEMM entry point that allocates nothing (its
split-K workspace is the library's static device array), against
lowbit_gemm_bf16 with a caller workspace and against the oracle: two calls in
a row, the second smaller, then the same pair again on the automatic choice,
and the size the static array cannot take."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_add_amd as lb
from block_scaled_fp4_add_amd import synth

from . import checkers
from .gpu_util import banner, dev_u8, host_f64

pytestmark = pytest.mark.gpu


def _operands(orc, M, N, K, fmt, seed):
    A = synth.activation(M, K, seed, outliers=True)
    W = synth.weight(N, K, seed)
    a, sfa = orc.quantize(synth.bits(A), fmt, orc.TILED)
    b, sfb = orc.quantize(synth.bits(W), fmt, orc.TILED)
    return a, sfa, b, sfb


@pytest.mark.parametrize("variant", [lb.VARIANT_SPLITK, lb.VARIANT_AUTO])
def test_noalloc_matches_workspace_entry(orc, variant):
    # each call smaller than the one before; the first splits the 128 x 384
    # schedule above 128 rows, the others the decode schedule
    for (M, N, K, fmt) in ((300, 400, 4096, 0), (41, 1536, 6144, 1), (5, 512, 4096, 0)):
        banner(f"noalloc M={M} N={N} K={K} fmt={fmt} variant={variant}")
        need = lb.lowbit_gemm_workspace_bytes(M, N, K, fmt, variant)
        assert 0 < need <= lb.STATIC_SCRATCH_BYTES or variant == lb.VARIANT_AUTO
        a, sfa, b, sfb = _operands(orc, M, N, K, fmt, M + K)
        args = (dev_u8(a), dev_u8(b), dev_u8(sfa), dev_u8(sfb))
        kw = dict(fmt=fmt, sfa_layout=1, sfb_layout=1, alpha=0.5, variant=variant)
        ws = torch.full((max(need, 16),), 0xFF, dtype=torch.uint8, device="cuda")
        want = lb.lowbit_gemm_bf16(*args, workspace=ws, **kw)
        got = lb.lowbit_gemm_bf16_noalloc(*args, **kw)
        torch.cuda.synchronize()
        assert torch.equal(got, want), "the static scratch must give the caller-workspace result"
        ref, l1 = orc.gemm(a, b, sfa, sfb, M, N, K, fmt, 1, 1, alpha=0.5)
        ok, worst = checkers.gemm_within_tolerance(host_f64(got), ref, l1)
        banner(f"  worst err/tol {worst:.3g}")
        assert ok.all()


def test_noalloc_mxfp8_mma(orc):
    """MXFP8 on the scaled FP8 MFMA: its 256 x 256 split through the static
    array gives the caller-workspace result, explicitly and automatically."""
    M, N, K = 300, 400, 4096
    A, W = synth.activation(M, K, 9, outliers=True), synth.weight(N, K, 9)
    a, sfa = orc.quantize(synth.bits(A), orc.MXFP8, orc.LINEAR)
    b, sfb = orc.quantize(synth.bits(W), orc.MXFP8, orc.LINEAR)
    args = (dev_u8(a), dev_u8(b), dev_u8(sfa), dev_u8(sfb))
    for variant in (lb.VARIANT_SPLITK, lb.VARIANT_AUTO):
        banner(f"noalloc mxfp8 mma M={M} N={N} K={K} variant={variant}")
        need = lb.lowbit_gemm_workspace_bytes(M, N, K, lb.MXFP8_MMA, variant)
        assert 0 < need <= lb.STATIC_SCRATCH_BYTES
        ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
        want = lb.lowbit_gemm_bf16(*args, fmt=lb.MXFP8_MMA, variant=variant, workspace=ws)
        got = lb.lowbit_gemm_bf16_noalloc(*args, fmt=lb.MXFP8_MMA, variant=variant)
        torch.cuda.synchronize()
        assert torch.equal(got, want)


def test_noalloc_refuses_plans_beyond_the_array(orc):
    """Forced split-K of a product whose partials need more than the static
    array: refused with LOWBIT_ESHAPE before any launch."""
    M, N, K = 128, 32768, 1024
    assert lb.lowbit_gemm_workspace_bytes(M, N, K, 1, lb.VARIANT_SPLITK) > lb.STATIC_SCRATCH_BYTES
    a = torch.zeros((M, K // 2), dtype=torch.uint8, device="cuda")
    b = torch.zeros((N, K // 2), dtype=torch.uint8, device="cuda")
    sa = torch.full((lb.lowbit_sf_bytes(M, K, 1, 1),), 127, dtype=torch.uint8, device="cuda")
    sb = torch.full((lb.lowbit_sf_bytes(N, K, 1, 1),), 127, dtype=torch.uint8, device="cuda")
    with pytest.raises(lb.LowbitError) as e:
        lb.lowbit_gemm_bf16_noalloc(a, b, sa, sb, fmt=1, sfa_layout=1, sfb_layout=1, variant=lb.VARIANT_SPLITK)
    assert e.value.status == 3
    out = lb.lowbit_gemm_bf16_noalloc(a, b, sa, sb, fmt=1, sfa_layout=1, sfb_layout=1)   # auto: not split
    torch.cuda.synchronize()
    assert bool((out == 0).all())
