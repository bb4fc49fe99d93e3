"""GPU parity of LOWBIT_MXFP8_MMA: MXFP8 operands (the vLLM fused_wo_a page's
format) contracted on gfx950's scaled FP8 MFMA, as that page's MMA stage runs
its block-scaled MXFP8 contraction on the hardware MMA.  The instruction sums
a 32-element block's products in a window narrower than fp32, so this format
states its own accumulation term: |gpu - ref| <= 2^-7 |ref| + 2^-10 L1
(measured worst case 2^-11.4 L1, below).  The oracle is the exact MXFP8
contraction; operands are quantized by the oracle as MXFP8."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_add_amd as lb

from .gpu_util import banner, dev_u8, host_f64
from .test_gpu_gemm import run_gemm, split_workspace
from .test_gpu_mxfp8 import one_hot_operands, run_fp8_out

pytestmark = pytest.mark.gpu

MMA = lb.MXFP8_MMA
L1_MMA = 2.0 ** -10     # the stated accumulation term of the format


# above 128 rows with K % 128 == 0: the 256 x 256 schedule on the scaled FP8
# MFMA; ragged M and N, K of one superstep and of many, every epilogue
@pytest.mark.parametrize("M,N,K", [(129, 400, 512), (300, 1000, 1152), (257, 770, 128), (256, 256, 256),
                                   (1000, 520, 2048), (520, 96, 4096)])
@pytest.mark.parametrize("epi", [0, 1, 2, 3, 4])
def test_mma_prefill(orc, M, N, K, epi):
    run_gemm(orc, M, N, K, MMA, 0, 0, epi, 1, seed=M + N + K + epi, alpha=0.5, outliers=True, l1_coef=L1_MMA)


# the same schedule split along K (supersteps of 128 elements): ragged M and
# N, a last split shorter than the others; explicit, and automatic with the
# workspace offered
@pytest.mark.parametrize("M,N,K", [(300, 770, 2048), (600, 1000, 4096), (129, 96, 8192), (257, 400, 4224)])
def test_mma_prefill_splitk(orc, M, N, K):
    run_gemm(orc, M, N, K, MMA, 0, 0, 0, 2, seed=M + N + K + 11, alpha=0.5, outliers=True, l1_coef=L1_MMA)
    assert lb.lowbit_gemm_workspace_bytes(M, N, K, MMA, -1) > 0
    run_gemm(orc, M, N, K, MMA, 0, 0, 0, -1, seed=M + N + K + 12, workspace=True, l1_coef=L1_MMA)


@pytest.mark.parametrize("epi", [1, 2, 3, 4])
def test_mma_prefill_splitk_epilogues(orc, epi):
    run_gemm(orc, 300, 400, 4096, MMA, 0, 0, epi, 2, seed=epi + 50, outliers=True, l1_coef=L1_MMA)


# where the scaled FP8 MFMA does not run (the decode schedule, K % 128 != 0)
# the format is the exact path, under the exact rule
@pytest.mark.parametrize("M,N,K,variant", [(41, 4608, 1536, -1), (5, 40, 2144, 2), (200, 96, 1056, 1)])
def test_mma_elsewhere_is_the_exact_path(orc, M, N, K, variant):
    run_gemm(orc, M, N, K, MMA, 0, 0, 0, variant, seed=M + K, alpha=0.5, workspace=variant == -1)


@pytest.mark.parametrize("M,N,K,variant", [(200, 416, 1024, 1), (256, 256, 2048, 2)])
def test_mma_single_product_is_exact(orc, M, N, K, variant):
    """One product per output: nothing to add, so the scaled FP8 MFMA returns
    the closed form exactly, for every code and scale bytes 10..246."""
    banner(f"mxfp8 mma one-hot M={M} N={N} K={K} variant={variant}")
    a, sfa, b, sfb, exact = one_hot_operands(orc, M, N, K)
    ws = split_workspace(M, N, K, MMA, 2) if variant == 2 else None
    out = lb.lowbit_gemm_bf16(dev_u8(a), dev_u8(b), dev_u8(sfa), dev_u8(sfb), fmt=MMA, variant=variant,
                              workspace=ws)
    torch.cuda.synchronize()
    got = host_f64(out)
    normal = (np.abs(exact) >= 2.0 ** -126) & (np.abs(exact) < 2.0 ** 127)
    assert normal.sum() > M * N // 4
    assert not (normal & (got != exact)).any()


@pytest.mark.parametrize("M,N,K,variant", [(300, 800, 1024, 1), (129, 416, 576, 1), (300, 800, 4096, 2)])
@pytest.mark.parametrize("out_layout", [0, 2])
def test_mma_fp8_out(orc, M, N, K, variant, out_layout):
    run_fp8_out(orc, M, N, K, MMA, variant, out_layout, seed=M + K, l1_coef=L1_MMA)


def test_mma_fp8_out_prefill_workload_full(orc):
    """The MXFP8 prefill workload the benchmark times on this format, (4096,
    1024, 8192) with FP8 output and 128 x 4 scales, in its launch
    configuration (256 x 256 tiles, K split in four), every output."""
    assert lb.lowbit_gemm_workspace_bytes(4096, 1024, 8192, MMA, -1) == 4 * 32 * 128 * 4096
    run_fp8_out(orc, 4096, 1024, 8192, MMA, 2, 2, seed=79, alpha=1.0, l1_coef=L1_MMA)


def _partials(M, N, K, a, b, sa, sb):
    """Sum of the split-K fp32 partials of the scaled FP8 MFMA (no bf16 rounding)."""
    n = lb.lowbit_gemm_workspace_bytes(M, N, K, MMA, 2)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    lb.lowbit_gemm_bf16(dev_u8(a), dev_u8(b), dev_u8(sa), dev_u8(sb), fmt=MMA, variant=2, workspace=ws)
    torch.cuda.synchronize()
    w = ws.cpu().numpy().view(np.float32)
    tn, tm = N // 32, M // 32
    S = n // (4 * tn * tm * 1024)
    # tile (y, n / 32, m / 32) holds lane (r, c), float k at row r, column 8(k / 4) + 4c + k % 4
    t = w.reshape(S, tn, tm, 2, 32, 4, 4).sum(axis=0)          # (tn, tm, c, r, k/4, k%4)
    return t.transpose(1, 3, 0, 4, 2, 5).reshape(M, N), S


def test_mma_accumulation_within_the_stated_term(orc):
    """The stated term, pinned on the device's fp32 sums (split-K partials,
    before any bf16 rounding): random E4M3 codes over the whole range (both
    signs, subnormals) with block scales spread over 20 binades -- products
    spanning about 2^55 inside one block pair -- stay within 2^-10 L1; their
    worst case measured 2^-11.4 L1.  And the term is needed: small products
    beside large ones in one block do lose bits (the exact sum is not met)."""
    M = N = 256
    K = 1024
    rng = np.random.default_rng(7)
    table = np.array([orc.e4m3_value(c) for c in range(256)])
    fix = lambda x: np.where((x & 0x7F) == 0x7F, x ^ 1, x).astype(np.uint8)     # no NaN codes
    a, b = fix(rng.integers(0, 256, (M, K))), fix(rng.integers(0, 256, (N, K)))
    sa = rng.integers(117, 138, M * K // 32).astype(np.uint8)
    sb = rng.integers(117, 138, N * K // 32).astype(np.uint8)
    got, S = _partials(M, N, K, a, b, sa, sb)
    assert S >= 2
    av = table[a] * np.repeat(np.exp2(sa.reshape(M, -1).astype(np.float64) - 127), 32, axis=1)
    bv = table[b] * np.repeat(np.exp2(sb.reshape(N, -1).astype(np.float64) - 127), 32, axis=1)
    exact, l1 = av @ bv.T, np.abs(av) @ np.abs(bv).T
    r = np.abs(got - exact) / l1
    banner(f"  max err/L1 = 2^{np.log2(r.max()):.2f}")
    assert r.max() <= L1_MMA
    # one block pair per output row: +448 and -448 (they cancel) and 1.5 * 2^-6 elsewhere
    a = np.full((M, K), orc.e4m3_encode(1.5 * 2.0 ** -6), np.uint8)
    a[:, 0::32] = np.where(np.arange(K // 32) % 2 == 0, 0x7E, 0xFE)[None, :]
    b = np.full((N, K), 0x38, np.uint8)                                        # 1.0
    one = np.full(M * K // 32, 127, np.uint8)
    got, _ = _partials(M, N, K, a, b, one, one)
    exact = (K - K // 32) * 1.5 * 2.0 ** -6
    assert np.all(got < exact) and np.all(got > exact - L1_MMA * (K // 32 * 448 + exact))
