"""The benchmark's algorithmic work per launch (bytes for the HBM-bound
kernels, FLOPs for the GEMMs) against the workload figures worked out from
the tensor sizes: the roofline fractions bench.py reports divide by these."""
import pytest

import bench


def test_producer_bytes():
    # x, r read and r written in bf16 (6 B), FP4 codes (0.5 B) and one E4M3
    # scale per 16 elements, plus the weight row (2H) and the global scale (4 B)
    assert bench.producer_bytes(4096, 4096, 16) == 110_108_676
    assert bench.producer_bytes(2048, 5120, 16) == 2048 * 5120 * 6 + 2048 * 2560 + 2048 * 320 + 10240 + 4
    # MXFP8: one byte per element and one scale per 32
    assert bench.producer_bytes(4096, 4096, 32, 1.0) == 4096 * 4096 * 7 + 4096 * 128 + 8192 + 4


@pytest.mark.parametrize("shape,mb,half_ulp", [((41, 4608, 1536), 4.171, 5e-4), ((41, 6144, 1536), 5.551, 5e-4),
                                               ((41, 1536, 6144), 5.273, 5e-4), ((1, 17408, 5120), 47.39, 5e-3)])
def test_decode_gemm_bytes(shape, mb, half_ulp):
    # (M + N) K (1/2 + 1/32) operand bytes + 2 M N bf16 output, against the
    # figure rounded to its printed digits
    assert bench.gemm_bytes(*shape, 32) / 1e6 == pytest.approx(mb, abs=half_ulp)


@pytest.mark.parametrize("shape,mb", [((8192, 14336, 4096), 518.8), ((8192, 4096, 14336), 227.8)])
def test_prefill_gemm_bytes_and_flops(shape, mb):
    # operands + bias (2N) + residual in and bf16 out (4MN)
    assert bench.gemm_bytes(*shape, 32, epi_bias=True, epi_res=True) / 1e6 == pytest.approx(mb, abs=0.05)
    M, N, K = shape
    assert 2.0 * M * N * K / 1e9 == pytest.approx(962.07, abs=0.005)


def test_chain_gemm1_fp4_output_bytes():
    # NVFP4 operands (1/2 + 1/16 B per element), bias, FP4 output (1/2 + 1/16 B per output)
    M, N, K = 2048, 17408, 5120
    want = (M + N) * (K // 2 + K // 16) + 2 * N + M * N // 2 + M * N // 16
    assert bench.gemm_bytes(M, N, K, 16, epi_bias=True, out_fp4=True) == want
