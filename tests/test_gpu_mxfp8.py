"""GPU parity of the MXFP8 GEMM (E4M3 operands, 32-element blocks, UE8M0
scales: the vLLM fused_wo_a page, FusedWoAKernel.device_kernel main loop) and
of the FP8-output epilogue (the same kernel's output stage) against the
oracle.  The bf16 outputs follow the GEMM rule |gpu - ref| <= 2^-7 |ref| +
1e-6 L1; the FP8 outputs follow the interval rule of tests/checkers.py; a
probe with one product per output checks the operand dequantization bit for
bit against the closed form a * b * 2^(ea + eb)."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_add_amd as lb

from . import checkers
from .gpu_util import banner, dev_u8, host_f64, host_u8
from .test_gpu_gemm import operands, run_gemm, split_workspace

pytestmark = pytest.mark.gpu

F8 = 2

# K % 128 (one superstep of FP8 elements) == 0, 32, 64 and 96 all appear,
# with ragged M and N tails; the last ones reach more than 256 workgroups
SHAPES = [(8, 128, 256), (1, 32, 32), (5, 40, 96), (33, 70, 320), (1, 200, 1056), (128, 256, 512),
          (130, 200, 768), (200, 96, 1056), (3, 96, 2336), (40, 64, 4352), (100, 48, 4640), (70, 200, 2560),
          (96, 136, 1568), (41, 4608, 1536), (1, 8224, 544), (2, 9000, 1088)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("variant", [0, 1])
def test_mxfp8_gemm_plain(orc, M, N, K, variant):
    if variant == 0 and M > 128:
        pytest.skip("decode schedule holds at most 128 rows")
    run_gemm(orc, M, N, K, F8, 0, 0, 0, variant, seed=M + N + K + 1, alpha=0.5)


@pytest.mark.parametrize("epi", [1, 2, 3, 4])
@pytest.mark.parametrize("variant", [0, 1, 2])
def test_mxfp8_gemm_epilogues(orc, epi, variant):
    M = 150 if variant == 1 else 33
    run_gemm(orc, M, 264, 2080 if variant == 2 else 544, F8, 0, 0, epi, variant, seed=epi * 10 + variant,
             outliers=True)


# K % 128 == 0 runs the 256 x 256 schedule (prefill, exact bf16 form): ragged M and N, every epilogue
@pytest.mark.parametrize("M,N,K", [(129, 400, 512), (300, 1000, 1152), (257, 770, 128)])
@pytest.mark.parametrize("epi", [0, 1, 2, 3, 4])
def test_mxfp8_gemm_prefill_schedule(orc, M, N, K, epi):
    run_gemm(orc, M, N, K, F8, 0, 0, epi, 1, seed=M + N + K + epi, alpha=0.5, outliers=True)


@pytest.mark.parametrize("M,N,K", [(1, 32, 2048), (5, 40, 2144), (64, 96, 4352), (128, 264, 3072),
                                   (17, 1000, 6144), (3, 96, 17408)])
def test_mxfp8_gemm_splitk(orc, M, N, K):
    run_gemm(orc, M, N, K, F8, 0, 0, 0, 2, seed=M + N + K + 9, alpha=0.25)
    run_gemm(orc, M, N, K, F8, 0, 0, 0, -1, seed=M + N + K + 9, alpha=0.25, workspace=True)


# Above 128 rows MXFP8 with K % 128 == 0 splits the 256 x 256 schedule along
# K (supersteps of 128 elements): ragged M and N, a last split shorter than the
# others (4224 = 33 supersteps: 9, 9, 9, 6); explicit, and automatic with the workspace offered
@pytest.mark.parametrize("M,N,K", [(300, 770, 2048), (600, 1000, 4096), (129, 96, 8192), (257, 400, 4224)])
def test_mxfp8_gemm_prefill_splitk(orc, M, N, K):
    run_gemm(orc, M, N, K, F8, 0, 0, 0, 2, seed=M + N + K + 11, alpha=0.5, outliers=True)
    assert lb.lowbit_gemm_workspace_bytes(M, N, K, F8, -1) > 0      # 16 supersteps of 128 elements or more
    run_gemm(orc, M, N, K, F8, 0, 0, 0, -1, seed=M + N + K + 12, workspace=True)


@pytest.mark.parametrize("epi", [1, 2, 3, 4])
def test_mxfp8_gemm_prefill_splitk_epilogues(orc, epi):
    run_gemm(orc, 300, 400, 4096, F8, 0, 0, epi, 2, seed=epi + 50, outliers=True)


def one_hot_operands(orc, M, N, K):
    """A: row i holds one nonzero E4M3 code, at k_i; B: every element
    nonzero.  Every scale byte lies in 10..246, where E4M3 x 2^e is a normal
    bf16 value.  Returns the operands and the exact products."""
    nblk = K // 32
    i = np.arange(M)
    ki = (i * 37 + 5) % K
    ca = (1 + (i * 5) % 126) | np.where(i % 2 == 1, 0x80, 0)          # codes 0x01..0x7E, both signs
    a = np.zeros((M, K), np.uint8)
    a[i, ki] = ca
    sfa = (10 + (i[:, None] * 41 + np.arange(nblk)[None, :] * 7) % 237).astype(np.uint8)
    j = np.arange(N)[:, None]
    k = np.arange(K)[None, :]
    b = ((1 + (j * 7 + k * 3) % 126) | np.where((j + k) % 2 == 1, 0x80, 0)).astype(np.uint8)
    sfb = (10 + (j * 13 + np.arange(nblk)[None, :] * 29) % 237).astype(np.uint8)
    table = np.array([orc.e4m3_value(c) for c in range(256)])
    va = table[ca] * np.exp2(sfa[i, ki // 32].astype(np.float64) - 127)                 # (M,)
    vb = table[b[:, ki]] * np.exp2(sfb[:, ki // 32].astype(np.float64) - 127)          # (N, M)
    exact = va[:, None] * vb.T                                                          # (M, N)
    return a, sfa.reshape(-1), b, sfb.reshape(-1), exact


@pytest.mark.parametrize("M,N,K", [(128, 256, 96), (64, 200, 4128), (100, 96, 2080), (200, 416, 1024)])
@pytest.mark.parametrize("variant", [0, 1, 2])
def test_mxfp8_dequantization_is_exact(orc, M, N, K, variant):
    """One product per output: E4M3 x 2^ea times E4M3 x 2^eb has at most 8
    significant bits, so inside the normal range the bf16 output must equal
    the closed form exactly, for every code and for scale bytes 10..246."""
    if variant == 2 and lb.lowbit_gemm_workspace_bytes(M, N, K, F8, 2) == 0:
        pytest.skip("K too short to split")
    if variant == 0 and M > 128:
        pytest.skip("decode schedule holds at most 128 rows")
    banner(f"mxfp8 one-hot M={M} N={N} K={K} variant={variant}")
    a, sfa, b, sfb, exact = one_hot_operands(orc, M, N, K)
    ws = split_workspace(M, N, K, F8, 2) if variant == 2 else None
    out = lb.lowbit_gemm_bf16(dev_u8(a), dev_u8(b), dev_u8(sfa), dev_u8(sfb), fmt=F8, variant=variant, workspace=ws)
    torch.cuda.synchronize()
    got = host_f64(out)
    normal = (np.abs(exact) >= 2.0 ** -126) & (np.abs(exact) < 2.0 ** 127)
    assert normal.sum() > M * N // 4
    bad = normal & (got != exact)
    banner(f"  {int(normal.sum())} in range, {int(bad.sum())} differ")
    assert not bad.any(), np.argwhere(bad)[:5]
    ref, _ = orc.gemm(a, b, sfa, sfb, M, N, K, F8, 0, 0)
    assert np.array_equal(ref[normal], exact[normal])


# --- FP8-output epilogue ---------------------------------------------------------------------

def run_fp8_out(orc, M, N, K, fmt, variant, out_layout, seed, alpha=0.75, l1_coef=1e-6):
    banner(f"gemm_fp8 M={M} N={N} K={K} fmt={fmt} variant={variant} out_layout={out_layout} seed={seed}")
    ofmt = F8 if fmt == lb.MXFP8_MMA else fmt     # the oracle's format
    la, lb_ = (0, 0) if ofmt == F8 else (0, 1)
    a, sfa, b, sfb = operands(orc, M, N, K, ofmt, la, lb_, seed, outliers=True)
    ws = split_workspace(M, N, K, fmt, 2) if variant == 2 else None
    p_ref, s_ref, ref, l1 = orc.gemm_fp8_out(a, b, sfa, sfb, M, N, K, ofmt, la, lb_, alpha, out_layout, diag=True)
    p, s = lb.lowbit_gemm_fp8(dev_u8(a), dev_u8(b), dev_u8(sfa), dev_u8(sfb), fmt=fmt, sfa_layout=la,
                              sfb_layout=lb_, alpha=alpha, out_layout=out_layout, variant=variant, workspace=ws)
    torch.cuda.synchronize()
    assert tuple(p.shape) == (M, N) and s.numel() == s_ref.size
    rep = checkers.compare_fp8_out(orc, host_u8(p), host_u8(s), p_ref, s_ref, ref, l1, M, N, out_layout, l1_coef)
    banner(f"  report {dict(rep)}")
    assert rep.ok(), rep
    # the interval rule admits a neighbour only where the fp32 sum sits next
    # to a rounding boundary: nearly every byte matches the oracle's (the
    # scaled FP8 MFMA's wider accumulation term admits more)
    if l1_coef <= 1e-6:
        assert rep["code_diff"] <= max(8, M * N // 500) and rep["scale_diff"] <= max(2, rep["blocks"] // 500)


# (200, 160, 1056): NVFP4 with K % 64 == 32 (the 64-byte-stage prefill kernel)
FP8_OUT_SHAPES = [(1, 64, 256), (33, 288, 512), (130, 160, 320), (96, 4096, 512), (1, 8224, 256), (128, 160, 1024),
                  (200, 96, 2048), (300, 800, 1024), (129, 416, 576), (200, 160, 1056)]


@pytest.mark.parametrize("M,N,K", FP8_OUT_SHAPES)
@pytest.mark.parametrize("fmt", [0, 1, 2])
@pytest.mark.parametrize("out_layout", [0, 2])
def test_gemm_fp8_out(orc, M, N, K, fmt, out_layout):
    for variant in (0, 1):
        if variant == 0 and M > 128:
            continue
        run_fp8_out(orc, M, N, K, fmt, variant, out_layout, seed=M + N + fmt)


@pytest.mark.parametrize("M,N,K", [(1, 64, 2048), (96, 288, 4096), (128, 160, 6144), (300, 800, 4096)])
@pytest.mark.parametrize("fmt", [0, 1, 2])
@pytest.mark.parametrize("out_layout", [0, 2])
def test_gemm_fp8_out_splitk(orc, M, N, K, fmt, out_layout):
    if M > 128 and fmt == 1:
        pytest.skip("MXFP4 splits K at most 128 rows")
    run_fp8_out(orc, M, N, K, fmt, 2, out_layout, seed=M + K + fmt)


def test_mxfp8_fp8_out_prefill_workload_full(orc):
    """The MXFP8 prefill workload the benchmark times, (4096, 1024, 8192) with
    FP8 output and 128 x 4 scales, in its launch configuration (the 256 x 256
    schedule split in four along K), every output compared."""
    assert lb.lowbit_gemm_workspace_bytes(4096, 1024, 8192, F8, -1) == lb.lowbit_gemm_workspace_bytes(
        4096, 1024, 8192, F8, 2) > 0
    run_fp8_out(orc, 4096, 1024, 8192, F8, 2, 2, seed=79, alpha=1.0)


@pytest.mark.parametrize("M", [5, 200])
def test_gemm_fp8_out_nvfp4_half_chunk_k(orc, M):
    """NVFP4 with K % 32 == 16 runs the decode schedule in 128-row slices."""
    run_fp8_out(orc, M, 192, 1552, 0, -1, 2, seed=M)


def test_gemm_fp8_out_special_values(orc):
    """All-ones MXFP8 operands with unit scales: every output alpha * K =
    0.75 * 256 = 192, scale byte 126 (2^-1) and code 0x7C (384 = 1.5 x 2^8)
    in every schedule; zero operands give scale byte 0 and zero codes."""
    M, N, K = 40, 64, 256
    a = np.full((M, K), 0x38, np.uint8)
    b = np.full((N, K), 0x38, np.uint8)
    sfa = np.full(M * K // 32, 127, np.uint8)
    sfb = np.full(N * K // 32, 127, np.uint8)
    for variant in (0, 1):
        p, s = lb.lowbit_gemm_fp8(dev_u8(a), dev_u8(b), dev_u8(sfa), dev_u8(sfb), fmt=F8, alpha=0.75,
                                  variant=variant)
        torch.cuda.synchronize()
        assert (host_u8(p) == 0x7C).all() and (host_u8(s) == 126).all()
        p, s = lb.lowbit_gemm_fp8(dev_u8(np.zeros_like(a)), dev_u8(b), dev_u8(sfa), dev_u8(sfb), fmt=F8,
                                  variant=variant)
        torch.cuda.synchronize()
        assert (host_u8(p) == 0).all() and (host_u8(s) == 0).all()


def test_gemm_fp8_out_errors(orc):
    a, sfa, b, sfb = operands(orc, 8, 96, 256, F8, 0, 0, 1)
    args = (dev_u8(a), dev_u8(b), dev_u8(sfa), dev_u8(sfb))
    with pytest.raises(lb.LowbitError) as e:
        lb.lowbit_gemm_fp8(*args, fmt=F8, out_layout=1)              # TILED output scales
    assert e.value.status == 1
    with pytest.raises(lb.LowbitError) as e:
        lb.lowbit_gemm_fp8(*args, fmt=F8, sfa_layout=1)             # MXFP8 operands: LINEAR only
    assert e.value.status == 1
