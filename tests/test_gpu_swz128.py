"""GPU parity of the 128 x 4 swizzled scale layout (LOWBIT_SF_SWZ128, the
producer page's swizzled output) against the oracle: the fused producer in both
kernel forms, the quantizer and the dequantizer, NVFP4 and MXFP4, every byte of
the scale buffer compared (padding included, which must be zero)."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_add_amd as lb
from block_scaled_fp4_add_amd import synth

from .gpu_util import banner, dev_bf16, dev_f32, host_bits, host_u8

pytestmark = pytest.mark.gpu
EPS = 1e-6
SWZ = lb.SWZ128


# row-split form below 256 rows, a workgroup per row above; M % 128 != 0 for
# padding rows, blocks per row % 4 != 0 for padding blocks
@pytest.mark.parametrize("M,H", [(1, 64), (8, 256), (33, 1120), (130, 5120), (300, 1568), (2049, 512),
                                 (520, 5632), (4096, 4096)])
@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_producer_bit_exact(orc, M, H, fmt, dtype):
    if H % (16 if fmt == 0 else 32):
        pytest.skip("H is not a whole number of blocks")
    banner(f"producer swz128 M={M} H={H} fmt={fmt} dtype={dtype}")
    odt = orc.F16 if dtype == torch.float16 else orc.BF16
    x, r, w = synth.producer_inputs(M, H, 19 * M + H, outliers=True, dtype=dtype)
    xb, rb, wb = synth.bits(x), synth.bits(r), synth.bits(w)
    gs = 0.6875 if fmt == 0 else 1.0
    ref = orc.add_rmsnorm_quant(xb, rb, wb, EPS, fmt, orc.SWZ128, gs=gs, dtype=odt)
    rd = dev_bf16(r)
    packed = torch.full((M, H // 2), 0xAA, dtype=torch.uint8, device="cuda")
    sf = torch.full((lb.lowbit_sf_bytes(M, H, fmt, SWZ),), 0xAA, dtype=torch.uint8, device="cuda")
    lb.lowbit_add_rmsnorm_quant(dev_bf16(x), rd, dev_bf16(w), EPS, fmt, SWZ,
                                global_scale=dev_f32(gs) if fmt == 0 else None, out_packed=packed, out_sf=sf)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(rd), ref["residual"])
    assert np.array_equal(host_u8(sf), ref["sf"])
    assert np.array_equal(host_u8(packed), ref["packed"])


@pytest.mark.parametrize("rows,K", [(1, 64), (7, 160), (41, 1536), (300, 2560), (1000, 5120)])
@pytest.mark.parametrize("fmt", [0, 1])
def test_quantize_and_dequantize_bit_exact(orc, rows, K, fmt):
    if K % (16 if fmt == 0 else 32):
        pytest.skip("K is not a whole number of blocks")
    banner(f"quantize swz128 rows={rows} K={K} fmt={fmt}")
    x = synth.activation(rows, K, 7 * rows + K, outliers=True)
    rp, rs = orc.quantize(synth.bits(x), fmt, orc.SWZ128)
    sf = torch.full((lb.lowbit_sf_bytes(rows, K, fmt, SWZ),), 0xAA, dtype=torch.uint8, device="cuda")
    p, s = lb.lowbit_quantize(dev_bf16(x), fmt, SWZ, out_sf=sf)
    torch.cuda.synchronize()
    assert np.array_equal(host_u8(p), rp) and np.array_equal(host_u8(s), rs)
    ref, _ = orc.dequantize(rp, rs, rows, K, fmt, orc.SWZ128)
    out = lb.lowbit_dequantize(p, s, fmt, SWZ)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(out), ref)


def test_gemm_rejects_the_layout():
    a = torch.zeros((32, 128), dtype=torch.uint8, device="cuda")
    s = torch.zeros(512, dtype=torch.uint8, device="cuda")
    with pytest.raises(lb.LowbitError):
        lb.lowbit_gemm_bf16(a, a, s, s, fmt=lb.MXFP4, sfa_layout=SWZ)
