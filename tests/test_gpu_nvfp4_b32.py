"""GPU parity of the NVFP4 rule on 32-element blocks (LOWBIT_NVFP4_B32: E4M3
block scales with the global scale folded in, LINEAR scales) against the
oracle: the fused producer in both of its kernel forms, the quantizer and the
dequantizer, bf16 and fp16 tensors, every byte compared."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_add_amd as lb
from block_scaled_fp4_add_amd import synth

from .gpu_util import banner, dev_bf16, dev_f32, host_bits, host_u8

pytestmark = pytest.mark.gpu
EPS = 1e-6
B32 = lb.NVFP4_B32


def _gs(orc, xb, rb, wb, odt):
    d = orc.add_rmsnorm_quant(xb, rb, wb, EPS, orc.NVFP4, orc.LINEAR, diag=True, dtype=odt)
    return float(np.float32(2688.0 / np.abs(d["y"]).max()))


# row-split form below 256 rows, a workgroup per row above; ragged row lengths
@pytest.mark.parametrize("M,H", [(1, 64), (8, 256), (33, 1024), (5, 5120), (300, 1536), (2049, 512),
                                 (520, 5632), (4096, 4096)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_producer_bit_exact(orc, M, H, dtype):
    banner(f"producer nvfp4_b32 M={M} H={H} dtype={dtype}")
    odt = orc.F16 if dtype == torch.float16 else orc.BF16
    x, r, w = synth.producer_inputs(M, H, 17 * M + H, outliers=True, dtype=dtype)
    xb, rb, wb = synth.bits(x), synth.bits(r), synth.bits(w)
    gs = _gs(orc, xb, rb, wb, odt)
    ref = orc.add_rmsnorm_quant(xb, rb, wb, EPS, orc.NVFP4_B32, orc.LINEAR, gs=gs, dtype=odt)
    rd = dev_bf16(r)
    packed = torch.full((M, H // 2), 0xAA, dtype=torch.uint8, device="cuda")
    sf = torch.full((lb.lowbit_sf_bytes(M, H, B32, lb.LINEAR),), 0xAA, dtype=torch.uint8, device="cuda")
    lb.lowbit_add_rmsnorm_quant(dev_bf16(x), rd, dev_bf16(w), EPS, B32, lb.LINEAR, global_scale=dev_f32(gs),
                                out_packed=packed, out_sf=sf)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(rd), ref["residual"])
    assert np.array_equal(host_u8(sf), ref["sf"])
    assert np.array_equal(host_u8(packed), ref["packed"])


@pytest.mark.parametrize("rows,K", [(1, 64), (7, 160), (41, 1536), (300, 2560), (1000, 5120)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_quantize_bit_exact(orc, rows, K, dtype):
    banner(f"quantize nvfp4_b32 rows={rows} K={K} dtype={dtype}")
    odt = orc.F16 if dtype == torch.float16 else orc.BF16
    x = synth.activation(rows, K, 5 * rows + K, outliers=True, dtype=dtype)
    gs = 0.8125
    rp, rs = orc.quantize(synth.bits(x), orc.NVFP4_B32, orc.LINEAR, gs=gs, dtype=odt)
    p, s = lb.lowbit_quantize(dev_bf16(x), B32, lb.LINEAR, global_scale=dev_f32(gs))
    torch.cuda.synchronize()
    assert np.array_equal(host_u8(p), rp) and np.array_equal(host_u8(s), rs)


def test_dequantize_bit_exact(orc):
    rows, K = 37, 1024
    rng = np.random.default_rng(3)
    packed = rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)
    sf = rng.integers(0, 0x7F, rows * K // 32, dtype=np.uint8)   # finite E4M3 bytes
    gs = 3.5
    ref, _ = orc.dequantize(packed, sf, rows, K, orc.NVFP4_B32, orc.LINEAR, gs=gs)
    out = lb.lowbit_dequantize(torch.from_numpy(packed).cuda(), torch.from_numpy(sf).cuda(), B32, lb.LINEAR,
                               global_scale=dev_f32(gs))
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(out), ref)


def test_rejections_on_device():
    x = torch.zeros((4, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lb.LowbitError):   # LINEAR scales only
        lb.lowbit_quantize(x, B32, lb.TILED, out_sf=torch.empty(64, dtype=torch.uint8, device="cuda"))
    a = torch.zeros((32, 128), dtype=torch.uint8, device="cuda")
    s = torch.zeros(32 * 8, dtype=torch.uint8, device="cuda")
    with pytest.raises(lb.LowbitError):   # no GEMM for this format
        lb.lowbit_gemm_bf16(a, a, s, s, fmt=B32)
