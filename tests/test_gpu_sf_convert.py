"""GPU parity of the scale relayout (lowbit_sf_convert) against the oracle,
every destination byte compared (padding included, which must be zero), with
garbage in the source's padding and a sentinel past the destination's end;
and the flow it serves: the FlashRT page's GEMM takes operand scales in the
128 x 4 layout, converted here into the TILED layout the GEMM reads."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_add_amd as lb
from block_scaled_fp4_add_amd import synth

from .gpu_util import DEV, banner, dev_bf16, dev_u8, host_bits, host_u8

pytestmark = pytest.mark.gpu
LIN, TIL, SWZ = lb.LINEAR, lb.TILED, lb.SWZ128
BLOCK = {0: 16, 1: 32, 2: 32, 3: 32}
PAIRS = {0: [(a, b) for a in (LIN, TIL, SWZ) for b in (LIN, TIL, SWZ)],
         1: [(a, b) for a in (LIN, TIL, SWZ) for b in (LIN, TIL, SWZ)],
         2: [(LIN, SWZ), (SWZ, LIN), (SWZ, SWZ)],
         3: [(LIN, LIN)]}
CASES = [(fmt, ls, ld) for fmt, pairs in PAIRS.items() for ls, ld in pairs]
SENTINEL = 64


def _run(orc, rows, nblk, fmt, ls, ld, src_off=0, dst_off=0, seed=0):
    K = nblk * BLOCK[fmt]
    sb, db = lb.lowbit_sf_bytes(rows, K, fmt, ls), lb.lowbit_sf_bytes(rows, K, fmt, ld)
    src = np.random.default_rng(seed).integers(0, 256, size=sb, dtype=np.uint8)   # padding is garbage
    ref = orc.sf_convert(src, rows, K, fmt, ls, ld)
    sbuf = torch.zeros(sb + src_off, dtype=torch.uint8, device=DEV)
    sbuf[src_off:] = dev_u8(src)
    dbuf = torch.full((db + dst_off + SENTINEL,), 0xAA, dtype=torch.uint8, device=DEV)
    out = lb.lowbit_sf_convert(sbuf[src_off:], rows, K, fmt, ls, ld, out=dbuf[dst_off:dst_off + db])
    torch.cuda.synchronize()
    assert out.data_ptr() == dbuf[dst_off:].data_ptr()
    got = host_u8(dbuf)
    assert np.array_equal(got[dst_off:dst_off + db], ref)
    assert (got[:dst_off] == 0xAA).all() and (got[dst_off + db:] == 0xAA).all()


@pytest.mark.parametrize("rows,nblk", [(1, 1), (3, 2), (37, 5), (130, 13), (300, 8), (1000, 320), (4097, 257)])
@pytest.mark.parametrize("fmt,ls,ld", CASES)
def test_relayout_bit_exact(orc, rows, nblk, fmt, ls, ld):
    banner(f"sf_convert rows={rows} nblk={nblk} fmt={fmt} {ls}->{ld}")
    _run(orc, rows, nblk, fmt, ls, ld, seed=rows + nblk)


@pytest.mark.parametrize("src_off,dst_off", [(1, 0), (0, 1), (3, 2)])
@pytest.mark.parametrize("fmt,ls,ld", [(0, SWZ, TIL), (1, TIL, LIN), (0, SWZ, LIN), (2, LIN, SWZ)])
def test_relayout_any_alignment(orc, src_off, dst_off, fmt, ls, ld):
    banner(f"sf_convert offsets {src_off}/{dst_off} fmt={fmt} {ls}->{ld}")
    _run(orc, 259, 11, fmt, ls, ld, src_off, dst_off, seed=5)


# the weight scales of the benchmarked GEMMs: (N, K) of the MXFP4 prefill pair and the NVFP4 chain
@pytest.mark.parametrize("rows,K,fmt", [(14336, 4096, 1), (4096, 14336, 1), (17408, 5120, 0), (5120, 17408, 0)])
def test_relayout_weight_scales_full_size(orc, rows, K, fmt):
    banner(f"sf_convert full size rows={rows} K={K} fmt={fmt}")
    _run(orc, rows, K // BLOCK[fmt], fmt, SWZ, TIL, seed=K)


@pytest.mark.parametrize("M,N,K,fmt", [(41, 1536, 6144, 1), (300, 1000, 2048, 0), (2048, 768, 1536, 1),
                                       (129, 384, 1024, 0)])
def test_gemm_on_converted_128x4_scales(M, N, K, fmt):
    """Both operands quantized with 128 x 4 scales, as the FlashRT page's
    contract hands them over, converted to TILED: the same scale bytes as
    quantizing into TILED directly, hence the same GEMM output bit for bit."""
    banner(f"gemm on converted 128x4 scales M={M} N={N} K={K} fmt={fmt}")
    a, b = dev_bf16(synth.activation(M, K, M + K, outliers=True)), dev_bf16(synth.weight(N, K, N + K))
    pa, sa_swz = lb.lowbit_quantize(a, fmt, SWZ)
    pb, sb_swz = lb.lowbit_quantize(b, fmt, SWZ)
    _, sa_til = lb.lowbit_quantize(a, fmt, TIL)
    _, sb_til = lb.lowbit_quantize(b, fmt, TIL)
    sa = lb.lowbit_sf_convert(sa_swz, M, K, fmt, SWZ, TIL)
    sb = lb.lowbit_sf_convert(sb_swz, N, K, fmt, SWZ, TIL)
    torch.cuda.synchronize()
    assert torch.equal(sa, sa_til) and torch.equal(sb, sb_til)
    got = lb.lowbit_gemm_bf16(pa, pb, sa, sb, fmt=fmt, sfa_layout=TIL, sfb_layout=TIL)
    ref = lb.lowbit_gemm_bf16(pa, pb, sa_til, sb_til, fmt=fmt, sfa_layout=TIL, sfb_layout=TIL)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(got), host_bits(ref))


def test_fp8_output_scales_feed_an_mxfp8_operand():
    """The FP8-output GEMM's 128 x 4 scales, converted to LINEAR, are the
    bytes its LINEAR output carries, and take the place of an MXFP8 operand's
    scales."""
    M, N, K = 300, 512, 1024
    banner(f"fp8 out 128x4 -> LINEAR M={M} N={N} K={K}")
    a, b = dev_bf16(synth.activation(M, K, 3)), dev_bf16(synth.weight(N, K, 4))
    pa, sa = lb.lowbit_quantize(a, lb.MXFP8, LIN)
    pb, sb = lb.lowbit_quantize(b, lb.MXFP8, LIN)
    q_lin, s_lin = lb.lowbit_gemm_fp8(pa, pb, sa, sb, out_layout=LIN)
    q_swz, s_swz = lb.lowbit_gemm_fp8(pa, pb, sa, sb, out_layout=SWZ)
    s_conv = lb.lowbit_sf_convert(s_swz, M, N, lb.MXFP8, SWZ, LIN)
    torch.cuda.synchronize()
    assert torch.equal(q_lin, q_swz) and torch.equal(s_conv, s_lin)
    # (M, N) as the A operand of a second MXFP8 GEMM against a (64, N) weight
    w = dev_bf16(synth.weight(64, N, 6))
    pw, sw = lb.lowbit_quantize(w, lb.MXFP8, LIN)
    got = lb.lowbit_gemm_bf16(q_swz, pw, s_conv, sw, fmt=lb.MXFP8)
    ref = lb.lowbit_gemm_bf16(q_lin, pw, s_lin, sw, fmt=lb.MXFP8)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(got), host_bits(ref))
