"""Device checks of the hardware conversions the exactness of the HIP path
rests on, and the bf16 / fp16 producer gate.

* E2M1 encoding (v_cvt_scalef32_pk_fp4_f32 at unit scale): every bf16 value
  of magnitude below 8 goes through the MXFP4 quantizer in blocks whose
  first element is 6, so the block's UE8M0 scale is 2^0 and each value is
  rounded as it is; the codes must equal the oracle's round-to-nearest-even,
  saturating, sign-keeping encoder's.
* FP4 times block scale inside the GEMM: a GEMM whose B operand is one-hot
  (B row n is the code for 1.0 at column n, unit scale) reads every A element
  back, A holding all sixteen codes under every finite E4M3 scale byte
  (NVFP4: v_cvt_scalef32_pk_f16_fp4 plus the mantissa multiply) or under a
  wide range of UE8M0 bytes (MXFP4: the scaled MFMA).  Every such product
  has at most six significant bits and lies inside bf16's normal range, so
  the bf16 output must equal the dequantized value exactly.
* The FlashRT README's validation gate: the bf16 quantizer entry must give
  the same bytes as the fp16 entry on the same values, at the decode widths
  5120, 6144 and 17408.
"""
import numpy as np
import pytest
import torch

import block_scaled_fp4_add_amd as lb
from block_scaled_fp4_add_amd import synth

from .gpu_util import banner, dev_bf16, dev_f32, dev_u8, host_f64, host_u8

pytestmark = pytest.mark.gpu


def test_e2m1_encoding_exhaustive(orc):
    pos = np.arange(0, 0x4100, dtype=np.uint16)                 # bf16 bit patterns of 0 .. just below 8
    vals = np.concatenate([pos, pos | 0x8000]).astype(np.uint16)
    per = 31
    nblk = ((vals.size + per - 1) // per + 15) // 16 * 16       # rows of 16 blocks (512 elements)
    blocks = np.zeros((nblk, 32), np.uint16)
    blocks[:, 0] = 0x40C0                                       # 6.0: floor(log2 amax) = 2, scale 2^0
    flat = np.concatenate([vals, np.zeros(nblk * per - vals.size, np.uint16)])
    blocks[:, 1:] = flat.reshape(nblk, per)
    x = synth.from_bits(blocks.reshape(-1, 32 * 16))
    ref_p, ref_s = orc.quantize(synth.bits(x), orc.MXFP4, orc.LINEAR)
    assert (ref_s == 127).all()
    p, s = lb.lowbit_quantize(dev_bf16(x), lb.MXFP4, lb.LINEAR)
    torch.cuda.synchronize()
    banner(f"e2m1 exhaustive: {vals.size} values")
    assert np.array_equal(host_u8(s), ref_s)
    assert np.array_equal(host_u8(p), ref_p)


def _one_hot_b(orc, N, K, fmt):
    """B (N, K): row n holds 1.0 (code 0x2) at column n, zero elsewhere, unit scales."""
    codes = np.zeros((N, K), np.uint8)
    codes[np.arange(N), np.arange(N)] = 0x2
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    unit = 0x38 if fmt == orc.NVFP4 else 127
    B = 16 if fmt == orc.NVFP4 else 32
    return packed, unit, B


def _scaled_rows(orc, scale_bytes, K, fmt, layout):
    """A rows: block 2j holds codes 0..15 in order, block 2j+1 in reverse (for
    NVFP4 a block is sixteen elements, so each block holds every code); every
    block of row i carries scale byte scale_bytes[i]."""
    rows = scale_bytes.size
    B = 16 if fmt == orc.NVFP4 else 32
    pattern = np.concatenate([np.arange(16), np.arange(15, -1, -1)]).astype(np.uint8)
    codes = np.tile(pattern, (rows, K // 32))
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    nblk = K // B
    sf = np.zeros(orc.sf_bytes(rows, K, fmt, layout), np.uint8)
    for i in range(rows):
        for kb in range(nblk):
            sf[orc.sf_offset(i, kb, nblk, fmt, layout)] = scale_bytes[i]
    return packed, sf


def _gemm_reads_back(orc, fmt, scale_bytes, K, layout, variant):
    rows = scale_bytes.size
    a, sfa = _scaled_rows(orc, scale_bytes, K, fmt, layout)
    b, unit, B = _one_hot_b(orc, K, K, fmt)
    sfb = np.full(orc.sf_bytes(K, K, fmt, orc.LINEAR), unit, np.uint8)
    _, want = orc.dequantize(a, sfa, rows, K, fmt, layout)       # the exact products (binary64)
    out = torch.empty((rows, K), dtype=torch.bfloat16, device="cuda")
    # the decode schedule holds at most 128 rows: run it over slices
    step = 128 if variant == 0 else rows
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        a_s, sfa_s = _scaled_rows(orc, scale_bytes[r0:r1], K, fmt, layout)
        lb.lowbit_gemm_bf16(dev_u8(a_s), dev_u8(b), dev_u8(sfa_s), dev_u8(sfb), fmt=fmt, sfa_layout=layout,
                            sfb_layout=orc.LINEAR, alpha=1.0, out=out[r0:r1], variant=variant)
    torch.cuda.synchronize()
    # compared as values: a sum that starts from +0 cannot reproduce the sign
    # of a zero product, and the contract does not ask it to
    got = host_f64(out)
    bad = np.argwhere(got != want)
    assert bad.size == 0, [(int(i), int(k), hex(int(scale_bytes[i])), float(got[i, k]), float(want[i, k]))
                           for i, k in bad[:8]]
    return got


@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("variant", [0, 1])
def test_nvfp4_products_exhaustive(orc, layout, variant):
    """Every E2M1 code times every finite E4M3 scale byte, both signs of the
    scale (0x00-0x7E, 0x80-0xFE), read back through the GEMM."""
    sb = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], np.uint8)
    banner(f"nvfp4 products: {sb.size} scale bytes x 16 codes, layout={layout} variant={variant}")
    got = _gemm_reads_back(orc, orc.NVFP4, sb, 32, layout, variant)
    assert np.count_nonzero(got) > 0


@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("variant", [0, 1])
def test_mxfp4_products_scale_range(orc, layout, variant):
    """Every E2M1 code under UE8M0 bytes 2..252 (2^-125 .. 2^125: every
    product a normal bf16 number), read back through the scaled MFMA."""
    sb = np.arange(2, 253, dtype=np.uint8)
    banner(f"mxfp4 products: {sb.size} scale bytes x 16 codes, layout={layout} variant={variant}")
    got = _gemm_reads_back(orc, orc.MXFP4, sb, 64, layout, variant)
    assert np.count_nonzero(got) > 0


@pytest.mark.parametrize("K", [5120, 6144, 17408])
@pytest.mark.parametrize("rows", [1, 41])
@pytest.mark.parametrize("fmt,layout", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_bf16_entry_matches_fp16_entry(orc, K, rows, fmt, layout):
    """lowbit_quantize(x) and lowbit_quantize_fp16(x as fp16) write the same
    bytes (values drawn in bf16, those below 2^-14 set to zero, so that the
    fp16 copy holds them exactly), and both equal the oracle's."""
    x = synth.activation(rows, K, seed=rows * 7 + K, outliers=True)
    # bf16 values below fp16's normal range (2^-14) lose bits in fp16: zero them
    x = torch.where(x.abs() < 2.0 ** -14, torch.zeros_like(x), x)
    xh = x.to(torch.float16)
    assert torch.equal(xh.float(), x.float()), "the fp16 copy must hold the bf16 values exactly"
    gs = 2.5 if fmt == 0 else None
    p16, s16 = lb.lowbit_quantize(dev_bf16(x), fmt, layout, global_scale=dev_f32(gs) if gs else None)
    ph, sh = lb.lowbit_quantize_fp16(xh.to("cuda"), fmt, layout, global_scale=dev_f32(gs) if gs else None)
    torch.cuda.synchronize()
    assert torch.equal(p16, ph) and torch.equal(s16, sh)
    ref_p, ref_s = orc.quantize(synth.bits(x), fmt, layout, gs=gs or 1.0)
    assert np.array_equal(host_u8(p16), ref_p) and np.array_equal(host_u8(s16), ref_s)
