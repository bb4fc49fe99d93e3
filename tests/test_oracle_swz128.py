"""Pins of the oracle's 128 x 4 swizzled scale layout (SWZ128, the add + RMSNorm
+ FP4 producer page's swizzled output): the offsets are a bijection onto the
used bytes, each 128-row x 4-block tile fills one 512-byte span, the 16 bytes at
16r of a tile are rows r, r+32, r+64, r+96 (four blocks each), and a quantized
tensor carries the same scale bytes as its LINEAR form with zero padding."""
import numpy as np
import pytest

from oracle import oracle as orc
from block_scaled_fp4_add_amd import synth

SWZ = orc.SWZ128


@pytest.mark.parametrize("rows", [1, 127, 128, 129, 300])
@pytest.mark.parametrize("nblk", [1, 3, 4, 5, 17])
def test_offsets_are_a_tiled_bijection(rows, nblk):
    fmt, B = orc.NVFP4, 16
    size = orc.sf_bytes(rows, nblk * B, fmt, SWZ)
    ktiles, mtiles = -(-nblk // 4), -(-rows // 128)
    assert size == mtiles * ktiles * 512
    offs = np.array([[orc.sf_offset(r, kb, nblk, fmt, SWZ) for kb in range(nblk)] for r in range(rows)])
    assert len(set(offs.ravel().tolist())) == rows * nblk
    assert offs.min() >= 0 and offs.max() < size
    for r in range(rows):
        for kb in range(nblk):
            t = (r // 128) * ktiles + kb // 4
            assert t * 512 <= offs[r, kb] < (t + 1) * 512


def test_sixteen_byte_groups_hold_four_rows():
    nblk = 8
    inv = {}
    for r in range(256):
        for kb in range(nblk):
            inv[orc.sf_offset(r, kb, nblk, orc.MXFP4, SWZ)] = (r, kb)
    for tile_r in range(2):
        for tile_k in range(2):
            base = (tile_r * 2 + tile_k) * 512
            for rr in range(32):
                got = [inv[base + 16 * rr + i] for i in range(16)]
                want = [(tile_r * 128 + rr + 32 * g, tile_k * 4 + j) for g in range(4) for j in range(4)]
                assert got == want


@pytest.mark.parametrize("fmt", [orc.NVFP4, orc.MXFP4, orc.NVFP4_B32])
def test_same_scales_as_linear_with_zero_padding(fmt):
    M, H = 150, 800 if fmt == orc.NVFP4 else 1120
    x, r, w = synth.producer_inputs(M, H, 9, outliers=True)
    args = (synth.bits(x), synth.bits(r), synth.bits(w), 1e-6)
    if fmt == orc.NVFP4_B32:
        with pytest.raises(ValueError):   # its scales are LINEAR only
            orc.add_rmsnorm_quant(*args, fmt, SWZ)
        return
    lin = orc.add_rmsnorm_quant(*args, fmt, orc.LINEAR)
    swz = orc.add_rmsnorm_quant(*args, fmt, SWZ)
    assert np.array_equal(lin["packed"], swz["packed"])
    nblk = H // orc.block_size(fmt)
    offs = np.array([[orc.sf_offset(m, kb, nblk, fmt, SWZ) for kb in range(nblk)] for m in range(M)])
    assert np.array_equal(swz["sf"][offs], lin["sf"].reshape(M, nblk))
    used = np.zeros(swz["sf"].size, bool)
    used[offs.ravel()] = True
    assert not np.any(swz["sf"][~used])
