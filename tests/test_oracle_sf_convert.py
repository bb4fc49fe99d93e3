"""Pins of the oracle's scale relayout (orc_sf_convert): the FlashRT page's GEMM
takes its operand scales in the 128 x 4 layout ("Tensor Contract"), the
library's GEMM in TILED or LINEAR, and the relayout moves each (row, block)
byte between them.  Pinned by
  - byte positions written out by hand from the layout definitions (the
    library header's text: 128 x 4 tiles at 16 (r % 32) + 4 ((r % 128) / 32) +
    kb % 4; TILED words per format), not through the oracle's offset function;
  - the quantizer: quantizing in layout A and converting to B gives the bytes
    that quantizing in B gives, padding included, for every ordered pair;
  - the FP8-output GEMM: its 128 x 4 scales converted to LINEAR are its LINEAR
    scales;
  - the source's padding bytes are never read, and A -> B -> A is the identity."""
import itertools

import numpy as np
import pytest

from oracle import oracle as orc
from block_scaled_fp4_add_amd import synth

LIN, TIL, SWZ = orc.LINEAR, orc.TILED, orc.SWZ128


def _linear(rows, nblk, seed):
    return np.random.default_rng(seed).integers(1, 256, size=rows * nblk, dtype=np.uint8)


def test_hand_positions_linear_to_swz128():
    # rows 0, 1, 2, 33, 130 of a 131-row, 6-block operand (NVFP4, k = 96)
    rows, nblk = 131, 6
    lin = _linear(rows, nblk, 1)
    out = orc.sf_convert(lin, rows, nblk * 16, orc.NVFP4, LIN, SWZ)
    assert out.size == 2 * 2 * 512            # 2 row tiles x 2 block tiles
    L = lin.reshape(rows, nblk)
    # row tile 0, block tile 0: row r < 32 at 16 r, row 32 + r at 16 r + 4
    assert out[0:4].tolist() == L[0, 0:4].tolist()
    assert out[16:20].tolist() == L[1, 0:4].tolist()
    assert out[32:36].tolist() == L[2, 0:4].tolist()
    assert out[16 + 4:16 + 8].tolist() == L[33, 0:4].tolist()
    # block tile 1 of row tile 0 starts at 512: blocks 4, 5 and two zero pads
    assert out[512:516].tolist() == [L[0, 4], L[0, 5], 0, 0]
    # row tile 1 (rows 128..130) starts at 1024; row 130 is r % 32 = 2, group 0
    assert out[1024 + 32:1024 + 36].tolist() == L[130, 0:4].tolist()
    assert out[1024 + 48:1024 + 52].tolist() == [0, 0, 0, 0]   # row 131: padding
    assert out[1024 + 512 + 32:1024 + 512 + 36].tolist() == [L[130, 4], L[130, 5], 0, 0]
    # every byte not named by a (row, block) is zero
    assert int(np.count_nonzero(out)) == rows * nblk


def test_hand_positions_linear_to_tiled():
    rows, nblk = 33, 8
    lin = _linear(rows, nblk, 2)
    L = lin.reshape(rows, nblk)
    # NVFP4: word c * 32 + r holds blocks 4c .. 4c + 3 of row r
    nv = orc.sf_convert(lin, rows, nblk * 16, orc.NVFP4, LIN, TIL)
    assert nv.size == 2 * 256
    assert nv[4 * 5:4 * 5 + 4].tolist() == L[5, 0:4].tolist()
    assert nv[4 * (32 + 5):4 * (32 + 5) + 4].tolist() == L[5, 4:8].tolist()
    assert nv[256:260].tolist() == L[32, 0:4].tolist()        # row 32 opens group 1
    # MXFP4: word h * 32 + r holds blocks 2h, 2h + 1, 2h + 4, 2h + 5 of row r
    mx = orc.sf_convert(lin, rows, nblk * 32, orc.MXFP4, LIN, TIL)
    assert mx[4 * 7:4 * 7 + 4].tolist() == [L[7, 0], L[7, 1], L[7, 4], L[7, 5]]
    assert mx[4 * 39:4 * 39 + 4].tolist() == [L[7, 2], L[7, 3], L[7, 6], L[7, 7]]
    assert int(np.count_nonzero(nv)) == int(np.count_nonzero(mx)) == rows * nblk


@pytest.mark.parametrize("fmt,rows,K", [(orc.NVFP4, 37, 80), (orc.NVFP4, 130, 272),
                                        (orc.MXFP4, 37, 160), (orc.MXFP4, 129, 544)])
def test_matches_the_quantizer_in_every_layout(fmt, rows, K):
    x = synth.bits(synth.activation(rows, K, 11, outliers=True))
    sf = {lay: orc.quantize(x, fmt, lay)[1] for lay in (LIN, TIL, SWZ)}
    for a, b in itertools.permutations((LIN, TIL, SWZ), 2):
        assert np.array_equal(orc.sf_convert(sf[a], rows, K, fmt, a, b), sf[b]), (a, b)


def test_fp8_output_scales_swz128_to_linear():
    M, N, K = 70, 96, 64
    a = synth.bits(synth.activation(M, K, 5))
    b = synth.bits(synth.weight(N, K, 5))
    (pa, sa), (pb, sb) = orc.quantize(a, orc.MXFP8, LIN), orc.quantize(b, orc.MXFP8, LIN)
    args = (pa, pb, sa, sb, M, N, K, orc.MXFP8, LIN, LIN, 1.0)
    lin = orc.gemm_fp8_out(*args, LIN)[1]
    swz = orc.gemm_fp8_out(*args, SWZ)[1]
    assert np.array_equal(orc.sf_convert(swz, M, N, orc.MXFP8, SWZ, LIN), lin)
    assert np.array_equal(orc.sf_convert(lin, M, N, orc.MXFP8, LIN, SWZ), swz)


@pytest.mark.parametrize("fmt", [orc.NVFP4, orc.MXFP4])
def test_source_padding_is_not_read_and_round_trip(fmt):
    rows, nblk = 45, 11
    K = nblk * orc.block_size(fmt)
    lin = _linear(rows, nblk, 3)
    for lay in (TIL, SWZ):
        clean = orc.sf_convert(lin, rows, K, fmt, LIN, lay)
        dirty = clean.copy()
        dirty[clean == 0] = 0xEE           # every padding byte (data bytes are nonzero)
        assert np.array_equal(orc.sf_convert(dirty, rows, K, fmt, lay, LIN), lin)
        other = SWZ if lay == TIL else TIL
        there = orc.sf_convert(dirty, rows, K, fmt, lay, other)
        assert np.array_equal(orc.sf_convert(there, rows, K, fmt, other, lay), clean)
