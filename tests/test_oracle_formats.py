"""Pins of the oracle's element formats and scale layouts against things other
than the oracle: the format definitions enumerated independently here with
exact rationals, torch's own bf16 / float8_e4m3fn conversions, hand-worked
blocks (tests/golden/hand_blocks.json) and layout invariants."""
import json
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --- independent enumerations of the formats (from bit fields, exact) ---------------------

def e2m1_exact(code):
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    v = Fraction(m, 2) if e == 0 else Fraction(2 + m, 2) * Fraction(2) ** (e - 1)
    return -v if s else v


def e4m3_exact(b):
    s, e, m = (b >> 7) & 1, (b >> 3) & 15, b & 7
    if e == 15 and m == 7:
        return None
    v = Fraction(m, 8) * Fraction(1, 64) if e == 0 else Fraction(8 + m, 8) * Fraction(2) ** (e - 7)
    return -v if s else v


def brute_nearest(a: Fraction, grid):
    """grid: list of (value, code) with value >= 0; nearest, ties -> even code;
    beyond the largest value saturate."""
    best = None
    for val, code in grid:
        d = abs(a - val)
        if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
            best = (d, code)
    return best[1]


E2M1_GRID = [(e2m1_exact(c), c) for c in range(8)]
E4M3_GRID = [(e4m3_exact(c), c) for c in range(0x7F)]


def f32(x):
    return float(np.float32(x))


def next_up(x):
    return float(np.nextafter(np.float32(x), np.float32(np.inf)))


def next_down(x):
    return float(np.nextafter(np.float32(x), np.float32(-np.inf)))


def test_e2m1_decode_table(orc):
    for c in range(16):
        assert orc.e2m1_value(c) == float(e2m1_exact(c))
        assert math.copysign(1.0, orc.e2m1_value(c)) == (-1.0 if c & 8 else 1.0)


def test_e2m1_round_trip(orc):
    for c in range(16):
        assert orc.e2m1_encode(orc.e2m1_value(c)) == c


def test_e2m1_midpoints_and_neighbours(orc):
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    for m in mids:
        for v in (next_down(m), m, next_up(m)):
            for s in (1.0, -1.0):
                want = brute_nearest(abs(Fraction(v)), E2M1_GRID) | (8 if s < 0 else 0)
                assert orc.e2m1_encode(s * v) == want, (s * v)


def test_e2m1_sweep_against_brute_force(orc):
    rng = np.random.default_rng(7)
    vals = np.concatenate([
        rng.uniform(-8, 8, 4000),
        np.ldexp(rng.uniform(0.5, 1.0, 2000), rng.integers(-30, 4, 2000)) * rng.choice([-1, 1], 2000),
        np.array([0.0, -0.0, 6.0, -6.0, 7.99, 100.0, -1e30, 1e-45]),
    ]).astype(np.float32)
    for v in vals:
        sign = 8 if math.copysign(1.0, float(v)) < 0 else 0
        want = brute_nearest(abs(Fraction(float(v))), E2M1_GRID) | sign
        assert orc.e2m1_encode(float(v)) == want, float(v)


def test_e4m3_decode_table(orc):
    for b in range(256):
        want = e4m3_exact(b)
        got = orc.e4m3_value(b)
        if want is None:
            assert math.isnan(got)
        else:
            assert got == float(want)
    assert orc.e4m3_value(0x7E) == 448.0  # FLOAT8_E4M3_MAX on the FlashInfer page


def test_e4m3_round_trip(orc):
    for b in range(256):
        if (b & 0x7F) == 0x7F:
            continue
        assert orc.e4m3_encode(orc.e4m3_value(b)) == b


def test_e4m3_midpoints_against_brute_force(orc):
    for c in range(0x7E):
        lo, hi = e4m3_exact(c), e4m3_exact(c + 1)
        mid = float((lo + hi) / 2)
        for v in (next_down(mid), mid, next_up(mid)):
            want = brute_nearest(Fraction(v), E4M3_GRID)
            assert orc.e4m3_encode(v) == want, v
    # saturation above the largest finite value
    for v in (448.0, 449.0, 464.0, 1e6, float("inf")):
        assert orc.e4m3_encode(v) == 0x7E


def test_e4m3_against_torch(orc):
    rng = np.random.default_rng(11)
    vals = np.concatenate([np.ldexp(rng.uniform(1.0, 2.0, 5000), rng.integers(-12, 9, 5000)),
                           rng.uniform(0, 460, 2000)]).astype(np.float32)
    vals = vals[vals < 464.0]  # torch's conversion turns larger values into NaN instead of saturating
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([orc.e4m3_encode(float(v)) for v in vals], dtype=np.uint8)
    assert np.array_equal(got, ref)


def test_ue8m0_values(orc):
    for b in range(255):
        assert orc.ue8m0_value(b) == math.ldexp(1.0, b - 127)
    assert math.isnan(orc.ue8m0_value(255))


def test_bf16_rounding_against_torch(orc):
    rng = np.random.default_rng(3)
    vals = np.concatenate([rng.standard_normal(5000) * 10,
                           np.ldexp(rng.uniform(1, 2, 2000), rng.integers(-130, 120, 2000))])
    vals = vals.astype(np.float32)
    # exact ties: low half 0x8000 with both parities of the kept bit
    ties = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x40490000 | 0x8000], dtype=np.uint32).view(np.float32)
    vals = np.concatenate([vals, ties])
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.f32_to_bf16(float(v)) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, ref)
    for b in (0x3F80, 0xC2F7, 0x0001, 0x7F7F):
        assert orc.bf16_to_f32(b) == struct.unpack("<f", struct.pack("<I", b << 16))[0]


# --- scale layouts ---------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("rows,nblk", [(1, 8), (32, 8), (41, 48), (64, 160), (33, 13), (7, 3)])
def test_tiled_layout_is_a_bijection(orc, fmt, rows, nblk):
    B = 16 if fmt == 0 else 32
    size = orc.sf_bytes(rows, nblk * B, fmt, 1)
    assert size == ((rows + 31) // 32) * ((nblk + 7) // 8) * 256
    seen = set()
    for r in range(rows):
        for kb in range(nblk):
            off = orc.sf_offset(r, kb, nblk, fmt, 1)
            assert 0 <= off < size
            assert off not in seen
            seen.add(off)


def test_tiled_layout_mxfp4_word_holds_the_blocks_of_one_lane(orc):
    """MXFP4: word h*32 + r of a group holds blocks 2h, 2h+1, 2h+4, 2h+5 of
    row r in bytes 0..3 (the four 32-blocks one MFMA lane half consumes over
    256 elements)."""
    nblk = 24
    for r in (0, 5, 31, 32, 63):
        for t in range(nblk // 8):
            for h in (0, 1):
                blocks = [8 * t + 2 * h, 8 * t + 2 * h + 1, 8 * t + 2 * h + 4, 8 * t + 2 * h + 5]
                offs = [orc.sf_offset(r, kb, nblk, 1, 1) for kb in blocks]
                assert offs[0] % 4 == 0 and offs == [offs[0] + j for j in range(4)]
                assert (offs[0] % 256) // 4 == h * 32 + r % 32
    # a 32-row x 8-block tile is 256 contiguous bytes, rows adjacent per word
    assert orc.sf_offset(0, 0, 8, 1, 1) == 0
    assert orc.sf_offset(1, 0, 8, 1, 1) == 4
    assert orc.sf_offset(0, 2, 8, 1, 1) == 128
    assert orc.sf_offset(0, 4, 8, 1, 1) == 2
    assert orc.sf_offset(31, 7, 8, 1, 1) == 255
    assert orc.sf_offset(32, 0, 8, 1, 1) == 256
    assert orc.sf_offset(0, 8, 16, 1, 1) == 256


def test_tiled_layout_nvfp4_word_holds_the_blocks_of_one_lane(orc):
    """NVFP4: word c*32 + r of a group holds blocks 4c .. 4c+3 of row r in
    bytes 0..3 (the four 16-blocks one lane half reads in a 128-element
    stage)."""
    nblk = 24
    for r in (0, 5, 31, 32, 63):
        for t in range(nblk // 8):
            for c in (0, 1):
                offs = [orc.sf_offset(r, 8 * t + 4 * c + j, nblk, 0, 1) for j in range(4)]
                assert offs[0] % 4 == 0 and offs == [offs[0] + j for j in range(4)]
                assert (offs[0] % 256) // 4 == c * 32 + r % 32
    assert orc.sf_offset(0, 0, 8, 0, 1) == 0
    assert orc.sf_offset(0, 3, 8, 0, 1) == 3
    assert orc.sf_offset(0, 4, 8, 0, 1) == 128
    assert orc.sf_offset(1, 0, 8, 0, 1) == 4
    assert orc.sf_offset(31, 7, 8, 0, 1) == 255
    assert orc.sf_offset(32, 0, 8, 0, 1) == 256
    assert orc.sf_offset(0, 8, 16, 0, 1) == 256


def test_linear_layout(orc):
    assert orc.sf_bytes(5, 64, 0, 0) == 20
    assert orc.sf_offset(3, 2, 4, 1, 0) == 14
    assert orc.sf_offset(3, 2, 4, 0, 0) == 14


# --- hand-worked blocks ------------------------------------------------------------------------

def _hand_blocks():
    with open(os.path.join(GOLDEN, "hand_blocks.json")) as f:
        return json.load(f)["blocks"]


@pytest.mark.parametrize("blk", _hand_blocks(), ids=lambda b: b["name"])
def test_hand_worked_blocks(orc, blk):
    fmt = orc.NVFP4 if blk["fmt"] == "nvfp4" else orc.MXFP4
    x = torch.tensor(blk["x"], dtype=torch.float32)
    xb = x.to(torch.bfloat16)
    assert torch.equal(xb.float(), x), "fixture values must be bf16-exact"
    bits = xb.view(torch.int16).numpy().view(np.uint16).reshape(1, -1)
    for layout in (orc.LINEAR, orc.TILED):
        packed, sf = orc.quantize(bits, fmt, layout, gs=blk["gs"])
        assert sf[orc.sf_offset(0, 0, 1, fmt, layout)] == blk["scale_byte"]
        codes = np.empty(bits.shape[1], np.uint8)
        codes[0::2] = packed[0] & 15
        codes[1::2] = packed[0] >> 4
        assert codes.tolist() == blk["codes"]
        if "packed" in blk:
            assert packed[0].tolist() == blk["packed"]
        if layout == orc.TILED:
            nz = np.flatnonzero(sf)
            assert set(nz.tolist()) <= {0}, "tiled padding must be zero"


# --- fp16 (the producer's and quantizer's other input format) -------------------------------

def test_f16_widening_exhaustive_against_numpy(orc):
    """Every binary16 bit pattern widens exactly as numpy's float16 does."""
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float32)
    got = np.array([orc.f16_to_f32(int(b)) for b in pats], dtype=np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f16_rounding_against_numpy(orc):
    """fp32 -> fp16 nearest-even against numpy's conversion: every finite fp16
    value, the midpoints between neighbours (exact ties, both parities), one
    fp32 ulp either side of them, the overflow boundary and random values
    from the subnormal range to beyond 65504."""
    fin = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float32)
    mids = ((fin[:-1].astype(np.float64) + fin[1:].astype(np.float64)) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (fin[:-1].astype(np.float64) + fin[1:]) / 2)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    rng = np.random.default_rng(11)
    rnd = np.ldexp(rng.uniform(1, 2, 20000), rng.integers(-26, 18, 20000)).astype(np.float32)
    edge = np.array([65504.0, 65519.996, 65520.0, 65536.0, 1e6, np.inf, 2.0 ** -24, 2.0 ** -25,
                     3 * 2.0 ** -26, 2.0 ** -26, 2.0 ** -14 - 2.0 ** -25], dtype=np.float32)
    vals = np.concatenate([fin, mids, up, dn, rnd, edge])
    vals = np.concatenate([vals, -vals])
    with np.errstate(over="ignore"):   # the overflow cases are meant to become infinities
        ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([orc.f32_to_f16(float(v)) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, ref)
