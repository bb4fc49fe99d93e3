"""Pins of the oracle's block-scaled GEMM and its epilogues against: exact
rational brute force on tiny shapes (decoding the nibbles and scale bytes from
their bit fields here, independently), closed forms (all-ones operands,
one-hot rows, a scale byte raised by one), a K=32 block worked by hand, and
math.erf for the GELU epilogue."""
import math
from fractions import Fraction

import numpy as np
import pytest

from block_scaled_fp4_add_amd import synth


def e2m1_exact(code):
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    v = Fraction(m, 2) if e == 0 else Fraction(2 + m, 2) * Fraction(2) ** (e - 1)
    return -v if s else v


def scale_exact(fmt, b):
    if fmt == 1:
        return Fraction(2) ** (int(b) - 127)
    e, m = (b >> 3) & 15, b & 7
    return Fraction(m, 8) * Fraction(1, 64) if e == 0 else Fraction(8 + m, 8) * Fraction(2) ** (e - 7)


def dequant_exact(packed, sf, rows, K, fmt, layout, orc):
    B = 16 if fmt == 0 else 32
    out = []
    for r in range(rows):
        row = []
        for k in range(K):
            byte = int(packed[r, k // 2])
            code = byte & 15 if k % 2 == 0 else byte >> 4
            sb = int(sf[orc.sf_offset(r, k // B, K // B, fmt, layout)])
            row.append(e2m1_exact(code) * scale_exact(fmt, sb))
        out.append(row)
    return out


def random_operand(rng, rows, K, fmt, orc, layout):
    """Random packed codes and random (moderate) scale bytes."""
    B = 16 if fmt == 0 else 32
    packed = rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)
    sf = np.zeros(orc.sf_bytes(rows, K, fmt, layout), np.uint8)
    for r in range(rows):
        for kb in range(K // B):
            sb = rng.integers(118, 136) if fmt == 1 else rng.integers(0x08, 0x70)
            sf[orc.sf_offset(r, kb, K // B, fmt, layout)] = sb
    return packed, sf


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (3, 2, 64), (4, 3, 128), (2, 4, 96)])
def test_gemm_brute_force_exact(orc, fmt, M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K + fmt)
    la, lb = orc.LINEAR, orc.TILED
    a, sfa = random_operand(rng, M, K, fmt, orc, la)
    b, sfb = random_operand(rng, N, K, fmt, orc, lb)
    A = dequant_exact(a, sfa, M, K, fmt, la, orc)
    Bm = dequant_exact(b, sfb, N, K, fmt, lb, orc)
    alpha = 0.75
    ref, l1 = orc.gemm(a, b, sfa, sfb, M, N, K, fmt, la, lb, alpha=alpha)
    for m in range(M):
        for n in range(N):
            exact = Fraction(alpha) * sum(A[m][k] * Bm[n][k] for k in range(K))
            absum = Fraction(alpha) * sum(abs(A[m][k] * Bm[n][k]) for k in range(K))
            assert abs(Fraction(ref[m, n]) - exact) <= absum * Fraction(1, 2 ** 50)
            assert abs(Fraction(l1[m, n]) - absum) <= absum * Fraction(1, 2 ** 50)


def test_gemm_all_ones_closed_form(orc):
    for fmt, unit in ((1, 127), (0, 0x38)):
        M, N, K = 3, 5, 256
        a = np.full((M, K // 2), 0x22, np.uint8)  # code 2 = 1.0 in both nibbles
        b = np.full((N, K // 2), 0x22, np.uint8)
        sfa = np.full(orc.sf_bytes(M, K, fmt, 0), unit, np.uint8)
        sfb = np.full(orc.sf_bytes(N, K, fmt, 0), unit, np.uint8)
        ref, l1 = orc.gemm(a, b, sfa, sfb, M, N, K, fmt, 0, 0, alpha=0.5)
        assert np.all(ref == 0.5 * K) and np.all(l1 == 0.5 * K)


def test_gemm_one_hot_selects_row(orc):
    rng = np.random.default_rng(1)
    M, N, K, fmt = 2, 4, 128, 1
    b, sfb = random_operand(rng, N, K, fmt, orc, 1)
    Bm = dequant_exact(b, sfb, N, K, fmt, 1, orc)
    a = np.zeros((M, K // 2), np.uint8)
    a[0, 37 // 2] = 0x2 << 4       # element 37 (odd -> high nibble) = 1.0
    a[1, 64 // 2] = 0xC            # element 64 = -2.0
    sfa = np.full(orc.sf_bytes(M, K, fmt, 0), 127, np.uint8)
    ref, _ = orc.gemm(a, b, sfa, sfb, M, N, K, fmt, 0, 1)
    for n in range(N):
        assert ref[0, n] == float(Bm[n][37])
        assert ref[1, n] == float(-2 * Bm[n][64])


def test_gemm_scale_plus_one_doubles_block(orc):
    rng = np.random.default_rng(2)
    M, N, K, fmt = 2, 3, 128, 1
    a, sfa = random_operand(rng, M, K, fmt, orc, 0)
    b, sfb = random_operand(rng, N, K, fmt, orc, 0)
    ref0, _ = orc.gemm(a, b, sfa, sfb, M, N, K, fmt, 0, 0)
    A = dequant_exact(a, sfa, M, K, fmt, 0, orc)
    Bm = dequant_exact(b, sfb, N, K, fmt, 0, orc)
    sfa2 = sfa.copy()
    sfa2[orc.sf_offset(1, 2, K // 32, fmt, 0)] += 1  # row 1, block 2 (k 64..95)
    ref1, _ = orc.gemm(a, b, sfa2, sfb, M, N, K, fmt, 0, 0)
    assert np.array_equal(ref1[0], ref0[0])
    for n in range(N):
        blk = sum(A[1][k] * Bm[n][k] for k in range(64, 96))
        assert Fraction(ref1[1, n]) - Fraction(ref0[1, n]) == blk


def test_gemm_k32_by_hand(orc):
    # A: 6, -6, 0.5, 1.5 at scale 2 -> 12, -12, 1, 3 ; B: 1, 1, 2, -4 at scale 1/2 -> .5, .5, 1, -2
    # dot = 6 - 6 + 1 - 6 = -5
    a = np.zeros((1, 16), np.uint8)
    a[0, 0] = 0x7 | (0xF << 4)
    a[0, 1] = 0x1 | (0x3 << 4)
    b = np.zeros((1, 16), np.uint8)
    b[0, 0] = 0x2 | (0x2 << 4)
    b[0, 1] = 0x4 | (0xE << 4)
    sfa = np.array([128], np.uint8)
    sfb = np.array([126], np.uint8)
    ref, l1 = orc.gemm(a, b, sfa, sfb, 1, 1, 32, 1, 0, 0)
    assert ref[0, 0] == -5.0 and l1[0, 0] == 19.0  # |6|+|-6|+|1|+|-6|


def test_epilogues(orc):
    rng = np.random.default_rng(3)
    M, N, K, fmt = 3, 4, 64, 0
    a, sfa = random_operand(rng, M, K, fmt, orc, 0)
    b, sfb = random_operand(rng, N, K, fmt, orc, 0)
    bias = synth.bits(synth.bias(N, seed=3))
    res = synth.bits(synth.residual(M, N, seed=3))
    base, _ = orc.gemm(a, b, sfa, sfb, M, N, K, fmt, 0, 0, alpha=0.25)
    bf = np.array([orc.bf16_to_f32(int(v)) for v in bias])
    rf = np.array([[orc.bf16_to_f32(int(v)) for v in row] for row in res])
    got_b, _ = orc.gemm(a, b, sfa, sfb, M, N, K, fmt, 0, 0, alpha=0.25, epi=orc.EPI_BIAS, bias=bias)
    got_r, _ = orc.gemm(a, b, sfa, sfb, M, N, K, fmt, 0, 0, alpha=0.25, epi=orc.EPI_RESIDUAL,
                        residual=res)
    got_br, _ = orc.gemm(a, b, sfa, sfb, M, N, K, fmt, 0, 0, alpha=0.25,
                         epi=orc.EPI_BIAS_RESIDUAL, bias=bias, residual=res)
    got_g, _ = orc.gemm(a, b, sfa, sfb, M, N, K, fmt, 0, 0, alpha=0.25, epi=orc.EPI_BIAS_GELU,
                        bias=bias)
    assert np.array_equal(got_b, base + bf[None, :])
    assert np.array_equal(got_r, base + rf)
    assert np.array_equal(got_br, (base + bf[None, :]) + rf)
    t = base + bf[None, :]
    gelu = np.vectorize(lambda v: 0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0))))(t)
    assert np.allclose(got_g, gelu, rtol=1e-15, atol=1e-300)
    assert got_g.min() >= -0.17 and np.all(got_g[t > 5] > 0.99999 * t[t > 5])


def test_gemm_entries_match_full(orc):
    rng = np.random.default_rng(4)
    M, N, K = 5, 7, 96
    for fmt in (0, 1):
        a, sfa = random_operand(rng, M, K, fmt, orc, 1)
        b, sfb = random_operand(rng, N, K, fmt, orc, 0)
        full, l1 = orc.gemm(a, b, sfa, sfb, M, N, K, fmt, 1, 0, alpha=2.0)
        im = np.array([0, 4, 2, 3], np.int64)
        jn = np.array([6, 0, 3, 3], np.int64)
        got, gl1 = orc.gemm_entries(a, b, sfa, sfb, M, N, K, fmt, 1, 0, im, jn, alpha=2.0)
        assert np.array_equal(got, full[im, jn]) and np.array_equal(gl1, l1[im, jn])


def test_gelu_fp4_output_is_nvfp4_of_the_gelu(orc):
    """The FP4-out epilogue must equal: reference GELU values rounded to fp32,
    then the NVFP4 block rule along N (checked block by block)."""
    rng = np.random.default_rng(5)
    M, N, K = 3, 64, 128
    a, sfa = random_operand(rng, M, K, 0, orc, 0)
    b, sfb = random_operand(rng, N, K, 0, orc, 0)
    bias = synth.bits(synth.bias(N, seed=5))
    alpha = 1.0 / 4096
    ref, _ = orc.gemm(a, b, sfa, sfb, M, N, K, 0, 0, 0, alpha=alpha, epi=orc.EPI_BIAS_GELU, bias=bias)
    out = orc.gemm_gelu_fp4(a, b, sfa, sfb, M, N, K, 0, 0, 0, alpha, bias, 1.0, orc.TILED, diag=True)
    assert np.array_equal(out["y"], ref.astype(np.float32))
    codes = np.empty((M, N), np.uint8)
    codes[:, 0::2] = out["packed"] & 15
    codes[:, 1::2] = out["packed"] >> 4
    for m in range(M):
        for kb in range(N // 16):
            sb = int(out["sf"][orc.sf_offset(m, kb, N // 16, orc.NVFP4, orc.TILED)])
            y = out["y"][m, kb * 16:(kb + 1) * 16]
            assert np.array_equal(orc.encode_with_scale(y, 0, 1.0, sb), codes[m, kb * 16:(kb + 1) * 16])
            assert sb == orc.e4m3_encode(min(np.float32(np.abs(y).max()) / np.float32(6), 448.0))


# --- MXFP8 operands (E4M3 elements, UE8M0 32-blocks, LINEAR scales) -------------------------

def e4m3_exact(b):
    s, e, m = (b >> 7) & 1, (b >> 3) & 15, b & 7
    v = Fraction(m, 8) * Fraction(1, 64) if e == 0 else Fraction(8 + m, 8) * Fraction(2) ** (e - 7)
    return -v if s else v


def random_mxfp8(rng, rows, K):
    packed = rng.integers(0, 256, (rows, K), dtype=np.uint8)
    packed[(packed & 0x7F) == 0x7F] = 0x7E                      # no NaN codes
    sf = rng.integers(118, 136, rows * (K // 32), dtype=np.uint8)
    return packed, sf


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (3, 2, 64), (2, 4, 160)])
def test_gemm_mxfp8_brute_force_exact(orc, M, N, K):
    """MXFP8 GEMM against exact rationals decoded from the bit fields here."""
    rng = np.random.default_rng(M * 31 + N * 7 + K)
    a, sfa = random_mxfp8(rng, M, K)
    b, sfb = random_mxfp8(rng, N, K)
    A = [[e4m3_exact(int(a[m, k])) * Fraction(2) ** (int(sfa[m * (K // 32) + k // 32]) - 127) for k in range(K)]
         for m in range(M)]
    Bm = [[e4m3_exact(int(b[n, k])) * Fraction(2) ** (int(sfb[n * (K // 32) + k // 32]) - 127) for k in range(K)]
          for n in range(N)]
    alpha = 1.25
    ref, l1 = orc.gemm(a, b, sfa, sfb, M, N, K, orc.MXFP8, orc.LINEAR, orc.LINEAR, alpha=alpha)
    for m in range(M):
        for n in range(N):
            exact = Fraction(alpha) * sum(A[m][k] * Bm[n][k] for k in range(K))
            absum = Fraction(alpha) * sum(abs(A[m][k] * Bm[n][k]) for k in range(K))
            assert abs(Fraction(ref[m, n]) - exact) <= absum * Fraction(1, 2 ** 50)
            assert abs(Fraction(l1[m, n]) - absum) <= absum * Fraction(1, 2 ** 50)


def test_gemm_mxfp8_closed_forms(orc):
    """All elements 1.0 (0x38) at unit scale give alpha * K; raising one row's
    first scale byte by one adds exactly that block's contribution again."""
    M, N, K = 2, 3, 96
    a = np.full((M, K), 0x38, np.uint8)
    b = np.full((N, K), 0x38, np.uint8)
    sfa = np.full(M * 3, 127, np.uint8)
    sfb = np.full(N * 3, 127, np.uint8)
    ref, _ = orc.gemm(a, b, sfa, sfb, M, N, K, orc.MXFP8, orc.LINEAR, orc.LINEAR, alpha=0.5)
    assert np.all(ref == 0.5 * K)
    sfa[3] = 128                     # row 1, block 0: doubled
    ref, _ = orc.gemm(a, b, sfa, sfb, M, N, K, orc.MXFP8, orc.LINEAR, orc.LINEAR, alpha=1.0)
    assert np.all(ref[0] == K) and np.all(ref[1] == K + 32)
