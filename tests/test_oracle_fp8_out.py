"""Pins of the oracle's FP8-output GEMM epilogue (the vLLM fused_wo_a page,
FusedWoAKernel.device_kernel output epilogue: the reduced sum rounded to bf16,
a 32-column block maximum, an MX scale, E4M3 elements; the scale bytes in the
page's 128 x 4 layout or row-major) against hand-worked blocks and closed
forms."""
import numpy as np
import pytest

F8 = 2          # MXFP8 operands and output
LIN, SWZ = 0, 2


def e4m3(v):
    """The E4M3 code of an exactly representable value (by search of the grid)."""
    from oracle import oracle as orc
    c = orc.e4m3_encode(v)
    assert orc.e4m3_value(c) == v
    return c


def operands_from(rows):
    """MXFP8 operand (len(rows), K) from rows of (value, scale_byte) per
    32-element block: each row is a list of blocks, each block a dict
    {k: value} of exactly representable E4M3 values under that block's scale."""
    n = len(rows)
    nblk = len(rows[0])
    K = 32 * nblk
    packed = np.zeros((n, K), np.uint8)
    sf = np.zeros(n * nblk, np.uint8)
    for i, blocks in enumerate(rows):
        for b, (sbyte, elems) in enumerate(blocks):
            sf[i * nblk + b] = sbyte
            for k, v in elems.items():
                packed[i, 32 * b + k] = e4m3(v)
    return packed, sf, K


def test_bf16_rounding_comes_before_the_e4m3_rounding(orc):
    """Output 0 is exactly 1 + 2^-4 + 2^-10: bf16 holds 1.0625, an E4M3
    midpoint between 1.0 and 1.125, which rounds to the even code 0x38 (1.0);
    rounding the exact value straight to E4M3 would give 0x39.  Output 1 is
    300, so the block maximum keeps the scale at 2^0 (byte 127) and 300
    itself encodes as 288 (0x79)."""
    one = 127
    # A: one row, two blocks; block 1 scaled by 2^-5 holds 2^-5 (= 2^-10 in value)
    a, sfa, K = operands_from([[(one, {0: 1.0, 1: 0.0625, 3: 256.0, 4: 32.0, 5: 8.0, 6: 4.0}),
                                (one - 5, {0: 2.0 ** -5})]])
    # B: row 0 sums a[0] + a[1] + a[32]; row 1 sums a[3..6]; rows 2..31 zero
    brows = [[(one, {0: 1.0, 1: 1.0}), (one, {0: 1.0})],
             [(one, {3: 1.0, 4: 1.0, 5: 1.0, 6: 1.0}), (one, {})]] + [[(one, {}), (one, {})]] * 30
    b, sfb, _ = operands_from(brows)
    p, s, ref, _ = orc.gemm_fp8_out(a, b, sfa, sfb, 1, 32, K, F8, LIN, LIN, 1.0, LIN, diag=True)
    assert ref[0, 0] == 1 + 2 ** -4 + 2 ** -10 and ref[0, 1] == 300.0
    assert list(s) == [127]
    assert p[0, 0] == 0x38 and p[0, 1] == 0x79 and (p[0, 2:] == 0).all()


@pytest.mark.parametrize("layout", [LIN, SWZ])
def test_constant_output(orc, layout):
    """All-ones operands (code 0x38, unit scales) give alpha * K everywhere:
    alpha = 0.75, K = 256 -> 192, e = floor(log2 192) - 8 = -1 (byte 126),
    192 * 2 = 384 = 1.5 * 2^8 -> code 0x7C, in every block of either layout."""
    M, N, K = 5, 64, 256
    a = np.full((M, K), 0x38, np.uint8)
    b = np.full((N, K), 0x38, np.uint8)
    sfa = np.full(M * K // 32, 127, np.uint8)
    sfb = np.full(N * K // 32, 127, np.uint8)
    p, s = orc.gemm_fp8_out(a, b, sfa, sfb, M, N, K, F8, LIN, LIN, 0.75, layout)
    assert (p == 0x7C).all()
    used = np.array([orc.sf_offset(m, kb, N // 32, F8, layout) for m in range(M) for kb in range(N // 32)])
    assert (s[used] == 126).all()
    mask = np.ones(s.size, bool)
    mask[used] = False
    assert (s[mask] == 0).all()                 # 128 x 4 padding written zero


def test_zero_and_negative_blocks(orc):
    """A block of zero outputs gets scale byte 0 and zero codes; negating A
    keeps the scales and sets every code's sign bit."""
    M, N, K = 2, 64, 64
    rng = np.random.default_rng(1)
    a = rng.integers(0x30, 0x50, (M, K)).astype(np.uint8)     # positive E4M3 values
    b = rng.integers(0x30, 0x50, (N, K)).astype(np.uint8)
    b[32:] = 0                                                # outputs 32..63 are zero
    sfa = np.full(M * 2, 127, np.uint8)
    sfb = np.full(N * 2, 127, np.uint8)
    p, s = orc.gemm_fp8_out(a, b, sfa, sfb, M, N, K, F8, LIN, LIN, 1.0, LIN)
    assert (s.reshape(M, 2)[:, 1] == 0).all() and (p[:, 32:] == 0).all()
    pn, sn = orc.gemm_fp8_out(a | 0x80, b, sfa, sfb, M, N, K, F8, LIN, LIN, 1.0, LIN)
    assert np.array_equal(sn, s)
    assert np.array_equal(pn[:, :32], p[:, :32] | 0x80)


@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_output_tracks_the_gemm(orc, fmt):
    """For operands of every GEMM format the dequantized FP8 output follows
    the binary64 GEMM to bf16-then-E4M3 precision (OCP clipping of values in
    (448, 512) * 2^e included), and each scale byte is floor(log2 of the
    block's largest bf16 output) - 8 + 127."""
    from block_scaled_fp4_add_amd import synth
    M, N, K = 7, 96, 512
    A = synth.activation(M, K, 9, outliers=True)
    W = synth.weight(N, K, 9)
    a, sfa = orc.quantize(synth.bits(A), fmt, LIN)
    b, sfb = orc.quantize(synth.bits(W), fmt, LIN)
    p, s, ref, _ = orc.gemm_fp8_out(a, b, sfa, sfb, M, N, K, fmt, LIN, LIN, 0.5, LIN, diag=True)
    _, dq = orc.dequantize(p, s, M, N, F8, LIN)
    blk = np.abs(ref).reshape(M, N // 32, 32).max(axis=2)
    e = np.floor(np.log2(blk)) - 8
    assert np.array_equal(s.reshape(M, -1).astype(int), (e + 127).astype(int))
    amax = np.repeat(blk, 32, axis=1)
    assert np.all(np.abs(dq - ref) <= 2.0 ** -3 * np.abs(ref) + 2.0 ** -7 * np.abs(ref) + 2.0 ** -10 * amax)
