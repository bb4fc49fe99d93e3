"""Pins of the oracle's inverse-RoPE + MX quantizer (the vLLM fused_wo_a page,
FusedWoAKernel.device_kernel, activation quant stage) against facts that do
not depend on its own code: special angles that reduce it to the plain MX
quantizer (itself pinned by hand blocks and exhaustive format checks), the
rotation's invariants, a forward rotation undone in binary64, the position
indexing, and closed forms of the 1e-10 floor."""
import numpy as np
import pytest
import torch

from block_scaled_fp4_add_amd import synth

FMTS = [(2, 8), (1, 2)]      # (format, emax): MXFP8 (E4M3 elements), MXFP4 (E2M1)


def table(P, R, angles):
    """A rope table, each row cos(angles[p]) || sin(angles[p]) in fp32."""
    ang = np.broadcast_to(np.asarray(angles, np.float64), (P, R // 2))
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def bf16_bits(a):
    """bf16 bit patterns (uint16) of float values, round to nearest even."""
    return synth.bits(torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16))


def rows_x(T, heads, D, seed):
    return synth.bits(synth.activation(T * heads, D, seed, outliers=True)).reshape(T, heads, D)


@pytest.mark.parametrize("fmt,emax", FMTS)
def test_no_rope_is_the_plain_mx_quantizer(orc, fmt, emax):
    """R = 0: no element is rotated; every block whose maximum is at least
    1e-10 quantizes exactly as the plain MX quantizer does."""
    T, heads, D = 5, 3, 256
    x = rows_x(T, heads, D, 11)
    p, s = orc.rope_quant(x, np.zeros(T, np.int64), np.zeros((1, 0), np.float32), heads, fmt, orc.LINEAR)
    q, qs = orc.quantize(x.reshape(T * heads, D), fmt, orc.LINEAR)
    assert np.array_equal(p, q) and np.array_equal(s, qs)


@pytest.mark.parametrize("fmt,emax", FMTS)
def test_zero_angle_is_the_identity(orc, fmt, emax):
    T, heads, D, R, P = 4, 2, 128, 64, 7
    x = rows_x(T, heads, D, 12)
    pos = np.array([0, 6, 3, 3], np.int64)
    p, s = orc.rope_quant(x, pos, table(P, R, 0.0), heads, fmt, orc.LINEAR)
    q, qs = orc.quantize(x.reshape(T * heads, D), fmt, orc.LINEAR)
    assert np.array_equal(p, q) and np.array_equal(s, qs)


@pytest.mark.parametrize("fmt,emax", FMTS)
def test_quarter_turn_swaps_and_negates_pairs(orc, fmt, emax):
    """cos = 0, sin = 1: (even, odd) -> (odd, -even) exactly, so the result is
    the plain quantizer on the pair-swapped, partly negated row."""
    T, heads, D, R = 3, 2, 96, 64
    x = rows_x(T, heads, D, 13)
    tab = np.concatenate([np.zeros((1, R // 2)), np.ones((1, R // 2))], axis=1).astype(np.float32)
    p, s = orc.rope_quant(x, np.zeros(T, np.int64), tab, heads, fmt, orc.LINEAR)
    z = x.reshape(T * heads, D).copy()
    nope = D - R
    ev, od = z[:, nope::2].copy(), z[:, nope + 1::2].copy()
    z[:, nope::2] = od
    z[:, nope + 1::2] = ev ^ np.uint16(0x8000)          # bf16 negation: the sign bit
    q, qs = orc.quantize(z, fmt, orc.LINEAR)
    assert np.array_equal(p, q) and np.array_equal(s, qs)


@pytest.mark.parametrize("fmt,emax", FMTS)
def test_half_turn_flips_every_sign(orc, fmt, emax):
    """cos = -1, sin = 0 on a row that is all rope: every value negated, so
    the scales stay and every code gets its sign bit flipped."""
    T, heads, D = 2, 2, 64
    x = rows_x(T, heads, D, 14)
    tab = np.concatenate([-np.ones((1, D // 2)), np.zeros((1, D // 2))], axis=1).astype(np.float32)
    p, s = orc.rope_quant(x, np.zeros(T, np.int64), tab, heads, fmt, orc.LINEAR)
    q, qs = orc.quantize(x.reshape(T * heads, D), fmt, orc.LINEAR)
    assert np.array_equal(s, qs)
    flip = np.uint8(0x80) if fmt == 2 else np.uint8(0x88)   # sign bit of each element (two per FP4 byte)
    assert np.array_equal(p, q ^ flip)


def test_rotation_is_the_inverse_and_keeps_pair_norms(orc):
    """Rows rotated forward in binary64 by the angle of their token's position
    come back (to bf16 precision) after the oracle's inverse rotation; a
    forward rotation there would double the angle instead.  Each rotated pair
    keeps its norm to fp32 precision."""
    T, heads, D, R, P = 6, 2, 128, 64, 50
    rng = np.random.default_rng(3)
    theta = rng.uniform(-np.pi, np.pi, (P, R // 2))
    pos = rng.integers(0, P, T)
    x0 = rng.standard_normal((T, heads, D))
    xr = x0.copy()
    nope = D - R
    for t in range(T):
        c, s = np.cos(theta[pos[t]]), np.sin(theta[pos[t]])
        e, o = x0[t, :, nope::2], x0[t, :, nope + 1::2]
        xr[t, :, nope::2] = e * c - o * s           # forward RoPE
        xr[t, :, nope + 1::2] = o * c + e * s
    xb = bf16_bits(xr)
    _, _, y, _ = orc.rope_quant(xb, pos, table(P, R, theta), heads, 2, orc.LINEAR, diag=True)
    y = y.reshape(T, heads, D).astype(np.float64)
    xin = synth.from_bits(xb.reshape(-1, D)).float().numpy().reshape(T, heads, D).astype(np.float64)
    assert np.allclose(y[..., :nope], xin[..., :nope], rtol=0, atol=0)        # nope part untouched
    assert np.allclose(y, x0, rtol=2 ** -7, atol=2 ** -7)                    # back to the unrotated row
    n_in = xin[..., nope::2] ** 2 + xin[..., nope + 1::2] ** 2
    n_out = y[..., nope::2] ** 2 + y[..., nope + 1::2] ** 2
    assert np.allclose(n_out, n_in, rtol=4e-6, atol=1e-12)


def test_positions_index_the_table_and_are_held_in_range(orc):
    """Token t uses table row positions[t]; a position outside [0, P) reads
    the nearest end row."""
    T, heads, D, R, P = 5, 1, 64, 32, 4
    ang = np.array([0.0, np.pi / 2, np.pi, 0.0])[:, None] * np.ones((1, R // 2))
    x = rows_x(T, heads, D, 15)
    pos = np.array([1, 2, -5, 9, 0], np.int64)      # -5 -> row 0 (identity), 9 -> row 3 (identity)
    _, _, y, _ = orc.rope_quant(x, pos, table(P, R, ang), heads, 2, orc.LINEAR, diag=True)
    xin = synth.from_bits(x.reshape(-1, D)).float().numpy()
    nope = D - R
    e, o = xin[:, nope::2], xin[:, nope + 1::2]
    # token 0 -> row 1 (a quarter turn), token 1 -> row 2 (a half turn); fp32
    # cos(pi/2) and sin(pi) are about 1e-16, not zero
    assert np.allclose(y[0, nope::2], o[0], atol=1e-6) and np.allclose(y[0, nope + 1::2], -e[0], atol=1e-6)
    assert np.allclose(y[1, nope::2], -e[1], atol=1e-6) and np.allclose(y[1, nope + 1::2], -o[1], atol=1e-6)
    for t in (2, 3, 4):
        assert np.array_equal(y[t], xin[t])


@pytest.mark.parametrize("fmt,emax", FMTS)
def test_block_maximum_floor(orc, fmt, emax):
    """The page floors the block maximum at 1e-10: an all-zero block gets
    e = floor(log2 fl32(1e-10)) - emax = -34 - emax (byte 85 for MXFP8, 91 for
    MXFP4) and zero codes; a block of 1e-12 values gets the same scale, each
    value then 1e-12 * 2^(34 + emax)."""
    D = 64
    x = np.zeros((1, 1, D), np.float32)
    x[0, 0, 32:] = 1e-12
    xb = bf16_bits(x)
    v = float(synth.from_bits(xb.reshape(-1)[32:33]).float()[0])      # 1e-12 as bf16
    p, s, y, am = orc.rope_quant(xb, np.zeros(1, np.int64), np.zeros((1, 0), np.float32), 1, fmt, orc.LINEAR,
                                 diag=True)
    assert list(s) == [127 - 34 - emax] * 2
    assert np.float32(am[0, 0]) == np.float32(1e-10)
    scaled = v * 2.0 ** (34 + emax)
    if fmt == 2:
        assert (p[0, :32] == 0).all()
        assert (p[0, 32:] == orc.e4m3_encode(scaled)).all()
    else:
        assert (p[0, :16] == 0).all()
        c = orc.e2m1_encode(scaled)
        assert (p[0, 16:] == (c | (c << 4))).all()


@pytest.mark.parametrize("fmt,emax", FMTS)
def test_dequantized_output_tracks_the_rotated_row(orc, fmt, emax):
    """Dequantizing the output gives back the rotated fp32 row to the element
    format's precision under the OCP MX scale (values in (448, 512) * 2^e and
    (6, 8) * 2^e clip): E4M3 within 1/8 relative plus its subnormal step,
    E2M1 within half the block maximum -- the quantizer and the rotation line
    up."""
    T, heads, D, R, P = 4, 3, 256, 64, 9
    rng = np.random.default_rng(5)
    x = rows_x(T, heads, D, 16)
    p, s, y, _ = orc.rope_quant(x, rng.integers(0, P, T), table(P, R, rng.uniform(-3, 3, (P, R // 2))),
                                heads, fmt, orc.LINEAR, diag=True)
    _, dq = orc.dequantize(p, s, T * heads, D, fmt, orc.LINEAR)
    y = y.astype(np.float64)
    blk = np.abs(y).reshape(T * heads, D // 32, 32).max(axis=2)
    amax = np.repeat(blk, 32, axis=1)
    tol = (2.0 ** -3 * np.abs(y) + 2.0 ** -10 * amax) if fmt == 2 else amax / 2.0
    assert np.all(np.abs(dq - y) <= tol + 1e-30)
