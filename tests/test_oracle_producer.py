"""Pins of the oracle's fused producer (add + RMSNorm + FP4 quant) and of its
quantize / dequantize pair, against: torch's bf16 add (the residual
invariant), a 60-digit Decimal evaluation of rstd, hand-worked constant rows
(tests/golden/producer_constant_rows.json), the MXFP4 idempotence of
quantize(dequantize(.)), and dequantization error bounds that follow from the
format definitions."""
import json
import os
import struct
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch

from block_scaled_fp4_add_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
EPS = 1e-6


def f32bits(x):
    return struct.unpack("<I", struct.pack("<f", float(x)))[0]


def codes_of(packed):
    c = np.empty((packed.shape[0], packed.shape[1] * 2), np.uint8)
    c[:, 0::2] = packed & 15
    c[:, 1::2] = packed >> 4
    return c


@pytest.mark.parametrize("fmt", [0, 1])
def test_residual_is_bf16_sum(orc, fmt):
    x, r, w = synth.producer_inputs(16, 512, seed=5, outliers=True)
    out = orc.add_rmsnorm_quant(synth.bits(x), synth.bits(r), synth.bits(w), EPS, fmt, orc.LINEAR)
    ref = (x.float() + r.float()).to(torch.bfloat16)
    assert np.array_equal(out["residual"], synth.bits(ref))


def test_rstd_against_decimal(orc):
    getcontext().prec = 60
    x, r, w = synth.producer_inputs(24, 320, seed=9)
    out = orc.add_rmsnorm_quant(synth.bits(x), synth.bits(r), synth.bits(w), EPS, 0, orc.LINEAR,
                                diag=True)
    h = (x.float() + r.float()).numpy()  # fp32 sum, as the producer squares it
    eps = Decimal(float(np.float32(EPS)))
    exact_hits = 0
    for m in range(h.shape[0]):
        S = sum(Decimal(float(v)) * Decimal(float(v)) for v in h[m])
        want = np.float32(float(1 / (S / h.shape[1] + eps).sqrt()))
        got = out["rstd"][m]
        ulps = abs(int(f32bits(got)) - int(f32bits(want)))
        assert ulps <= 1
        exact_hits += ulps == 0
    assert exact_hits >= h.shape[0] - 1


def test_y_definition_and_amax(orc):
    x, r, w = synth.producer_inputs(8, 256, seed=4, outliers=True)
    out = orc.add_rmsnorm_quant(synth.bits(x), synth.bits(r), synth.bits(w), EPS, 1, orc.LINEAR,
                                diag=True)
    hb = (x.float() + r.float()).to(torch.bfloat16).float()
    rstd = torch.from_numpy(out["rstd"]).unsqueeze(1)
    y = (hb * rstd) * w.float()  # torch fp32 elementwise: two separately rounded products
    assert np.array_equal(out["y"], y.numpy())
    amax = np.abs(out["y"]).reshape(8, -1, 32).max(axis=2)
    assert np.array_equal(out["amax"], amax)


def _constant_rows():
    with open(os.path.join(GOLDEN, "producer_constant_rows.json")) as f:
        return json.load(f)["rows"]


@pytest.mark.parametrize("row", _constant_rows(), ids=lambda r: r["name"])
@pytest.mark.parametrize("fmt", [0, 1])
def test_constant_row_closed_form(orc, row, fmt):
    H = row["H"]
    x = torch.full((1, H), row["c"], dtype=torch.bfloat16)
    r = torch.zeros((1, H), dtype=torch.bfloat16)
    w = torch.ones((H,), dtype=torch.bfloat16)
    for layout in (orc.LINEAR, orc.TILED):
        out = orc.add_rmsnorm_quant(synth.bits(x), synth.bits(r), synth.bits(w), EPS, fmt, layout,
                                    diag=True)
        assert f32bits(out["rstd"][0]) == int(row["rstd_bits"], 16)
        assert all(f32bits(v) == int(row["y_bits"], 16) for v in out["y"][0])
        want = row["nv"] if fmt == 0 else row["mx"]
        nblk = H // (16 if fmt == 0 else 32)
        for kb in range(nblk):
            assert out["sf"][orc.sf_offset(0, kb, nblk, fmt, layout)] == want["scale_byte"]
        assert (codes_of(out["packed"]) == want["code"]).all()


def test_producer_equals_quantize_of_its_y_for_mxfp4(orc):
    """MXFP4 ignores the global scale, so the producer's codes must be the
    quantizer's codes of y -- when y is bf16-exact.  Use w such that y is the
    bf16 value itself: rows where rstd == 1 exactly are rare, so instead check
    the block rule through orc.encode_with_scale on the producer's own y."""
    x, r, w = synth.producer_inputs(4, 256, seed=12)
    out = orc.add_rmsnorm_quant(synth.bits(x), synth.bits(r), synth.bits(w), EPS, 1, orc.LINEAR,
                                diag=True)
    codes = codes_of(out["packed"])
    for m in range(4):
        for kb in range(8):
            sb = out["sf"][m * 8 + kb]
            c = orc.encode_with_scale(out["y"][m, kb * 32:(kb + 1) * 32], 1, 1.0, int(sb))
            assert np.array_equal(c, codes[m, kb * 32:(kb + 1) * 32])
            # OCP MX rule: the scale's binade is the amax's binade minus 2
            a = float(out["amax"][m, kb])
            e = int(sb) - 127
            assert 2.0 ** (e + 2) <= a < 2.0 ** (e + 3)


def test_nvfp4_scale_rule_with_global_scale(orc):
    x, r, w = synth.producer_inputs(4, 128, seed=13, outliers=True)
    gs = 2688.0 / 30.0
    out = orc.add_rmsnorm_quant(synth.bits(x), synth.bits(r), synth.bits(w), EPS, 0, orc.LINEAR,
                                gs=np.float32(gs), diag=True)
    gs32 = np.float32(gs)
    for m in range(4):
        for kb in range(8):
            s_pre = min(np.float32(np.float32(gs32 * out["amax"][m, kb]) / np.float32(6.0)),
                        np.float32(448.0))
            assert out["spre"][m, kb] == s_pre
            # the chosen E4M3 byte is the nearest to s_pre (brute force over codes)
            sb = int(out["sf"][m * 8 + kb])
            vals = np.array([orc.e4m3_value(c) for c in range(0x7F)])
            d = np.abs(vals - float(s_pre))
            assert d[sb] == d.min()


@pytest.mark.parametrize("K", [64, 256, 5120])
def test_mxfp4_quantize_dequantize_idempotent(orc, K):
    x = synth.activation(6, K, seed=21, outliers=True)
    p, s = orc.quantize(synth.bits(x), 1, orc.TILED)
    xq, _ = orc.dequantize(p, s, 6, K, 1, orc.TILED)
    p2, s2 = orc.quantize(xq, 1, orc.TILED)
    assert np.array_equal(p, p2) and np.array_equal(s, s2)


@pytest.mark.parametrize("fmt", [0, 1])
def test_dequantize_error_bound(orc, fmt):
    """|x - dequant(quant(x))| <= half a grid step at the block scale, except
    for values clipped at 6*scale (MXFP4's OCP rule clips up to amax < 8*scale)."""
    K = 512
    x = synth.activation(8, K, seed=22)
    p, s = orc.quantize(synth.bits(x), fmt, orc.LINEAR)
    _, xq = orc.dequantize(p, s, 8, K, fmt, orc.LINEAR)
    B = 16 if fmt == 0 else 32
    xf = x.double().numpy()
    for m in range(8):
        for kb in range(K // B):
            sb = s[m * (K // B) + kb]
            scale = orc.e4m3_value(sb) if fmt == 0 else orc.ue8m0_value(sb)
            blk = slice(kb * B, (kb + 1) * B)
            err = np.abs(xf[m, blk] - xq[m, blk])
            mag = np.abs(xf[m, blk]) / scale
            step = np.where(mag < 2, 0.5, np.where(mag < 4, 1.0, 2.0))
            clipped = mag > 6
            bound = np.where(clipped, (mag - 6) * scale, 0.5 * step * scale)
            # NVFP4's scale is rounded to E4M3, so v = x/scale may exceed 6 slightly
            assert np.all(err <= bound * (1 + 1e-12) + 1e-30)


def test_nvfp4_dequantize_divides_by_global_scale(orc):
    x = synth.activation(2, 64, seed=23)
    gs = np.float32(3.0)
    p, s = orc.quantize(synth.bits(x), 0, orc.LINEAR, gs=gs)
    _, x1 = orc.dequantize(p, s, 2, 64, 0, orc.LINEAR, gs=1.0)
    bits, x3 = orc.dequantize(p, s, 2, 64, 0, orc.LINEAR, gs=gs)
    want = (x1 / 3.0).astype(np.float32)
    assert np.array_equal(x3.astype(np.float32), want)
    assert np.array_equal(bits, synth.bits(torch.from_numpy(want).to(torch.bfloat16)))


@pytest.mark.parametrize("fmt,gs", [(0, 1.0), (0, 0.3), (1, 1.0), (2, 1.0), (3, 7.0)])
def test_dequantize_fp16_output_is_numpys_rounding(orc, fmt, gs):
    """The fp16 output of the dequantizer (the README's dequantize_fp4_sfa_fp16)
    is numpy's IEEE rounding of the binary32 value, for every code under scale
    bytes that reach fp16 overflow (infinity) and its subnormals."""
    rows, K = 64, 256
    B = orc.block_size(fmt)
    rng = np.random.default_rng(fmt * 10 + int(gs))
    width = K if fmt == orc.MXFP8 else K // 2
    packed = rng.integers(0, 256, size=(rows, width), dtype=np.uint8)
    if fmt == orc.MXFP8:
        packed[(packed & 0x7F) == 0x7F] = 0x7E           # no E4M3 NaN codes
    if fmt in (orc.MXFP4, orc.MXFP8):
        # UE8M0 bytes from 2^-40 to 2^25: fp16 subnormals, zeros and overflow to infinity
        sf = rng.integers(127 - 40, 127 + 26, size=rows * (K // B), dtype=np.uint8)
    else:
        sf = rng.integers(0, 0x7F, size=rows * (K // B), dtype=np.uint8)   # every E4M3 scale but NaN
    bits, f64 = orc.dequantize(packed, sf, rows, K, fmt, orc.LINEAR, gs=gs, dtype=orc.F16)
    with np.errstate(over="ignore"):   # overflow to infinity is the case under test
        want = f64.astype(np.float32).astype(np.float16).view(np.uint16)
    assert np.array_equal(bits, want)
    if fmt in (orc.MXFP4, orc.MXFP8):
        assert (want & 0x7FFF == 0x7C00).any() and ((want & 0x7C00) == 0).any()   # both ends reached
    bf, f64b = orc.dequantize(packed, sf, rows, K, fmt, orc.LINEAR, gs=gs)
    assert np.array_equal(f64b, f64)


# --- fp16 tensors ----------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", [0, 1])
def test_residual_is_fp16_sum(orc, fmt):
    """With fp16 tensors the residual is numpy's fp16 rounding of the fp32 sum."""
    x, r, w = synth.producer_inputs(16, 512, seed=15, outliers=True, dtype=torch.float16)
    out = orc.add_rmsnorm_quant(synth.bits(x), synth.bits(r), synth.bits(w), EPS, fmt, orc.LINEAR,
                                dtype=orc.F16)
    ref = (x.numpy().astype(np.float32) + r.numpy().astype(np.float32)).astype(np.float16)
    assert np.array_equal(out["residual"], ref.view(np.uint16))


def test_fp16_y_definition(orc):
    """y = fl32(fl32(fp16(h) * rstd) * w) with fp16 h and w, in numpy fp32."""
    x, r, w = synth.producer_inputs(8, 256, seed=14, outliers=True, dtype=torch.float16)
    out = orc.add_rmsnorm_quant(synth.bits(x), synth.bits(r), synth.bits(w), EPS, 0, orc.LINEAR,
                                diag=True, dtype=orc.F16)
    hb = (x.numpy().astype(np.float32) + r.numpy().astype(np.float32)).astype(np.float16).astype(np.float32)
    y = (hb * out["rstd"][:, None]) * w.numpy().astype(np.float32)
    assert np.array_equal(out["y"], y.astype(np.float32))


def test_fp16_and_bf16_agree_on_common_values(orc):
    """Values exact in both formats (small integers times powers of two within
    range) give identical codes and scales through the fp16 and bf16 paths of
    the quantizer and the producer."""
    rng = np.random.default_rng(21)
    v = (rng.integers(-64, 65, (12, 256)) * np.ldexp(1.0, rng.integers(-6, 4, (12, 1)))).astype(np.float32)
    xb = torch.from_numpy(v).to(torch.bfloat16)
    xh = torch.from_numpy(v).to(torch.float16)
    assert torch.equal(xb.float(), xh.float())
    for fmt in (0, 1):
        pb, sb = orc.quantize(synth.bits(xb), fmt, orc.TILED)
        ph, sh = orc.quantize(synth.bits(xh), fmt, orc.TILED, dtype=orc.F16)
        assert np.array_equal(pb, ph) and np.array_equal(sb, sh)
    zb, zh = torch.zeros_like(xb), torch.zeros_like(xh)
    wb = torch.ones(256, dtype=torch.bfloat16)
    wh = torch.ones(256, dtype=torch.float16)
    for fmt in (0, 1):
        ob = orc.add_rmsnorm_quant(synth.bits(xb), synth.bits(zb), synth.bits(wb), EPS, fmt, orc.LINEAR)
        oh = orc.add_rmsnorm_quant(synth.bits(xh), synth.bits(zh), synth.bits(wh), EPS, fmt, orc.LINEAR,
                                   dtype=orc.F16)
        assert np.array_equal(ob["packed"], oh["packed"]) and np.array_equal(ob["sf"], oh["sf"])


# --- MXFP8 (E4M3 elements, UE8M0 32-blocks) ------------------------------------------------

def _e4m3_bits(v):
    """E4M3 byte of a value exactly on the grid (torch's own conversion)."""
    return int(torch.tensor([v], dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)[0])


def test_mxfp8_hand_worked_blocks(orc):
    """Blocks worked out by hand from the OCP MX rule (e = floor(log2 amax) - 8,
    E4M3 elements nearest-even, saturating at 448, sign kept)."""
    rows = []
    want_sf, want_codes = [], []
    # all zero: scale byte 0, every element 0
    rows.append([0.0] * 32)
    want_sf.append(0)
    want_codes.append([0] * 32)
    # one outlier 1000 and 31 x 0.01 (bf16 0.010009765625): floor(log2 1000) = 9,
    # e = 1 (X = 2); 1000 / 2 = 500 saturates to 448 (0x7E); 0.01000977 / 2 =
    # 0.00500488 = 2.5625 steps of the subnormal step 2^-9 -> 3 steps (0x03)
    rows.append([1000.0] + [0.01] * 31)
    want_sf.append(128)
    want_codes.append([0x7E] + [0x03] * 31)
    # exact grid: amax 448 gives e = 0 (X = 1); grid values keep their codes, a
    # negative value its sign, and -0.001 (0.512 of the subnormal step) rounds
    # to 1 step with its sign (0x81)
    grid = [448.0, -448.0, 1.0, -1.125, 0.015625, 240.0, -0.001953125, 3.5]
    vals = grid + [-0.001] + [0.0] * 23
    rows.append(vals)
    want_sf.append(127)
    want_codes.append([_e4m3_bits(v) for v in grid] + [0x81] + [0] * 23)
    # amax 512 moves to the next binade: e = 1 (X = 2), elements 256 and 8
    rows.append([512.0, 16.0] + [0.0] * 30)
    want_sf.append(128)
    want_codes.append([_e4m3_bits(256.0), _e4m3_bits(8.0)] + [0] * 30)
    x = torch.tensor(rows, dtype=torch.float32).to(torch.bfloat16)
    p, s = orc.quantize(synth.bits(x), orc.MXFP8, orc.LINEAR)
    assert s.tolist() == want_sf
    assert p.tolist() == want_codes


@pytest.mark.parametrize("K", [64, 256, 5120])
def test_mxfp8_quantize_dequantize_idempotent(orc, K):
    """Dequantized MXFP8 values (at most 4 significant bits: exact in bf16)
    quantize back to the same values."""
    x = synth.activation(6, K, seed=23, outliers=True)
    p, s = orc.quantize(synth.bits(x), orc.MXFP8, orc.LINEAR)
    xq, f1 = orc.dequantize(p, s, 6, K, orc.MXFP8, orc.LINEAR)
    assert np.array_equal(synth.from_bits(xq).double().numpy(), f1)   # bf16-exact
    p2, s2 = orc.quantize(xq, orc.MXFP8, orc.LINEAR)
    _, f2 = orc.dequantize(p2, s2, 6, K, orc.MXFP8, orc.LINEAR)
    assert np.array_equal(f1, f2)


def test_mxfp8_dequantize_error_bound(orc):
    """|x - dq(q(x))| <= half an E4M3 step at the element's binade (relative
    2^-4 for normal elements), or 448 * X saturation, from the definitions."""
    x = synth.activation(16, 1024, seed=24, outliers=True)
    p, s = orc.quantize(synth.bits(x), orc.MXFP8, orc.LINEAR)
    _, f = orc.dequantize(p, s, 16, 1024, orc.MXFP8, orc.LINEAR)
    xv = x.double().numpy()
    X = np.repeat(np.ldexp(1.0, (s.reshape(16, -1).astype(np.int32) - 127)), 32, axis=1)
    v = np.abs(xv) / X
    step = np.ldexp(1.0, (np.maximum(np.floor(np.log2(np.maximum(v, 1e-300))), -6) - 3).astype(np.int32))
    bound = np.where(v > 448, v - 448, step / 2) * X
    assert np.all(np.abs(xv - f) <= bound * (1 + 1e-12))


def test_mxfp8_producer_equals_quantize_of_its_y(orc):
    """The fused producer's MXFP8 codes are the quantizer's codes of its own y."""
    x, r, w = synth.producer_inputs(8, 512, seed=25, outliers=True)
    out = orc.add_rmsnorm_quant(synth.bits(x), synth.bits(r), synth.bits(w), EPS, orc.MXFP8, orc.LINEAR,
                                diag=True)
    assert out["packed"].shape == (8, 512)
    y = out["y"].reshape(-1, 32)
    for i in range(y.shape[0]):
        codes, _ = orc.encode_with_scale(y[i], orc.MXFP8, 1.0, int(out["sf"][i]), with_v=True)
        assert np.array_equal(codes, out["packed"].reshape(-1, 32)[i])


def test_mxfp8_rejects_tiled_scales(orc):
    x = synth.activation(2, 64, seed=1)
    with pytest.raises(ValueError):
        orc.quantize(synth.bits(x), orc.MXFP8, orc.TILED)
