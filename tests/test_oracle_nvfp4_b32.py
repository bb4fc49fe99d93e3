"""Pins of the oracle's NVFP4 rule on 32-element blocks (format 3: E4M3 block
scales with the global scale folded in, as the add + RMSNorm + FP4 producer's
page allows by its E4M3 scale-format override at block size 32).  Each pin ties
the format to something fixed outside it: the separately pinned 16-block NVFP4
path, hand-computed blocks, or closed forms of E2M1 and E4M3."""
import numpy as np
import pytest

from oracle import oracle as orc
from block_scaled_fp4_add_amd import synth

B32 = orc.NVFP4_B32


def _bf16(vals):
    return np.array([orc.f32_to_bf16(float(v)) for v in np.ravel(vals)], np.uint16).reshape(np.shape(vals))


def _codes(packed):
    p = np.asarray(packed, np.uint8)
    out = np.zeros(p.shape[:-1] + (2 * p.shape[-1],), np.uint8)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out


@pytest.mark.parametrize("gs", [1.0, 0.37, 1000.0])
def test_equal_half_amax_reduces_to_16_blocks(gs):
    """When both 16-element halves of every 32-block share one amax, the 32-block
    scale is the 16-block scale of either half and the codes are the same."""
    rng = np.random.default_rng(7)
    rows, K = 6, 256
    x = rng.normal(0, 1, (rows, K)).astype(np.float32)
    peak = rng.uniform(4.0, 9.0, (rows, K // 32)).astype(np.float32)
    sign = rng.choice([-1.0, 1.0], (rows, K // 32, 2)).astype(np.float32)
    for b in range(K // 32):
        x[:, 32 * b] = peak[:, b] * sign[:, b, 0]
        x[:, 32 * b + 16] = peak[:, b] * sign[:, b, 1]
    xb = _bf16(x)
    p16, s16 = orc.quantize(xb, orc.NVFP4, orc.LINEAR, gs=gs)
    p32, s32 = orc.quantize(xb, B32, orc.LINEAR, gs=gs)
    assert np.array_equal(p16, p32)
    s16 = s16.reshape(rows, K // 16)
    s32 = s32.reshape(rows, K // 32)
    assert np.array_equal(s32, s16[:, 0::2]) and np.array_equal(s32, s16[:, 1::2])


def test_hand_block_spans_32_elements():
    """First half 0.5 and 1.0, the block's amax 12 in the second half: gs = 1,
    s = 12/6 = 2 (E4M3 0x40), inv = 0.5.  0.5 -> 0.25, a tie between E2M1 0
    and 0.5 that goes to the even code 0; 1.0 -> 0.5 (code 1); 12 -> 6 (code 7);
    -3 -> -1.5 (code 0xB)."""
    y = np.array([0.5] * 8 + [1.0] * 8 + [12.0] + [-3.0] * 15, np.float32)
    p, s = orc.quantize(_bf16(y[None, :]), B32, orc.LINEAR)
    assert s.tolist() == [0x40]
    want = [0] * 8 + [1] * 8 + [7] + [0xB] * 15
    assert _codes(p)[0].tolist() == want
    # the 16-block rule scales the first half by its own amax instead
    p16, s16 = orc.quantize(_bf16(y[None, :]), orc.NVFP4, orc.LINEAR)
    assert s16.tolist()[0] != 0x40


def test_scale_saturates_at_448_and_zero_block():
    """gs * amax / 6 above 448 clamps to E4M3 0x7E; an all-zero block has scale 0
    and every code 0."""
    y = np.zeros((2, 32), np.float32)
    y[0, 5] = 3.0e4
    p, s = orc.quantize(_bf16(y), B32, orc.LINEAR, gs=1.0)
    assert s.tolist() == [0x7E, 0x00]
    assert not np.any(_codes(p)[1])


def test_dequantize_closed_form():
    """x = E2M1 * E4M3(scale) / gs: byte 0x71 holds codes 1 (0.5) and 7 (6);
    scale 0x40 = 2, gs = 4 -> 0.25 and 3.0, exact in bf16."""
    packed = np.full((1, 16), 0x71, np.uint8)
    sf = np.array([0x40], np.uint8)
    bf, f64 = orc.dequantize(packed, sf, 1, 32, B32, orc.LINEAR, gs=4.0)
    assert f64[0, 0::2].tolist() == [0.25] * 16 and f64[0, 1::2].tolist() == [3.0] * 16
    assert [orc.bf16_to_f32(int(b)) for b in bf[0, :2]] == [0.25, 3.0]


def test_producer_same_y_and_amax_over_32():
    """The fused producer computes the same y in both block sizes; the 32-block
    amax is the larger of its two 16-block amaxes."""
    M, H = 5, 640
    x, r, w = synth.producer_inputs(M, H, 3, outliers=True)
    args = (synth.bits(x), synth.bits(r), synth.bits(w), 1e-6)
    d16 = orc.add_rmsnorm_quant(*args, orc.NVFP4, orc.LINEAR, gs=2.5, diag=True)
    d32 = orc.add_rmsnorm_quant(*args, B32, orc.LINEAR, gs=2.5, diag=True)
    assert np.array_equal(d16["residual"], d32["residual"])
    assert np.array_equal(d16["y"].view(np.uint32), d32["y"].view(np.uint32))
    assert np.array_equal(d32["amax"], np.maximum(d16["amax"][:, 0::2], d16["amax"][:, 1::2]))


def test_round_trip_of_representable_values():
    """Values E2M1 * s with one E4M3-exact s per block survive quantize ->
    dequantize when the block holds a 6 * s element (then the scale is s)."""
    rng = np.random.default_rng(11)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    rows, K = 4, 128
    s = np.float32(2.0) ** rng.integers(-4, 5, (rows, K // 32))
    q = grid[rng.integers(0, 8, (rows, K))] * rng.choice([-1, 1], (rows, K))
    q[:, ::32] = 6.0
    y = (q.reshape(rows, K // 32, 32) * s[..., None]).reshape(rows, K).astype(np.float32)
    p, sf = orc.quantize(_bf16(y), B32, orc.LINEAR)
    _, f64 = orc.dequantize(p, sf, rows, K, B32, orc.LINEAR)
    assert np.array_equal(f64, y.astype(np.float64))


def test_rejections():
    x = np.zeros((2, 64), np.uint16)
    with pytest.raises(ValueError):
        orc.quantize(x, B32, orc.TILED)           # LINEAR scales only
    with pytest.raises(ValueError):
        orc.quantize(np.zeros((2, 48), np.uint16), B32, orc.LINEAR)   # K % 32
