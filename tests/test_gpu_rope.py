"""GPU parity of the inverse-RoPE + MX quantizer (vLLM fused_wo_a page,
FusedWoAKernel.device_kernel activation quant stage) against the oracle, bit
for bit: the rotation is the same fp32 operation sequence on both sides and
the scale and element encodings are exact.  Inputs follow the page's decode
rows (1 to 96 tokens of several heads) with a 512-element head whose last 64
elements carry RoPE, a table of standard RoPE frequencies over 4096
positions, and random positions."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_add_amd as lb
from block_scaled_fp4_add_amd import synth

from . import checkers
from .gpu_util import banner, dev_bf16, host_u8

pytestmark = pytest.mark.gpu


def rope_table(P, R, base=10000.0):
    """cos || sin rows of the standard RoPE angles pos * base^(-2i/R), fp32."""
    inv = base ** (-np.arange(0, R, 2, dtype=np.float64) / R)
    ang = np.arange(P, dtype=np.float64)[:, None] * inv[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def run(orc, T, heads, D, R, P, fmt, layout, seed, positions=None, zero_rows=()):
    banner(f"rope_quant T={T} heads={heads} D={D} R={R} P={P} fmt={fmt} layout={layout} seed={seed}")
    x = synth.activation(T * heads, D, seed, outliers=True)
    for r in zero_rows:
        x[r] = 0
    x3 = x.reshape(T, heads, D)
    rng = np.random.default_rng(seed)
    pos = rng.integers(0, max(P, 1), T).astype(np.int64) if positions is None else np.asarray(positions, np.int64)
    tab = rope_table(P, R) if R > 0 else np.zeros((max(P, 1), 0), np.float32)
    ref_p, ref_s = orc.rope_quant(synth.bits(x3), pos, tab, heads, fmt, layout)
    p, s = lb.lowbit_rope_quant(dev_bf16(x3), torch.from_numpy(pos).to("cuda"),
                                torch.from_numpy(tab).to("cuda") if R > 0 else None, fmt, layout)
    torch.cuda.synchronize()
    assert np.array_equal(host_u8(s), ref_s), "scale bytes differ"
    assert np.array_equal(host_u8(p), ref_p), "element codes differ"
    if layout == lb.TILED:
        assert checkers.tiled_padding_is_zero(orc, host_u8(s), T * heads, D // 32, fmt)


@pytest.mark.parametrize("T,heads", [(1, 16), (7, 8), (41, 16), (96, 16), (96, 3)])
@pytest.mark.parametrize("fmt,layout", [(2, 0), (1, 0), (1, 1), (1, 2)])
def test_rope_quant_decode_rows(orc, T, heads, fmt, layout):
    run(orc, T, heads, 512, 64, 4096, fmt, layout, seed=T * 31 + heads)


@pytest.mark.parametrize("D,R", [(512, 0), (64, 64), (96, 36), (256, 8), (1024, 128), (32, 2)])
@pytest.mark.parametrize("fmt", [2, 1])
def test_rope_quant_slices(orc, D, R, fmt):
    """No rope, an all-rope row, a rotary slice starting inside an 8-element
    vector (D - R = 60), short and long heads."""
    run(orc, 9, 5, D, R, 300, fmt, 0, seed=D + R)


def test_rope_quant_positions_held_in_range_and_zero_rows(orc):
    """Out-of-range positions read the nearest end row; all-zero rows give the
    page's floored scale byte (127 - 34 - 8 for MXFP8) with zero codes."""
    run(orc, 6, 4, 512, 64, 128, 2, 0, seed=5, positions=[-3, 0, 127, 128, 5000, 64], zero_rows=(0, 7))
    run(orc, 6, 4, 512, 64, 128, 1, 1, seed=6, positions=[-3, 0, 127, 128, 5000, 64], zero_rows=(1, 23))


def test_rope_quant_empty_and_errors(orc):
    x = torch.zeros((0, 4, 512), dtype=torch.bfloat16, device="cuda")
    p, s = lb.lowbit_rope_quant(x, torch.zeros(0, dtype=torch.int64, device="cuda"),
                                torch.zeros((8, 64), dtype=torch.float32, device="cuda"))
    assert p.numel() == 0
    x = torch.zeros((2, 4, 100), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lb.LowbitError) as e:
        lb.lowbit_rope_quant(x, torch.zeros(2, dtype=torch.int64, device="cuda"),
                             torch.zeros((8, 64), dtype=torch.float32, device="cuda"),
                             out_packed=torch.empty((8, 100), dtype=torch.uint8, device="cuda"),
                             out_sf=torch.empty(64, dtype=torch.uint8, device="cuda"))
    assert e.value.status == 3                                    # D % 32
    x = torch.zeros((2, 4, 512), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lb.LowbitError) as e:
        lb.lowbit_rope_quant(x, torch.zeros(2, dtype=torch.int64, device="cuda"),
                             torch.zeros((8, 64), dtype=torch.float32, device="cuda"), fmt=lb.MXFP8,
                             layout=lb.TILED)
    assert e.value.status == 1                                    # MXFP8 scales: LINEAR only
