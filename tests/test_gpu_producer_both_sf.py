"""GPU parity of the producer that writes its block scales in two layouts in
one pass (lowbit_add_rmsnorm_quant_both_sf and its fp16 form; the padded
layout TILED or the 128 x 4 swizzle, plus a row-major copy): the codes, the
residual and each scale buffer against the oracle run in that layout, and the
two scale buffers against each other byte for byte."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_add_amd as lb
from block_scaled_fp4_add_amd import synth

from . import checkers
from .gpu_util import banner, dev_bf16, dev_f32, host_bits, host_u8

pytestmark = pytest.mark.gpu
EPS = 1e-6


def run_both(orc, M, H, fmt, seed, use_gs, dtype=torch.bfloat16, layout=1):
    banner(f"producer both layouts M={M} H={H} fmt={fmt} layout={layout} seed={seed} gs={use_gs} dtype={dtype}")
    odt = orc.F16 if dtype == torch.float16 else orc.BF16
    x, r, w = synth.producer_inputs(M, H, seed, outliers=True, dtype=dtype)
    xb, rb, wb = synth.bits(x), synth.bits(r), synth.bits(w)
    gs = 1.0
    if use_gs:
        d = orc.add_rmsnorm_quant(xb, rb, wb, EPS, orc.NVFP4, orc.LINEAR, diag=True, dtype=odt)
        gs = float(np.float32(2688.0 / np.abs(d["y"]).max()))
    refs = {lay: orc.add_rmsnorm_quant(xb, rb, wb, EPS, fmt, lay, gs=gs, diag=True, dtype=odt)
            for lay in (layout, orc.LINEAR)}
    xd, rd, wd = dev_bf16(x), dev_bf16(r), dev_bf16(w)
    packed = torch.full((M, H // 2), 0xAA, dtype=torch.uint8, device="cuda")
    sf_t = torch.full((lb.lowbit_sf_bytes(M, H, fmt, layout),), 0xAA, dtype=torch.uint8, device="cuda")
    sf_l = torch.full((lb.lowbit_sf_bytes(M, H, fmt, lb.LINEAR),), 0xAA, dtype=torch.uint8, device="cuda")
    outs = lb.lowbit_add_rmsnorm_quant_both_sf(xd, rd, wd, EPS, fmt, layout,
                                               global_scale=dev_f32(gs) if use_gs else None,
                                               out_packed=packed, out_sf=sf_t, out_sf_linear=sf_l)
    assert outs[0] is packed and outs[1] is sf_t and outs[2] is sf_l
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(rd), refs[orc.LINEAR]["residual"])
    nblk = H // (16 if fmt == orc.NVFP4 else 32)
    got_t, got_l = host_u8(sf_t), host_u8(sf_l)
    for lay, got in ((layout, got_t), (orc.LINEAR, got_l)):
        ref = refs[lay]
        spre = ref["spre"] if fmt == orc.NVFP4 else ref["amax"]
        rep = checkers.compare_quantized(orc, fmt, gs, host_u8(packed), got, ref["packed"], ref["sf"],
                                         ref["y"], ref["v"], spre, M, H, lay)
        banner(f"  layout {lay} report {dict(rep)}")
        assert rep.ok(), rep
    if layout == orc.TILED:
        assert checkers.tiled_padding_is_zero(orc, got_t, M, nblk, fmt)
    else:
        assert np.array_equal(got_t, refs[layout]["sf"])          # padding included
        assert checkers.swz_padding_is_zero(orc, got_t, M, nblk, fmt)
    # one pass, one scale per block: the padded layout gathered to row-major equals the linear copy
    assert np.array_equal(checkers.gather_scales(orc, got_t, M, nblk, fmt, layout),
                          got_l.reshape(M, nblk))


# both producer forms (row-split below 256 rows, a workgroup per row above),
# M % 32 != 0 for TILED padding rows, nblk % 8 != 0 for padding blocks, and the
# 4096 x 4096 workload the benchmark times
SHAPES = [(1, 64), (8, 256), (33, 1024), (5, 5120), (70, 4096), (300, 1536), (257, 2560), (520, 5632),
          (2049, 512), (1000, 5120), (4096, 4096)]


@pytest.mark.parametrize("M,H", SHAPES)
@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("layout", [1, 2])
def test_both_layouts_bf16(orc, M, H, fmt, layout):
    if layout == 2 and M * H > 2 ** 22:
        pytest.skip("the 128 x 4 form is checked up to 4M elements")
    run_both(orc, M, H, fmt, seed=11 * M + H, use_gs=(fmt == 0), layout=layout)


@pytest.mark.parametrize("M,H", [(8, 256), (33, 1024), (300, 1536), (2049, 512)])
@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("layout", [1, 2])
def test_both_layouts_fp16(orc, M, H, fmt, layout):
    run_both(orc, M, H, fmt, seed=13 * M + H, use_gs=(fmt == 0), dtype=torch.float16, layout=layout)


def test_both_layouts_fp16_by_name(orc):
    M, H = 40, 640
    x, r, w = synth.producer_inputs(M, H, 5, dtype=torch.float16)
    r2 = r.clone()
    p1, t1, l1 = lb.lowbit_add_rmsnorm_quant_both_sf_fp16(dev_bf16(x), dev_bf16(r), dev_bf16(w), EPS, lb.MXFP4)
    p2, t2, l2 = lb.lowbit_add_rmsnorm_quant_both_sf(dev_bf16(x), dev_bf16(r2), dev_bf16(w), EPS, lb.MXFP4)
    torch.cuda.synchronize()
    assert torch.equal(p1, p2) and torch.equal(t1, t2) and torch.equal(l1, l2)


@pytest.mark.parametrize("layout", [1, 2])
def test_both_layouts_match_single_layout_calls(orc, layout):
    """The one-pass form writes what the padded-layout and the LINEAR calls write."""
    M, H = 300, 2048
    x, r, w = synth.producer_inputs(M, H, 21)
    xd, wd = dev_bf16(x), dev_bf16(w)
    gsd = dev_f32(0.75)
    res = [dev_bf16(r) for _ in range(3)]
    pb, tb, lb_ = lb.lowbit_add_rmsnorm_quant_both_sf(xd, res[0], wd, EPS, lb.NVFP4, layout, global_scale=gsd)
    pt, st = lb.lowbit_add_rmsnorm_quant(xd, res[1], wd, EPS, lb.NVFP4, layout, global_scale=gsd)
    pl, sl = lb.lowbit_add_rmsnorm_quant(xd, res[2], wd, EPS, lb.NVFP4, lb.LINEAR, global_scale=gsd)
    torch.cuda.synchronize()
    assert torch.equal(pb, pt) and torch.equal(pb, pl)
    assert torch.equal(tb, st) and torch.equal(lb_, sl)
    assert torch.equal(res[0], res[1]) and torch.equal(res[0], res[2])


def test_both_layouts_argument_errors():
    M, H = 4, 256
    x = torch.zeros((M, H), dtype=torch.bfloat16, device="cuda")
    r = x.clone()
    w = torch.ones(H, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lb.LowbitError):   # MXFP8 has no TILED layout
        lb.lowbit_add_rmsnorm_quant_both_sf(x, r, w, EPS, lb.MXFP8, out_packed=torch.empty(
            (M, H), dtype=torch.uint8, device="cuda"), out_sf=torch.empty(64, dtype=torch.uint8, device="cuda"))
    with pytest.raises(lb.LowbitError):   # the second copy is LINEAR: the first must be a padded layout
        lb.lowbit_add_rmsnorm_quant_both_sf(x, r, w, EPS, lb.MXFP4, lb.LINEAR)
    with pytest.raises(lb.LowbitError):   # global scale with MXFP4
        lb.lowbit_add_rmsnorm_quant_both_sf(x, r, w, EPS, lb.MXFP4, global_scale=dev_f32(1.0))
