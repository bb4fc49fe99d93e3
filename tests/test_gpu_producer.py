"""GPU parity of the memory-bound kernels against the CPU oracle: the fused
add + RMSNorm + FP4 producer, the quantizer and the dequantizer.  Calls go
through the C ABI (ctypes binding); inputs are seeded and synthetic."""
import json
import os

import numpy as np
import pytest
import torch

import block_scaled_fp4_add_amd as lb
from block_scaled_fp4_add_amd import synth

from . import checkers
from .gpu_util import banner, dev_bf16, dev_f32, dev_u8, host_bits, host_u8

pytestmark = pytest.mark.gpu
EPS = 1e-6
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _odt(orc, dtype):
    return orc.F16 if dtype == torch.float16 else orc.BF16


def _gs_for(orc, x, r, w, M, H, dtype=torch.bfloat16):
    """NVFP4 global scale 6*448/amax(y), amax from the oracle's own y."""
    d = orc.add_rmsnorm_quant(synth.bits(x), synth.bits(r), synth.bits(w), EPS, orc.NVFP4, orc.LINEAR,
                              diag=True, dtype=_odt(orc, dtype))
    return float(np.float32(2688.0 / np.abs(d["y"]).max()))


def run_producer(orc, M, H, fmt, layout, seed, outliers=False, use_gs=False, dtype=torch.bfloat16):
    banner(f"producer M={M} H={H} fmt={fmt} layout={layout} seed={seed} gs={use_gs} dtype={dtype}")
    x, r, w = synth.producer_inputs(M, H, seed, outliers=outliers, dtype=dtype)
    gs = _gs_for(orc, x, r, w, M, H, dtype) if (use_gs and fmt == orc.NVFP4) else 1.0
    ref = orc.add_rmsnorm_quant(synth.bits(x), synth.bits(r), synth.bits(w), EPS, fmt, layout,
                                gs=gs, diag=True, dtype=_odt(orc, dtype))
    xd, rd, wd = dev_bf16(x), dev_bf16(r), dev_bf16(w)
    sf_n = lb.lowbit_sf_bytes(M, H, fmt, layout)
    packed = torch.full((M, H // 2), 0xAA, dtype=torch.uint8, device="cuda")
    sf = torch.full((sf_n,), 0xAA, dtype=torch.uint8, device="cuda")
    lb.lowbit_add_rmsnorm_quant(xd, rd, wd, EPS, fmt, layout,
                                global_scale=dev_f32(gs) if (use_gs and fmt == lb.NVFP4) else None,
                                out_packed=packed, out_sf=sf)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(rd), ref["residual"]), "residual must be the rounded x + r bit-exact"
    spre = ref["spre"] if fmt == orc.NVFP4 else ref["amax"]
    rep = checkers.compare_quantized(orc, fmt, gs, host_u8(packed), host_u8(sf), ref["packed"], ref["sf"],
                                     ref["y"], ref["v"], spre, M, H, layout)
    banner(f"  report {dict(rep)}")
    assert rep.ok(), rep
    if layout == orc.TILED:
        assert checkers.tiled_padding_is_zero(orc, host_u8(sf), M, H // (16 if fmt == 0 else 32), fmt)
    return rep


SMALL = [(8, 256), (1, 64), (3, 320), (33, 1024), (5, 5120), (1, 5120), (17, 17408), (2, 32768),
         (70, 4096)]


@pytest.mark.parametrize("M,H", SMALL)
@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("layout", [0, 1])
def test_producer_small(orc, M, H, fmt, layout):
    run_producer(orc, M, H, fmt, layout, seed=M * 7 + H, outliers=True, use_gs=(fmt == 0))


# Many rows: one workgroup per row (NW = ceil(H/1024) waves, two 16-byte
# vectors per thread).  Rows of 1..6 waves, with H % 1024 != 0 so that the
# second vector of some threads lies past the row's end; M % 32 != 0 for the
# TILED padding rows.  More than 1280 rows of 4096 < H <= 6144 take three
# vectors per thread in 4 waves: (4200, 6144), (1300, 4160) (the third vector
# of most threads past the row's end), (1281, 5632); (520, 5632) keeps two.
MANY_ROWS = [(256, 64), (300, 1536), (257, 2560), (2100, 3584), (520, 5632), (4200, 6144), (2049, 512),
         (4500, 4096), (256, 16384), (300, 11264), (1300, 4160), (1281, 5632)]


@pytest.mark.parametrize("M,H", MANY_ROWS)
@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("layout", [0, 1])
def test_producer_many_rows(orc, M, H, fmt, layout):
    run_producer(orc, M, H, fmt, layout, seed=M + 3 * H, outliers=True, use_gs=(fmt == 0))


# fp16 tensors (lowbit_add_rmsnorm_quant_fp16): both kernel forms, both
# formats and layouts, ragged rows of the workgroup form included
FP16_SHAPES = [(8, 256), (1, 5120), (33, 1024), (300, 1536), (2049, 512), (520, 5632), (4500, 4096)]


@pytest.mark.parametrize("M,H", FP16_SHAPES)
@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("layout", [0, 1])
def test_producer_fp16(orc, M, H, fmt, layout):
    run_producer(orc, M, H, fmt, layout, seed=M + 5 * H, outliers=True, use_gs=(fmt == 0),
                 dtype=torch.float16)


def test_producer_tiny_mxfp4_workload(orc):
    """8 rows x 256, MXFP4, linear scales (the tiny end-to-end workload)."""
    c = synth.TINY_MXFP4
    run_producer(orc, c["M"], c["H"], orc.MXFP4, orc.LINEAR, seed=c["seed"])


def test_producer_nvfp4_4096x4096_full(orc):
    """The memory-bound benchmark workload in full: 4096 x 4096, NVFP4 with
    1% outlier channels and the global scale 6*448/amax."""
    c = synth.NVFP4_PRODUCER
    rep = run_producer(orc, c["M"], c["H"], orc.NVFP4, orc.LINEAR, seed=c["seed"], outliers=True,
                       use_gs=True)
    # in-window differences must stay rare
    assert rep["code_diff_in_window"] + rep["scale_diff_in_window"] <= 0.001 * rep["blocks"]


def test_producer_chain_rows(orc):
    """Producer rows of the NVFP4 chain workload (H = 5120) at M = 1, 128, 2048, TILED scales."""
    c = synth.NVFP4_CHAIN
    for M in c["Ms"]:
        run_producer(orc, M, c["H"], orc.NVFP4, orc.TILED, seed=c["seed"] + M, outliers=True, use_gs=True)


def test_producer_constant_rows(orc):
    with open(os.path.join(GOLDEN, "producer_constant_rows.json")) as f:
        rows = json.load(f)["rows"]
    for row in rows:
        H = row["H"]
        for fmt in (0, 1):
            x = torch.full((1, H), row["c"], dtype=torch.bfloat16)
            r = torch.zeros((1, H), dtype=torch.bfloat16)
            w = torch.ones((H,), dtype=torch.bfloat16)
            packed, sf = lb.lowbit_add_rmsnorm_quant(dev_bf16(x), dev_bf16(r), dev_bf16(w), EPS, fmt, 0)
            want = row["nv"] if fmt == 0 else row["mx"]
            assert (host_u8(sf) == want["scale_byte"]).all()
            assert (checkers.unpack_codes(host_u8(packed)) == want["code"]).all()


def test_producer_empty_is_noop(orc):
    z = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    w = torch.ones(256, dtype=torch.bfloat16, device="cuda")
    p, s = lb.lowbit_add_rmsnorm_quant(z, z.clone(), w, EPS, 1, 0)
    assert p.numel() == 0


# --- quantize / dequantize ------------------------------------------------------------------

QSHAPES = [(1, 64), (7, 160), (41, 1536), (128, 5120), (5, 17408), (33, 256), (100, 96)]


@pytest.mark.parametrize("rows,K", QSHAPES)
@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("layout", [0, 1])
def test_quantize_bit_exact(orc, rows, K, fmt, layout):
    if K % (16 if fmt == 0 else 32):
        pytest.skip("K not a multiple of the block")
    banner(f"quantize rows={rows} K={K} fmt={fmt} layout={layout}")
    x = synth.activation(rows, K, seed=rows + K, outliers=True)
    gs = 3.25 if fmt == 0 else 1.0
    ref_p, ref_s = orc.quantize(synth.bits(x), fmt, layout, gs=gs)
    p, s = lb.lowbit_quantize(dev_bf16(x), fmt, layout, global_scale=dev_f32(gs) if fmt == 0 else None)
    torch.cuda.synchronize()
    assert np.array_equal(host_u8(p), ref_p)
    assert np.array_equal(host_u8(s), ref_s)


@pytest.mark.parametrize("rows,K", QSHAPES + [(300, 2560), (1000, 5120)])
@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("layout", [0, 1])
def test_quantize_fp16_bit_exact(orc, rows, K, fmt, layout):
    if K % (16 if fmt == 0 else 32):
        pytest.skip("K not a multiple of the block")
    banner(f"quantize fp16 rows={rows} K={K} fmt={fmt} layout={layout}")
    x = synth.activation(rows, K, seed=rows + 3 * K, outliers=True, dtype=torch.float16)
    gs = 3.25 if fmt == 0 else 1.0
    ref_p, ref_s = orc.quantize(synth.bits(x), fmt, layout, gs=gs, dtype=orc.F16)
    p, s = lb.lowbit_quantize_fp16(dev_bf16(x), fmt, layout, global_scale=dev_f32(gs) if fmt == 0 else None)
    torch.cuda.synchronize()
    assert np.array_equal(host_u8(p), ref_p)
    assert np.array_equal(host_u8(s), ref_s)


@pytest.mark.parametrize("rows", [1, 41, 128])
@pytest.mark.parametrize("K", [5120, 6144, 17408])
@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("layout", [0, 1, 2])
def test_bf16_entry_matches_the_fp16_chain(rows, K, fmt, layout):
    """The FlashRT README's validation gate at the decode widths: quantizing a
    bf16 tensor directly gives, byte for byte, what converting it to fp16 and
    quantizing that gives.  Values below fp16's normal range (|x| < 2^-14),
    which the conversion would round, are set to zero first, so the two
    inputs hold the same numbers."""
    banner(f"bf16 entry vs fp16 chain rows={rows} K={K} fmt={fmt} layout={layout}")
    x = synth.activation(rows, K, seed=rows * 7 + K, outliers=True)
    x = torch.where(x.float().abs() < 2.0 ** -14, torch.zeros_like(x), x)
    x16 = x.half()
    assert torch.equal(x16.float(), x.float())
    gs = dev_f32(5.5) if fmt == 0 else None
    p, s = lb.lowbit_quantize(dev_bf16(x), fmt, layout, global_scale=gs)
    p16, s16 = lb.lowbit_quantize_fp16(dev_bf16(x16), fmt, layout, global_scale=gs)
    torch.cuda.synchronize()
    assert torch.equal(p, p16) and torch.equal(s, s16)


def test_quantize_hand_blocks(orc):
    with open(os.path.join(GOLDEN, "hand_blocks.json")) as f:
        blocks = json.load(f)["blocks"]
    for blk in blocks:
        fmt = 0 if blk["fmt"] == "nvfp4" else 1
        x = torch.tensor(blk["x"], dtype=torch.float32).to(torch.bfloat16).reshape(1, -1)
        p, s = lb.lowbit_quantize(dev_bf16(x), fmt, 0,
                                  global_scale=dev_f32(blk["gs"]) if fmt == 0 else None)
        torch.cuda.synchronize()
        assert int(host_u8(s)[0]) == blk["scale_byte"], blk["name"]
        assert checkers.unpack_codes(host_u8(p))[0].tolist() == blk["codes"], blk["name"]


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("layout", [0, 1])
def test_dequantize_bit_exact(orc, fmt, layout):
    rows, K = 37, 512
    rng = np.random.default_rng(fmt * 2 + layout)
    packed = rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)
    nb = orc.sf_bytes(rows, K, fmt, layout)
    if fmt == 0:
        sf = rng.integers(0, 0x7F, nb, dtype=np.uint8)       # finite E4M3 (no NaN code)
        gs = 0.75
    else:
        sf = rng.integers(100, 150, nb, dtype=np.uint8)
        gs = 1.0
    want, _ = orc.dequantize(packed, sf, rows, K, fmt, layout, gs=gs)
    out = lb.lowbit_dequantize(dev_u8(packed), dev_u8(sf), fmt, layout,
                               global_scale=dev_f32(gs) if fmt == 0 else None)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(out), want)


@pytest.mark.parametrize("fmt,layout,gs", [(0, 0, 0.75), (0, 1, 0.01), (0, 2, 1.0), (1, 0, 1.0), (1, 1, 1.0),
                                           (1, 2, 1.0), (2, 0, 1.0), (3, 0, 3.0)])
@pytest.mark.parametrize("rows,K", [(37, 512), (300, 1024)])
def test_dequantize_fp16_bit_exact(orc, fmt, layout, gs, rows, K):
    """fp16 output ([FRT] dequantize_fp4_sfa_fp16) against the oracle, every
    value, with scales that take the results past fp16's largest value
    (infinity) and into its subnormals."""
    banner(f"dequantize fp16 fmt={fmt} layout={layout} gs={gs} rows={rows} K={K}")
    rng = np.random.default_rng(fmt * 8 + layout + rows)
    width = K if fmt == 2 else K // 2
    packed = rng.integers(0, 256, (rows, width), dtype=np.uint8)
    if fmt == 2:
        packed[(packed & 0x7F) == 0x7F] = 0x7E           # no E4M3 NaN codes
    nb = orc.sf_bytes(rows, K, fmt, layout)
    if fmt in (0, 3):
        sf = rng.integers(0, 0x7F, nb, dtype=np.uint8)   # finite E4M3 (no NaN code)
    else:
        sf = rng.integers(127 - 40, 127 + 26, nb, dtype=np.uint8)
    want, _ = orc.dequantize(packed, sf, rows, K, fmt, layout, gs=gs, dtype=orc.F16)
    out = lb.lowbit_dequantize_fp16(dev_u8(packed), dev_u8(sf), fmt, layout,
                                    global_scale=dev_f32(gs) if fmt in (0, 3) else None)
    torch.cuda.synchronize()
    assert out.dtype == torch.float16
    assert np.array_equal(host_bits(out), want)


def test_argument_errors_on_device():
    x = torch.zeros((4, 100), dtype=torch.bfloat16, device="cuda")
    p = torch.empty((4, 50), dtype=torch.uint8, device="cuda")
    s = torch.empty(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(lb.LowbitError) as e:
        lb.lowbit_quantize(x, 1, 0, out_packed=p, out_sf=s)          # K % 32 != 0
    assert e.value.status == 3
    with pytest.raises(lb.LowbitError) as e:
        lb.lowbit_quantize(x, 1, 0)          # no scale buffer can be sized: NULL -> invalid argument
    assert e.value.status == 1
    w = torch.ones(48, dtype=torch.bfloat16, device="cuda")
    x = torch.zeros((4, 48), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lb.LowbitError) as e:
        lb.lowbit_add_rmsnorm_quant(x, x.clone(), w, EPS, 0, 0)   # H < 64
    assert e.value.status == 3
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.ones(64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lb.LowbitError) as e:
        lb.lowbit_add_rmsnorm_quant(x, x.clone(), w, EPS, 1, 0, global_scale=dev_f32(1.0))
    assert e.value.status == 1


# --- MXFP8 (E4M3 elements, UE8M0 32-blocks, LINEAR scales) ----------------------------------

def _mxfp8_compare(orc, got_p, got_s, ref_p, ref_s, y):
    """Scales bit-exact except where amax lies within 2^-20 of a power of two;
    elements bit-exact except where the pre-rounding value lies within 2^-20
    relative of an E4M3 midpoint (re-derived from the device's scale byte)."""
    assert got_p.shape == ref_p.shape and got_s.shape == ref_s.shape
    bad = np.nonzero((got_s != ref_s))[0]
    for b in bad:   # scale differs: only allowed at a binade boundary, then re-encode
        blk = y.reshape(-1, 32)[b]
        amax = float(np.abs(blk).max())
        assert amax > 0 and abs(amax / 2.0 ** np.round(np.log2(amax)) - 1) <= 2.0 ** -20, b
        codes = orc.encode_with_scale(blk, orc.MXFP8, 1.0, int(got_s[b]))
        assert np.array_equal(codes, got_p.reshape(-1, 32)[b])
    ok = np.ones(ref_s.size, bool)
    ok[bad] = False
    gp, rp = got_p.reshape(-1, 32)[ok], ref_p.reshape(-1, 32)[ok]
    diff = np.nonzero(gp != rp)
    if diff[0].size:
        yb = y.reshape(-1, 32)[ok]
        X = np.ldexp(1.0, ref_s[ok].astype(np.int32) - 127)[:, None]
        v = (yb / X)[diff]
        # the two candidate codes must be neighbours and v within 2^-20 of their midpoint
        lo = np.array([orc.e4m3_value(int(c)) for c in rp[diff]])
        hi = np.array([orc.e4m3_value(int(c)) for c in gp[diff]])
        assert np.all(np.abs(v - (lo + hi) / 2) <= 2.0 ** -20 * np.abs(v)), (v, lo, hi)
    return diff[0].size + bad.size


MXFP8_SHAPES = [(8, 256), (1, 5120), (33, 1024), (300, 1536), (2049, 512), (4500, 4096), (5, 17408)]


@pytest.mark.parametrize("M,H", MXFP8_SHAPES)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_producer_mxfp8(orc, M, H, dtype):
    banner(f"producer mxfp8 M={M} H={H} dtype={dtype}")
    x, r, w = synth.producer_inputs(M, H, M + 7 * H, outliers=True, dtype=dtype)
    ref = orc.add_rmsnorm_quant(synth.bits(x), synth.bits(r), synth.bits(w), EPS, orc.MXFP8, orc.LINEAR,
                                diag=True, dtype=_odt(orc, dtype))
    rd = dev_bf16(r)
    p, s = lb.lowbit_add_rmsnorm_quant(dev_bf16(x), rd, dev_bf16(w), EPS, lb.MXFP8, lb.LINEAR)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(rd), ref["residual"])
    n = _mxfp8_compare(orc, host_u8(p), host_u8(s), ref["packed"], ref["sf"], ref["y"])
    assert n <= 0.001 * ref["sf"].size


@pytest.mark.parametrize("rows,K", [(1, 64), (7, 160), (41, 1536), (128, 5120), (300, 2560), (5, 17408)])
def test_quantize_mxfp8_bit_exact(orc, rows, K):
    banner(f"quantize mxfp8 rows={rows} K={K}")
    x = synth.activation(rows, K, seed=rows + 11 * K, outliers=True)
    ref_p, ref_s = orc.quantize(synth.bits(x), orc.MXFP8, orc.LINEAR)
    p, s = lb.lowbit_quantize(dev_bf16(x), lb.MXFP8, lb.LINEAR)
    torch.cuda.synchronize()
    assert np.array_equal(host_u8(p), ref_p)
    assert np.array_equal(host_u8(s), ref_s)


def test_dequantize_mxfp8_bit_exact(orc):
    rows, K = 37, 512
    rng = np.random.default_rng(8)
    packed = rng.integers(0, 256, (rows, K), dtype=np.uint8)
    packed[(packed & 0x7F) == 0x7F] = 0x7E          # no NaN codes
    sf = rng.integers(100, 150, orc.sf_bytes(rows, K, orc.MXFP8, orc.LINEAR), dtype=np.uint8)
    want, _ = orc.dequantize(packed, sf, rows, K, orc.MXFP8, orc.LINEAR)
    out = lb.lowbit_dequantize(dev_u8(packed), dev_u8(sf), lb.MXFP8, lb.LINEAR)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(out), want)


def test_mxfp8_element_encoding_exhaustive(orc):
    """Every bf16 value with |v| <= 510 (and -0), as elements of blocks that
    start with 448 (so e = 0 and v is encoded as it is; values above 448
    saturate): the device's E4M3 codes equal the oracle's nearest-even,
    saturating encoder's."""
    pos = np.arange(0, 0x43FF + 1, dtype=np.uint16)            # bf16 bit patterns 0 .. 510
    vals = np.concatenate([pos, pos | 0x8000]).astype(np.uint16)
    per = 31
    nblk = ((vals.size + per - 1) // per + 15) // 16 * 16        # rows of 16 blocks (512 elements)
    blocks = np.zeros((nblk, 32), np.uint16)
    blocks[:, 0] = 0x43E0                                        # 448
    flat = np.concatenate([vals, np.zeros(nblk * per - vals.size, np.uint16)])
    blocks[:, 1:] = flat.reshape(nblk, per)
    rows = blocks.reshape(-1, 32 * 16)
    x = synth.from_bits(rows)
    ref_p, ref_s = orc.quantize(synth.bits(x), orc.MXFP8, orc.LINEAR)
    p, s = lb.lowbit_quantize(dev_bf16(x), lb.MXFP8, lb.LINEAR)
    torch.cuda.synchronize()
    assert (ref_s == 127).all()
    assert np.array_equal(host_u8(s), ref_s)
    assert np.array_equal(host_u8(p), ref_p)


def test_producer_accepts_leading_dims(orc):
    """(batch, tokens, H) tensors are rows of H: the same bytes as the 2-D call."""
    x, r, w = synth.producer_inputs(24, 512, 77, outliers=True)
    r3 = dev_bf16(r).reshape(2, 12, 512).clone()
    p3, s3 = lb.lowbit_add_rmsnorm_quant(dev_bf16(x).reshape(2, 12, 512), r3, dev_bf16(w), EPS, lb.NVFP4,
                                         lb.LINEAR)
    r2 = dev_bf16(r)
    p2, s2 = lb.lowbit_add_rmsnorm_quant(dev_bf16(x), r2, dev_bf16(w), EPS, lb.NVFP4, lb.LINEAR)
    torch.cuda.synchronize()
    assert p3.shape == (2, 12, 256)
    assert torch.equal(p3.reshape(24, 256), p2) and torch.equal(s3, s2)
    assert torch.equal(r3.reshape(24, 512), r2)
    q3, t3 = lb.lowbit_quantize(dev_bf16(x).reshape(4, 6, 512), lb.MXFP4, lb.TILED)
    q2, t2 = lb.lowbit_quantize(dev_bf16(x), lb.MXFP4, lb.TILED)
    torch.cuda.synchronize()
    assert q3.shape == (4, 6, 256) and torch.equal(q3.reshape(24, 256), q2) and torch.equal(t3, t2)


def test_binding_rejects_short_buffers():
    """Buffers smaller than the contract needs are refused before any launch:
    a LINEAR-sized scale buffer handed over for the padded layouts, short
    packed outputs, a weight of the wrong length, short GEMM operands."""
    x = torch.zeros((40, 512), dtype=torch.bfloat16, device="cuda")
    w = torch.ones(512, dtype=torch.bfloat16, device="cuda")
    lin = torch.empty(lb.lowbit_sf_bytes(40, 512, lb.NVFP4, lb.LINEAR), dtype=torch.uint8, device="cuda")
    for layout in (lb.TILED, lb.SWZ128):
        with pytest.raises(ValueError):
            lb.lowbit_quantize(x, lb.NVFP4, layout, out_sf=lin)
        with pytest.raises(ValueError):
            lb.lowbit_add_rmsnorm_quant(x, x.clone(), w, EPS, lb.NVFP4, layout, out_sf=lin)
    with pytest.raises(ValueError):
        lb.lowbit_quantize(x, lb.NVFP4, lb.LINEAR, out_packed=torch.empty((40, 255), dtype=torch.uint8,
                                                                          device="cuda"))
    with pytest.raises(ValueError):
        lb.lowbit_add_rmsnorm_quant(x, x.clone(), w[:256], EPS, lb.NVFP4, lb.LINEAR)
    a, sa = lb.lowbit_quantize(x, lb.MXFP4, lb.TILED)
    with pytest.raises(ValueError):
        lb.lowbit_gemm_bf16(a, a, sa[:100], sa, fmt=lb.MXFP4, sfa_layout=lb.TILED, sfb_layout=lb.TILED)
    with pytest.raises(ValueError):
        lb.lowbit_gemm_bias_bf16(a, a, sa, sa, torch.zeros(39, dtype=torch.bfloat16, device="cuda"),
                                 fmt=lb.MXFP4, sfa_layout=lb.TILED, sfb_layout=lb.TILED)
    with pytest.raises(ValueError):
        lb.lowbit_gemm_residual_bf16(a, a, sa, sa, torch.zeros((40, 39), dtype=torch.bfloat16, device="cuda"),
                                     fmt=lb.MXFP4, sfa_layout=lb.TILED, sfb_layout=lb.TILED)
    with pytest.raises(ValueError):
        lb.lowbit_dequantize(a, sa[:10], lb.MXFP4, lb.TILED)
    torch.cuda.synchronize()


def test_dequantize_and_gemm_accept_leading_dims(orc):
    """A packed (batch, tokens, K/2) tensor is rows x K for the dequantizer
    and the GEMM (the shape lowbit_quantize returns for 3-D input)."""
    x = synth.activation(24, 512, 91, outliers=True)
    W = synth.weight(64, 512, 91)
    p3, s3 = lb.lowbit_quantize(dev_bf16(x).reshape(2, 12, 512), lb.NVFP4, lb.TILED)
    p2, s2 = lb.lowbit_quantize(dev_bf16(x), lb.NVFP4, lb.TILED)
    b, sb = lb.lowbit_quantize(dev_bf16(W), lb.NVFP4, lb.TILED)
    d3 = lb.lowbit_dequantize(p3, s3, lb.NVFP4, lb.TILED)
    d2 = lb.lowbit_dequantize(p2, s2, lb.NVFP4, lb.TILED)
    g3 = lb.lowbit_gemm_bf16(p3, b, s3, sb, fmt=lb.NVFP4, sfa_layout=lb.TILED, sfb_layout=lb.TILED)
    g2 = lb.lowbit_gemm_bf16(p2, b, s2, sb, fmt=lb.NVFP4, sfa_layout=lb.TILED, sfb_layout=lb.TILED)
    torch.cuda.synchronize()
    assert d3.shape == (2, 12, 512) and torch.equal(d3.reshape(24, 512), d2)
    assert g3.shape == (2, 12, 64) and torch.equal(g3.reshape(24, 64), g2)
