"""Parity rules between the HIP path and the CPU oracle.

* Residuals and the quantizer's codes/scales: bit-exact.
* Producer codes and scales: bit-exact, except where the oracle's fp32
  pre-rounding value lies within 2^-20 (relative) of a rounding boundary:
    - codes: v_i near an E2M1 midpoint (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5);
    - NVFP4 scales: s_pre near a midpoint of two consecutive E4M3 values;
    - MXFP4 scales: amax near a power of two (the binade decides the byte).
  When a scale byte differs inside its window the block's codes are
  re-derived (by the oracle) from the device's scale byte and must then match
  (again modulo the code window).  Such cases are counted and reported.
* GEMM bf16 outputs: |gpu - ref| <= 2^-7 |ref| + 1e-6 * L1, with ref the
  oracle's unrounded binary64 value and L1 = |alpha| sum_k |a_k b_k|.
* FP4-output epilogue: as the producer, with the window widened by the GEMM's
  own accumulation budget and by the device GELU's error:
  2^-20 |y| + GELU_REL |y| + 1.13e-6 L1 in units of y (1.13 bounds the slope
  of GELU; GELU_REL bounds the fp32 evaluation's relative error under a
  one-ulp model of the hardware reciprocal and power of two, see
  tests/test_gelu_form.py).
"""
import numpy as np

E2M1_MIDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
WIN = 2.0 ** -20
GELU_REL = 4.5e-6   # relative error bound of the device GELU for z >= -9


def fp4_out_windows(ref, gs_out, rows, N):
    """Extra window terms of the FP4-output epilogue, from the oracle's
    diagnostics (y, v, l1): codes in units of v, scales in units of s_pre."""
    l1 = ref["l1"]
    inv = np.abs(ref["v"]) / np.maximum(np.abs(ref["y"]), 1e-30)
    code_extra = 1.13e-6 * l1 * inv + GELU_REL * np.abs(ref["v"])
    blk_l1 = l1.reshape(rows, N // 16, 16).max(axis=2)
    scale_extra = 1.13e-6 * blk_l1 * gs_out / 6.0 + GELU_REL * np.abs(ref["spre"])
    return code_extra, scale_extra


def unpack_codes(packed):
    p = np.asarray(packed, dtype=np.uint8)
    c = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.uint8)
    c[..., 0::2] = p & 15
    c[..., 1::2] = p >> 4
    return c


def tiled_in_group(fmt, r, j):
    """Byte of block j (0..7) of row r inside its 256-byte TILED group: one
    word per (lane half, row) holding the four blocks that lane half reads
    (MXFP4: blocks {2h, 2h+1, 2h+4, 2h+5} in word h*32 + r; NVFP4: blocks
    4c..4c+3 in word c*32 + r)."""
    if fmt == 0:
        return ((j // 4) * 32 + r % 32) * 4 + j % 4
    return (((j // 2) % 2) * 32 + r % 32) * 4 + (j % 2) + 2 * (j // 4)


def swz_offsets(orc, rows, nblk, fmt):
    """Byte offsets of the (rows, nblk) scales in the 128 x 4 swizzle, from
    the oracle's layout function."""
    return np.array([[orc.sf_offset(m, kb, nblk, fmt, orc.SWZ128) for kb in range(nblk)] for m in range(rows)],
                    dtype=np.int64).reshape(rows, nblk)


def gather_scales(orc, sf, rows, nblk, fmt, layout):
    """(rows, nblk) scale bytes from a buffer in any layout."""
    sf = np.asarray(sf, dtype=np.uint8)
    if layout == orc.LINEAR:
        return sf[: rows * nblk].reshape(rows, nblk)
    if layout == orc.SWZ128:
        return sf[swz_offsets(orc, rows, nblk, fmt)]
    r = np.arange(rows)[:, None]
    kb = np.arange(nblk)[None, :]
    ktiles = (nblk + 7) // 8
    j = kb % 8
    off = ((r // 32) * ktiles + kb // 8) * 256 + tiled_in_group(fmt, r, j)
    return sf[off]


def tiled_padding_is_zero(orc, sf, rows, nblk, fmt):
    sf = np.asarray(sf, dtype=np.uint8)
    used = np.zeros(sf.size, bool)
    r = np.arange(rows)[:, None]
    kb = np.arange(nblk)[None, :]
    ktiles = (nblk + 7) // 8
    j = kb % 8
    off = ((r // 32) * ktiles + kb // 8) * 256 + tiled_in_group(fmt, r, j)
    used[off.ravel()] = True
    return not np.any(sf[~used])


def swz_padding_is_zero(orc, sf, rows, nblk, fmt):
    sf = np.asarray(sf, dtype=np.uint8)
    used = np.zeros(sf.size, bool)
    used[swz_offsets(orc, rows, nblk, fmt).ravel()] = True
    return not np.any(sf[~used])


def near_e2m1_boundary(v, extra=0.0):
    a = np.abs(np.asarray(v, dtype=np.float64))
    d = np.min(np.abs(a[..., None] - E2M1_MIDS), axis=-1)
    return d <= WIN * a + extra


_E4M3_MIDS = None


def e4m3_midpoints(orc):
    global _E4M3_MIDS
    if _E4M3_MIDS is None:
        vals = np.array([orc.e4m3_value(c) for c in range(0x7F)])
        _E4M3_MIDS = 0.5 * (vals[:-1] + vals[1:])
    return _E4M3_MIDS


def near_scale_boundary(orc, fmt, pre, extra=0.0):
    pre = np.abs(np.asarray(pre, dtype=np.float64))
    if fmt == orc.NVFP4:
        mids = e4m3_midpoints(orc)
        idx = np.clip(np.searchsorted(mids, pre), 1, len(mids) - 1)
        d = np.minimum(np.abs(pre - mids[idx - 1]), np.abs(pre - mids[idx]))
        return d <= WIN * pre + extra
    with np.errstate(divide="ignore"):
        p2 = np.exp2(np.round(np.log2(np.where(pre > 0, pre, 1.0))))
    return (pre > 0) & (np.abs(pre - p2) <= WIN * pre + extra)


class Report(dict):
    def ok(self):
        return self["hard_failures"] == 0


def compare_quantized(orc, fmt, gs, gpu_packed, gpu_sf, orc_packed, orc_sf, y, v, spre, rows, K,
                      layout, code_extra=None, scale_extra=None):
    """Compare device codes/scales with the oracle's under the window rule.
    y, v: oracle fp32 values (rows, K); spre: oracle pre-rounding scale values
    (rows, K/B) (s_pre for NVFP4, amax for MXFP4).  code_extra / scale_extra:
    optional absolute window widening (arrays broadcastable to v / spre)."""
    B = 16 if fmt == orc.NVFP4 else 32
    nblk = K // B
    gs_ = gather_scales(orc, gpu_sf, rows, nblk, fmt, layout)
    os_ = gather_scales(orc, orc_sf, rows, nblk, fmt, layout)
    gc = unpack_codes(np.asarray(gpu_packed).reshape(rows, K // 2))
    oc = unpack_codes(np.asarray(orc_packed).reshape(rows, K // 2))
    rep = Report(blocks=rows * nblk, scale_diff_in_window=0, code_diff_in_window=0, hard_failures=0,
                 examples=[])
    sdiff = gs_ != os_
    if np.any(sdiff):
        v = np.array(v, dtype=np.float32, copy=True)
        near = near_scale_boundary(orc, fmt, spre, 0.0 if scale_extra is None else scale_extra)
        bad = sdiff & ~near
        rep["hard_failures"] += int(bad.sum())
        for m, kb in zip(*np.nonzero(bad)):
            if len(rep["examples"]) < 5:
                rep["examples"].append(("scale", int(m), int(kb), int(gs_[m, kb]), int(os_[m, kb]),
                                        float(spre[m, kb])))
        # re-derive the codes of in-window blocks from the device's scale byte
        for m, kb in zip(*np.nonzero(sdiff & near)):
            rep["scale_diff_in_window"] += 1
            sl = slice(kb * B, (kb + 1) * B)
            codes, vv = orc.encode_with_scale(y[m, sl], fmt, gs, int(gs_[m, kb]), with_v=True)
            oc[m, sl] = codes
            v[m, sl] = vv
    cdiff = gc != oc
    if np.any(cdiff):
        extra = 0.0 if code_extra is None else np.broadcast_to(code_extra, v.shape)[cdiff]
        near = near_e2m1_boundary(v[cdiff], extra)
        rep["code_diff_in_window"] += int(near.sum())
        rep["hard_failures"] += int((~near).sum())
        idx = np.argwhere(cdiff)[~near][:5]
        for m, k in idx:
            rep["examples"].append(("code", int(m), int(k), int(gc[m, k]), int(oc[m, k]), float(v[m, k])))
    return rep


def gemm_within_tolerance(gpu, ref, l1, l1_coef=1e-6):
    """Elementwise GEMM tolerance rule; returns (ok_mask, worst ratio).
    l1_coef: the accumulation term (1e-6; the scaled FP8 MFMA format states
    a wider one)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    tol = 2.0 ** -7 * np.abs(ref) + l1_coef * l1
    err = np.abs(gpu - ref)
    ok = err <= tol
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(tol > 0, err / tol, np.where(err > 0, np.inf, 0.0))
    return ok, float(np.max(ratio)) if ratio.size else 0.0


# --- FP8-output epilogue ---------------------------------------------------------------------
# The device rounds its fp32 sum alpha * t to bf16 and quantizes the bf16
# values; the oracle does the same from the binary64 sum.  t differs from the
# exact sum by the fp32 accumulation (<= 1e-6 L1) and alpha * t by one more fp32
# rounding, so the device's bf16 value is one of the bf16 roundings of
# [ref - e, ref + e], e = 2^-22 |ref| + 1e-6 L1.  Rounding is monotone, so
# the block maximum, the scale byte (a function of the binade of the block
# maximum) and each code (under the device's scale byte) must lie between
# those of the interval's ends.

def bf16_of_f32(x):
    """Round-to-nearest-even bf16 value (as float64) of float32 values."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def mx8_scale_byte(amax):
    """Scale byte of an MXFP8 block maximum: max(biased exponent - 8, 0)."""
    eb = (np.ascontiguousarray(amax, dtype=np.float32).view(np.uint32) >> 23) & 0xFF
    return np.maximum(eb.astype(np.int64) - 8, 0)


def gather_mx8_scales(orc, sf, rows, nblk, layout):
    sf = np.asarray(sf, dtype=np.uint8)
    off = (np.arange(rows * nblk, dtype=np.int64).reshape(rows, nblk) if layout == orc.LINEAR
           else swz_offsets(orc, rows, nblk, orc.MXFP8))
    return sf[off], off


def compare_fp8_out(orc, gpu_packed, gpu_sf, orc_packed, orc_sf, ref, l1, rows, N, layout, l1_coef=1e-6):
    """Device FP8-output codes and scales against the oracle's under the
    interval rule above; reports exact matches and hard failures, and (for a
    padded layout) that every byte outside the covered blocks is zero."""
    nblk = N // 32
    ref = np.asarray(ref, dtype=np.float64)
    e = 2.0 ** -22 * np.abs(ref) + l1_coef * np.asarray(l1, dtype=np.float64)
    lo = bf16_of_f32((ref - e).astype(np.float32))
    hi = bf16_of_f32((ref + e).astype(np.float32))
    straddle = (lo <= 0) & (hi >= 0)
    amin = np.where(straddle, 0.0, np.minimum(np.abs(lo), np.abs(hi)))
    amax = np.maximum(np.abs(lo), np.abs(hi))
    b_lo = mx8_scale_byte(amin.reshape(rows, nblk, 32).max(axis=2))
    b_hi = mx8_scale_byte(amax.reshape(rows, nblk, 32).max(axis=2))
    gs, off = gather_mx8_scales(orc, gpu_sf, rows, nblk, layout)
    os_, _ = gather_mx8_scales(orc, orc_sf, rows, nblk, layout)
    gs = gs.astype(np.int64)
    rep = Report(blocks=rows * nblk, scale_diff=int((gs != os_).sum()), code_diff=0, hard_failures=0,
                 padding_nonzero=0, examples=[])
    bad_s = (gs < b_lo) | (gs > b_hi)
    rep["hard_failures"] += int(bad_s.sum())
    for m, kb in list(zip(*np.nonzero(bad_s)))[:5]:
        rep["examples"].append(("scale", int(m), int(kb), int(gs[m, kb]), int(os_[m, kb]), int(b_lo[m, kb]),
                                int(b_hi[m, kb])))
    gp = np.asarray(gpu_packed, dtype=np.uint8).reshape(rows, N)
    op = np.asarray(orc_packed, dtype=np.uint8).reshape(rows, N)
    rep["code_diff"] = int((gp != op).sum())
    sb = gs.astype(np.uint8).reshape(-1)
    c_lo = orc.mxfp8_encode_blocks(lo.reshape(-1, 32).astype(np.float32), sb).reshape(rows, N)
    c_hi = orc.mxfp8_encode_blocks(hi.reshape(-1, 32).astype(np.float32), sb).reshape(rows, N)
    table = np.array([orc.e4m3_value(c) for c in range(256)])
    v_dev, v_lo, v_hi = table[gp], table[c_lo], table[c_hi]
    bad_c = ~((v_dev >= np.minimum(v_lo, v_hi)) & (v_dev <= np.maximum(v_lo, v_hi)))
    bad_c &= ~np.repeat(bad_s, 32, axis=1)            # a wrong scale is already counted
    rep["hard_failures"] += int(bad_c.sum())
    for m, k in np.argwhere(bad_c)[:5]:
        rep["examples"].append(("code", int(m), int(k), int(gp[m, k]), int(op[m, k]), float(ref[m, k])))
    if layout != orc.LINEAR:
        used = np.zeros(np.asarray(gpu_sf).size, bool)
        used[off.ravel()] = True
        rep["padding_nonzero"] = int(np.count_nonzero(np.asarray(gpu_sf)[~used]))
        rep["hard_failures"] += rep["padding_nonzero"]
    return rep
