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


def gather_scales(orc, sf, rows, nblk, fmt, layout):
    """(rows, nblk) scale bytes from a buffer in either layout."""
    sf = np.asarray(sf, dtype=np.uint8)
    if layout == orc.LINEAR:
        return sf[: rows * nblk].reshape(rows, nblk)
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


def gemm_within_tolerance(gpu, ref, l1):
    """Elementwise GEMM tolerance rule; returns (ok_mask, worst ratio)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    tol = 2.0 ** -7 * np.abs(ref) + 1e-6 * l1
    err = np.abs(gpu - ref)
    ok = err <= tol
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(tol > 0, err / tol, np.where(err > 0, np.inf, 0.0))
    return ok, float(np.max(ratio)) if ratio.size else 0.0
