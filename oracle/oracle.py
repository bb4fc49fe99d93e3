"""ctypes front end of the CPU oracle (oracle/lowbit_oracle.c).

TEST INFRASTRUCTURE ONLY.  Imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg; never by the product package.  All arrays are
numpy host arrays; bf16 and fp16 tensors travel as their uint16 bit patterns
(dtype BF16 = 0 or F16 = 1 says which).

Enum values: fmt NVFP4 = 0 (16-blocks, E4M3 scales), MXFP4 = 1 (32-blocks,
UE8M0 scales), MXFP8 = 2 (32-blocks, UE8M0 scales, E4M3 elements, one byte
each; LINEAR scales only, no GEMM), NVFP4_B32 = 3 (the NVFP4 rule on
32-blocks: E4M3 scales with the global scale; LINEAR scales only, no GEMM);
layout LINEAR = 0, TILED = 1, SWZ128 = 2 (the page's 128 x 4 swizzle); epilogue NONE = 0, BIAS = 1,
RESIDUAL = 2, BIAS_RESIDUAL = 3, BIAS_GELU = 4.
"""
import ctypes
import os

import numpy as np

from . import build as _build

NVFP4, MXFP4, MXFP8, NVFP4_B32 = 0, 1, 2, 3
LINEAR, TILED, SWZ128 = 0, 1, 2
EPI_NONE, EPI_BIAS, EPI_RESIDUAL, EPI_BIAS_RESIDUAL, EPI_BIAS_GELU = 0, 1, 2, 3, 4
BF16, F16 = 0, 1

_lib = None

_u8p = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
_u16p = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")
_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int


def block_size(fmt: int) -> int:
    return 16 if fmt == NVFP4 else 32


def row_bytes(fmt: int, n: int) -> int:
    """Bytes of a packed row of n elements: two FP4 codes per byte, one MXFP8 byte each."""
    return n if fmt == MXFP8 else n // 2


def lib():
    """Load the oracle library, compiling it first if it is not built yet."""
    global _lib
    if _lib is not None:
        return _lib
    if (not os.path.exists(_build.LIB)
            or os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC)):
        _build.build()
    L = ctypes.CDLL(_build.LIB)
    L.orc_bf16_to_f32.restype = ctypes.c_float
    L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
    L.orc_f32_to_bf16.restype = ctypes.c_uint16
    L.orc_f32_to_bf16.argtypes = [ctypes.c_float]
    L.orc_e2m1_value.restype = ctypes.c_double
    L.orc_e2m1_value.argtypes = [ctypes.c_uint8]
    L.orc_e2m1_encode.restype = ctypes.c_uint8
    L.orc_e2m1_encode.argtypes = [ctypes.c_float]
    L.orc_e4m3_value.restype = ctypes.c_double
    L.orc_e4m3_value.argtypes = [ctypes.c_uint8]
    L.orc_e4m3_encode.restype = ctypes.c_uint8
    L.orc_e4m3_encode.argtypes = [ctypes.c_float]
    L.orc_ue8m0_value.restype = ctypes.c_double
    L.orc_ue8m0_value.argtypes = [ctypes.c_uint8]
    L.orc_sf_bytes.restype = _i64
    L.orc_sf_bytes.argtypes = [_i64, _i64, _int, _int]
    L.orc_sf_offset.restype = _i64
    L.orc_sf_offset.argtypes = [_i64, _i64, _i64, _int, _int]
    L.orc_sf_convert.restype = None
    L.orc_sf_convert.argtypes = [_u8p, _int, _u8p, _int, _i64, _i64, _int]
    L.orc_encode_with_scale.restype = None
    L.orc_encode_with_scale.argtypes = [_f32p, _int, _int, ctypes.c_float, ctypes.c_uint8, _u8p, _vp]
    L.orc_add_rmsnorm_quant.restype = _int
    L.orc_f16_to_f32.restype = ctypes.c_float
    L.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
    L.orc_f32_to_f16.restype = ctypes.c_uint16
    L.orc_f32_to_f16.argtypes = [ctypes.c_float]
    L.orc_add_rmsnorm_quant_dt.restype = _int
    L.orc_add_rmsnorm_quant_dt.argtypes = [_u16p, _u16p, _u16p, _i64, _i64, ctypes.c_float, _int, _int,
                                           ctypes.c_float, _u8p, _u8p, _vp, _vp, _vp, _vp, _vp, _int]
    L.orc_quantize_dt.restype = _int
    L.orc_quantize_dt.argtypes = [_u16p, _i64, _i64, _int, _int, ctypes.c_float, _u8p, _u8p, _vp, _int]
    L.orc_add_rmsnorm_quant.argtypes = [_u16p, _u16p, _u16p, _i64, _i64, ctypes.c_float, _int, _int,
                                        ctypes.c_float, _u8p, _u8p, _vp, _vp, _vp, _vp, _vp]
    L.orc_quantize.restype = _int
    L.orc_quantize.argtypes = [_u16p, _i64, _i64, _int, _int, ctypes.c_float, _u8p, _u8p, _vp]
    L.orc_dequantize.restype = _int
    L.orc_dequantize.argtypes = [_u8p, _u8p, _i64, _i64, _int, _int, ctypes.c_float, _vp, _vp]
    L.orc_dequantize_dt.restype = _int
    L.orc_dequantize_dt.argtypes = [_u8p, _u8p, _i64, _i64, _int, _int, ctypes.c_float, _vp, _vp, _int]
    L.orc_gemm.restype = _int
    L.orc_gemm.argtypes = [_u8p, _u8p, _u8p, _u8p, _i64, _i64, _i64, _int, _int, _int,
                           ctypes.c_double, _int, _vp, _vp, _f64p, _vp]
    L.orc_gemm_entries.restype = _int
    L.orc_gemm_entries.argtypes = [_u8p, _u8p, _u8p, _u8p, _i64, _i64, _i64, _int, _int, _int,
                                   ctypes.c_double, _int, _vp, _vp, _i64, _i64p, _i64p, _f64p, _vp]
    L.orc_gemm_gelu_fp4.restype = _int
    L.orc_gemm_gelu_fp4.argtypes = [_u8p, _u8p, _u8p, _u8p, _i64, _i64, _i64, _int, _int, _int,
                                    ctypes.c_double, _u16p, ctypes.c_float, _int, _u8p, _u8p,
                                    _vp, _vp, _vp, _vp, _vp]
    L.orc_rope_quant.restype = _int
    L.orc_rope_quant.argtypes = [_u16p, _i64p, _f32p, _i64, _i64, _i64, _i64, _i64, _int, _int, _u8p, _u8p,
                                 _vp, _vp]
    L.orc_gemm_fp8_out.restype = _int
    L.orc_gemm_fp8_out.argtypes = [_u8p, _u8p, _u8p, _u8p, _i64, _i64, _i64, _int, _int, _int,
                                   ctypes.c_double, _int, _u8p, _u8p, _vp, _vp]
    L.orc_mxfp8_encode_blocks.restype = None
    L.orc_mxfp8_encode_blocks.argtypes = [_f32p, _i64, _u8p, _u8p]
    L.orc_num_threads.restype = _int
    L.orc_num_threads.argtypes = []
    L.orc_set_num_threads.restype = None
    L.orc_set_num_threads.argtypes = [_int]
    _lib = L
    return L


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# --- scalar formats -------------------------------------------------------------------------

def e2m1_value(code: int) -> float:
    return lib().orc_e2m1_value(code)


def e2m1_encode(v: float) -> int:
    return lib().orc_e2m1_encode(v)


def e4m3_value(b: int) -> float:
    return lib().orc_e4m3_value(b)


def e4m3_encode(v: float) -> int:
    return lib().orc_e4m3_encode(v)


def ue8m0_value(b: int) -> float:
    return lib().orc_ue8m0_value(b)


def f32_to_bf16(v: float) -> int:
    return lib().orc_f32_to_bf16(v)


def bf16_to_f32(b: int) -> float:
    return lib().orc_bf16_to_f32(b)


def f32_to_f16(v: float) -> int:
    return lib().orc_f32_to_f16(v)


def f16_to_f32(b: int) -> float:
    return lib().orc_f16_to_f32(b)


def sf_bytes(rows: int, k: int, fmt: int, layout: int) -> int:
    return lib().orc_sf_bytes(rows, k, fmt, layout)


def sf_offset(row: int, kb: int, nblk: int, fmt: int, layout: int) -> int:
    return lib().orc_sf_offset(row, kb, nblk, fmt, layout)


def sf_convert(sf, rows: int, k: int, fmt: int, src_layout: int, dst_layout: int):
    """Scale bytes of a (rows, k) operand in dst_layout, from src_layout."""
    src = _c(sf, np.uint8)
    assert src.size >= sf_bytes(rows, k, fmt, src_layout)
    out = np.empty(sf_bytes(rows, k, fmt, dst_layout), dtype=np.uint8)
    lib().orc_sf_convert(src, src_layout, out, dst_layout, rows, k, fmt)
    return out


def encode_with_scale(y, fmt: int, gs: float, sbyte: int, with_v: bool = False):
    """Codes of the block y under a given scale byte (and the pre-rounding v)."""
    y = _c(y, np.float32)
    out = np.zeros(y.size, dtype=np.uint8)
    v = np.zeros(y.size, dtype=np.float32)
    lib().orc_encode_with_scale(y, y.size, fmt, gs, sbyte, out, _ptr(v))
    return (out, v) if with_v else out


# --- tensor entry points --------------------------------------------------------------------

def add_rmsnorm_quant(x, residual, weight, eps, fmt, layout, gs=1.0, diag=False, dtype=BF16):
    """Fused producer.  x, residual: uint16 (M, H) bf16 bits (fp16 bits with
    dtype F16); weight uint16 (H,).
    Returns a dict with the updated residual, packed codes, scales and, when
    diag is set, y / v / amax / s_pre / rstd."""
    x = _c(x, np.uint16)
    res = np.array(residual, dtype=np.uint16, copy=True, order="C")
    w = _c(weight, np.uint16)
    M, H = x.shape
    B = block_size(fmt)
    packed = np.zeros((M, row_bytes(fmt, H)), dtype=np.uint8)
    sf = np.zeros(sf_bytes(M, H, fmt, layout), dtype=np.uint8)
    d = {}
    if diag:
        d = dict(y=np.zeros((M, H), np.float32), v=np.zeros((M, H), np.float32),
                 amax=np.zeros((M, H // B), np.float32), spre=np.zeros((M, H // B), np.float32),
                 rstd=np.zeros(M, np.float32))
    rc = lib().orc_add_rmsnorm_quant_dt(
        x, res, w, M, H, eps, fmt, layout, gs, packed, sf,
        _ptr(d.get("y")), _ptr(d.get("v")), _ptr(d.get("amax")), _ptr(d.get("spre")),
        _ptr(d.get("rstd")), dtype)
    if rc:
        raise ValueError(f"oracle add_rmsnorm_quant rejected its arguments (rc={rc})")
    out = dict(residual=res, packed=packed, sf=sf)
    out.update(d)
    return out


def quantize(x, fmt, layout, gs=1.0, diag=False, dtype=BF16):
    """Quantizer.  x: uint16 (rows, K) bf16 bits (fp16 bits with dtype F16)."""
    x = _c(x, np.uint16)
    rows, K = x.shape
    packed = np.zeros((rows, row_bytes(fmt, K)), dtype=np.uint8)
    sf = np.zeros(sf_bytes(rows, K, fmt, layout), dtype=np.uint8)
    spre = np.zeros((rows, K // block_size(fmt)), np.float32) if diag else None
    rc = lib().orc_quantize_dt(x, rows, K, fmt, layout, gs, packed, sf, _ptr(spre), dtype)
    if rc:
        raise ValueError(f"oracle quantize rejected its arguments (rc={rc})")
    return (packed, sf, spre) if diag else (packed, sf)


def rope_quant(x, positions, rope, heads, fmt, layout, diag=False):
    """Inverse RoPE + MX quantization (the vLLM fused_wo_a page's activation
    quant stage).  x: uint16 bf16 bits (T, heads, D); positions: int64 (T);
    rope: fp32 (P, R), each row cos || sin.  Returns packed (T*heads, D or
    D/2), scales, and with diag the rotated fp32 rows and the floored block
    maxima."""
    x = _c(x, np.uint16)
    positions = _c(positions, np.int64)
    rope = _c(rope, np.float32)
    T, H, D = x.shape
    assert H == heads
    P, R = rope.shape if rope.size else (0, 0)
    rows = T * heads
    packed = np.zeros((rows, row_bytes(fmt, D)), np.uint8)
    sf = np.zeros(sf_bytes(rows, D, fmt, layout), np.uint8)
    y = np.zeros((rows, D), np.float32) if diag else None
    am = np.zeros((rows, D // 32), np.float32) if diag else None
    rc = lib().orc_rope_quant(x, positions, rope if rope.size else np.zeros(1, np.float32), T, heads, D, R,
                              P, fmt, layout, packed, sf, _ptr(y), _ptr(am))
    if rc:
        raise ValueError(f"oracle rope_quant rejected its arguments (rc={rc})")
    return (packed, sf, y, am) if diag else (packed, sf)


def dequantize(packed, sf, rows, K, fmt, layout, gs=1.0, dtype=BF16):
    """Dequantizer: bf16 bits (fp16 bits with dtype F16) and the binary64 values."""
    packed = _c(packed, np.uint8)
    sf = _c(sf, np.uint8)
    out = np.zeros((rows, K), dtype=np.uint16)
    f64 = np.zeros((rows, K), dtype=np.float64)
    rc = lib().orc_dequantize_dt(packed, sf, rows, K, fmt, layout, gs, _ptr(out), _ptr(f64), dtype)
    if rc:
        raise ValueError(f"oracle dequantize rejected its arguments (rc={rc})")
    return out, f64


def gemm(a, b, sfa, sfb, M, N, K, fmt, layout_a, layout_b, alpha=1.0, epi=EPI_NONE,
         bias=None, residual=None):
    """Reference D = epilogue(alpha * Ahat . Bhat^T) in binary64 and its L1 budget."""
    a, b, sfa, sfb = (_c(t, np.uint8) for t in (a, b, sfa, sfb))
    bias = None if bias is None else _c(bias, np.uint16)
    residual = None if residual is None else _c(residual, np.uint16)
    ref = np.zeros((M, N), np.float64)
    l1 = np.zeros((M, N), np.float64)
    rc = lib().orc_gemm(a, b, sfa, sfb, M, N, K, fmt, layout_a, layout_b, alpha, epi,
                        _ptr(bias), _ptr(residual), ref, _ptr(l1))
    if rc:
        raise ValueError(f"oracle gemm rejected its arguments (rc={rc})")
    return ref, l1


def gemm_entries(a, b, sfa, sfb, M, N, K, fmt, layout_a, layout_b, idx_m, idx_n, alpha=1.0,
                 epi=EPI_NONE, bias=None, residual=None):
    a, b, sfa, sfb = (_c(t, np.uint8) for t in (a, b, sfa, sfb))
    bias = None if bias is None else _c(bias, np.uint16)
    residual = None if residual is None else _c(residual, np.uint16)
    idx_m = _c(idx_m, np.int64)
    idx_n = _c(idx_n, np.int64)
    ref = np.zeros(idx_m.size, np.float64)
    l1 = np.zeros(idx_m.size, np.float64)
    rc = lib().orc_gemm_entries(a, b, sfa, sfb, M, N, K, fmt, layout_a, layout_b, alpha, epi,
                                _ptr(bias), _ptr(residual), idx_m.size, idx_m, idx_n, ref, _ptr(l1))
    if rc:
        raise ValueError(f"oracle gemm_entries rejected its arguments (rc={rc})")
    return ref, l1


def gemm_gelu_fp4(a, b, sfa, sfb, M, N, K, fmt, layout_a, layout_b, alpha, bias, gs_out,
                  out_layout, diag=False):
    a, b, sfa, sfb = (_c(t, np.uint8) for t in (a, b, sfa, sfb))
    bias = _c(bias, np.uint16)
    packed = np.zeros((M, N // 2), np.uint8)
    sf = np.zeros(sf_bytes(M, N, NVFP4, out_layout), np.uint8)
    d = {}
    if diag:
        d = dict(y=np.zeros((M, N), np.float32), v=np.zeros((M, N), np.float32),
                 l1=np.zeros((M, N), np.float64), spre=np.zeros((M, N // 16), np.float32),
                 amax=np.zeros((M, N // 16), np.float32))
    rc = lib().orc_gemm_gelu_fp4(a, b, sfa, sfb, M, N, K, fmt, layout_a, layout_b, alpha, bias,
                                 gs_out, out_layout, packed, sf, _ptr(d.get("y")),
                                 _ptr(d.get("v")), _ptr(d.get("l1")), _ptr(d.get("spre")),
                                 _ptr(d.get("amax")))
    if rc:
        raise ValueError(f"oracle gemm_gelu_fp4 rejected its arguments (rc={rc})")
    out = dict(packed=packed, sf=sf)
    out.update(d)
    return out


def gemm_fp8_out(a, b, sfa, sfb, M, N, K, fmt, layout_a, layout_b, alpha, out_layout, diag=False):
    """GEMM with the FP8 output epilogue: bf16(alpha * A.B^T) quantized as
    MXFP8 along N.  Returns packed (M, N), scales, and with diag the
    unrounded binary64 values and their L1 budget."""
    a, b, sfa, sfb = (_c(t, np.uint8) for t in (a, b, sfa, sfb))
    packed = np.zeros((M, N), np.uint8)
    sf = np.zeros(sf_bytes(M, N, MXFP8, out_layout), np.uint8)
    ref = np.zeros((M, N), np.float64) if diag else None
    l1 = np.zeros((M, N), np.float64) if diag else None
    rc = lib().orc_gemm_fp8_out(a, b, sfa, sfb, M, N, K, fmt, layout_a, layout_b, alpha, out_layout, packed, sf,
                                _ptr(ref), _ptr(l1))
    if rc:
        raise ValueError(f"oracle gemm_fp8_out rejected its arguments (rc={rc})")
    return (packed, sf, ref, l1) if diag else (packed, sf)


def mxfp8_encode_blocks(y, sbytes):
    """E4M3 codes of 32-value blocks y (nblocks, 32) under the scale bytes."""
    y = _c(y, np.float32)
    sbytes = _c(sbytes, np.uint8)
    codes = np.zeros(y.shape, np.uint8)
    lib().orc_mxfp8_encode_blocks(y, sbytes.size, sbytes, codes)
    return codes


def num_threads() -> int:
    return lib().orc_num_threads()


def set_num_threads(n: int) -> None:
    """Threads of the following oracle calls (OpenMP)."""
    lib().orc_set_num_threads(int(n))
