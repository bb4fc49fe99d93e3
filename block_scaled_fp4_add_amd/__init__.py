"""Python binding of liblowbit.so, the MI355X (gfx950) low-bit linear hot path.

Argument marshalling only: every step of the computation runs in the HIP
kernels of liblowbit.so (see include/lowbit.h for the contract of each call).
PyTorch supplies device memory and the current stream.  Outputs may be passed
in; when omitted they are allocated here (the C ABI itself never allocates).

If the native library is missing, every call raises: there is no fallback.
"""
import ctypes
import os

import numpy as np
import torch

NVFP4, MXFP4, MXFP8 = 0, 1, 2   # MXFP8: LINEAR scales (its GEMM output also takes SWZ128)
NVFP4_B32 = 3                   # the NVFP4 rule on 32-blocks: the same three calls, LINEAR scales
MXFP8_MMA = 4                   # GEMM operands: MXFP8 bytes and scales, contracted on the scaled FP8 MFMA
LINEAR, TILED, SWZ128 = 0, 1, 2   # SWZ128: the 128 x 4 swizzle (quantizer outputs, FP8 GEMM output)
VARIANT_AUTO, VARIANT_DECODE, VARIANT_PREFILL, VARIANT_SPLITK = -1, 0, 1, 2

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblowbit.so")

_STATUS = {0: "ok", 1: "invalid argument", 2: "misaligned pointer", 3: "unsupported shape",
           4: "device is not gfx950", 5: "HIP runtime error"}

# exported symbols (the entry points of include/lowbit.h)
EXPORTS = (
    "lowbit_status_str", "lowbit_sf_bytes", "lowbit_add_rmsnorm_quant", "lowbit_quantize",
    "lowbit_add_rmsnorm_quant_fp16", "lowbit_quantize_fp16",
    "lowbit_add_rmsnorm_quant_both_sf", "lowbit_add_rmsnorm_quant_both_sf_fp16",
    "lowbit_dequantize", "lowbit_gemm_bf16", "lowbit_gemm_bias_bf16", "lowbit_gemm_residual_bf16",
    "lowbit_gemm_bias_residual_bf16", "lowbit_gemm_bias_gelu_bf16", "lowbit_gemm_bias_gelu_fp4",
    "lowbit_gemm_pick_variant", "lowbit_gemm_workspace_bytes", "lowbit_gemm_bf16_noalloc",
    "lowbit_rope_quant", "lowbit_gemm_fp8", "lowbit_sf_convert", "lowbit_dequantize_fp16",
)
STATIC_SCRATCH_BYTES = 16 << 20   # LOWBIT_STATIC_SCRATCH_BYTES


class LowbitError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: {_STATUS.get(status, 'unknown status')} (status {status})")


_lib = None
_vp, _i64, _int, _f32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t


def lib():
    """The loaded liblowbit.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"liblowbit.so is not built ({LIB_PATH}); run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        L.lowbit_status_str.restype = ctypes.c_char_p
        L.lowbit_status_str.argtypes = [_int]
        L.lowbit_sf_bytes.restype = ctypes.c_size_t
        L.lowbit_sf_bytes.argtypes = [_i64, _i64, _int, _int]
        L.lowbit_add_rmsnorm_quant.restype = _int
        L.lowbit_add_rmsnorm_quant.argtypes = [_vp, _vp, _vp, _i64, _i64, _f32, _int, _int, _vp, _vp, _vp, _vp]
        L.lowbit_quantize.restype = _int
        L.lowbit_quantize.argtypes = [_vp, _i64, _i64, _int, _int, _vp, _vp, _vp, _vp]
        L.lowbit_add_rmsnorm_quant_fp16.restype = _int
        L.lowbit_add_rmsnorm_quant_fp16.argtypes = L.lowbit_add_rmsnorm_quant.argtypes
        for name in ("lowbit_add_rmsnorm_quant_both_sf", "lowbit_add_rmsnorm_quant_both_sf_fp16"):
            getattr(L, name).restype = _int
            getattr(L, name).argtypes = [_vp, _vp, _vp, _i64, _i64, _f32, _int, _int, _vp, _vp, _vp, _vp, _vp]
        L.lowbit_quantize_fp16.restype = _int
        L.lowbit_quantize_fp16.argtypes = L.lowbit_quantize.argtypes
        L.lowbit_rope_quant.restype = _int
        L.lowbit_rope_quant.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _int, _int, _vp, _vp, _vp]
        L.lowbit_dequantize.restype = _int
        L.lowbit_dequantize.argtypes = [_vp, _vp, _i64, _i64, _int, _int, _vp, _vp, _vp]
        L.lowbit_dequantize_fp16.restype = _int
        L.lowbit_dequantize_fp16.argtypes = L.lowbit_dequantize.argtypes
        L.lowbit_sf_convert.restype = _int
        L.lowbit_sf_convert.argtypes = [_vp, _int, _vp, _int, _i64, _i64, _int, _vp]
        head = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _int, _int, _f32]
        tail = [_int, _vp, _sz, _vp]   # variant, workspace, workspace_bytes, stream
        L.lowbit_gemm_bf16.argtypes = head + [_vp] + tail
        L.lowbit_gemm_bias_bf16.argtypes = head + [_vp, _vp] + tail
        L.lowbit_gemm_bf16_noalloc.argtypes = head + [_vp, _int, _vp]
        L.lowbit_gemm_residual_bf16.argtypes = head + [_vp, _vp] + tail
        L.lowbit_gemm_bias_residual_bf16.argtypes = head + [_vp, _vp, _vp] + tail
        L.lowbit_gemm_bias_gelu_bf16.argtypes = head + [_vp, _vp] + tail
        L.lowbit_gemm_bias_gelu_fp4.argtypes = head + [_vp, _vp, _vp, _vp, _int] + tail
        L.lowbit_gemm_fp8.argtypes = head + [_vp, _vp, _int] + tail
        for n in ("lowbit_gemm_bf16", "lowbit_gemm_bf16_noalloc", "lowbit_gemm_bias_bf16", "lowbit_gemm_residual_bf16",
                  "lowbit_gemm_bias_residual_bf16", "lowbit_gemm_bias_gelu_bf16",
                  "lowbit_gemm_bias_gelu_fp4", "lowbit_gemm_fp8"):
            getattr(L, n).restype = _int
        L.lowbit_gemm_pick_variant.restype = _int
        L.lowbit_gemm_pick_variant.argtypes = [_i64, _i64, _i64, _int, _int, _sz]
        L.lowbit_gemm_workspace_bytes.restype = _sz
        L.lowbit_gemm_workspace_bytes.argtypes = [_i64, _i64, _i64, _int, _int]
        _lib = L
    return _lib


def _check(fn, status):
    if status != 0:
        raise LowbitError(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, dtype, name):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def block_size(fmt):
    return 16 if fmt == NVFP4 else 32


def _row_bytes(fmt, k):
    """Packed bytes of a row of k elements: one per MXFP8 element, else two codes a byte."""
    return k if fmt in (MXFP8, MXFP8_MMA) else k // 2


def _at_least(t, n, name):
    """Every buffer handed to the library must hold what the contract writes or reads."""
    if n > 0 and t.numel() < n:
        raise ValueError(f"{name} holds {t.numel()} elements, the call needs {n}")


def _rows_of(t):
    """Leading dimensions of a tensor fold into rows; the last one is the row."""
    lead = tuple(t.shape[:-1])
    return lead, (int(np.prod(lead)) if lead else 1), int(t.shape[-1])


def lowbit_sf_bytes(rows, k, fmt, layout):
    return int(lib().lowbit_sf_bytes(rows, k, fmt, layout))


def _alloc_q(rows, k, fmt, layout, device, out_packed, out_sf, lead=None):
    """Outputs the caller did not pass: packed codes shaped like the input's
    leading dims (rows when none are given) and the flat scale buffer."""
    if out_packed is None:
        shape = (tuple(lead) if lead is not None else (rows,)) + (k if fmt == MXFP8 else k // 2,)
        out_packed = torch.empty(shape, dtype=torch.uint8, device=device)
    if out_sf is None:
        out_sf = torch.empty(lowbit_sf_bytes(rows, k, fmt, layout), dtype=torch.uint8, device=device)
    return out_packed, out_sf


def _check_q_out(out_packed, out_sf, rows, k, fmt, layout):
    _need(out_packed, torch.uint8, "out_packed")
    _need(out_sf, torch.uint8, "out_sf")
    _at_least(out_packed, rows * _row_bytes(fmt, k), "out_packed")
    _at_least(out_sf, lowbit_sf_bytes(rows, k, fmt, layout), "out_sf")


def _in_dtype(t, name):
    if t.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError(f"{name} must be bfloat16 or float16, got {t.dtype}")
    return t.dtype


def lowbit_add_rmsnorm_quant(input, residual, weight, eps=1e-6, fmt=NVFP4, layout=LINEAR,
                             global_scale=None, out_packed=None, out_sf=None, stream=None):
    """residual += input (in place); y = RMSNorm(residual) * weight; y -> FP4.
    bf16 tensors call lowbit_add_rmsnorm_quant, fp16 ones
    lowbit_add_rmsnorm_quant_fp16 (input, residual and weight share the dtype).
    Returns (packed (M, H/2) uint8, scales uint8)."""
    dt = _in_dtype(input, "input")
    _need(input, dt, "input")
    _need(residual, dt, "residual")
    _need(weight, dt, "weight")
    if global_scale is not None:
        _need(global_scale, torch.float32, "global_scale")
        _at_least(global_scale, 1, "global_scale")
    if residual.shape != input.shape:
        raise ValueError(f"residual shape {tuple(residual.shape)} differs from input {tuple(input.shape)}")
    lead, M, H = _rows_of(input)   # leading dims are rows
    if weight.numel() != H:
        raise ValueError(f"weight has {weight.numel()} elements, the rows have {H}")
    out_packed, out_sf = _alloc_q(M, H, fmt, layout, input.device, out_packed, out_sf, lead)
    _check_q_out(out_packed, out_sf, M, H, fmt, layout)
    name = "lowbit_add_rmsnorm_quant" if dt == torch.bfloat16 else "lowbit_add_rmsnorm_quant_fp16"
    _check(name, getattr(lib(), name)(
        _ptr(input), _ptr(residual), _ptr(weight), M, H, eps, fmt, layout, _ptr(global_scale),
        _ptr(out_packed), _ptr(out_sf), _stream(stream)))
    return out_packed, out_sf


def lowbit_add_rmsnorm_quant_fp16(input, residual, weight, eps=1e-6, fmt=NVFP4, layout=LINEAR,
                                  global_scale=None, out_packed=None, out_sf=None, stream=None):
    """The fp16 producer by name (lowbit_add_rmsnorm_quant dispatches on dtype)."""
    _need(input, torch.float16, "input")
    return lowbit_add_rmsnorm_quant(input, residual, weight, eps, fmt, layout, global_scale, out_packed,
                                    out_sf, stream)


def lowbit_add_rmsnorm_quant_both_sf(input, residual, weight, eps=1e-6, fmt=NVFP4, layout=TILED,
                                     global_scale=None, out_packed=None, out_sf=None, out_sf_linear=None,
                                     stream=None):
    """The producer with its scales in two layouts, one pass: `layout`
    (TILED or SWZ128) and a LINEAR copy.  bf16 tensors call
    lowbit_add_rmsnorm_quant_both_sf, fp16 ones the _fp16 entry point.
    Returns (packed uint8, scales in `layout` uint8, LINEAR scales uint8)."""
    dt = _in_dtype(input, "input")
    _need(input, dt, "input")
    _need(residual, dt, "residual")
    _need(weight, dt, "weight")
    if global_scale is not None:
        _need(global_scale, torch.float32, "global_scale")
        _at_least(global_scale, 1, "global_scale")
    if residual.shape != input.shape:
        raise ValueError(f"residual shape {tuple(residual.shape)} differs from input {tuple(input.shape)}")
    lead, M, H = _rows_of(input)
    if weight.numel() != H:
        raise ValueError(f"weight has {weight.numel()} elements, the rows have {H}")
    out_packed, out_sf = _alloc_q(M, H, fmt, layout, input.device, out_packed, out_sf, lead)
    if out_sf_linear is None:
        out_sf_linear = torch.empty(lowbit_sf_bytes(M, H, fmt, LINEAR), dtype=torch.uint8, device=input.device)
    _check_q_out(out_packed, out_sf, M, H, fmt, layout)
    _need(out_sf_linear, torch.uint8, "out_sf_linear")
    _at_least(out_sf_linear, lowbit_sf_bytes(M, H, fmt, LINEAR), "out_sf_linear")
    name = "lowbit_add_rmsnorm_quant_both_sf" + ("" if dt == torch.bfloat16 else "_fp16")
    _check(name, getattr(lib(), name)(
        _ptr(input), _ptr(residual), _ptr(weight), M, H, eps, fmt, layout, _ptr(global_scale),
        _ptr(out_packed), _ptr(out_sf), _ptr(out_sf_linear), _stream(stream)))
    return out_packed, out_sf, out_sf_linear


def lowbit_add_rmsnorm_quant_both_sf_fp16(input, residual, weight, eps=1e-6, fmt=NVFP4, layout=TILED,
                                          global_scale=None, out_packed=None, out_sf=None, out_sf_linear=None,
                                          stream=None):
    """The fp16 form by name (lowbit_add_rmsnorm_quant_both_sf dispatches on dtype)."""
    _need(input, torch.float16, "input")
    return lowbit_add_rmsnorm_quant_both_sf(input, residual, weight, eps, fmt, layout, global_scale, out_packed,
                                            out_sf, out_sf_linear, stream)


def lowbit_quantize(x, fmt=NVFP4, layout=LINEAR, global_scale=None, out_packed=None, out_sf=None,
                    stream=None):
    """x (rows, K) bf16 or fp16 -> (packed (rows, K/2) uint8, scales uint8)."""
    dt = _in_dtype(x, "x")
    _need(x, dt, "x")
    if global_scale is not None:
        _need(global_scale, torch.float32, "global_scale")
        _at_least(global_scale, 1, "global_scale")
    lead, rows, K = _rows_of(x)           # leading dims are rows
    out_packed, out_sf = _alloc_q(rows, K, fmt, layout, x.device, out_packed, out_sf, lead)
    _check_q_out(out_packed, out_sf, rows, K, fmt, layout)
    name = "lowbit_quantize" if dt == torch.bfloat16 else "lowbit_quantize_fp16"
    _check(name, getattr(lib(), name)(
        _ptr(x), rows, K, fmt, layout, _ptr(global_scale), _ptr(out_packed), _ptr(out_sf),
        _stream(stream)))
    return out_packed, out_sf


def lowbit_quantize_fp16(x, fmt=NVFP4, layout=LINEAR, global_scale=None, out_packed=None, out_sf=None,
                         stream=None):
    """The fp16 quantizer by name (lowbit_quantize dispatches on dtype)."""
    _need(x, torch.float16, "x")
    return lowbit_quantize(x, fmt, layout, global_scale, out_packed, out_sf, stream)


def lowbit_rope_quant(x, positions, rope, fmt=MXFP8, layout=LINEAR, out_packed=None, out_sf=None, stream=None):
    """Inverse RoPE on the last R elements of each head row, then MX
    quantization with the 1e-10 floor on the block maximum.  x: bf16
    (T, heads, D); positions: int64 (T); rope: fp32 (P, R), each row
    cos || sin (R = 0: pass an empty (P, 0) tensor or None).  Returns
    (packed (T*heads, D) for MXFP8 or (T*heads, D/2) for MXFP4, scales)."""
    _need(x, torch.bfloat16, "x")
    if x.dim() != 3:
        raise ValueError(f"x must be (tokens, heads, head_dim), got {tuple(x.shape)}")
    T, heads, D = (int(v) for v in x.shape)
    if rope is None or rope.numel() == 0:
        R, P, rope, positions = 0, 0, None, None
    else:
        _need(rope, torch.float32, "rope")
        if rope.dim() != 2:
            raise ValueError(f"rope must be (positions, rope_dim), got {tuple(rope.shape)}")
        P, R = (int(v) for v in rope.shape)
        _need(positions, torch.int64, "positions")
        if positions.numel() != T:
            raise ValueError(f"positions has {positions.numel()} entries for {T} tokens")
    rows = T * heads
    out_packed, out_sf = _alloc_q(rows, D, fmt, layout, x.device, out_packed, out_sf)
    _check_q_out(out_packed, out_sf, rows, D, fmt, layout)
    _check("lowbit_rope_quant", lib().lowbit_rope_quant(
        _ptr(x), _ptr(positions), _ptr(rope), T, heads, D, R, P, fmt, layout, _ptr(out_packed), _ptr(out_sf),
        _stream(stream)))
    return out_packed, out_sf


def lowbit_dequantize(packed, sf, fmt=NVFP4, layout=LINEAR, global_scale=None, out=None, stream=None):
    """packed (..., K/2) (MXFP8: (..., K)) + scales -> bf16 (..., K)."""
    return _dequantize("lowbit_dequantize", torch.bfloat16, packed, sf, fmt, layout, global_scale, out, stream)


def lowbit_dequantize_fp16(packed, sf, fmt=NVFP4, layout=LINEAR, global_scale=None, out=None, stream=None):
    """packed (..., K/2) (MXFP8: (..., K)) + scales -> fp16 (..., K)."""
    return _dequantize("lowbit_dequantize_fp16", torch.float16, packed, sf, fmt, layout, global_scale, out, stream)


def _dequantize(fn, dtype, packed, sf, fmt, layout, global_scale, out, stream):
    _need(packed, torch.uint8, "packed")
    _need(sf, torch.uint8, "sf")
    lead, rows, kb = _rows_of(packed)
    K = kb * (1 if fmt == MXFP8 else 2)
    _at_least(sf, lowbit_sf_bytes(rows, K, fmt, layout), "sf")
    if global_scale is not None:
        _need(global_scale, torch.float32, "global_scale")
        _at_least(global_scale, 1, "global_scale")
    if out is None:
        out = torch.empty(lead + (K,), dtype=dtype, device=packed.device)
    _need(out, dtype, "out")
    _at_least(out, rows * K, "out")
    _check(fn, getattr(lib(), fn)(
        _ptr(packed), _ptr(sf), rows, K, fmt, layout, _ptr(global_scale), _ptr(out), _stream(stream)))
    return out


def lowbit_sf_convert(sf, rows, k, fmt=NVFP4, src_layout=SWZ128, dst_layout=TILED, out=None, stream=None):
    """Scale bytes of a (rows, k) operand rewritten from src_layout into
    dst_layout (destination padding zero), e.g. 128 x 4 weight scales into the
    TILED layout the GEMM reads."""
    _need(sf, torch.uint8, "sf")
    _at_least(sf, lowbit_sf_bytes(rows, k, fmt, src_layout), "sf")
    if out is None:
        out = torch.empty(lowbit_sf_bytes(rows, k, fmt, dst_layout), dtype=torch.uint8, device=sf.device)
    _need(out, torch.uint8, "out")
    _at_least(out, lowbit_sf_bytes(rows, k, fmt, dst_layout), "out")
    _check("lowbit_sf_convert", lib().lowbit_sf_convert(
        _ptr(sf), src_layout, _ptr(out), dst_layout, rows, k, fmt, _stream(stream)))
    return out


def _gemm_head(a, b, sfa, sfb, fmt, sfa_layout, sfb_layout, alpha):
    """Sizes of a GEMM call: A (..., K/2) with its leading dims as the M rows,
    B (N, K/2); every buffer checked against the contract's sizes."""
    for t, n in ((a, "a"), (b, "b"), (sfa, "sfa"), (sfb, "sfb")):
        _need(t, torch.uint8, n)
    _, M, ka = _rows_of(a)
    _, N, kb = _rows_of(b)
    per = 1 if fmt in (MXFP8, MXFP8_MMA) else 2     # elements per packed byte
    K = ka * per
    if kb * per != K:
        raise ValueError("a and b disagree on K")
    # sizes are checked for the layouts the GEMM takes; any other layout or
    # format is the C ABI's to refuse (LOWBIT_EINVAL)
    if (fmt in (NVFP4, MXFP4) and sfa_layout in (LINEAR, TILED) and sfb_layout in (LINEAR, TILED)) or \
            (fmt in (MXFP8, MXFP8_MMA) and sfa_layout == LINEAR and sfb_layout == LINEAR):
        _at_least(sfa, lowbit_sf_bytes(M, K, fmt, sfa_layout), "sfa")
        _at_least(sfb, lowbit_sf_bytes(N, K, fmt, sfb_layout), "sfb")
    return M, N, K, [_ptr(a), _ptr(b), _ptr(sfa), _ptr(sfb), M, N, K, fmt, sfa_layout, sfb_layout,
                     float(alpha)]


def _ws(workspace):
    """(pointer, bytes) of an optional uint8 device workspace for split-K."""
    if workspace is None:
        return None, 0
    _need(workspace, torch.uint8, "workspace")
    return _ptr(workspace), workspace.numel()


def lowbit_gemm_workspace_bytes(M, N, K, fmt=NVFP4, variant=VARIANT_AUTO):
    """Workspace bytes the split-K schedule needs (0: it would not run)."""
    return int(lib().lowbit_gemm_workspace_bytes(M, N, K, fmt, variant))


def _out_bf16(out, a, M, N):
    if out is None:
        out = torch.empty(tuple(a.shape[:-1]) + (N,), dtype=torch.bfloat16, device=a.device)
    _need(out, torch.bfloat16, "out")
    if out.numel() != M * N:
        raise ValueError(f"out has {out.numel()} elements, the product has {M} x {N}")
    return out


def _bias(bias, N):
    _need(bias, torch.bfloat16, "bias")
    if bias.numel() != N:
        raise ValueError(f"bias has {bias.numel()} elements, the product has {N} columns")


def _residual(residual, M, N):
    _need(residual, torch.bfloat16, "residual")
    if residual.numel() != M * N:
        raise ValueError(f"residual has {residual.numel()} elements, the product has {M} x {N}")


def lowbit_gemm_bf16(a, b, sfa, sfb, fmt=NVFP4, sfa_layout=LINEAR, sfb_layout=LINEAR, alpha=1.0,
                     out=None, variant=VARIANT_AUTO, workspace=None, stream=None):
    M, N, K, head = _gemm_head(a, b, sfa, sfb, fmt, sfa_layout, sfb_layout, alpha)
    out = _out_bf16(out, a, M, N)
    _check("lowbit_gemm_bf16", lib().lowbit_gemm_bf16(*head, _ptr(out), variant, *_ws(workspace), _stream(stream)))
    return out


def lowbit_gemm_bf16_noalloc(a, b, sfa, sfb, fmt=NVFP4, sfa_layout=LINEAR, sfb_layout=LINEAR, alpha=1.0,
                             out=None, variant=VARIANT_AUTO, stream=None):
    """lowbit_gemm_bf16 with its split-K workspace in the library's static
    device array (nothing allocated by the call; pass `out` to allocate
    nothing here either).  Calls overlapping on one device race on the array."""
    M, N, K, head = _gemm_head(a, b, sfa, sfb, fmt, sfa_layout, sfb_layout, alpha)
    out = _out_bf16(out, a, M, N)
    _check("lowbit_gemm_bf16_noalloc",
           lib().lowbit_gemm_bf16_noalloc(*head, _ptr(out), variant, _stream(stream)))
    return out


def lowbit_gemm_bias_bf16(a, b, sfa, sfb, bias, fmt=NVFP4, sfa_layout=LINEAR, sfb_layout=LINEAR,
                          alpha=1.0, out=None, variant=VARIANT_AUTO, workspace=None, stream=None):
    M, N, K, head = _gemm_head(a, b, sfa, sfb, fmt, sfa_layout, sfb_layout, alpha)
    _bias(bias, N)
    out = _out_bf16(out, a, M, N)
    _check("lowbit_gemm_bias_bf16",
           lib().lowbit_gemm_bias_bf16(*head, _ptr(bias), _ptr(out), variant, *_ws(workspace), _stream(stream)))
    return out


def lowbit_gemm_residual_bf16(a, b, sfa, sfb, residual, fmt=NVFP4, sfa_layout=LINEAR,
                              sfb_layout=LINEAR, alpha=1.0, out=None, variant=VARIANT_AUTO, workspace=None,
                              stream=None):
    M, N, K, head = _gemm_head(a, b, sfa, sfb, fmt, sfa_layout, sfb_layout, alpha)
    _residual(residual, M, N)
    out = _out_bf16(out, a, M, N)
    _check("lowbit_gemm_residual_bf16",
           lib().lowbit_gemm_residual_bf16(*head, _ptr(residual), _ptr(out), variant, *_ws(workspace), _stream(stream)))
    return out


def lowbit_gemm_bias_residual_bf16(a, b, sfa, sfb, bias, residual, fmt=NVFP4, sfa_layout=LINEAR,
                                   sfb_layout=LINEAR, alpha=1.0, out=None, variant=VARIANT_AUTO,
                                   workspace=None, stream=None):
    M, N, K, head = _gemm_head(a, b, sfa, sfb, fmt, sfa_layout, sfb_layout, alpha)
    _bias(bias, N)
    _residual(residual, M, N)
    out = _out_bf16(out, a, M, N)
    _check("lowbit_gemm_bias_residual_bf16", lib().lowbit_gemm_bias_residual_bf16(
        *head, _ptr(bias), _ptr(residual), _ptr(out), variant, *_ws(workspace), _stream(stream)))
    return out


def lowbit_gemm_bias_gelu_bf16(a, b, sfa, sfb, bias, fmt=NVFP4, sfa_layout=LINEAR, sfb_layout=LINEAR,
                               alpha=1.0, out=None, variant=VARIANT_AUTO, workspace=None, stream=None):
    M, N, K, head = _gemm_head(a, b, sfa, sfb, fmt, sfa_layout, sfb_layout, alpha)
    _bias(bias, N)
    out = _out_bf16(out, a, M, N)
    _check("lowbit_gemm_bias_gelu_bf16",
           lib().lowbit_gemm_bias_gelu_bf16(*head, _ptr(bias), _ptr(out), variant, *_ws(workspace), _stream(stream)))
    return out


def lowbit_gemm_bias_gelu_fp4(a, b, sfa, sfb, bias, fmt=NVFP4, sfa_layout=LINEAR, sfb_layout=LINEAR,
                              alpha=1.0, out_global_scale=None, out_packed=None, out_sf=None,
                              out_layout=LINEAR, variant=VARIANT_AUTO, workspace=None, stream=None):
    """GELU(alpha * A.B^T + bias) quantized to NVFP4 along N.  Returns (packed, scales)."""
    M, N, K, head = _gemm_head(a, b, sfa, sfb, fmt, sfa_layout, sfb_layout, alpha)
    _bias(bias, N)
    if out_global_scale is not None:
        _need(out_global_scale, torch.float32, "out_global_scale")
        _at_least(out_global_scale, 1, "out_global_scale")
    out_packed, out_sf = _alloc_q(M, N, NVFP4, out_layout, a.device, out_packed, out_sf,
                                  tuple(a.shape[:-1]))
    _check_q_out(out_packed, out_sf, M, N, NVFP4, out_layout)
    _check("lowbit_gemm_bias_gelu_fp4", lib().lowbit_gemm_bias_gelu_fp4(
        *head, _ptr(bias), _ptr(out_global_scale), _ptr(out_packed), _ptr(out_sf), out_layout, variant,
        *_ws(workspace), _stream(stream)))
    return out_packed, out_sf


def lowbit_gemm_fp8(a, b, sfa, sfb, fmt=MXFP8, sfa_layout=LINEAR, sfb_layout=LINEAR, alpha=1.0,
                    out_packed=None, out_sf=None, out_layout=LINEAR, variant=VARIANT_AUTO, workspace=None,
                    stream=None):
    """bf16(alpha * A.B^T) quantized to MXFP8 along N (E4M3 bytes (M, N) and
    UE8M0 scales in out_layout: LINEAR or SWZ128).  Returns (packed, scales)."""
    M, N, K, head = _gemm_head(a, b, sfa, sfb, fmt, sfa_layout, sfb_layout, alpha)
    out_packed, out_sf = _alloc_q(M, N, MXFP8, out_layout, a.device, out_packed, out_sf, tuple(a.shape[:-1]))
    _check_q_out(out_packed, out_sf, M, N, MXFP8, out_layout)
    _check("lowbit_gemm_fp8", lib().lowbit_gemm_fp8(
        *head, _ptr(out_packed), _ptr(out_sf), out_layout, variant, *_ws(workspace), _stream(stream)))
    return out_packed, out_sf


def lowbit_gemm_pick_variant(M, N, K, fmt=NVFP4, variant=VARIANT_AUTO, workspace_bytes=0):
    return int(lib().lowbit_gemm_pick_variant(M, N, K, fmt, variant, workspace_bytes))
