"""The C ABI on the host, no GPU needed: liblowbit.so loads, exports every
entry point include/lowbit.h declares, and its host-side logic (scale buffer
sizes, schedule choice, argument checks in the documented order) behaves as
the header states.  No call here reaches a kernel launch: every argument set
is rejected before the device check, or, where it passes every check and
no GPU is visible, the device check itself answers."""
import ctypes
import os
import re

import pytest

import torch

import block_scaled_fp4_add_amd as lb

HEADER = os.path.join(os.path.dirname(__file__), "..", "include", "lowbit.h")
OK, EINVAL, EALIGN, ESHAPE, EDEVICE, EHIP = 0, 1, 2, 3, 4, 5
# argument sets that pass every check reach the device check; they are only
# made where no GPU is visible (host pointers must never reach a kernel)
NO_DEVICE = torch.cuda.device_count() == 0


def declared():
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\w[\w\s\*]*?\b(lowbit_\w+)\(", text, flags=re.M)))


def test_header_declares_the_binding_exports():
    assert declared() == sorted(lb.EXPORTS)


def test_library_exports_every_declared_symbol():
    raw = ctypes.CDLL(lb.LIB_PATH)
    for name in declared():
        assert hasattr(raw, name), name


def test_status_strings():
    L = lb.lib()
    for s, text in ((OK, b"ok"), (EINVAL, b"invalid argument"), (EALIGN, b"misaligned pointer"),
                    (ESHAPE, b"unsupported shape"), (EDEVICE, b"device is not gfx950")):
        assert L.lowbit_status_str(s) == text


def test_sf_bytes_matches_the_oracle(orc):
    L = lb.lib()
    for rows, K in ((1, 64), (41, 1536), (33, 5120), (8192, 14336), (7, 96)):
        for fmt in (0, 1):
            if K % (16 if fmt == 0 else 32):
                continue
            for layout in (0, 1):
                assert L.lowbit_sf_bytes(rows, K, fmt, layout) == orc.sf_bytes(rows, K, fmt, layout)
    # MXFP8: 32-blocks, LINEAR and (for the FP8 GEMM output) the 128 x 4 swizzle
    assert L.lowbit_sf_bytes(33, 5120, 2, 0) == 33 * 160 == orc.sf_bytes(33, 5120, 2, 0)
    assert L.lowbit_sf_bytes(33, 5120, 2, 1) == 0
    assert L.lowbit_sf_bytes(33, 5120, 2, 2) == 128 * 160 == orc.sf_bytes(33, 5120, 2, 2)
    # the 128 x 4 swizzle: FP4 GEMM formats, quantization side
    for rows, K, fmt in ((1, 64, 0), (129, 1120, 1), (300, 5120, 0)):
        assert L.lowbit_sf_bytes(rows, K, fmt, 2) == orc.sf_bytes(rows, K, fmt, 2)
    assert L.lowbit_sf_bytes(33, 5120, 3, 2) == 0
    # the NVFP4 rule on 32-blocks: LINEAR only
    assert L.lowbit_sf_bytes(33, 5120, 3, 0) == 33 * 160 == orc.sf_bytes(33, 5120, 3, 0)
    assert L.lowbit_sf_bytes(33, 5120, 3, 1) == 0


def test_pick_variant():
    L = lb.lib()
    assert L.lowbit_gemm_pick_variant(41, 4608, 1536, 1, -1, 0) == 0      # small M: decode schedule
    assert L.lowbit_gemm_pick_variant(128, 4608, 1536, 1, -1, 0) == 0
    assert L.lowbit_gemm_pick_variant(129, 4608, 1536, 1, -1, 0) == 1     # prefill schedule
    assert L.lowbit_gemm_pick_variant(8192, 4096, 14336, 0, -1, 0) == 1
    assert L.lowbit_gemm_pick_variant(8192, 4096, 14336, 1, 0, 0) < 0     # decode needs M <= 128
    assert L.lowbit_gemm_pick_variant(1, 17408, 5120, 1, 1, 0) == 1       # prefill accepts any M
    assert L.lowbit_gemm_pick_variant(300, 64, 48, 0, -1, 0) == 0         # NVFP4, K % 32 == 16: decode
    assert L.lowbit_gemm_pick_variant(300, 64, 48, 0, 1, 0) < 0           # ... and never prefill
    assert L.lowbit_gemm_pick_variant(8, 128, 256, 1, 3, 0) < 0           # no such variant


def splitk_plan(M, N, K, fmt=1):
    """The split-K plan the library documents, written out.  Above 128
    rows see below.  NVFP4 with
    64 < M <= 128 and K % 64 == 0 splits the 128 x 384 schedule: about one
    workgroup per CU (256 over the 384-column tiles), at least two
    128-element stages per split, K of at least 32 stages.  Otherwise the
    decode schedule: twice as many workgroups as CUs, at least four
    supersteps (1024 elements) per split, K of at least 16 supersteps.  No
    empty split; bytes = splits x 32-column tiles x M-tiles x 32 x 32 floats."""
    tiles, mt = -(-N // 32), -(-M // 32)
    if fmt == 4:            # MXFP8 on the scaled FP8 MFMA splits as MXFP8 does
        fmt = 2
    if M > 128:
        # above 128 rows: NVFP4 (K % 64 == 0) with at most 128 tiles of
        # 128 x 384 splits its 128-element stages, 16 or more each; MXFP8
        # (K % 128 == 0) with at most 128 tiles of 256 x 256 its 128-element
        # supersteps, 8 or more each; about one workgroup per CU
        if not ((fmt == 0 and K % 64 == 0) or (fmt == 2 and K % 128 == 0)):
            return 1, 0
        nst = K // 128 if fmt == 2 else -(-K // 128)
        tnv = -(-M // 256) * -(-N // 256) if fmt == 2 else -(-M // 128) * -(-N // 384)
        S = 1 if 2 * tnv > 256 else min(256 // tnv, nst // (8 if fmt == 2 else 16))
        if S <= 1:
            return 1, 0
        per = -(-nst // S)
        S = -(-nst // per)
        return (S, S * tiles * mt * 1024 * 4) if S > 1 else (1, 0)
    if fmt == 0 and 64 < M <= 128 and K % 64 == 0:
        nst = -(-K // 128)
        S = min(256 // -(-N // 384), nst // 2)
        if nst < 32:
            S = 1
        if S > 1:
            per = -(-nst // S)
            S = -(-nst // per)
            if S > 1:
                return S, S * tiles * mt * 1024 * 4
    nss = -(-K // (128 if fmt == 2 else 256))
    S = min(-(-512 // tiles), nss // 4)
    if nss < 16:
        S = 1
    if S <= 1:
        return 1, 0
    per = -(-nss // S)
    S = -(-nss // per)
    return S, S * tiles * mt * 1024 * 4


def test_splitk_nvfp4_chain_plans():
    """The chain's 128-token GEMMs split the NVFP4 128 x 384 schedule: 46
    column tiles x 5 splits of 8 stages, and 14 x 17 splits of 8 stages."""
    assert splitk_plan(128, 17408, 5120, 0)[0] == 5 and splitk_plan(128, 5120, 17408, 0)[0] == 17
    assert lb.lib().lowbit_gemm_workspace_bytes(128, 17408, 5120, 0, -1) == 5 * 544 * 4 * 4096


@pytest.mark.parametrize("M,N,K", [(41, 4608, 1536), (41, 6144, 1536), (41, 1536, 6144), (1, 17408, 5120),
                                   (1, 5120, 17408), (128, 5120, 17408), (128, 17408, 5120), (5, 40, 512), (2, 64, 4096),
                                   (100, 264, 1536), (65, 400, 4096), (97, 96, 2304)])
def test_splitk_workspace_and_choice(M, N, K):
    L = lb.lib()
    for fmt in (0, 1):
        S, need = splitk_plan(M, N, K, fmt)
        assert L.lowbit_gemm_workspace_bytes(M, N, K, fmt, -1) == need
        if need:
            assert L.lowbit_gemm_pick_variant(M, N, K, fmt, -1, need) == 2       # offered enough: split
            assert L.lowbit_gemm_pick_variant(M, N, K, fmt, -1, need - 1) == 0   # too little: decode
        else:
            assert L.lowbit_gemm_pick_variant(M, N, K, fmt, -1, 1 << 30) == 0
        forced = L.lowbit_gemm_workspace_bytes(M, N, K, fmt, 2)
        assert forced >= need and forced > 0
        assert L.lowbit_gemm_pick_variant(M, N, K, fmt, 2, 0) == 2
    assert L.lowbit_gemm_workspace_bytes(M, N, K, 1, 0) == 0 and L.lowbit_gemm_workspace_bytes(M, N, K, 1, 1) == 0
    assert L.lowbit_gemm_workspace_bytes(200, N, K, 1, 2) == 0             # MXFP4 split-K needs M <= 128
    assert L.lowbit_gemm_pick_variant(200, N, K, 1, 2, 1 << 30) < 0


@pytest.mark.parametrize("M,N,K,fmt", [(4096, 1024, 8192, 2), (4096, 1024, 8192, 4), (4096, 1024, 8192, 0),
                                       (600, 1000, 4096, 0), (300, 770, 2048, 4), (4096, 1024, 8160, 4),
                                       (2048, 7168, 4096, 4),
                                       (300, 770, 2048, 2), (2048, 5120, 17408, 0), (2048, 17408, 5120, 0),
                                       (8192, 4096, 14336, 1), (129, 96, 8192, 0), (4096, 1024, 8160, 2),
                                       (1000, 400, 4096 + 32, 0), (200, 384, 1024, 0), (257, 400, 4160, 0),
                                       (300, 400, 1984, 0)])
def test_splitk_above_128_rows(M, N, K, fmt):
    """Above 128 rows only NVFP4 (K % 64 == 0, 128 x 384 tiles) and MXFP8
    (K % 128 == 0, exact or on the scaled FP8 MFMA, 256 x 256 tiles) split,
    and the automatic choice only with at most 128 such tiles: (4096, 1024,
    8192) has 96 tiles of 128 x 384 and splits in two, 64 of 256 x 256 and
    splits in four; the chain's 2048-token GEMMs (224 and 736 tiles) and
    MXFP4 never do."""
    L = lb.lib()
    S, need = splitk_plan(M, N, K, fmt)
    assert L.lowbit_gemm_workspace_bytes(M, N, K, fmt, -1) == need
    if need:
        assert L.lowbit_gemm_pick_variant(M, N, K, fmt, -1, need) == 2
        assert L.lowbit_gemm_pick_variant(M, N, K, fmt, -1, need - 1) == 1   # too little: prefill
    else:
        assert L.lowbit_gemm_pick_variant(M, N, K, fmt, -1, 1 << 30) == 1
    nv_ok = (fmt == 0 and K % 64 == 0) or (fmt in (2, 4) and K % 128 == 0)
    forced = L.lowbit_gemm_workspace_bytes(M, N, K, fmt, 2)
    assert (forced > 0) == nv_ok and forced >= need
    assert (L.lowbit_gemm_pick_variant(M, N, K, fmt, 2, 0) == 2) == nv_ok
    if (M, N, K, fmt) == (4096, 1024, 8192, 0):
        assert S == 2 and need == 2 * 32 * 128 * 4096
    if (M, N, K) == (4096, 1024, 8192) and fmt in (2, 4):
        assert S == 4 and need == 4 * 32 * 128 * 4096
    if (M, N, K) == (257, 400, 4160):   # 33 stages, the last a half one: 2 splits of 17 and 16
        assert S == 2
    if (M, N) in ((2048, 5120), (2048, 17408)) or fmt == 1:
        assert need == 0


class Buf:
    """An aligned host buffer: stands in for operand pointers in calls that
    are rejected before any memory is touched."""

    def __init__(self, n=1 << 16):
        self.raw = ctypes.create_string_buffer(n + 512)
        self.base = (ctypes.addressof(self.raw) + 255) & ~255

    def at(self, off=0):
        return ctypes.c_void_p(self.base + off)


@pytest.fixture
def buf():
    return Buf()


def quant(L, buf, rows, K, fmt=1, layout=0, gs=None, x=0, p=0, s=0):
    return L.lowbit_quantize(buf.at(x), rows, K, fmt, layout, gs, buf.at(p), buf.at(s), None)


def test_quantize_argument_order(buf):
    L = lb.lib()
    assert quant(L, buf, 4, 64, fmt=4) == EINVAL                           # format
    assert quant(L, buf, 4, 64, fmt=3, layout=1) == EINVAL                 # 32-block NVFP4: LINEAR only
    assert quant(L, buf, 4, 48, fmt=3) == ESHAPE                           # 32-block NVFP4: K % 32
    assert quant(L, buf, 4, 64, fmt=2, layout=1) == EINVAL                 # MXFP8: LINEAR scales only
    assert quant(L, buf, 4, 64, fmt=2, gs=buf.at()) == EINVAL              # MXFP8 has no global scale
    assert quant(L, buf, 4, 48, fmt=2) == ESHAPE                           # MXFP8: K % 32
    assert quant(L, buf, 4, 64, layout=5) == EINVAL                        # layout
    assert quant(L, buf, 4, 64, fmt=1, gs=buf.at()) == EINVAL              # MXFP4 has no global scale
    assert L.lowbit_quantize(None, 4, 64, 1, 0, None, buf.at(), buf.at(), None) == EINVAL
    assert quant(L, buf, -1, 64) == ESHAPE
    assert quant(L, buf, 4, 48) == ESHAPE                                  # K % 32
    assert quant(L, buf, 4, 8, fmt=0) == ESHAPE                            # K below one block
    assert quant(L, buf, 4, 64, x=2) == EALIGN                             # input not 16-byte aligned
    assert quant(L, buf, 4, 64, layout=1, s=1) == EALIGN                   # tiled scales need 4 bytes
    assert quant(L, buf, 0, 64) == OK                                      # empty: nothing to do
    if NO_DEVICE:
        assert quant(L, buf, 4, 64) == EDEVICE                             # all checks pass: no device
        assert quant(L, buf, 4, 64, fmt=3, gs=buf.at()) == EDEVICE         # 32-block NVFP4 takes gs


def conv(L, buf, rows, k, fmt=0, ls=2, ld=1, s=0, d=4096):
    return L.lowbit_sf_convert(buf.at(s), ls, buf.at(d), ld, rows, k, fmt, None)


def test_sf_convert_argument_order(buf):
    L = lb.lib()
    assert conv(L, buf, 4, 64, fmt=4) == EINVAL                  # format
    assert conv(L, buf, 4, 64, ls=3) == EINVAL                   # layout
    assert conv(L, buf, 4, 64, fmt=2, ld=1) == EINVAL            # MXFP8 has no TILED layout
    assert conv(L, buf, 4, 64, fmt=3, ls=2, ld=0) == EINVAL      # 32-block NVFP4: LINEAR only
    assert conv(L, buf, -1, 64) == ESHAPE
    assert L.lowbit_sf_convert(None, 2, buf.at(), 1, 4, 64, 0, None) == EINVAL
    assert L.lowbit_sf_convert(buf.at(), 2, None, 1, 4, 64, 0, None) == EINVAL
    assert conv(L, buf, 4, 40) == ESHAPE                         # k % 16
    assert conv(L, buf, 4, 0) == ESHAPE                          # k below one block
    assert conv(L, buf, 4, 48, fmt=1, ls=0) == ESHAPE            # MXFP4: k % 32
    assert conv(L, buf, 1 << 40, 64) == ESHAPE                   # more than 8 GiB of output
    # overlapping buffers: the 512-byte 128 x 4 source and the 256-byte TILED output
    assert conv(L, buf, 4, 64, s=0, d=256) == EINVAL
    assert conv(L, buf, 4, 64, s=128, d=0) == EINVAL
    if NO_DEVICE:
        assert conv(L, buf, 4, 64, s=256, d=0) == EDEVICE        # adjacent the other way
    assert conv(L, buf, 0, 64) == OK                             # empty: nothing to do
    if NO_DEVICE:
        assert conv(L, buf, 4, 64, s=0, d=512) == EDEVICE        # adjacent, not overlapping
        assert conv(L, buf, 4, 64, fmt=2, ls=2, ld=0) == EDEVICE  # MXFP8 128 x 4 -> LINEAR
        assert conv(L, buf, 4, 64, fmt=3, ls=0, ld=0) == EDEVICE  # 32-block NVFP4 copy
        assert conv(L, buf, 4, 64, s=1, d=4097) == EDEVICE       # any alignment


def test_dequantize_argument_order(buf):
    """Both dequantizers (bf16 and fp16 output) check their arguments alike."""
    L = lb.lib()
    for fn in (L.lowbit_dequantize, L.lowbit_dequantize_fp16):
        def dq(rows, K, fmt=1, layout=0, gs=None, p=0, s=0, o=0):
            return fn(buf.at(p), buf.at(s), rows, K, fmt, layout, gs, buf.at(o), None)
        assert dq(4, 64, fmt=5) == EINVAL                           # format
        assert dq(4, 64, fmt=2, layout=1) == EINVAL                 # MXFP8: LINEAR scales only
        assert dq(4, 64, gs=buf.at()) == EINVAL                     # MXFP4 has no global scale
        assert dq(-1, 64) == ESHAPE
        assert fn(None, buf.at(), 4, 64, 1, 0, None, buf.at(), None) == EINVAL
        assert dq(4, 48) == ESHAPE                                  # K % 32
        assert dq(0, 64) == OK                                      # empty: nothing to do
        assert dq(4, 64, o=2) == EALIGN                             # output 16 bytes
        assert dq(4, 64, p=8) == EALIGN                             # packed 16 bytes
        if NO_DEVICE:
            assert dq(4, 64) == EDEVICE
            assert dq(4, 64, fmt=0, layout=2, gs=buf.at()) == EDEVICE   # NVFP4, 128 x 4, global scale


def test_producer_argument_order(buf):
    L = lb.lib()

    def call(M, H, fmt=1, layout=0, gs=None, eps=1e-6, x=0):
        return L.lowbit_add_rmsnorm_quant(buf.at(x), buf.at(), buf.at(), M, H, eps, fmt, layout, gs,
                                          buf.at(), buf.at(), None)

    assert call(4, 256, fmt=7) == EINVAL
    assert call(4, 256, fmt=1, gs=buf.at()) == EINVAL
    assert call(4, 48) == ESHAPE                     # H < 64
    assert call(4, 100) == ESHAPE                    # H % block
    assert call(4, 65536) == ESHAPE                  # longer rows than the kernel's limit
    assert call(4, 256, x=8) == EALIGN
    assert call(0, 256) == OK
    if NO_DEVICE:
        assert call(4, 256) == EDEVICE


def test_producer_both_sf_argument_order(buf):
    L = lb.lib()

    def call(M, H, fmt=1, gs=None, lin=True, x=0, fp16=False, layout=1):
        fn = L.lowbit_add_rmsnorm_quant_both_sf_fp16 if fp16 else L.lowbit_add_rmsnorm_quant_both_sf
        return fn(buf.at(x), buf.at(), buf.at(), M, H, 1e-6, fmt, layout, gs, buf.at(), buf.at(),
                  buf.at() if lin else None, None)

    for fp16 in (False, True):
        assert call(4, 256, fmt=2, fp16=fp16) == EINVAL            # MXFP8: no TILED layout
        assert call(4, 256, fmt=2, layout=2, fp16=fp16) == EINVAL  # nor a second copy beside LINEAR scales
        assert call(4, 256, layout=0, fp16=fp16) == EINVAL         # the first layout must be a padded one
        assert call(4, 256, layout=3, fp16=fp16) == EINVAL
        assert call(4, 256, fmt=7, fp16=fp16) == EINVAL
        assert call(4, 256, fmt=3, fp16=fp16) == EINVAL            # 32-block NVFP4: no TILED layout
        assert call(4, 256, fmt=1, gs=buf.at(), fp16=fp16) == EINVAL
        assert call(4, 256, lin=False, fp16=fp16) == EINVAL        # no LINEAR buffer
        assert call(4, 48, fp16=fp16) == ESHAPE
        assert call(4, 256, x=8, fp16=fp16) == EALIGN
        assert call(0, 256, lin=False, fp16=fp16) == OK            # M == 0: nothing is written
        if NO_DEVICE:
            assert call(4, 256, fp16=fp16) == EDEVICE
            assert call(4, 256, fmt=0, gs=buf.at(), fp16=fp16) == EDEVICE
            assert call(4, 256, fmt=0, gs=buf.at(), layout=2, fp16=fp16) == EDEVICE


def test_gemm_argument_order(buf):
    L = lb.lib()
    a, b, sa, sb, out = buf.at(0), buf.at(4096), buf.at(8192), buf.at(12288), buf.at(16384)

    def call(M, N, K, fmt=1, la=0, lb_=0, variant=-1, o=out, a_=a, ws=None, wsb=0):
        return L.lowbit_gemm_bf16(a_, b, sa, sb, M, N, K, fmt, la, lb_, 1.0, o, variant, ws, wsb, None)

    assert call(8, 128, 256, fmt=3) == EINVAL                # 32-block NVFP4: no GEMM
    assert call(8, 128, 256, fmt=5) == EINVAL
    assert call(8, 128, 256, fmt=4, la=1) == EINVAL          # MXFP8 on the FP8 MFMA: LINEAR scales only
    assert call(8, 128, 48, fmt=4) == ESHAPE                 # ... K % 32
    assert L.lowbit_sf_bytes(33, 5120, 4, 0) == L.lowbit_sf_bytes(33, 5120, 2, 0) == 33 * 160
    assert quant(L, buf, 4, 64, fmt=4) == EINVAL             # a GEMM format only
    assert call(8, 128, 256, la=2) == EINVAL                 # 128 x 4 swizzle: no GEMM
    assert call(8, 128, 256, fmt=2, la=1) == EINVAL          # MXFP8 operands: LINEAR scales only
    assert call(8, 128, 256, fmt=2, lb_=1) == EINVAL
    assert call(8, 128, 48, fmt=2) == ESHAPE                 # MXFP8: K % 32
    assert call(8, 128, 256, variant=3) == EINVAL
    assert call(8, 128, 256, wsb=64) == EINVAL               # workspace bytes without a workspace
    assert call(8, 128, 1024, variant=2) == EINVAL           # split-K without its workspace
    assert call(8, 128, 1024, variant=2, ws=buf.at(32768), wsb=100) == EINVAL
    assert call(8, 128, 256, variant=2, ws=buf.at(32768), wsb=1 << 20) == ESHAPE   # one superstep: no split
    assert call(200, 128, 1024, variant=2, ws=buf.at(32768), wsb=1 << 20) == ESHAPE  # MXFP4 above 128 rows
    assert call(200, 128, 1056, fmt=2, variant=2, ws=buf.at(32768), wsb=1 << 30) == ESHAPE  # MXFP8: K % 128
    assert call(200, 128, 1040, fmt=0, variant=2, ws=buf.at(32768), wsb=1 << 30) == ESHAPE  # NVFP4: K % 64
    # above 64 NVFP4 rows the split runs the 128 x 384 schedule, which reads
    # LINEAR scales as aligned words
    assert L.lowbit_gemm_bf16(a, b, buf.at(8193), sb, 300, 400, 4096, 0, 0, 0, 1.0, out, 2, buf.at(32768),
                              1 << 30, None) == EALIGN
    assert L.lowbit_gemm_bf16(a, b, sa, buf.at(12290), 100, 400, 4096, 0, 0, 0, 1.0, out, 2, buf.at(32768),
                              1 << 30, None) == EALIGN
    assert call(8, 128, 1024, variant=2, ws=buf.at(32772), wsb=1 << 15) == EALIGN   # workspace alignment
    assert call(0, 128, 1024, variant=2) == OK               # empty: nothing to run
    assert call(8, 128, 256, o=None) == EINVAL
    assert call(-1, 128, 256) == ESHAPE
    assert call(8, 128, 48) == ESHAPE                        # K % 32
    assert call(200, 128, 256, variant=0) == ESHAPE          # decode schedule needs M <= 128
    assert call(8, 128, 256, a_=buf.at(4)) == EALIGN
    assert call(0, 128, 256) == OK
    if NO_DEVICE:
        assert call(8, 128, 256) == EDEVICE
        assert call(8, 128, 256, fmt=2) == EDEVICE
        assert call(8, 128, 1024, variant=2, ws=buf.at(32768), wsb=1 << 15) == EDEVICE
        assert call(300, 400, 4096, fmt=0, variant=2, ws=buf.at(32768), wsb=1 << 30) == EDEVICE
        assert call(300, 400, 4096, fmt=2, variant=2, ws=buf.at(32768), wsb=1 << 30) == EDEVICE
        # the automatic split with misaligned LINEAR scales runs unsplit instead
        assert L.lowbit_gemm_bf16(a, b, buf.at(8193), sb, 300, 400, 4096, 0, 0, 0, 1.0, out, -1,
                                  buf.at(32768), 1 << 30, None) == EDEVICE
    # epilogues that need an operand reject its absence
    assert L.lowbit_gemm_bias_bf16(a, b, sa, sb, 8, 128, 256, 1, 0, 0, 1.0, None, out, -1, None, 0,
                                   None) == EINVAL
    assert L.lowbit_gemm_residual_bf16(a, b, sa, sb, 8, 128, 256, 1, 0, 0, 1.0, None, out, -1,
                                       None, 0, None) == EINVAL
    # FP4 out: N must be a multiple of the NVFP4 block
    assert L.lowbit_gemm_bias_gelu_fp4(a, b, sa, sb, 8, 120, 256, 1, 0, 0, 1.0, buf.at(20480), None,
                                       buf.at(24576), buf.at(28672), 0, -1, None, 0, None) == ESHAPE


def test_gemm_fp4_out_takes_fp4_operands(buf):
    """The GELU -> NVFP4 output GEMM takes NVFP4 or MXFP4 operands; MXFP8
    (exact or on the FP8 MFMA) is refused before anything else is checked."""
    L = lb.lib()
    for fmt in (2, 4):
        assert L.lowbit_gemm_bias_gelu_fp4(buf.at(0), buf.at(4096), buf.at(8192), buf.at(12288), 8, 128, 256, fmt,
                                           0, 0, 1.0, buf.at(16384), None, buf.at(20480), buf.at(24576), 0, -1,
                                           None, 0, None) == EINVAL
    if NO_DEVICE:
        assert L.lowbit_gemm_bias_gelu_fp4(buf.at(0), buf.at(4096), buf.at(8192), buf.at(12288), 8, 128, 256, 1,
                                           0, 0, 1.0, buf.at(16384), None, buf.at(20480), buf.at(24576), 0, -1,
                                           None, 0, None) == EDEVICE


def test_gemm_fp8_argument_order(buf):
    L = lb.lib()
    a, b, sa, sb = buf.at(0), buf.at(4096), buf.at(8192), buf.at(12288)

    def call(M=8, N=128, K=256, fmt=2, ol=0, p=16384, sf=True, variant=-1):
        return L.lowbit_gemm_fp8(a, b, sa, sb, M, N, K, fmt, 0, 0, 1.0, buf.at(p),
                                 buf.at(20480) if sf else None, ol, variant, None, 0, None)

    assert call(ol=1) == EINVAL                       # output scales: LINEAR or the 128 x 4 swizzle
    assert call(ol=3) == EINVAL
    assert call(sf=False) == EINVAL
    assert call(fmt=3) == EINVAL
    assert call(N=112) == ESHAPE                      # N % 32
    assert call(K=48) == ESHAPE
    assert call(variant=2) == EINVAL                  # split-K without its workspace
    assert call(p=16392) == EALIGN                    # packed output 16-byte aligned
    assert call(M=0) == OK
    if NO_DEVICE:
        for fmt in (0, 1, 2):
            for ol in (0, 2):
                assert call(fmt=fmt, ol=ol) == EDEVICE


def test_rope_quant_argument_order(buf):
    L = lb.lib()

    def call(T=2, heads=4, D=512, R=64, P=16, fmt=2, layout=0, x=0, pos=True, rope=True, p=4096):
        return L.lowbit_rope_quant(buf.at(x), buf.at(8192) if pos else None, buf.at(12288) if rope else None,
                                   T, heads, D, R, P, fmt, layout, buf.at(p), buf.at(16384), None)

    assert call(fmt=0) == EINVAL                      # NVFP4: not an MX format
    assert call(fmt=3) == EINVAL
    assert call(fmt=2, layout=1) == EINVAL            # MXFP8: LINEAR scales only
    assert call(pos=False) == EINVAL                  # rope without positions
    assert call(rope=False) == EINVAL
    assert call(T=-1) == ESHAPE
    assert call(heads=0) == ESHAPE
    assert call(D=100) == ESHAPE                      # D % 32
    assert call(R=63) == ESHAPE                       # odd rotary slice
    assert call(R=576) == ESHAPE                      # R > D
    assert call(P=0) == ESHAPE
    assert call(x=4) == EALIGN
    assert call(p=8) == EALIGN
    assert call(T=0) == OK
    assert call(R=0, pos=False, rope=False, T=0) == OK
    if NO_DEVICE:
        assert call() == EDEVICE
        assert call(fmt=1, layout=2) == EDEVICE       # MXFP4 takes the FP4 layouts
        assert call(R=0, pos=False, rope=False) == EDEVICE


def test_binding_fails_loudly_without_the_library(monkeypatch):
    monkeypatch.setattr(lb, "LIB_PATH", "/nonexistent/liblowbit.so")
    monkeypatch.setattr(lb, "_lib", None)
    with pytest.raises(RuntimeError):
        lb.lib()
