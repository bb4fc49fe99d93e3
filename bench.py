"""Benchmark of the low-bit linear hot path on one MI355X.

One step = one pass of every stage of the path over one batch of resident,
seeded synthetic input:
  1. fused add + RMSNorm + NVFP4 quant, 4096 x 4096 (outlier channels, global
     scale 6*448/amax)                                   -- HBM-bound
  2. MXFP4 prefill GEMM + bias + residual, (8192, 14336, 4096)
  3. MXFP4 prefill GEMM + bias + residual, (8192, 4096, 14336)   -- MFMA-bound
  4. NVFP4 chain at M = 2048: producer (H = 5120) -> GEMM N = 17408 with
     bias + GELU emitting NVFP4 -> GEMM N = 5120 (K = 17408) to bf16

value = 100 * (sum of the stages' roofline times) / (measured step time): the
step's throughput as a percentage of the one-GPU roofline (HBM 8 TB/s for
the producer, dense FP4 MFMA 10.1 PFLOP/s for the GEMMs).  Per-kernel GB/s and
TFLOP/s are printed on stderr and carried in "kernels".

Prints ONE JSON line on stdout.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import block_scaled_fp4_add_amd as lb  # noqa: E402
from block_scaled_fp4_add_amd import synth  # noqa: E402

HBM_PEAK = 8.0e12          # B/s, MI355X published
FP4_PEAK = 10.1e15         # FLOP/s dense FP4/FP6 MFMA, published
FP16_PEAK = 2.5e15         # FLOP/s dense fp16/bf16 MFMA, published
FP8_PEAK = 5.0e15          # FLOP/s dense FP8 MFMA, published
EPS = 1e-6
COPY_PROBE_BYTES = 1 << 30
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
METRIC = "fused add-RMSNorm-FP4 quant GB/s + FP4 GEMM TFLOPS, as % of 1-GPU roofline"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def producer_bytes(M, H, B, elem_bytes=0.5):
    # x read, r read, r written (bf16) + the codes (half a byte per FP4
    # element, one per MXFP8 element) + one scale byte per block + the weight
    # row and the global scale once per launch
    return M * H * 6 + int(M * H * elem_bytes) + M * H // B + 2 * H + 4


def rope_bytes(T, heads, D, R, elem_bytes):
    # x read (bf16) + the elements (one byte MXFP8, half a byte MXFP4) + a scale
    # byte per 32, per element; each token's table row and position once
    return T * heads * D * 2 + int(T * heads * D * elem_bytes) + T * heads * D // 32 + T * (R * 4 + 8)


ROPE_D, ROPE_R, ROPE_P = 512, 64, 4096   # head, rotary slice, table rows of the RoPE workloads


def rope_stage(name, T, heads, fmt, dev):
    """The inverse-RoPE + MX quantizer over T tokens of `heads` heads."""
    x = synth.activation(T * heads, ROPE_D, 77, outliers=True).reshape(T, heads, ROPE_D).to(dev)
    inv = 10000.0 ** (-np.arange(0, ROPE_R, 2, dtype=np.float64) / ROPE_R)
    ang = np.arange(ROPE_P, dtype=np.float64)[:, None] * inv[None, :]
    tab = torch.from_numpy(np.concatenate([np.cos(ang), np.sin(ang)], 1).astype(np.float32)).to(dev)
    pos = torch.from_numpy(np.random.default_rng(7).integers(0, ROPE_P, T).astype(np.int64)).to(dev)
    pk = torch.empty((T * heads, ROPE_D if fmt == lb.MXFP8 else ROPE_D // 2), dtype=torch.uint8, device=dev)
    sf = torch.empty(lb.lowbit_sf_bytes(T * heads, ROPE_D, fmt, lb.LINEAR), dtype=torch.uint8, device=dev)

    def fn(x=x, pos=pos, tab=tab, pk=pk, sf=sf):
        lb.lowbit_rope_quant(x, pos, tab, fmt, lb.LINEAR, out_packed=pk, out_sf=sf)

    return Stage(name, fn, "hbm", rope_bytes(T, heads, ROPE_D, ROPE_R, 1.0 if fmt == lb.MXFP8 else 0.5), "B",
                 HBM_PEAK)


WOA_N = 1024   # output columns of the MXFP8 GEMM workloads (synthetic: the page gives no head geometry)


def mxfp8_gemm_stage(name, M, N, K, dev, bound, workspace=None, fmt=None):
    """MXFP8 operands (E4M3 elements, UE8M0 scales per 32) through the GEMM
    with the FP8 output epilogue: bf16(A.B^T) quantized to MXFP8 along N,
    scale bytes in the 128 x 4 layout.  With fmt MXFP8 the operands are
    dequantized exactly to bf16 and contracted on bf16 MFMAs, so the executed
    peak is bf16's; with MXFP8_MMA they run on the scaled FP8 MFMA.  The
    roofline prices the format at the FP8 peak (MFMA-bound) or its bytes at
    HBM (decode)."""
    fmt = lb.MXFP8 if fmt is None else fmt
    A = synth.activation(M, K, 79, outliers=True).to(dev)
    a, sa = lb.lowbit_quantize(A, lb.MXFP8, lb.LINEAR)
    # decode: one weight copy per launch of a graph replay, so that the
    # last-level cache does not serve the weights
    wsets = []
    for i in range(DECODE_REPS if bound == "hbm" else 1):
        W = synth.weight(N, K, 79 + i).to(dev)
        wsets.append(lb.lowbit_quantize(W, lb.MXFP8, lb.LINEAR))
    pk = torch.empty((M, N), dtype=torch.uint8, device=dev)
    sf = torch.empty(lb.lowbit_sf_bytes(M, N, lb.MXFP8, lb.SWZ128), dtype=torch.uint8, device=dev)
    it = {"i": 0}

    def fn(a=a, sa=sa, pk=pk, sf=sf, wsets=wsets, it=it, ws=workspace):
        b, sb = wsets[it["i"] % len(wsets)]
        it["i"] += 1
        lb.lowbit_gemm_fp8(a, b, sa, sb, fmt=fmt, out_packed=pk, out_sf=sf, out_layout=lb.SWZ128,
                           workspace=ws)

    if bound == "mfma" and fmt == lb.MXFP8_MMA:
        return Stage(name, fn, "mfma", 2.0 * M * N * K, "FLOP", FP8_PEAK)
    if bound == "mfma":
        return Stage(name, fn, "mfma", 2.0 * M * N * K, "FLOP", FP8_PEAK, own_peak=FP16_PEAK, own_dtype="bf16")
    nbytes = (M + N) * (K + K // 32) + M * N + M * N // 32
    return Stage(name, fn, "hbm", nbytes, "B", HBM_PEAK)


def gemm_bytes(M, N, K, B, epi_bias=False, epi_res=False, out_fp4=False):
    b = (M + N) * (K // 2 + K // B)
    b += 2 * N if epi_bias else 0
    b += 2 * M * N if epi_res else 0
    b += (M * N // 2 + M * N // 16) if out_fp4 else 2 * M * N
    return b


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000   # hipEventDisableSystemFence, hip_runtime_api.h


class HipEvents:
    """Timing-only HIP events recorded on torch's current stream (the stream
    every lowbit call is launched on), created with hipEventDisableSystemFence.
    HIP documents that flag for events used only to measure time: a default
    event's system-scope release writes back and invalidates the caches when
    it is recorded, and that cost lands on the kernels around it (measured on
    the 4096 x 4096 producer: 24.7 us per launch between default events, 22.9
    us between these, 21.1 us back to back).  The functions come from the HIP
    runtime torch itself loaded, so the stream handle is valid for them."""

    def __init__(self):
        import ctypes
        with open("/proc/self/maps") as f:
            paths = sorted({line.split()[-1] for line in f if "libamdhip64.so" in line})
        if len(paths) != 1:
            raise RuntimeError(f"expected one HIP runtime in the process, found {paths}")
        path = paths[0]
        log(f"[bench] HIP events from {path}")
        self.ct = ctypes
        self.L = ctypes.CDLL(path)
        self.live = []

    def record(self):
        ct = self.ct
        e = ct.c_void_p()
        if self.L.hipEventCreateWithFlags(ct.byref(e), ct.c_uint(HIP_EVENT_DISABLE_SYSTEM_FENCE)) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        if self.L.hipEventRecord(e, ct.c_void_p(torch.cuda.current_stream().cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")
        self.live.append(e)
        return e

    def elapsed_ms(self, a, b):
        ct = self.ct
        ms = ct.c_float()
        if self.L.hipEventSynchronize(b) != 0 or self.L.hipEventElapsedTime(ct.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def release(self):
        for e in self.live:
            self.L.hipEventDestroy(e)
        self.live = []


EVENTS = None


class Stage:
    """A kernel launch with its per-launch HIP-event timing on torch's stream
    (the stream every lowbit call is launched on)."""

    def __init__(self, name, fn, bound, work, unit_work, roof, own_peak=None, own_dtype=None, reps=1):
        self.name, self.fn, self.bound, self.work, self.unit_work, self.roof = name, fn, bound, work, unit_work, roof
        # the peak of the arithmetic the kernel executes (the NVFP4 GEMM runs fp16
        # MFMAs on exactly dequantized operands); the step value prices every GEMM at FP4
        self.own_peak = roof if own_peak is None else own_peak
        self.own_dtype = own_dtype
        self.reps = reps          # launches per call of fn (a graph replay holds several)
        self.times = []

    def mean_s(self):
        return float(np.mean([EVENTS.elapsed_ms(a, b) for a, b in self.times])) * 1e-3 / self.reps

    def ideal_s(self):
        return self.work / self.roof


def run_pass(stages, timed):
    """One pass over the stages.  Timed: one HIP event on the launch stream
    before the first stage and one after each stage, so that a stage's time
    runs from the event that ends the previous stage to its own (consecutive
    stages share an event, one event's overhead per stage)."""
    if not timed:
        for s in stages:
            s.fn()
        return
    prev = EVENTS.record()
    for s in stages:
        s.fn()
        e = EVENTS.record()
        s.times.append((prev, e))
        prev = e


def build_stages():
    dev = "cuda"
    stages = []

    # 1. producer, NVFP4 4096 x 4096, rotated over 4 input sets (256 MiB) so
    #    that the 256 MiB last-level cache cannot hold the step's inputs
    c = synth.NVFP4_PRODUCER
    M, H = c["M"], c["H"]
    sets = []
    for i in range(4):
        x, r, w = synth.producer_inputs(M, H, c["seed"] + 100 * i, outliers=True)
        sets.append((x.to(dev), r.to(dev), w.to(dev)))
    # global scale 6*448/amax(y): a calibration input, measured once with the
    # path itself at gs = 1 via dequantization of its own output
    x0, r0, w0 = synth.producer_inputs(M, H, c["seed"], outliers=True)
    p, s = lb.lowbit_add_rmsnorm_quant(x0.to(dev), r0.to(dev), w0.to(dev), EPS, lb.NVFP4, lb.LINEAR)
    amax = lb.lowbit_dequantize(p, s, lb.NVFP4, lb.LINEAR).float().abs().max().item()
    gs = torch.tensor([2688.0 / amax], dtype=torch.float32, device=dev)
    pk = torch.empty((M, H // 2), dtype=torch.uint8, device=dev)
    sf = torch.empty(lb.lowbit_sf_bytes(M, H, lb.NVFP4, lb.LINEAR), dtype=torch.uint8, device=dev)
    it = {"i": 0}

    def producer():
        x, r, w = sets[it["i"] % 4]
        it["i"] += 1
        lb.lowbit_add_rmsnorm_quant(x, r, w, EPS, lb.NVFP4, lb.LINEAR, global_scale=gs, out_packed=pk,
                                    out_sf=sf)

    stages.append(Stage("add_rmsnorm_nvfp4_4096x4096", producer, "hbm", producer_bytes(M, H, 16),
                        "B", HBM_PEAK))

    # 2-3. MXFP4 prefill GEMMs with bias + residual (operands quantized by the path itself)
    c = synth.MXFP4_PREFILL
    for (M, N, K) in c["shapes"]:
        A = synth.activation(M, K, c["seed"], outliers=True).to(dev)
        Wt = synth.weight(N, K, c["seed"]).to(dev)
        a, sfa = lb.lowbit_quantize(A, lb.MXFP4, lb.TILED)
        b, sfb = lb.lowbit_quantize(Wt, lb.MXFP4, lb.TILED)
        del A, Wt
        bias = synth.bias(N, c["seed"]).to(dev)
        res = synth.residual(M, N, c["seed"]).to(dev)
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

        def gemm(a=a, b=b, sfa=sfa, sfb=sfb, bias=bias, res=res, out=out):
            lb.lowbit_gemm_bias_residual_bf16(a, b, sfa, sfb, bias, res, fmt=lb.MXFP4, sfa_layout=lb.TILED,
                                              sfb_layout=lb.TILED, out=out)

        stages.append(Stage(f"mxfp4_gemm_bias_residual_{M}x{N}x{K}", gemm, "mfma", 2.0 * M * N * K, "FLOP",
                            FP4_PEAK))

    # 4. NVFP4 chain at M = 2048
    c = synth.NVFP4_CHAIN
    H, N1, M = c["H"], c["N1"], 2048
    x, r, w = (t.to(dev) for t in synth.producer_inputs(M, H, c["seed"] + M, outliers=True))
    W1 = synth.weight(N1, H, c["seed"], index=10).to(dev)
    W2 = synth.weight(H, N1, c["seed"], index=11).to(dev)
    bias1 = synth.bias(N1, c["seed"], index=12).to(dev)
    gs1 = torch.tensor([2688.0 / W1.float().abs().max().item()], device=dev)
    gs2 = torch.tensor([2688.0 / W2.float().abs().max().item()], device=dev)
    b1, sfb1 = lb.lowbit_quantize(W1, lb.NVFP4, lb.TILED, global_scale=gs1)
    b2, sfb2 = lb.lowbit_quantize(W2, lb.NVFP4, lb.TILED, global_scale=gs2)
    del W1, W2
    p, s = lb.lowbit_add_rmsnorm_quant(x, r.clone(), w, EPS, lb.NVFP4, lb.TILED)
    amax = lb.lowbit_dequantize(p, s, lb.NVFP4, lb.TILED).float().abs().max().item()
    gsA = torch.tensor([2688.0 / amax], dtype=torch.float32, device=dev)
    alpha1 = 1.0 / (gsA.item() * gs1.item())
    alpha2 = 1.0 / gs2.item()
    a1 = torch.empty((M, H // 2), dtype=torch.uint8, device=dev)
    sa1 = torch.empty(lb.lowbit_sf_bytes(M, H, lb.NVFP4, lb.TILED), dtype=torch.uint8, device=dev)
    a2 = torch.empty((M, N1 // 2), dtype=torch.uint8, device=dev)
    sa2 = torch.empty(lb.lowbit_sf_bytes(M, N1, lb.NVFP4, lb.TILED), dtype=torch.uint8, device=dev)
    out2 = torch.empty((M, H), dtype=torch.bfloat16, device=dev)

    def chain_producer():
        lb.lowbit_add_rmsnorm_quant(x, r, w, EPS, lb.NVFP4, lb.TILED, global_scale=gsA, out_packed=a1,
                                    out_sf=sa1)

    def chain_gemm1():
        lb.lowbit_gemm_bias_gelu_fp4(a1, b1, sa1, sfb1, bias1, fmt=lb.NVFP4, sfa_layout=lb.TILED,
                                     sfb_layout=lb.TILED, alpha=alpha1, out_packed=a2, out_sf=sa2,
                                     out_layout=lb.TILED)

    def chain_gemm2():
        lb.lowbit_gemm_bf16(a2, b2, sa2, sfb2, fmt=lb.NVFP4, sfa_layout=lb.TILED, sfb_layout=lb.TILED,
                            alpha=alpha2, out=out2)

    stages.append(Stage(f"chain_add_rmsnorm_nvfp4_{M}x{H}", chain_producer, "hbm",
                        producer_bytes(M, H, 16), "B", HBM_PEAK))
    stages.append(Stage(f"chain_nvfp4_gemm_gelu_fp4_{M}x{N1}x{H}", chain_gemm1, "mfma",
                        2.0 * M * N1 * H, "FLOP", FP4_PEAK, FP16_PEAK, "fp16"))
    stages.append(Stage(f"chain_nvfp4_gemm_{M}x{H}x{N1}", chain_gemm2, "mfma", 2.0 * M * H * N1, "FLOP",
                        FP4_PEAK, FP16_PEAK, "fp16"))
    return stages


def build_variant_stages():
    """Format variants of the step's kernels, timed beside the step and
    reported apart from `value`, at the 4096 x 4096 producer workload with 4
    rotating input sets like the bf16 stage: the NVFP4 producer on fp16
    tensors (same draws, rounded to fp16), the producer with MXFP8 output, and
    the NVFP4 producer writing both scale layouts in one pass; then the
    inverse-RoPE + MX quantizer at a prefill size.  Each is replayed from a
    HIP graph of DECODE_REPS launches, so that the binding's per-call host
    work does not stand in for these 20-30 us kernels."""
    dev = "cuda"
    c = synth.NVFP4_PRODUCER
    M, H = c["M"], c["H"]
    sets = []
    for i in range(4):
        x, r, w = synth.producer_inputs(M, H, c["seed"] + 100 * i, outliers=True, dtype=torch.float16)
        sets.append((x.to(dev), r.to(dev), w.to(dev)))
    x0, r0, w0 = synth.producer_inputs(M, H, c["seed"], outliers=True, dtype=torch.float16)
    p, s = lb.lowbit_add_rmsnorm_quant(x0.to(dev), r0.to(dev), w0.to(dev), EPS, lb.NVFP4, lb.LINEAR)
    amax = lb.lowbit_dequantize(p, s, lb.NVFP4, lb.LINEAR).float().abs().max().item()
    gs = torch.tensor([2688.0 / amax], dtype=torch.float32, device=dev)
    pk = torch.empty((M, H // 2), dtype=torch.uint8, device=dev)
    sf = torch.empty(lb.lowbit_sf_bytes(M, H, lb.NVFP4, lb.LINEAR), dtype=torch.uint8, device=dev)
    it = {"i": 0}

    def producer():
        x, r, w = sets[it["i"] % 4]
        it["i"] += 1
        lb.lowbit_add_rmsnorm_quant_fp16(x, r, w, EPS, lb.NVFP4, lb.LINEAR, global_scale=gs, out_packed=pk,
                                         out_sf=sf)

    stages = [graphed(Stage(f"add_rmsnorm_nvfp4_fp16_{M}x{H}", producer, "hbm", producer_bytes(M, H, 16), "B",
                            HBM_PEAK))]

    # the same bf16 workload quantized to MXFP8 (E4M3 elements, one byte each)
    bsets = []
    for i in range(4):
        x, r, w = synth.producer_inputs(M, H, c["seed"] + 100 * i, outliers=True)
        bsets.append((x.to(dev), r.to(dev), w.to(dev)))
    pk8 = torch.empty((M, H), dtype=torch.uint8, device=dev)
    sf8 = torch.empty(lb.lowbit_sf_bytes(M, H, lb.MXFP8, lb.LINEAR), dtype=torch.uint8, device=dev)
    it8 = {"i": 0}

    def producer8():
        x, r, w = bsets[it8["i"] % 4]
        it8["i"] += 1
        lb.lowbit_add_rmsnorm_quant(x, r, w, EPS, lb.MXFP8, lb.LINEAR, out_packed=pk8, out_sf=sf8)

    stages.append(graphed(Stage(f"add_rmsnorm_mxfp8_{M}x{H}", producer8, "hbm", producer_bytes(M, H, 32, 1.0), "B",
                                HBM_PEAK)))

    # the bf16 NVFP4 producer writing TILED and LINEAR scales in one pass: one
    # more scale byte per block (4096 rows and 256 blocks per row: no padding)
    pkb = torch.empty((M, H // 2), dtype=torch.uint8, device=dev)
    sft = torch.empty(lb.lowbit_sf_bytes(M, H, lb.NVFP4, lb.TILED), dtype=torch.uint8, device=dev)
    sfl = torch.empty(lb.lowbit_sf_bytes(M, H, lb.NVFP4, lb.LINEAR), dtype=torch.uint8, device=dev)
    itb = {"i": 0}

    def producer_both():
        x, r, w = bsets[itb["i"] % 4]
        itb["i"] += 1
        lb.lowbit_add_rmsnorm_quant_both_sf(x, r, w, EPS, lb.NVFP4, lb.TILED, global_scale=gs, out_packed=pkb,
                                            out_sf=sft, out_sf_linear=sfl)

    stages.append(graphed(Stage(f"add_rmsnorm_nvfp4_both_sf_{M}x{H}", producer_both, "hbm",
                                producer_bytes(M, H, 16) + M * H // 16, "B", HBM_PEAK)))
    # inverse RoPE + MX quantization at a prefill size: 4096 tokens x 16 heads of 512
    stages.append(graphed(rope_stage("rope_quant_mxfp8_4096x16x512", 4096, 16, lb.MXFP8, dev)))
    stages.append(graphed(rope_stage("rope_quant_mxfp4_4096x16x512", 4096, 16, lb.MXFP4, dev)))
    # the MXFP8 GEMM with FP8 output on the RoPE workload's rows: 4096 tokens x 16 heads of 512, with
    # the workspace its plan asks for (its 64 tiles of 256 x 256 fill 1/4 of the CUs: K splits in four)
    need = lb.lowbit_gemm_workspace_bytes(4096, WOA_N, 8192, lb.MXFP8, -1)
    ws8 = torch.empty(max(need, 16), dtype=torch.uint8, device=dev) if need else None
    stages.append(graphed(mxfp8_gemm_stage(f"mxfp8_gemm_fp8out_4096x{WOA_N}x8192", 4096, WOA_N, 8192, dev, "mfma",
                                           workspace=ws8)))
    # the same on the scaled FP8 MFMA (LOWBIT_MXFP8_MMA: 64 tiles of 256 x 256, K split in four)
    need = lb.lowbit_gemm_workspace_bytes(4096, WOA_N, 8192, lb.MXFP8_MMA, -1)
    wsm = torch.empty(max(need, 16), dtype=torch.uint8, device=dev) if need else None
    stages.append(graphed(mxfp8_gemm_stage(f"mxfp8_mma_gemm_fp8out_4096x{WOA_N}x8192", 4096, WOA_N, 8192, dev,
                                           "mfma", workspace=wsm, fmt=lb.MXFP8_MMA)))
    return stages


DECODE_REPS = 8   # launches per graph replay: one per rotating weight copy


def graphed(stage):
    """The stage as a HIP graph of DECODE_REPS launches (captured from torch's
    stream, onto which every lowbit call launches), replayed by stage.fn.  A
    decode step is a launch-bound loop: replaying it as a graph measures the
    kernels back to back, not the host's launch overhead (the library
    allocates nothing and never synchronizes, so its calls capture as they
    are).  The stage runs once eagerly first.

    The graph holds raw device pointers of every tensor the captured calls
    touch, and every later capture starts with torch.cuda.empty_cache(),
    which returns freed blocks to the driver: the eager function, whose
    closure owns those tensors, stays referenced by the stage for as long as
    the graph can be replayed."""
    log(f"[bench] capturing {stage.name}")
    stage.fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(DECODE_REPS):
            stage.fn()
    torch.cuda.synchronize()
    stage.eager_fn = stage.fn          # keeps the captured tensors alive
    stage.fn, stage.reps, stage.graph = g.replay, DECODE_REPS, g
    return stage


def build_decode_stages():
    """The decode-shaped workloads, timed beside the step and reported apart
    from `value`: the four MXFP4 decode GEMMs (with a split-K workspace
    offered, and without) and the NVFP4 chain at 1 and 128 tokens (producer,
    GEMM1 with GELU -> FP4, GEMM2, the GEMMs with the workspace offered).
    These are HBM-bound (the weights dominate); each rotates over enough
    weight copies that the 256 MiB last-level cache cannot hold them, as a
    decode step sees them."""
    dev = "cuda"
    stages = []
    lay = lb.TILED

    def rotating(N, K, fmt, seed, copies=8):
        # one quantized weight, copied to `copies` distinct buffers: every
        # decode stage rotates its own copies, and together they cycle well over
        # a gigabyte through the last-level cache
        W = synth.weight(N, K, seed).to(dev)
        b, sfb = lb.lowbit_quantize(W, fmt, lay)
        del W
        return [(b.clone(), sfb.clone()) for _ in range(copies)]

    # one split-K workspace for every decode GEMM (the automatic choice splits
    # K where the library's plan says so; each stage also runs without it)
    c = synth.MXFP4_DECODE
    need = [lb.lowbit_gemm_workspace_bytes(M, N, K, f, lb.VARIANT_AUTO) for (M, N, K) in c["shapes"]
            for f in (lb.NVFP4, lb.MXFP4)]
    need += [lb.lowbit_gemm_workspace_bytes(M, N, K, lb.NVFP4, lb.VARIANT_AUTO)
             for M in (1, 128) for (N, K) in ((synth.NVFP4_CHAIN["N1"], synth.NVFP4_CHAIN["H"]),
                                              (synth.NVFP4_CHAIN["H"], synth.NVFP4_CHAIN["N1"]))]
    need += [lb.lowbit_gemm_workspace_bytes(96, WOA_N, 8192, lb.MXFP8, lb.VARIANT_AUTO)]
    wspace = torch.empty(max(need + [16]), dtype=torch.uint8, device=dev)
    for (M, N, K) in c["shapes"]:
        A = synth.activation(M, K, c["seed"]).to(dev)
        a, sfa = lb.lowbit_quantize(A, lb.MXFP4, lay)
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        for use_ws in (True, False):
            wts = rotating(N, K, lb.MXFP4, c["seed"])   # own copies: the other stage leaves nothing warm
            it = {"i": 0}

            def gemm(a=a, sfa=sfa, wts=wts, out=out, it=it, ws=wspace if use_ws else None):
                b, sfb = wts[it["i"] % len(wts)]
                it["i"] += 1
                lb.lowbit_gemm_bf16(a, b, sfa, sfb, fmt=lb.MXFP4, sfa_layout=lay, sfb_layout=lay, out=out,
                                    workspace=ws)

            stages.append(graphed(Stage(f"mxfp4_decode_gemm_{M}x{N}x{K}" + ("" if use_ws else "_no_workspace"),
                                        gemm, "hbm", gemm_bytes(M, N, K, 32), "B", HBM_PEAK)))
    # the NVFP4 chain as the workload defines it: weights quantized with
    # gs_B = 6*448/amax(B), activations with gs_A = 6*448/amax(y) (calibrated
    # once with the path itself at gs = 1), alpha = 1/(gs_A gs_B) for GEMM1 and
    # 1/gs_B for GEMM2 (GEMM1 writes its FP4 output with gs_out = 1)
    c = synth.NVFP4_CHAIN
    H, N1 = c["H"], c["N1"]

    def rotating_gs(N, K, seed, index, copies=8):
        W = synth.weight(N, K, seed, index=index).to(dev)
        gsb = 2688.0 / W.float().abs().max().item()
        b, sfb = lb.lowbit_quantize(W, lb.NVFP4, lay, global_scale=torch.tensor([gsb], device=dev))
        del W
        return [(b.clone(), sfb.clone()) for _ in range(copies)], gsb

    w1, gsb1 = rotating_gs(N1, H, c["seed"], 10)
    w2, gsb2 = rotating_gs(H, N1, c["seed"], 11)
    bias1 = synth.bias(N1, c["seed"], index=12).to(dev)
    for M in (1, 128):
        x, r, w = (t.to(dev) for t in synth.producer_inputs(M, H, c["seed"] + M, outliers=True))
        p, s = lb.lowbit_add_rmsnorm_quant(x, r.clone(), w, EPS, lb.NVFP4, lay)
        amax = lb.lowbit_dequantize(p, s, lb.NVFP4, lay).float().abs().max().item()
        gs1 = torch.tensor([2688.0 / amax], dtype=torch.float32, device=dev)
        alpha1, alpha2 = 1.0 / (gs1.item() * gsb1), 1.0 / gsb2
        a1 = torch.empty((M, H // 2), dtype=torch.uint8, device=dev)
        sa1 = torch.empty(lb.lowbit_sf_bytes(M, H, lb.NVFP4, lay), dtype=torch.uint8, device=dev)
        a2 = torch.empty((M, N1 // 2), dtype=torch.uint8, device=dev)
        sa2 = torch.empty(lb.lowbit_sf_bytes(M, N1, lb.NVFP4, lay), dtype=torch.uint8, device=dev)
        out2 = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
        it = {"i": 0, "j": 0}

        def prod(x=x, r=r, w=w, a1=a1, sa1=sa1, gs1=gs1):
            lb.lowbit_add_rmsnorm_quant(x, r, w, EPS, lb.NVFP4, lay, global_scale=gs1, out_packed=a1, out_sf=sa1)

        def g1(a1=a1, sa1=sa1, a2=a2, sa2=sa2, it=it, alpha1=alpha1):
            b, sfb = w1[it["j"] % len(w1)]
            it["j"] += 1
            lb.lowbit_gemm_bias_gelu_fp4(a1, b, sa1, sfb, bias1, fmt=lb.NVFP4, sfa_layout=lay, sfb_layout=lay,
                                         alpha=alpha1, out_packed=a2, out_sf=sa2, out_layout=lay,
                                         workspace=wspace)

        def g2(a2=a2, sa2=sa2, out2=out2, it=it, alpha2=alpha2):
            b, sfb = w2[it["i"] % len(w2)]
            it["i"] += 1
            lb.lowbit_gemm_bf16(a2, b, sa2, sfb, fmt=lb.NVFP4, sfa_layout=lay, sfb_layout=lay, alpha=alpha2,
                                out=out2, workspace=wspace)

        stages.append(graphed(Stage(f"chain_m{M}_add_rmsnorm_nvfp4_{M}x{H}", prod, "hbm", producer_bytes(M, H, 16),
                                    "B", HBM_PEAK)))
        stages.append(graphed(Stage(f"chain_m{M}_nvfp4_gemm_gelu_fp4_{M}x{N1}x{H}", g1, "hbm",
                                    gemm_bytes(M, N1, H, 16, epi_bias=True, out_fp4=True), "B", HBM_PEAK)))
        stages.append(graphed(Stage(f"chain_m{M}_nvfp4_gemm_{M}x{H}x{N1}", g2, "hbm", gemm_bytes(M, H, N1, 16),
                                    "B", HBM_PEAK)))
    # inverse RoPE + MXFP8 at the page's decode size: 96 tokens x 16 heads of 512
    stages.append(graphed(rope_stage("rope_quant_mxfp8_96x16x512", 96, 16, lb.MXFP8, dev)))
    stages.append(graphed(mxfp8_gemm_stage(f"mxfp8_gemm_fp8out_96x{WOA_N}x8192", 96, WOA_N, 8192, dev, "hbm",
                                           workspace=wspace)))
    return stages


def report(stages):
    kernels = {}
    for s in stages:
        t = s.mean_s()
        rate = s.work / t
        frac = s.ideal_s() / t
        kernels[s.name] = {"us": round(t * 1e6, 2),
                           ("GB/s" if s.unit_work == "B" else "TFLOP/s"):
                               round(rate / (1e9 if s.unit_work == "B" else 1e12), 1),
                           "roofline_frac": round(frac, 4)}
        if s.own_peak != s.roof:
            kernels[s.name][f"{s.own_dtype}_mfma_frac"] = round(s.work / t / s.own_peak, 4)
        log(f"[bench] {s.name}: {t * 1e6:.1f} us, "
            f"{rate / (1e9 if s.unit_work == 'B' else 1e12):.1f} {'GB/s' if s.unit_work == 'B' else 'TFLOP/s'}, "
            f"{100 * frac:.1f}% of roofline")
    return kernels


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_step_time(orc, stages, small):
    """Extrapolated oracle time of one step: the full 4096 x 4096 producer,
    timed, plus a rows x columns block (full K) of each GEMM, timed and scaled
    by its share of the GEMM's multiply-accumulates.  small: blocks 16x
    smaller (the one-core run)."""
    parts = []
    t_step = 0.0

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    # producers: the full NVFP4 4096 x 4096 workload, rate in bytes/s
    c = synth.NVFP4_PRODUCER
    x, r, w = synth.producer_inputs(c["M"], c["H"], c["seed"], outliers=True)
    xb, rb, wb = synth.bits(x), synth.bits(r), synth.bits(w)
    dt = timed(lambda: orc.add_rmsnorm_quant(xb, rb, wb, EPS, orc.NVFP4, orc.LINEAR, gs=1.0))
    rate_b = producer_bytes(c["M"], c["H"], 16) / dt
    t_step += sum(s.work for s in stages if s.unit_work == "B") / rate_b
    parts.append(f"producer {c['M']}x{c['H']} nvfp4 full ({dt:.2f} s)")

    def gemm_rate(M, N, K, fmt, Msub, Nsub, seed, gelu_fp4=False):
        if small:
            Msub, Nsub = Msub // 4, Nsub // 4
        A = synth.activation(Msub, K, seed, outliers=True)
        Wt = synth.weight(Nsub, K, seed)
        a, sfa = orc.quantize(synth.bits(A), fmt, orc.TILED)
        b, sfb = orc.quantize(synth.bits(Wt), fmt, orc.TILED)
        bias = synth.bits(synth.bias(Nsub, seed))
        if gelu_fp4:
            fn = lambda: orc.gemm_gelu_fp4(a, b, sfa, sfb, Msub, Nsub, K, fmt, orc.TILED, orc.TILED, 1.0,
                                           bias, 1.0, orc.TILED)
        else:
            res = synth.bits(synth.residual(Msub, Nsub, seed))
            fn = lambda: orc.gemm(a, b, sfa, sfb, Msub, Nsub, K, fmt, orc.TILED, orc.TILED, 1.0,
                                  orc.EPI_BIAS_RESIDUAL, bias, res)
        dt = timed(fn)
        parts.append(f"{'nvfp4' if fmt == orc.NVFP4 else 'mxfp4'} gemm{'-gelu-fp4' if gelu_fp4 else ''} "
                     f"{Msub}x{Nsub} of ({M},{N},{K}) ({dt:.2f} s)")
        return Msub * Nsub * K / dt

    gemm_stages = [s for s in stages if s.unit_work == "FLOP"]
    (M1, N1, K1), (M2, N2, K2) = synth.MXFP4_PREFILL["shapes"]
    ch = synth.NVFP4_CHAIN
    samples = [
        (gemm_stages[0], gemm_rate(M1, N1, K1, orc.MXFP4, 2048, 8192, 1)),
        (gemm_stages[1], gemm_rate(M2, N2, K2, orc.MXFP4, 2048, 4096, 2)),
        (gemm_stages[2], gemm_rate(2048, ch["N1"], ch["H"], orc.NVFP4, 1024, 8192, 3, gelu_fp4=True)),
        (gemm_stages[3], gemm_rate(2048, ch["H"], ch["N1"], orc.NVFP4, 1024, 4096, 4)),
    ]
    for st, mac_rate in samples:
        t_step += (st.work / 2) / mac_rate
    return t_step, parts


def oracle_config_seconds(orc, small=False):
    """Oracle seconds of each workload on the threads the oracle is set to:
    the tiny MXFP4 case, the 4096 x 4096 producer and the four decode GEMMs in
    full; the prefill GEMMs and the chain's GEMMs from a timed block scaled by
    its share of the multiply-accumulates (the chain at M = 1 and 128 in
    full).  small: the one-core pass -- each timed call runs on one thread
    (the inputs are prepared on all of them), the decode GEMMs on 8 rows, the
    prefill GEMMs on 32, the chain at M = 128 and 2048 on 8, each timed also
    on half its rows and extrapolated linearly in the row count."""
    out = {}
    threads = orc.num_threads()

    def timed(fn):
        if small:
            orc.set_num_threads(1)
        try:
            t0 = time.perf_counter()
            fn()
            return time.perf_counter() - t0
        finally:
            orc.set_num_threads(threads)

    c = synth.TINY_MXFP4
    x, r, w = synth.producer_inputs(c["M"], c["H"], c["seed"])
    W = synth.weight(c["N"], c["H"], c["seed"])

    def tiny():
        d = orc.add_rmsnorm_quant(synth.bits(x), synth.bits(r), synth.bits(w), EPS, orc.MXFP4, orc.LINEAR)
        b, sfb = orc.quantize(synth.bits(W), orc.MXFP4, orc.LINEAR)
        orc.gemm(d["packed"], b, d["sf"], sfb, c["M"], c["N"], c["H"], orc.MXFP4, orc.LINEAR, orc.LINEAR)
    out["tiny_mxfp4_m8_h256_gemm_8x128x256"] = round(timed(tiny), 5)

    c = synth.NVFP4_PRODUCER
    x, r, w = synth.producer_inputs(c["M"], c["H"], c["seed"], outliers=True)
    out["nvfp4_producer_4096x4096"] = round(timed(lambda: orc.add_rmsnorm_quant(
        synth.bits(x), synth.bits(r), synth.bits(w), EPS, orc.NVFP4, orc.LINEAR, gs=1.0)), 3)

    def gemm_s(M, N, K, fmt, epi=orc.EPI_NONE, rows=None, gelu_fp4=False, seed=9):
        Ms = M if rows is None else min(M, rows)
        A = synth.activation(Ms, K, seed)
        Wt = synth.weight(N, K, seed)
        a, sfa = orc.quantize(synth.bits(A), fmt, orc.TILED)
        b, sfb = orc.quantize(synth.bits(Wt), fmt, orc.TILED)
        bias = synth.bits(synth.bias(N, seed))
        res = synth.bits(synth.residual(Ms, N, seed))
        def run(rows):
            if gelu_fp4:
                return timed(lambda: orc.gemm_gelu_fp4(a, b, sfa, sfb, rows, N, K, fmt, orc.TILED, orc.TILED, 1.0,
                                                       bias, 1.0, orc.TILED))
            return timed(lambda: orc.gemm(a, b, sfa, sfb, rows, N, K, fmt, orc.TILED, orc.TILED, 1.0, epi, bias, res))
        dt = run(Ms)
        if not small or Ms == M:
            return dt * M / Ms
        # one-core samples are a few rows: the call's fixed cost (the B
        # operand's decode) is counted once, the rows' cost scaled
        half = run(Ms // 2)
        return dt + (dt - half) * (M - Ms) / (Ms - Ms // 2)

    for (M, N, K) in synth.MXFP4_DECODE["shapes"]:
        key = f"mxfp4_decode_gemm_{M}x{N}x{K}" + ("_extrapolated" if small and M > 8 else "")
        out[key] = round(gemm_s(M, N, K, orc.MXFP4, rows=8 if small else None), 3)
    for (M, N, K) in synth.MXFP4_PREFILL["shapes"]:
        out[f"mxfp4_prefill_gemm_bias_residual_{M}x{N}x{K}_extrapolated"] = round(
            gemm_s(M, N, K, orc.MXFP4, orc.EPI_BIAS_RESIDUAL, rows=32 if small else 256), 2)
    ch = synth.NVFP4_CHAIN
    for M in ch["Ms"]:
        x, r, w = synth.producer_inputs(M, ch["H"], ch["seed"] + M, outliers=True)
        tp = timed(lambda: orc.add_rmsnorm_quant(synth.bits(x), synth.bits(r), synth.bits(w), EPS, orc.NVFP4,
                                                 orc.TILED))
        rows = (None if M == 1 else 8) if small else (None if M <= 128 else 64)
        t1 = gemm_s(M, ch["N1"], ch["H"], orc.NVFP4, rows=rows, gelu_fp4=True)
        t2 = gemm_s(M, ch["H"], ch["N1"], orc.NVFP4, rows=rows)
        key = f"nvfp4_chain_m{M}" + ("_extrapolated" if rows else "")
        out[key] = round(tp + t1 + t2, 3)
    return out


def cpu_baseline(stages, step_ideal_s):
    """Time the CPU oracle, as it stands, on a bounded sample of every stage
    of the step and extrapolate each stage by its share of the work (bytes
    for the producers, multiply-accumulates for the GEMMs): once on all the
    host's cores and once on one core (smaller GEMM blocks), plus the oracle
    seconds of each workload.  A reported baseline, not a target."""
    from oracle import oracle as orc

    orc.lib()
    threads = orc.num_threads()
    t_all, parts = _oracle_step_time(orc, stages, small=False)
    orc.set_num_threads(1)
    try:
        t_one, parts1 = _oracle_step_time(orc, stages, small=True)
    finally:
        orc.set_num_threads(threads)
    configs = oracle_config_seconds(orc)
    log("[bench] cpu baseline: workloads on one core")
    configs1 = oracle_config_seconds(orc, small=True)
    return {"value": 100.0 * step_ideal_s / t_all, "unit": "% of 1-GPU roofline", "cores": threads,
            "kind": "oracle", "step_s": round(t_all, 2),
            "value_1core": 100.0 * step_ideal_s / t_one, "step_s_1core": round(t_one, 2),
            "nproc": os.cpu_count(), "cpu_model": cpu_model(),
            "sample": "; ".join(parts) + f"; extrapolated step time {t_all:.1f} s on {threads} threads",
            "sample_1core": "; ".join(parts1) + f"; extrapolated step time {t_one:.1f} s on 1 thread",
            "config_seconds": configs, "config_seconds_1core": configs1}


def source_digest():
    """sha256 over the kernel sources: counters taken on other sources do not apply."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_scaled_fp4_add_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp", ".cpp")):
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def measured_traffic(stage_name):
    """HBM bytes per launch of a stage from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, each scaled by the copy-kernel calibration), or
    None when there is none for this stage or the kernels changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != source_digest():
        return None
    k = t.get("kernels", {}).get(stage_name)
    return None if k is None else k.get("hbm_bytes_per_launch")


def copy_probe():
    """An elementwise kernel that reads and writes COPY_PROBE_BYTES each, three
    times (torch.add: a plain streaming kernel; copy_ would go to the runtime's
    blit path); 1 GiB so that what the fill leaves in L2 is negligible."""
    src = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.add(src, 1.0, out=dst)
    torch.cuda.synchronize()
    del src, dst


def counter_run(args):
    """Launches for a counter profiler (rocprofv3 --pmc): every selected stage
    args.counters times back to back, untimed, then the copy probe."""
    stages = build_stages()
    if not args.no_decode:
        stages += build_decode_stages() + build_variant_stages()
    sel = [k for k in args.only.split(",") if k]
    torch.cuda.synchronize()
    for s in stages:
        if sel and not any(k in s.name for k in sel):
            continue
        for _ in range(args.counters):
            s.fn()
        torch.cuda.synchronize()
        log(f"[bench] ran {s.name} x{args.counters}")
    if args.copy_probe:
        copy_probe()
        log("[bench] ran copy probe")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode-shaped workloads reported beside the step")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after the timed region, run a 1 GiB read + 1 GiB write elementwise kernel "
                         "three times: the known-size kernel that calibrates the HBM byte counters")
    ap.add_argument("--counters", type=int, default=0, metavar="REPS",
                    help="counter-collection run for a profiler: build the stages (the decode and format "
                         "variants too unless --no-decode), launch each selected stage REPS times with no "
                         "timing, then the copy probe if asked, and print no JSON line")
    ap.add_argument("--only", default="",
                    help="with --counters: comma-separated substrings; run only stages whose name has one")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    lb.lib()
    global EVENTS
    torch.cuda.init()
    EVENTS = HipEvents()
    if args.counters > 0:
        counter_run(args)
        return
    log("[bench] building inputs")
    stages = build_stages()
    torch.cuda.synchronize()
    log("[bench] warmup")
    for _ in range(args.warmup):
        run_pass(stages, False)
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run_pass(stages, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / args.steps * 1e3
    if args.copy_probe:
        copy_probe()
    ideal = sum(s.ideal_s() for s in stages)
    value = 100.0 * ideal / (wall / args.steps)
    kernels = report(stages)
    decode = None
    if not args.no_decode:
        # decode-shaped workloads: timed after the step, reported apart from `value`
        log("[bench] decode workloads")
        dstages = build_decode_stages()
        for _ in range(3):
            run_pass(dstages, False)
        for _ in range(args.steps):
            run_pass(dstages, True)
        torch.cuda.synchronize()
        decode = report(dstages)
    # format variants (fp16 producer), also apart from `value`
    log("[bench] variants")
    vstages = build_variant_stages()
    for _ in range(3):
        run_pass(vstages, False)
    for _ in range(args.steps):
        run_pass(vstages, True)
    torch.cuda.synchronize()
    variants = report(vstages)
    # dominant kernel: the one with the largest share of the step
    dom = max(stages, key=lambda s: s.mean_s())
    t = dom.mean_s()
    scale = 1e9 if dom.bound == "hbm" else 1e12
    # priced at the step's roof (FP4 for every GEMM, as `value` and `dtype`);
    # an NVFP4 GEMM's fraction of the fp16 MFMA peak it executes on rides beside
    roof = {"bound": dom.bound, "achieved": round(dom.work / t / scale, 2),
            "peak": dom.roof / scale, "unit": "GB/s" if dom.bound == "hbm" else "TFLOP/s",
            "frac": round(dom.work / t / dom.roof, 4), "traffic": measured_traffic(dom.name),
            "kernel": dom.name, "peak_dtype": "fp4" if dom.bound == "mfma" else "hbm"}
    if dom.own_peak != dom.roof:
        roof["executed_peak"] = dom.own_peak / scale
        roof["executed_dtype"] = dom.own_dtype
        roof["frac_of_executed_peak"] = round(dom.work / t / dom.own_peak, 4)
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        cpu = cpu_baseline(stages, ideal)
    line = {"metric": METRIC, "value": round(value, 3), "unit": "% of 1-GPU roofline", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp4_e2m1",
            "data": "synthetic",
            "config": {"workload": "nvfp4_add_rmsnorm_quant_m4096_h4096 + "
                                   "mxfp4_prefill_gemm_bias_residual (8192,14336,4096),(8192,4096,14336) + "
                                   "nvfp4_chain_m2048_h5120_n17408",
                       "parallelism": "none (1 GPU)"},
            "roofline": roof, "cpu_baseline": cpu, "kernels": kernels, "decode": decode,
            "variants": variants}
    print(json.dumps(line), flush=True)
    EVENTS.release()


if __name__ == "__main__":
    main()
