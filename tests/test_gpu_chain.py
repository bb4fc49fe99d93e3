"""The NVFP4 chain -- add + RMSNorm + quant (H = 5120) -> GEMM N = 17408 with a
bias + GELU epilogue emitting NVFP4 -> GEMM N = 5120, K = 17408 to bf16 -- at
M = 1, 128, 2048, checked stage by stage:

* the producer in full;
* each GEMM relaunched on sampled rows of the oracle's bytes of the previous
  stage;
* each GEMM at the full-M launch the benchmark times (decode with four M-tiles
  at M = 128, the prefill tiles at M = 2048), on sampled rows and every
  column, against the oracle fed with the bytes that launch consumed (the
  device producer's output for GEMM1, the device GEMM1's for GEMM2), under
  the same rules as everywhere else and with no allowance."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_add_amd as lb
from block_scaled_fp4_add_amd import synth

from . import checkers
from .gpu_util import banner, dev_bf16, dev_f32, dev_u8, host_f64, host_u8

pytestmark = pytest.mark.gpu
EPS = 1e-6


def linear_rows(orc, packed, sf, rows_idx, K, fmt, layout):
    """Sub-operand made of the listed rows, scales re-laid out LINEAR (test plumbing)."""
    B = 16 if fmt == 0 else 32
    full = checkers.gather_scales(orc, sf, packed.shape[0], K // B, fmt, layout)
    return np.ascontiguousarray(packed[rows_idx]), np.ascontiguousarray(full[rows_idx]).ravel()


@pytest.fixture(scope="module")
def weights(orc):
    c = synth.NVFP4_CHAIN
    H, N1, seed = c["H"], c["N1"], c["seed"]
    W1 = synth.weight(N1, H, seed, index=10)
    W2 = synth.weight(H, N1, seed, index=11)
    bias1 = synth.bias(N1, seed, index=12)
    gs1 = float(np.float32(2688.0 / W1.float().abs().max().item()))
    gs2 = float(np.float32(2688.0 / W2.float().abs().max().item()))
    b1, sfb1 = orc.quantize(synth.bits(W1), orc.NVFP4, orc.TILED, gs=gs1)
    b2, sfb2 = orc.quantize(synth.bits(W2), orc.NVFP4, orc.TILED, gs=gs2)
    return dict(H=H, N1=N1, bias1=bias1, gs1=gs1, gs2=gs2, b1=b1, sfb1=sfb1, b2=b2, sfb2=sfb2,
                d_b1=dev_u8(b1), d_sfb1=dev_u8(sfb1), d_b2=dev_u8(b2), d_sfb2=dev_u8(sfb2),
                d_bias1=dev_bf16(bias1))


@pytest.mark.parametrize("M", synth.NVFP4_CHAIN["Ms"])
def test_nvfp4_chain(orc, weights, M):
    W = weights
    H, N1 = W["H"], W["N1"]
    seed = synth.NVFP4_CHAIN["seed"] + M
    banner(f"chain M={M}")
    x, r, w = synth.producer_inputs(M, H, seed, outliers=True)
    y = orc.add_rmsnorm_quant(synth.bits(x), synth.bits(r), synth.bits(w), EPS, orc.NVFP4, orc.LINEAR,
                              diag=True)["y"]
    gsA = float(np.float32(2688.0 / np.abs(y).max()))
    # --- stage 1: producer
    pro = orc.add_rmsnorm_quant(synth.bits(x), synth.bits(r), synth.bits(w), EPS, orc.NVFP4, orc.TILED,
                                gs=gsA, diag=True)
    rd = dev_bf16(r)
    a1, sfa1 = lb.lowbit_add_rmsnorm_quant(dev_bf16(x), rd, dev_bf16(w), EPS, lb.NVFP4, lb.TILED,
                                           global_scale=dev_f32(gsA))
    torch.cuda.synchronize()
    rep = checkers.compare_quantized(orc, 0, gsA, host_u8(a1), host_u8(sfa1), pro["packed"], pro["sf"],
                                     pro["y"], pro["v"], pro["spre"], M, H, orc.TILED)
    banner(f"  producer {dict(rep)}")
    assert rep.ok(), rep

    # sampled rows: the first and last, tile edges, and random ones (every column is checked)
    edges = [r for r in (31, 32, 127, 128, 255, 256, 1023, 1024) if r < M]
    rows = np.arange(M) if M <= 4 else np.unique(np.r_[0, M - 1, edges,
                                                        np.random.default_rng(M).integers(0, M, 8)])
    alpha1 = 1.0 / (gsA * W["gs1"])
    alpha2 = 1.0 / W["gs2"]
    # --- stage 2: GEMM1 + bias + GELU -> NVFP4, device fed with the oracle's producer bytes
    a_sub, sfa_sub = linear_rows(orc, pro["packed"], pro["sf"], rows, H, 0, orc.TILED)
    g1 = orc.gemm_gelu_fp4(a_sub, W["b1"], sfa_sub, W["sfb1"], len(rows), N1, H, 0, 0, 1, alpha1,
                           synth.bits(W["bias1"]), 1.0, orc.LINEAR, diag=True)
    p1, s1 = lb.lowbit_gemm_bias_gelu_fp4(dev_u8(pro["packed"]), W["d_b1"], dev_u8(pro["sf"]), W["d_sfb1"],
                                          W["d_bias1"], fmt=0, sfa_layout=1, sfb_layout=1, alpha=alpha1,
                                          out_layout=lb.TILED)
    torch.cuda.synchronize()
    gp, gsf = linear_rows(orc, host_u8(p1), host_u8(s1), rows, N1, 0, orc.TILED)
    ce, se = checkers.fp4_out_windows(g1, 1.0, len(rows), N1)
    rep = checkers.compare_quantized(
        orc, 0, 1.0, gp, gsf, g1["packed"], g1["sf"], g1["y"], g1["v"], g1["spre"], len(rows), N1,
        orc.LINEAR, code_extra=ce, scale_extra=se)
    banner(f"  gemm1 fp4 {dict(rep)}")
    assert rep.ok(), rep
    # --- stage 3: GEMM2 -> bf16, device fed with the oracle's GEMM1 bytes (sampled rows)
    ref2, l12 = orc.gemm(g1["packed"], W["b2"], g1["sf"], W["sfb2"], len(rows), H, N1, 0, 0, 1,
                         alpha=alpha2)
    out2 = lb.lowbit_gemm_bf16(dev_u8(g1["packed"]), W["d_b2"], dev_u8(g1["sf"]), W["d_sfb2"], fmt=0,
                               sfa_layout=0, sfb_layout=1, alpha=alpha2)
    torch.cuda.synchronize()
    ok, worst = checkers.gemm_within_tolerance(host_f64(out2), ref2, l12)
    banner(f"  gemm2 worst {worst:.3g}")
    assert ok.all()
    # --- the full-M launches the benchmark times, each against the oracle fed
    # with the bytes that launch consumed
    p1d, s1d = lb.lowbit_gemm_bias_gelu_fp4(a1, W["d_b1"], sfa1, W["d_sfb1"], W["d_bias1"], fmt=0,
                                            sfa_layout=1, sfb_layout=1, alpha=alpha1, out_layout=lb.TILED)
    out_e2e = lb.lowbit_gemm_bf16(p1d, W["d_b2"], s1d, W["d_sfb2"], fmt=0, sfa_layout=1, sfb_layout=1,
                                  alpha=alpha2)
    torch.cuda.synchronize()
    a_dev, sfa_dev = linear_rows(orc, host_u8(a1), host_u8(sfa1), rows, H, 0, orc.TILED)
    g1d = orc.gemm_gelu_fp4(a_dev, W["b1"], sfa_dev, W["sfb1"], len(rows), N1, H, 0, 0, 1, alpha1,
                            synth.bits(W["bias1"]), 1.0, orc.LINEAR, diag=True)
    gp, gsf = linear_rows(orc, host_u8(p1d), host_u8(s1d), rows, N1, 0, orc.TILED)
    ce, se = checkers.fp4_out_windows(g1d, 1.0, len(rows), N1)
    rep = checkers.compare_quantized(
        orc, 0, 1.0, gp, gsf, g1d["packed"], g1d["sf"], g1d["y"], g1d["v"], g1d["spre"], len(rows), N1,
        orc.LINEAR, code_extra=ce, scale_extra=se)
    banner(f"  gemm1 at the full launch {dict(rep)}")
    assert rep.ok(), rep
    assert checkers.tiled_padding_is_zero(orc, host_u8(s1d), M, N1 // 16, 0)
    ref2d, l12d = orc.gemm(gp, W["b2"], gsf, W["sfb2"], len(rows), H, N1, 0, 0, 1, alpha=alpha2)
    got = host_f64(out_e2e)[rows]
    assert np.all(np.isfinite(got))
    ok, worst = checkers.gemm_within_tolerance(got, ref2d, l12d)
    banner(f"  gemm2 at the full launch: worst {worst:.3g}, violations {int((~ok).sum())}")
    assert ok.all(), f"{int((~ok).sum())} outputs out of tolerance (worst ratio {worst})"


@pytest.mark.parametrize("M", [1, 128])
def test_nvfp4_chain_splitk(orc, weights, M):
    """The decode chain with a workspace offered to both GEMMs (split-K where
    the plan splits: GEMM2, K = 17408), checked like the launches above on
    sampled rows and every column against the oracle fed with the device's
    own bytes."""
    W = weights
    H, N1 = W["H"], W["N1"]
    x, r, w = synth.producer_inputs(M, H, synth.NVFP4_CHAIN["seed"] + M, outliers=True)
    y = orc.add_rmsnorm_quant(synth.bits(x), synth.bits(r), synth.bits(w), EPS, orc.NVFP4, orc.LINEAR,
                              diag=True)["y"]
    gsA = float(np.float32(2688.0 / np.abs(y).max()))
    a1, sfa1 = lb.lowbit_add_rmsnorm_quant(dev_bf16(x), dev_bf16(r), dev_bf16(w), EPS, lb.NVFP4, lb.TILED,
                                           global_scale=dev_f32(gsA))
    alpha1, alpha2 = 1.0 / (gsA * W["gs1"]), 1.0 / W["gs2"]
    n1 = lb.lowbit_gemm_workspace_bytes(M, N1, H, 0, -1)
    n2 = lb.lowbit_gemm_workspace_bytes(M, H, N1, 0, -1)
    assert n2 > 0, "the down-projection splits K"
    ws = torch.empty(max(n1, n2), dtype=torch.uint8, device="cuda")
    p1, s1 = lb.lowbit_gemm_bias_gelu_fp4(a1, W["d_b1"], sfa1, W["d_sfb1"], W["d_bias1"], fmt=0, sfa_layout=1,
                                          sfb_layout=1, alpha=alpha1, out_layout=lb.TILED, workspace=ws)
    out = lb.lowbit_gemm_bf16(p1, W["d_b2"], s1, W["d_sfb2"], fmt=0, sfa_layout=1, sfb_layout=1, alpha=alpha2,
                              workspace=ws)
    torch.cuda.synchronize()
    rows = np.arange(M) if M <= 4 else np.unique(np.r_[0, 31, 32, 64, 100, M - 1])
    a_dev, sfa_dev = linear_rows(orc, host_u8(a1), host_u8(sfa1), rows, H, 0, orc.TILED)
    g1d = orc.gemm_gelu_fp4(a_dev, W["b1"], sfa_dev, W["sfb1"], len(rows), N1, H, 0, 0, 1, alpha1,
                            synth.bits(W["bias1"]), 1.0, orc.LINEAR, diag=True)
    gp, gsf = linear_rows(orc, host_u8(p1), host_u8(s1), rows, N1, 0, orc.TILED)
    ce, se = checkers.fp4_out_windows(g1d, 1.0, len(rows), N1)
    rep = checkers.compare_quantized(
        orc, 0, 1.0, gp, gsf, g1d["packed"], g1d["sf"], g1d["y"], g1d["v"], g1d["spre"], len(rows), N1,
        orc.LINEAR, code_extra=ce, scale_extra=se)
    banner(f"  split-K chain gemm1 {dict(rep)}")
    assert rep.ok(), rep
    ref2, l12 = orc.gemm(gp, W["b2"], gsf, W["sfb2"], len(rows), H, N1, 0, 0, 1, alpha=alpha2)
    ok, worst = checkers.gemm_within_tolerance(host_f64(out)[rows], ref2, l12)
    banner(f"  split-K chain gemm2 worst {worst:.3g}")
    assert ok.all()


def test_decode_chain_graph_replays(orc, weights):
    """The decode chain at M = 128 (producer, GEMM1 -> FP4, split-K GEMM2)
    captured in a HIP graph and replayed three times, with eager work and
    synchronisations between the replays: every replay matches the eager
    result bit for bit (the library allocates nothing and never
    synchronizes, so its calls capture as they are)."""
    W = weights
    M, H, N1 = 128, W["H"], W["N1"]
    x, r, w = synth.producer_inputs(M, H, 4242, outliers=True)
    xd, wd, r0 = dev_bf16(x), dev_bf16(w), dev_bf16(r)
    a1 = torch.empty((M, H // 2), dtype=torch.uint8, device="cuda")
    s1 = torch.empty(lb.lowbit_sf_bytes(M, H, 0, 1), dtype=torch.uint8, device="cuda")
    a2 = torch.empty((M, N1 // 2), dtype=torch.uint8, device="cuda")
    s2 = torch.empty(lb.lowbit_sf_bytes(M, N1, 0, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(lb.lowbit_gemm_workspace_bytes(M, H, N1, 0, -1), dtype=torch.uint8, device="cuda")
    assert ws.numel() > 0
    rd = r0.clone()
    gs = dev_f32(2.0)

    def step():
        lb.lowbit_add_rmsnorm_quant(xd, rd, wd, EPS, lb.NVFP4, lb.TILED, global_scale=gs, out_packed=a1,
                                    out_sf=s1)
        lb.lowbit_gemm_bias_gelu_fp4(a1, W["d_b1"], s1, W["d_sfb1"], W["d_bias1"], fmt=0, sfa_layout=1,
                                     sfb_layout=1, alpha=1e-3, out_packed=a2, out_sf=s2, out_layout=1)
        lb.lowbit_gemm_bf16(a2, W["d_b2"], s2, W["d_sfb2"], fmt=0, sfa_layout=1, sfb_layout=1, alpha=0.01,
                            out=out, workspace=ws)

    step()
    torch.cuda.synchronize()
    want = (rd.clone(), a1.clone(), s1.clone(), a2.clone(), s2.clone(), out.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for k in range(3):
        # eager work between the replays: the residual back to its input
        # value (the producer updates it in place) and the outputs cleared
        rd.copy_(r0)
        for t in (a1, s1, a2, s2, out, ws):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (rd, a1, s1, a2, s2, out)
        banner(f"  graph replay {k}")
        assert all(torch.equal(a, b) for a, b in zip(got, want)), f"replay {k} differs from the eager run"
