"""Seeded synthetic inputs for the low-bit linear hot path.

This module only draws numbers: it holds none of the method's arithmetic
(no normalisation, no quantisation, no matmul).  Both the HIP path and the
CPU oracle are fed from the same host tensors made here.

Recipe (the same for every workload):
  * values are drawn with ``torch.randn`` on the CPU from a
    ``torch.Generator`` seeded with ``seed * 1000 + tensor_index``, in fp32,
    scaled/shifted, then rounded to bf16 by ``Tensor.to(torch.bfloat16)``;
  * "outlier channels": ``round(0.01 * ncols)`` columns chosen by a seeded
    permutation are multiplied by 20 in fp32 before the bf16 rounding;
  * RMSNorm weights are ``1 + 0.1 * randn``; weights of the GEMMs are
    ``0.02 * randn``; biases ``0.1 * randn``; residuals ``randn``.
"""
import torch

# Workloads, named by what they are.  Sizes follow the decode / prefill rows of
# the pages (FlashRT README release-gate shapes; FlashInfer decode widths).
TINY_MXFP4 = dict(name="tiny_mxfp4_m8_h256_n128", M=8, H=256, N=128, seed=1001)
NVFP4_PRODUCER = dict(name="nvfp4_add_rmsnorm_quant_m4096_h4096", M=4096, H=4096, seed=1002)
MXFP4_DECODE = dict(name="mxfp4_decode_gemm",
                    shapes=[(41, 4608, 1536), (41, 6144, 1536), (41, 1536, 6144), (1, 17408, 5120)],
                    seed=1003)
MXFP4_PREFILL = dict(name="mxfp4_prefill_gemm_bias_residual",
                     shapes=[(8192, 14336, 4096), (8192, 4096, 14336)], seed=1004)
NVFP4_CHAIN = dict(name="nvfp4_chain_h5120_n17408", H=5120, N1=17408, Ms=[1, 128, 2048], seed=1005)


def _gen(seed: int, index: int) -> torch.Generator:
    return torch.Generator().manual_seed(seed * 1000 + index)


def outlier_columns(ncols: int, seed: int, index: int = 99) -> torch.Tensor:
    """Indices of round(0.01 * ncols) columns, from a seeded permutation."""
    k = int(round(0.01 * ncols))
    perm = torch.randperm(ncols, generator=_gen(seed, index))
    return torch.sort(perm[:k]).values


def normal_bf16(shape, seed: int, index: int, std: float = 1.0, mean: float = 0.0,
                outliers: bool = False, outlier_scale: float = 20.0,
                dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """bf16 (or `dtype`) CPU tensor of mean + std * N(0, 1), optional outlier columns."""
    t = torch.randn(*shape, generator=_gen(seed, index), dtype=torch.float32) * std + mean
    if outliers:
        cols = outlier_columns(shape[-1], seed, 100 + index)
        t[..., cols] *= outlier_scale
    return t.to(dtype)


def producer_inputs(M: int, H: int, seed: int, outliers: bool = False, dtype: torch.dtype = torch.bfloat16):
    """(input, residual, rmsnorm weight) as bf16 (or fp16) CPU tensors: the same
    fp32 draws either way, rounded to the requested 16-bit format."""
    x = normal_bf16((M, H), seed, 0, outliers=outliers, dtype=dtype)
    r = normal_bf16((M, H), seed, 1, dtype=dtype)
    w = normal_bf16((H,), seed, 2, std=0.1, mean=1.0, dtype=dtype)
    return x, r, w


def activation(M: int, K: int, seed: int, index: int = 3, outliers: bool = False,
               dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    return normal_bf16((M, K), seed, index, outliers=outliers, dtype=dtype)


def weight(N: int, K: int, seed: int, index: int = 4) -> torch.Tensor:
    return normal_bf16((N, K), seed, index, std=0.02)


def bias(N: int, seed: int, index: int = 5) -> torch.Tensor:
    return normal_bf16((N,), seed, index, std=0.1)


def residual(M: int, N: int, seed: int, index: int = 6) -> torch.Tensor:
    return normal_bf16((M, N), seed, index)


def bits(t: torch.Tensor):
    """uint16 numpy view of a bf16 (or fp16) tensor's bit patterns (host)."""
    return t.contiguous().view(torch.int16).numpy().view("uint16")


def from_bits(a) -> torch.Tensor:
    """bf16 CPU tensor from a uint16 numpy array of bit patterns."""
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
