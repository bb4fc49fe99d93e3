"""Host <-> device plumbing for the GPU parity tests (no arithmetic)."""
import numpy as np
import torch

from block_scaled_fp4_add_amd import synth

DEV = "cuda:0"


def dev_bf16(t_cpu_bf16):
    return t_cpu_bf16.contiguous().to(DEV)


def dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def dev_f32(x):
    return torch.tensor([x], dtype=torch.float32, device=DEV)


def host_u8(t):
    return t.cpu().numpy()


def host_bits(t):
    """uint16 bit patterns of a device bf16 tensor."""
    return synth.bits(t.cpu())


def host_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def banner(msg):
    print(f"[gpu-test] {msg}", flush=True)
