"""Shared helpers of the GPU parity tests."""

import numpy as np


def rel_fro(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / d) if d > 0 else float(np.linalg.norm(x))


def device():
    import torch
    return torch.device("cuda:0")


def to_dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(device())


def bf16_tensor(bits):
    """uint16 bfloat16 bit patterns -> device bfloat16 tensor (same bits)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device())


def log(msg):
    print(msg, flush=True)
