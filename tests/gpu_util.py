"""Helpers for the GPU tests: host arrays to device tensors, and announcing
each GPU step before it runs."""
from __future__ import annotations

import sys

import numpy as np


def say(*a):
    print("[gpu-step]", *a, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:        # bf16 bit patterns
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def host(t) -> np.ndarray:
    import torch
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def empty(shape, dtype: str):
    import torch
    dt = {"f32": torch.float32, "i32": torch.int32, "u8": torch.uint8}[dtype]
    return torch.empty(shape, dtype=dt, device="cuda")
