"""Helpers for the GPU tests: move host inputs (numpy; bf16 as uint16 bits)
onto the device byte for byte, and bring results back."""

import numpy as np
import torch

DEV = torch.device("cuda:0")


def bf(a):
    """uint16 bf16 bits -> device bfloat16 tensor (same bytes)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16)).view(torch.bfloat16).to(DEV)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def as_dtype(a, dtype):
    return bf(a) if dtype == "bf16" else dev(np.asarray(a, dtype=np.float32))


def host_bits(t):
    """device bfloat16 tensor -> uint16 bits on the host."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_f32(t):
    return t.float().cpu().numpy()
