"""Helpers for the GPU parity tests (device placement, canaries)."""
import numpy as np
import torch

DEV = "cuda:0"
CANARY = 64  # extra output elements that must stay untouched


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def out_with_canary(n, rows=None):
    """fp32 output buffer of n (or rows x n) elements plus a NaN canary tail;
    returns (full buffer, contiguous view of the output part)."""
    total = n if rows is None else rows * n
    buf = torch.full((total + CANARY,), float("nan"), dtype=torch.float32, device=DEV)
    view = buf[:total] if rows is None else buf[:total].view(rows, n)
    return buf, view


def canary_intact(buf, n_out):
    tail = buf[n_out:].cpu().numpy()
    return bool(np.all(np.isnan(tail)))


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()
