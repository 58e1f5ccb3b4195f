"""Helpers for the GPU parity tests (device placement, canaries)."""
import numpy as np
import torch

DEV = "cuda:0"
CANARY = 64  # extra output elements that must stay untouched

# Every launch shape (rows per lane, k-waves, workgroup waves) the vector-form
# GEMVs accept; 8 waves with 8 rows per lane is rejected (test_abi_cpu).
VECTOR_SHAPES = [(rpl, kw, wg) for rpl in (1, 2, 4, 8)
                 for kw, wg in ((1, 1), (1, 2), (2, 2), (1, 4), (2, 4), (4, 4), (1, 8), (2, 8))
                 if not (wg == 8 and rpl == 8)]


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
