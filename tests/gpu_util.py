"""Helpers shared by the GPU parity tests (imported only from GPU tests)."""
from __future__ import annotations

import sys

import numpy as np


def say(*a):
    """Name the case before a GPU step, so a crash still tells which one it was."""
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def lib():
    import coo_spmm_amd
    return coo_spmm_amd


def dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def assert_close(name, got, ref, abs_sum, rel=1e-5, atol=1e-6):
    """Per element |got - ref| <= rel * sum|terms| + atol (the layer's stated tolerance)."""
    got = np.asarray(got, np.float64)
    bad = np.abs(got - ref) > rel * abs_sum + atol
    if bad.any():
        idx = np.argwhere(bad)[:5]
        det = [(tuple(i), float(got[tuple(i)]), float(ref[tuple(i)]), float(abs_sum[tuple(i)])) for i in idx]
        raise AssertionError(f"{name}: {int(bad.sum())} of {bad.size} elements outside tolerance, e.g. {det}")
