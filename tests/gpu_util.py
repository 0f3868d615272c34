"""Helpers shared by the GPU parity tests (test code only)."""
import sys

import numpy as np

DEV = "cuda:0"


def say(*a):
    """Name the case before a GPU step, flushed, so a fault can be traced."""
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def x_dev(xvals, dtype):
    """x values (float32, already rounded to dtype) -> device tensor of that dtype."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(xvals, np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    elif dtype == "f16":
        t = t.to(torch.float16)
    return t.to(DEV)


def u32(t):
    """Device int32 tensor -> numpy uint32 (bit-identical)."""
    return t.cpu().numpy().view(np.uint32)


def u16(t):
    return t.cpu().numpy().view(np.uint16)


def f16_dev(bits_u16):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits_u16).view(np.int16)).to(DEV)


def check_close(y, ref, tol, what):
    y = np.asarray(y, np.float64)
    err = np.abs(y - ref)
    bad = err > tol
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError("%s: %d of %d outputs outside tolerance; first at %s: y=%r ref=%r tol=%r"
                             % (what, int(bad.sum()), bad.size, tuple(i), y[tuple(i)], ref[tuple(i)], tol[tuple(i)]))
    return float(err.max()), float((err / np.maximum(tol, 1e-300)).max())
