"""Small helpers shared by the GPU parity tests (host <-> device moves)."""

import sys

import numpy as np
import torch

DEV = "cuda"


def dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device=DEV, dtype=dtype)


def dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def host(t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def announce(*what):
    """Name the case before a GPU step, flushed, so a fault is attributable."""
    print("[gpu case]", *what, flush=True)
    sys.stdout.flush()
