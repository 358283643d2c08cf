"""Helpers for the GPU parity tests: device tensors from host arrays, poisoned outputs, logging."""
import sys

import numpy as np
import torch

DEV = "cuda:0"


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def up(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(DEV)


def down(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def poisoned(shape, dtype):
    """Output buffer holding a value no kernel writes, so unwritten elements show up: all-ones bytes
    for floats and bf16 bits (NaN) and for bytes, 0x5A5A5A5A for int32 (not -1, the top-k pad, and
    larger than any entry index here)."""
    t = torch.empty(shape, dtype=dtype, device=DEV)
    if dtype == torch.int32:
        t.fill_(0x5A5A5A5A)
    else:
        t.view(torch.uint8).fill_(0xFF)
    return t
