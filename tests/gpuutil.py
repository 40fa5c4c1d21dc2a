"""Shared helpers for the GPU parity tests (device buffers via torch)."""
import sys

import numpy as np


def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from sparse_sketching_amd import binding
    binding.load()                         # fails loudly without the library
    return torch.device("cuda", 0)


def to_dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev())


def sync():
    import torch
    torch.cuda.synchronize()


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()
