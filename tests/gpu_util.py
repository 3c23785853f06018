"""Helpers for GPU tests: device transfer and running the library on a Batch."""
import numpy as np
import pytest


def torch_cuda():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def dev(a, torch):
    """NumPy -> device tensor; uint16 (FP16 bits) becomes int16, int32 stays int32."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def host_bits(t):
    return t.cpu().numpy().view(np.uint16)


def host_f64(t):
    return t.cpu().view(__import__("torch").float16).numpy().astype(np.float64)


def say(msg):
    print(msg, flush=True)
