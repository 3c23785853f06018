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


def ramp_keys(b, top=8.0):
    """Scale each row's key at position p by 1 + (top - 1) * p / L, in the pool
    and in the step's new tokens alike, so that scores keep growing along the
    context and a running softmax maximum moves again and again.  Rows must
    not share blocks."""
    pool = b.pool.view(np.float16).copy()
    k_new = b.k_new.view(np.float16).copy()
    for r in range(b.rows):
        L, n = int(b.context_lens[r]), int(b.q_counts[r])
        first_new = L - n
        for p in range(first_new):
            pool[b.block_tables[r, p // 16], :, 0, :, p % 16, :] *= np.float16(1 + (top - 1) * p / L)
        for i in range(n):
            k_new[:, b.query_start[r] + i] *= np.float16(1 + (top - 1) * (first_new + i) / L)
    b.pool = pool.view(np.uint16)
    b.k_new = k_new.view(np.uint16)
    return b
