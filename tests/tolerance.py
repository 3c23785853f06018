"""Attention tolerance: an element passes when |gpu - ref| <= max(2e-3, 1e-2 * |ref|).

Reading of "max-abs 2e-3 and max-rel 1e-2": a pure relative bound cannot hold
near zero and a pure absolute bound is below FP16's half-ulp once |o| >= 8,
so an element must meet one of the two.  max-rel is reported over elements
with |ref| >= 0.2, where the two bounds cross.
"""
import numpy as np

ABS_TOL = 2e-3
REL_TOL = 1e-2


def compare(gpu, ref):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    err = np.abs(gpu - ref)
    bound = np.maximum(ABS_TOL, REL_TOL * np.abs(ref))
    bad = ~(err <= bound)  # NaN counts as bad
    big = np.abs(ref) >= 0.2
    max_rel = float(np.max(err[big] / np.abs(ref[big]))) if np.any(big) else 0.0
    return {"max_abs": float(np.nanmax(err)) if err.size else 0.0, "max_rel": max_rel,
            "bad": int(bad.sum()), "nan": int(np.isnan(gpu).sum()), "n": int(err.size)}


def assert_close(gpu, ref, what=""):
    s = compare(gpu, ref)
    assert s["bad"] == 0 and s["nan"] == 0, f"{what}: {s}"
    return s
