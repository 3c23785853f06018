"""Attention tolerance for "max-abs 2e-3 and max-rel 1e-2".

Both bounds hold wherever they can:
  * the absolute bound 2e-3 on every element with |ref| < 4.  FP16's half-ulp
    is at most 9.8e-4 there, so the output's own rounding leaves room for the
    arithmetic.  From |ref| = 4 on, the half-ulp reaches 1.95e-3 and an
    absolute bound of 2e-3 would leave the arithmetic no room at all;
  * the relative bound 1e-2 on every element with |ref| >= 0.2.  Below 0.2 it
    is tighter than the absolute bound, and it cannot hold at all near 0.
An element passes when both bounds that apply to it hold: |err| <= 2e-3 for
|ref| < 4, and |err| <= 1e-2 * |ref| for |ref| >= 4.  max_abs is reported over
|ref| < 4, and max_rel over |ref| >= 0.2.
"""
import numpy as np

ABS_TOL = 2e-3
REL_TOL = 1e-2
ABS_RANGE = 4.0   # |ref| below this: the absolute bound applies
REL_FLOOR = 0.2   # |ref| from this on: the relative bound applies


def bound(ref):
    a = np.abs(np.asarray(ref, dtype=np.float64))
    return np.where(a < ABS_RANGE, ABS_TOL, REL_TOL * a)


def compare(gpu, ref):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    err = np.abs(gpu - ref)
    bad = ~(err <= bound(ref))  # NaN counts as bad
    a = np.abs(ref)
    small, big = a < ABS_RANGE, a >= REL_FLOOR
    max_rel = float(np.max(err[big] / a[big])) if np.any(big) else 0.0
    max_abs = float(np.nanmax(err[small])) if np.any(small) else 0.0
    return {"max_abs": max_abs, "max_rel": max_rel, "max_err": float(np.nanmax(err)) if err.size else 0.0,
            "bad": int(bad.sum()), "nan": int(np.isnan(gpu).sum()), "n": int(err.size)}


def assert_close(gpu, ref, what=""):
    s = compare(gpu, ref)
    assert s["bad"] == 0 and s["nan"] == 0, f"{what}: {s}"
    assert s["max_abs"] <= ABS_TOL and s["max_rel"] <= REL_TOL, f"{what}: {s}"
    return s
