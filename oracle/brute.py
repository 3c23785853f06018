"""Pure-Python brute-force attention for tiny inputs.  TEST INFRASTRUCTURE ONLY.

Works on contiguous Python lists that never pass through a block table, so a
gather or indexing mistake in `oracle.paged` cannot hide behind it.
"""
from __future__ import annotations

import math


def attend_one(q, keys, values, scale):
    """softmax over j of (sum_d q[d] * keys[j][d]) * scale, applied to values.

    q: list of D floats; keys, values: lists of L lists of D floats.
    """
    scores = []
    for k in keys:
        acc = 0.0
        for d in range(len(q)):
            acc += q[d] * k[d]
        scores.append(acc * scale)
    top = max(scores)
    weights = [math.exp(s - top) for s in scores]
    total = math.fsum(weights)
    out = []
    for d in range(len(values[0])):
        out.append(math.fsum(weights[j] * values[j][d] for j in range(len(values))) / total)
    return out
