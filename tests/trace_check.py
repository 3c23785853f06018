"""Oracle check of the continuous-batching trace's decode outputs.

TEST INFRASTRUCTURE: used by the trace tests and by bench.py's oracle leg.

A trace row's context is rebuilt without reading anything a kernel wrote:
  * its shared prefix from the prefix blocks' contents, read back before the
    first kernel ran;
  * its private prompt tokens from the request's seeded draw;
  * each generated token from the seeded draw of the step that appended it.
The fp64 oracle then attends the step's query over that context.
"""
from __future__ import annotations

import numpy as np

import oracle.paged as opaged
from tests.tolerance import compare


def host_bits(torch, t):
    return t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


class TraceChecker:
    def __init__(self, tr):
        """Call before the trace's first step: reads the prefix blocks back."""
        torch = tr.torch
        self.tr = tr
        self.prefix = tr.prefix_ids.copy()
        ids = torch.from_numpy(self.prefix.astype(np.int64)).to(tr.dev)
        slab = host_bits(torch, tr.pool_d[ids, 0])  # [P, 2, H, 16, 128]
        # prefix tokens in logical order, [P * 16, H, 128] for keys and for values
        self.pre_k = slab[:, 0].transpose(0, 2, 1, 3).reshape(-1, tr.H, 128)
        self.pre_v = slab[:, 1].transpose(0, 2, 1, 3).reshape(-1, tr.H, 128)
        self.origin = {}   # (req, position) -> (step, index in that step)
        self.joins = {}    # req -> (prompt, shared)
        self._draws = {}   # step -> (k, v) host bits [n, H, 128]
        self.samples = []  # (step, reqs, lens, q bits, out bits)

    def record(self, snap):
        """Call after every step with its snapshot."""
        st = self.tr.log["steps"][-1]
        for j, (req, pos) in enumerate(zip(st["reqs"], st["new_pos"])):
            self.origin[(req, int(pos))] = (st["step"], j)
        for req, prompt, _, shared, _ in self.tr.log["joins"][len(self.joins):]:
            self.joins[req] = (prompt, shared)

    def keep(self, snap):
        """Keep a step's outputs (and its queries) for a later check."""
        torch = self.tr.torch
        _, _, q = self.tr.step_draws(snap["step"], len(snap["reqs"]))
        self.samples.append((snap["step"], list(snap["reqs"]), snap["lens"].copy(), host_bits(torch, q),
                             host_bits(torch, snap["out"])))

    def _step_kv(self, step):
        if step not in self._draws:
            torch = self.tr.torch
            n = len(self.tr.log["steps"][step]["reqs"])
            k, v, _ = self.tr.step_draws(step, n)
            self._draws[step] = (host_bits(torch, k), host_bits(torch, v))
        return self._draws[step]

    def context(self, req, L):
        """Keys and values of positions 0..L-1 of request req, float64 [H, L, 128]."""
        torch = self.tr.torch
        prompt, shared = self.joins[req]
        K = np.empty((L, self.tr.H, 128), dtype=np.uint16)
        V = np.empty_like(K)
        if shared:
            K[:shared], V[:shared] = self.pre_k[:shared], self.pre_v[:shared]
        if prompt > shared:
            k, v = self.tr.prompt_kv(req, shared, prompt)
            K[shared:prompt], V[shared:prompt] = host_bits(torch, k), host_bits(torch, v)
        for pos in range(prompt, L):
            step, j = self.origin[(req, pos)]
            k, v = self._step_kv(step)
            K[pos], V[pos] = k[j], v[j]
        f = lambda a: a.view(np.float16).transpose(1, 0, 2).astype(np.float64)
        return f(K), f(V)

    def check(self, rows=None, log=None):
        """Compare the kept samples' outputs (every row, or `rows` of each)
        with the oracle.  Returns totals over all compared elements."""
        tot = {"steps": 0, "rows": 0, "max_abs": 0.0, "max_rel": 0.0, "bad": 0, "nan": 0}
        for step, reqs, lens, q, out in self.samples:
            pick = range(len(reqs)) if rows is None else [j for j in rows if j < len(reqs)]
            for j in pick:
                L = int(lens[j])
                K, V = self.context(reqs[j], L)
                ref = opaged.attention(q[j:j + 1], K, V, [L - 1], self.tr.scale)[0]
                got = out[j].view(np.float16).astype(np.float64)
                s = compare(got, ref)
                tot["rows"] += 1
                tot["max_abs"] = max(tot["max_abs"], s["max_abs"])
                tot["max_rel"] = max(tot["max_rel"], s["max_rel"])
                tot["bad"] += s["bad"]
                tot["nan"] += s["nan"]
            tot["steps"] += 1
            if log:
                log(f"trace step {step}: {tot}")
        return tot
