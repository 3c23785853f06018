"""CPU oracle for paged KV-cache attention.

TEST INFRASTRUCTURE ONLY.  Only tests, the smoke check and the benchmark's
CPU-baseline leg may import anything under this package.  The library's
product path never calls it, and this package imports nothing from the
library: the two share no code.

Contents
  paged   append, gather and attention in float64 with NumPy, following the
          pages' statement of the problem (see each function's docstring).
  pool    a Python model of the block pool: a last-in-first-out free list
          with per-block reference counts.
  brute   pure-Python attention over contiguous key/value lists, for tiny
          inputs only.
  blocks  whole-block copies: copy-on-write inside the pool, swap out to and
          in from a host image.
  fp8     the 8-bit cache: E4M3 codes with a scale per (token, head), append
          and attention over the dequantized values.

Pins (what holds this oracle to something other than itself) live in
tests/test_oracle_*.py: the pages' printed block arithmetic, closed forms,
invariants and the brute force.  No function here is "parity unpinned".
"""
from . import blocks, brute, fp8, paged, pool  # noqa: F401
