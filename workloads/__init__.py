"""Seeded synthetic inputs for the paged KV-cache attention path.

This package draws lengths, block-id permutations and N(0,1) FP16 values, and
nothing else: it performs none of the append, gather, softmax or pooling
arithmetic that the library and its oracle each compute on their own.
"""
from .gen import *  # noqa: F401,F403
