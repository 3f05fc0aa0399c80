"""Relative-distance bucket rule for the learned relative attention bias.

The pages say only that HSTU adds a relative attention bias (aitrends.kr
article 100093, "HSTU sequential modelling"; news.bpdata.com article, "HSTU"),
and the workloads state "learned buckets of |i - j| (log-bucketed)".  Reading
taken: an integer log-linear rule with m mantissa bits (s = 2^m):

    b(delta) = delta                                   if delta < s
    b(delta) = s*(e - m + 1) + (delta >> (e - m)) - s  otherwise, e = floor(log2 delta)
    b       <- min(b, nb - 1);  delta < 0 -> 0

Distances below s get their own bucket; every octave [2^e, 2^(e+1)) above is
split into s equal-width buckets.  The rule is integer-only.

parity pins: hand values, continuity at octave edges, monotonicity and
agreement with an independent octave-table construction (tests/test_buckets.py).
"""
from __future__ import annotations

import numpy as np


def bucket(delta: int, mbits: int, nb: int) -> int:
    """Scalar bucket of one distance (pure Python integers)."""
    if delta < 0:
        delta = 0
    s = 1 << mbits
    if delta < s:
        b = delta
    else:
        e = delta.bit_length() - 1
        b = s * (e - mbits + 1) + (delta >> (e - mbits)) - s
    return min(b, nb - 1)


def bucket_np(delta: np.ndarray, mbits: int, nb: int) -> np.ndarray:
    """Vectorised bucket of an integer array of distances (int64 math)."""
    d = np.maximum(np.asarray(delta, dtype=np.int64), 0)
    s = np.int64(1 << mbits)
    # floor(log2 d) for d >= 1, computed exactly with integer comparisons.
    e = np.zeros_like(d)
    dd = d.copy()
    for sh in (32, 16, 8, 4, 2, 1):
        big = dd >= (np.int64(1) << sh)
        e = np.where(big, e + sh, e)
        dd = np.where(big, dd >> sh, dd)
    shift = np.maximum(e - mbits, 0)
    b_log = s * (e - mbits + 1) + (d >> shift) - s
    b = np.where(d < s, d, b_log)
    return np.minimum(b, nb - 1)
