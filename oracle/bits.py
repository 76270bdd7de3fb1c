"""Bits-per-weight ledger and packed buffer sizes.

mhpq.cn/news/1159370 §1.1 puts the ternary code at log2(3) ~ 1.585 bits and
§1.3 adds 16/128 = 0.125 bits for one fp16 scale per 128 weights, giving ~1.71;
§3.1 stores 2 bits per weight instead (0.415 bits wasted, for aligned decode).
"""

import math

import numpy as np


def information_bound_bits():
    """log2(3) + 16/128: the ternary code at its entropy bound plus the scale."""
    return math.log2(3.0) + 16.0 / 128.0


def dense_storage_bits():
    """2-bit codes plus one fp16 scale per 128 weights."""
    return 2.0 + 16.0 / 128.0


def storage24_bits():
    """2:4: a 4-bit index nibble and 2 sign bits per quad of 4, plus the scale."""
    return (4.0 + 2.0) / 4.0 + 16.0 / 128.0


def packed_bytes(fmt, n, k):
    """(code_bytes, meta_bytes, scale_bytes) of the packed planes of an [n, k] matrix.

    dense: codes n*k/4 bytes, no meta; "24": signs n*k/16 bytes, meta n*k/8 bytes.
    Scales are n*(k/128) fp16 values in both formats."""
    if n <= 0 or k <= 0 or n % 128 or k % 128:
        raise ValueError("n and k must be positive multiples of 128")
    scales = n * (k // 128) * 2
    if fmt == "dense":
        return n * k // 4, 0, scales
    if fmt == "24":
        return n * k // 16, n * k // 8, scales
    raise ValueError(f"unknown format {fmt!r}")


def entropy_bits(t):
    """Empirical entropy of the ternary symbols in t (bits per symbol)."""
    t = np.asarray(t).reshape(-1)
    h = 0.0
    for v in (-1, 0, 1):
        p = np.count_nonzero(t == v) / t.size
        if p > 0:
            h -= p * math.log2(p)
    return h
