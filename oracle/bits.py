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

    dense: codes n*k/4 bytes, no meta, n*(k/128) fp16 scales.  "24": signs
    n*k'/16 bytes, meta n*k'/8 bytes and n*(k'/128) fp16 scales for k' = k
    rounded up to a multiple of 512 (the stored format keeps four 128-groups
    per block and pads the last block with zero groups)."""
    if n <= 0 or k <= 0 or n % 128 or k % 128:
        raise ValueError("n and k must be positive multiples of 128")
    if fmt == "dense":
        return n * k // 4, 0, n * (k // 128) * 2
    if fmt == "24":
        kp = -(-k // 512) * 512
        return n * kp // 16, n * kp // 8, n * (kp // 128) * 2
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
