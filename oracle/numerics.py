"""fp16 and bf16 conversions written out with integer bit operations.

The pages fix the storage types (one fp16 scale per 128-group,
mhpq.cn/news/1159370 §1.3; bf16 activations) but not the rounding mode; the
plain reading is IEEE round-to-nearest-even, which is what this module does.
Encoding rounds the exact float64 value once (no double rounding through
float32).  Decoding is exact.

Pinned by tests/test_oracle_numerics.py: exhaustive 2^16 round trip, agreement
with numpy.float16 casts, and hand-worked tie cases.
"""

import numpy as np

# (exponent bits, stored mantissa bits)
_FMT = {"f16": (5, 10), "bf16": (8, 7)}


def _encode(x, fmt):
    """Round float64 array ``x`` to the 16-bit format ``fmt``; return uint16 bits."""
    ebits, mbits = _FMT[fmt]
    bias = (1 << (ebits - 1)) - 1
    emax_field = (1 << ebits) - 1

    x = np.ascontiguousarray(x, dtype=np.float64)
    bu = x.reshape(-1).view(np.uint64)
    sign = (bu >> np.uint64(63)).astype(np.int64)
    e64 = ((bu >> np.uint64(52)) & np.uint64(0x7FF)).astype(np.int64)
    m64 = (bu & np.uint64((1 << 52) - 1)).astype(np.int64)

    is_special = e64 == 0x7FF
    is_nan = is_special & (m64 != 0)

    # full significand and unbiased exponent of the float64 value: value = sig * 2^(e - 52)
    sig = np.where(e64 > 0, m64 | (1 << 52), m64)
    e = np.where(e64 > 0, e64 - 1023, -1022)

    te = e + bias  # target biased exponent if normal
    normal = te >= 1
    # number of low significand bits to drop
    shift = np.where(normal, 52 - mbits, 52 - mbits + (1 - te))
    shift = np.clip(shift, 0, 60)
    q = sig >> shift
    rem = sig - (q << shift)
    half = np.where(shift > 0, np.left_shift(np.int64(1), np.maximum(shift - 1, 0)), 0)
    round_up = (shift > 0) & ((rem > half) | ((rem == half) & ((q & 1) == 1)))
    q = q + round_up.astype(np.int64)
    # normal: field = (te - 1) << mbits + q  (q carries the hidden bit, so a carry out
    # of the mantissa bumps the exponent); subnormal: field = q
    field = np.where(normal, ((te - 1) << mbits) + q, q)
    overflow = field >= (emax_field << mbits)
    field = np.where(overflow, emax_field << mbits, field)
    field = np.where(sig == 0, 0, field)
    field = np.where(is_special & ~is_nan, emax_field << mbits, field)
    field = np.where(is_nan, (emax_field << mbits) | (1 << (mbits - 1)), field)
    out = (sign << (ebits + mbits)) | field
    return out.astype(np.uint16).reshape(x.shape)


def _decode(bits, fmt):
    """Exact float64 value of 16-bit patterns ``bits`` in format ``fmt``."""
    ebits, mbits = _FMT[fmt]
    bias = (1 << (ebits - 1)) - 1
    emax_field = (1 << ebits) - 1
    b = np.asarray(bits).astype(np.int64)
    sign = np.where((b >> (ebits + mbits)) & 1 == 1, -1.0, 1.0)
    ef = (b >> mbits) & emax_field
    mf = b & ((1 << mbits) - 1)
    with np.errstate(over="ignore"):
        normal = sign * np.ldexp(1.0 + mf / float(1 << mbits), ef - bias)
        sub = sign * np.ldexp(mf.astype(np.float64), 1 - bias - mbits)
    val = np.where(ef == 0, sub, normal)
    val = np.where((ef == emax_field) & (mf == 0), sign * np.inf, val)
    val = np.where((ef == emax_field) & (mf != 0), np.nan, val)
    return val


def f64_to_f16_bits(x):
    return _encode(x, "f16")


def f16_bits_to_f64(bits):
    return _decode(bits, "f16")


def f64_to_bf16_bits(x):
    return _encode(x, "bf16")


def bf16_bits_to_f64(bits):
    return _decode(bits, "bf16")
