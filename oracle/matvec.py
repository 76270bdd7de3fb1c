"""Ternary GEMV / GEMM / 2:4 GEMV definitions in float64.

What the decode and prefill paths compute (mhpq.cn/news/1159370 §4.2: read
the weight bits, expand the signs, multiply by the scale, then the matrix
product; the activations are already rotated, zwxr.cn/news/303439 §3.4):

    y'[m, n] = sum_g f16(scale[n, g]) * sum_{k in g} t[n, k] * x'[m, k]

with x' the exact bf16 values handed to the kernel and t in {-1, 0, +1}.
The vectorised forms dequantise and call numpy.matmul in float64; the
brute-force forms are explicit Python loops for tiny shapes.
"""

import numpy as np

from .numerics import bf16_bits_to_f64, f16_bits_to_f64
from .quant import GROUP, dense_from_24, load_24, split_planes, unpack_24, unpack_dense, untile_scales


def _x(x_bf16_bits):
    x = bf16_bits_to_f64(np.asarray(x_bf16_bits, dtype=np.uint16))
    return x.reshape(1, -1) if x.ndim == 1 else x


def dequant_dense(codes, scales, k):
    """W~[n, k] = f16(scale[n, k // 128]) * t[n, k], scales in the dense storage
    order [N/16, K/128, 16]."""
    t = unpack_dense(codes, k).astype(np.float64)
    s = f16_bits_to_f64(untile_scales(np.asarray(scales, dtype=np.uint16)))
    return t * np.repeat(s, GROUP, axis=1)


def gemv(x_bf16_bits, codes, scales, k):
    """y'[m, n] for activations x'[m, k] (bf16 bits) against dense codes."""
    return np.matmul(_x(x_bf16_bits), dequant_dense(codes, scales, k).T)


# the prefill GEMM is the same contraction for M rows of activations
gemm = gemv


def dequant_residual(codes, scales, k):
    """W~[n, k] = f16(s1[n, g]) t1[n, k] + f16(s2[n, g]) t2[n, k] for the
    two-plane format (groups of the planes interleaved, quant.interleave_planes)."""
    c1, c2 = split_planes(codes)
    s1, s2 = split_planes(scales)
    return dequant_dense(c1, s1, k) + dequant_dense(c2, s2, k)


def gemv_residual(x_bf16_bits, codes, scales, k):
    """y'[m, n] = sum_g sum_p f16(s_p[n, g]) sum_{k in g} t_p[n, k] x'[m, k] over
    both planes p of the two-plane format."""
    return np.matmul(_x(x_bf16_bits), dequant_residual(codes, scales, k).T)


def dequant_24(meta, signs, scales, k):
    """The stored 2:4 planes (lane-major) as a dense float64 matrix [N, K]."""
    meta_r, signs_r, scales_r = load_24(meta, signs, scales, k)
    idx0, idx1, neg0, neg1 = unpack_24(meta_r, signs_r, k)
    t = dense_from_24(idx0, idx1, neg0, neg1).astype(np.float64)
    s = f16_bits_to_f64(np.asarray(scales_r, dtype=np.uint16))
    return t * np.repeat(s, GROUP, axis=1)


def gemv24(x_bf16_bits, meta, signs, scales, k):
    """y'[m, n] = sum_g s[n, g] * sum_quads (+-x'[4q + idx0] +- x'[4q + idx1])."""
    return np.matmul(_x(x_bf16_bits), dequant_24(meta, signs, scales, k).T)


def gemv_bruteforce(x_bf16_bits, codes, scales, k):
    """Loop form of gemv: decode each 2-bit field by hand and accumulate."""
    x = _x(x_bf16_bits)
    codes = np.asarray(codes, dtype=np.uint32)
    st = np.asarray(scales, dtype=np.uint16)  # [N/16, G, 16]
    m_rows, n_rows = x.shape[0], codes.shape[0] * 16
    y = np.zeros((m_rows, n_rows))
    for m in range(m_rows):
        for n in range(n_rows):
            total = 0.0
            for g in range(k // GROUP):
                part = 0.0
                for kk in range(g * GROUP, (g + 1) * GROUP):
                    c = kk % GROUP
                    lane = 16 * (c // 32) + n % 16
                    word = int(codes[n // 16, g, 2 * lane + (c % 32) // 16])
                    r = c % 16
                    field = (word >> (4 * (r % 8) + (2 if r < 8 else 0))) & 3
                    if field == 1:
                        part += x[m, kk]
                    elif field == 3:
                        part -= x[m, kk]
                    elif field != 0:
                        raise ValueError("invalid code")
                total += float(f16_bits_to_f64(st[n // 16, g, n % 16])) * part
            y[m, n] = total
    return y


def gemv24_bruteforce(x_bf16_bits, meta, signs, scales, k):
    """Loop form of gemv24 on the stored lane-major planes: find each quad's
    words by hand and gather the two kept activations.  Quad qd of row n lies
    in group g = qd // 32 and lane column q = (qd % 32) // 8, at position
    e = qd % 8 of that lane's meta word and sign field."""
    x = _x(x_bf16_bits)
    meta = np.asarray(meta, dtype=np.uint32)  # [N/16, G4, 64, 4]
    signs = np.asarray(signs, dtype=np.uint32)  # [N/16, G4, 64, 2]
    s = f16_bits_to_f64(np.asarray(scales, dtype=np.uint16))  # [N/16, G4, 4, 4, 4]
    y = np.zeros((x.shape[0], meta.shape[0] * 16))
    for m in range(x.shape[0]):
        for n in range(meta.shape[0] * 16):
            nb, i = n // 16, n % 16
            total = 0.0
            for g in range(k // GROUP):
                b, j = g // 4, g % 4
                part = 0.0
                for qd in range(g * GROUP // 4, (g + 1) * GROUP // 4):
                    q, e = (qd % 32) // 8, qd % 8
                    lane = 16 * q + i
                    nib = (int(meta[nb, b, lane, j]) >> (4 * e)) & 0xF
                    i0, i1 = nib & 3, nib >> 2
                    field = (int(signs[nb, b, lane, j // 2]) >> (16 * (j % 2))) & 0xFFFF
                    n0 = (field >> e) & 1
                    n1 = (field >> (8 + e)) & 1
                    part += (-1.0 if n0 else 1.0) * x[m, 4 * qd + i0]
                    part += (-1.0 if n1 else 1.0) * x[m, 4 * qd + i1]
                total += float(s[nb, b, i // 4, j, i % 4]) * part
            y[m, n] = total
    return y
