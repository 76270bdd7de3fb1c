"""Hadamard matrices, the blockwise 128-point Walsh-Hadamard transform and the
2D block rotation of a weight matrix, in float64.

* The matrix is built twice: by the bit rule H[i][j] = (-1)^popcount(i & j)
  (dpshk.com/news/5289456 §2.1, the tip on constructing H) and by Sylvester's
  recursion H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]] (same section;
  mhpq.cn/news/1159370 §2.2; zwxr.cn/news/303439 §2.1).  Natural (Sylvester)
  order throughout.
* The activation transform is blockwise along K in blocks of 128 (the block
  size is fixed at 128 in dpshk.com/news/5289456 §2.1 and mhpq.cn §1.3),
  normalised by 1/sqrt(128) so that it is orthonormal and its own inverse
  (the kernel scale factor 1/sqrt(block) of dpshk.com §2.3).
* The fast form is log2(n) rounds of (a + b, a - b) butterflies
  (xxqk.cn/news/652513 §2; mhpq.cn §2.2), O(n log n).
* The weight rotation is W' = H B H^T / 128 per 128x128 block B
  (xxqk.cn §2 "W_h = H x W x H^T"; dpshk.com §2.1 and §3.2 step 3 apply it per
  128x128 sub-block; dpshk.com §2.3 divides by 128).  H is symmetric, so
  H B H^T = H B H.
"""

import numpy as np

BLOCK = 128


def _popcount(a):
    a = np.asarray(a, dtype=np.int64)
    c = np.zeros_like(a)
    while np.any(a):
        c += a & 1
        a = a >> 1
    return c


def hadamard_bitrule(n):
    """H[i][j] = (-1)^popcount(i & j) for 0 <= i, j < n (n a power of two)."""
    if n < 1 or (n & (n - 1)):
        raise ValueError("n must be a power of two")
    i = np.arange(n)
    return np.where(_popcount(i[:, None] & i[None, :]) % 2 == 0, 1.0, -1.0)


def hadamard_sylvester(n):
    """Sylvester recursion H_1 = [1], H_2m = [[H_m, H_m], [H_m, -H_m]]."""
    if n < 1 or (n & (n - 1)):
        raise ValueError("n must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def _check_blocks(x, n):
    x = np.asarray(x, dtype=np.float64)
    if x.shape[-1] % n:
        raise ValueError(f"last dimension {x.shape[-1]} is not a multiple of {n}")
    return x


def fwht_dense(x, n=BLOCK):
    """Blockwise orthonormal transform along the last axis by a dense matmul:
    out[..., n*b + i] = sum_j H[i][j] / sqrt(n) * x[..., n*b + j]."""
    x = _check_blocks(x, n)
    h = hadamard_bitrule(n) / np.sqrt(n)
    blocks = x.reshape(x.shape[:-1] + (x.shape[-1] // n, n))
    return np.matmul(blocks, h.T).reshape(x.shape)


def fwht_butterfly(x, n=BLOCK):
    """Same transform by log2(n) rounds of (a + b, a - b) butterflies, then 1/sqrt(n)."""
    x = _check_blocks(x, n)
    y = x.reshape(x.shape[:-1] + (x.shape[-1] // n, n)).copy()
    h = 1
    while h < n:
        y = y.reshape(y.shape[:-1] + (n // (2 * h), 2, h))
        a = y[..., 0, :].copy()
        b = y[..., 1, :].copy()
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        y = y.reshape(y.shape[:-3] + (n,))
        h *= 2
    return (y / np.sqrt(n)).reshape(x.shape)


def rotate_blocks(w, n=BLOCK):
    """2D rotation of a [N, K] weight matrix, block by block:
    W'[block] = H @ B @ H^T / n for every n x n block B (N, K multiples of n)."""
    w = np.asarray(w, dtype=np.float64)
    if w.ndim != 2 or w.shape[0] % n or w.shape[1] % n:
        raise ValueError(f"weight shape {w.shape} is not a multiple of {n} x {n}")
    h = hadamard_bitrule(n)
    out = np.empty_like(w)
    for a in range(0, w.shape[0], n):
        for b in range(0, w.shape[1], n):
            out[a:a + n, b:b + n] = h @ w[a:a + n, b:b + n] @ h.T / n
    return out
