"""Offline quantiser: absmean group scale, ternarisation and packing, dense and
2:4, in float64.

Definitions followed (where the pages leave a step open, the reading taken is
stated with the step):

* Group scale: the mean absolute value of the 128 contiguous K-elements of one
  row of one rotated 128x128 block (mhpq.cn/news/1159370 §1.1: take the group's
  mean absolute value as the scale; §1.3: one fp16 scale per 128 elements).
* Ternarise: divide by the scale, round, clip to {-1, 0, 1} (mhpq.cn §1.1).
  Written as a threshold at half the scale with a strict comparison, as in the
  sign(w) * (|w| > thr) step of dpshk.com/news/5289456 §3.2 step 5; a value at
  exactly s/2 gives 0 (round-half-even agrees).  The comparison uses the
  unrounded float64 scale; the stored scale is its fp16 rounding.
* Error-minimising variant: for each group choose the threshold theta and
  scale s that minimise ||w' - s t||^2 with t = sign(w') [|w'| >= theta]
  (a threshold-shaped ternarisation, dpshk.com/news/5289456 §3.2 steps 4-5;
  the threshold as the accuracy-critical choice, xxqk.cn/news/652513 §3,
  its per-block threshold search).
  For a kept set of j elements with magnitude sum S the best scale is S / j
  and the error is sum w'^2 - S^2 / j, so theta is the group magnitude that
  maximises S^2 / j over the kept sets {|w'| >= theta}.  The 0.38-quantile
  threshold of dpshk.com §3.2 step 4 is one member of this family (it keeps
  the largest 79 of 128).  Ties in S^2 / j go to the larger theta.
* Residual plane: the part of W' the first ternary plane misses, W' minus its
  fp16 scale times t, is ternarised again by the absmean rule (the residual
  calibration of xxqk.cn/news/652513 §3), giving W' ~ s1 t1 + s2 t2.
* 2:4: of every 4 consecutive K-elements keep the 2 largest |w'| and ternarise
  the survivors (mhpq.cn §1.2: prune with the 2:4 pattern, then ternarise what
  remains).  Kept elements are nonzero, so each carries only a sign; the group
  scale is the mean |w'| of the 64 kept elements of the group.
* Storage: 2 bits per weight (mhpq.cn §3.1), as a sign bit and a magnitude bit
  per weight (the sign/magnitude split of dpshk.com §2.2).  The arrangement of
  the fields inside the words is this implementation's choice: 16-row x
  128-column tiles whose word order matches the operand layout of the matrix
  instruction that consumes them.

Dense format (N a multiple of 16, K a multiple of 128):
  codes[N / 16][K / 128][128] uint32.  Tile (nb, g) covers rows 16 nb .. 16 nb + 15
  and columns 128 g .. 128 g + 127.  With l = 16 q + i (i = row in the tile,
  q = 0..3) and h = 0, 1, word 2 l + h of the tile holds row 16 nb + i, columns
  128 g + 32 q + 16 h + r for r = 0..15; the 2-bit field of r starts at bit
  4 (r mod 8) + 2 - 2 floor(r / 8), so fields r < 8 sit in bits 2-3 of nibble r
  and fields r >= 8 in bits 0-1 of nibble r - 8.  Field value: 0b00 -> 0,
  0b01 -> +1, 0b11 -> -1 (bit 0 = nonzero, bit 1 = negative); 0b10 is invalid.
  scales[N / 16][K / 128][16] fp16 bits, tile-major like the codes: the scale
  of row n and group g at [n // 16, g, n % 16] (tile_scales).
Residual (two-plane) format: the dense format of both planes with their
  groups interleaved along K (interleave_planes), codes [N/16][2 K/128][128] and
  scales [N/16][2 K/128][16].
2:4 format.  The words of a row (pack_24, unpack_24):
  meta word j of row n covers quads q = 8 j .. 8 j + 7 (q = k // 4): the
  nibble at bits 4 * (q % 8) holds idx0 (bits 0-1) and idx1 (bits 2-3),
  idx0 < idx1 the kept positions.  Sign word j covers quads 16 j .. 16 j + 15:
  bit q % 16 is set when the element at idx0 is negative, bit 16 + q % 16
  when the element at idx1 is.
  Stored lane-major (store_24, load_24): a 16-row tile and a block of four
  128-column groups together, G4 = ceil(G / 4) blocks per tile (G = K / 128;
  the groups of the last block past G are zero).  Lane l = 16 q + i stands
  for row i of the tile and the quads 32 g + 8 q .. 32 g + 8 q + 7 of each
  group g (its meta word 4 g + q), so that one lane finds its words for the
  four groups of a block side by side:
    meta[N / 16][G4][64][4] uint32: [nb, b, 16 q + i, j] = meta word
      4 g + q of row 16 nb + i, g = 4 b + j;
    signs[N / 16][G4][64][2] uint32: the 16-bit sign field of lane (i, q)
      and group g in the low half of [nb, b, 16 q + i, p] for g = 4 b + 2 p,
      in the high half for g = 4 b + 2 p + 1.  The field holds the lane's
      quads 32 g + 8 q + e, e = 0..7: bit e the idx0 sign, bit 8 + e the
      idx1 sign (bits 8 (q % 2) + e and 16 + 8 (q % 2) + e of sign word
      2 g + q // 2 of the row);
    scales[N / 16][G4][4][4][4] fp16 bits: [nb, b, q, j, r] = the scale of
      row 16 nb + 4 q + r and group 4 b + j.
"""

import numpy as np

from .hadamard import BLOCK, rotate_blocks
from .numerics import f16_bits_to_f64, f64_to_f16_bits

GROUP = 128
NEAR_REL = 1e-5

FIELD_OF_T = {0: 0b00, 1: 0b01, -1: 0b11}


def _check_w(w):
    w = np.asarray(w, dtype=np.float64)
    if w.ndim != 2 or w.shape[0] % BLOCK or w.shape[1] % BLOCK:
        raise ValueError(f"weight shape {w.shape} must be multiples of {BLOCK}")
    if not np.all(np.isfinite(w)):
        raise ValueError("weights must be finite")
    return w


def absmean_scales(wr):
    """s[n, g] = mean over the 128 elements of group g of row n of |W'|."""
    n, k = wr.shape
    return np.abs(wr).reshape(n, k // GROUP, GROUP).mean(axis=2)


def ternarize(wr, s):
    """t = +1 where W' > s/2, -1 where W' < -s/2, else 0 (s per 128-group)."""
    thr = np.repeat(s / 2.0, GROUP, axis=1)
    return np.where(wr > thr, 1, np.where(wr < -thr, -1, 0)).astype(np.int8)


def near_threshold(wr, s, rel=NEAR_REL):
    """Elements whose |W'| is within rel * s/2 of the threshold s/2."""
    thr = np.repeat(s / 2.0, GROUP, axis=1)
    return np.abs(np.abs(wr) - thr) <= rel * thr


def dense_location(n, k):
    """Tile index (nb, g), word index in the tile and bit position of the 2-bit
    field of element (n, k) of the dense format (arrays broadcast)."""
    n = np.asarray(n)
    k = np.asarray(k)
    i, nb = n % 16, n // 16
    g, kk = k // GROUP, k % GROUP
    q, h, r = kk // 32, (kk % 32) // 16, kk % 16
    word = 2 * (16 * q + i) + h
    bit = 4 * (r % 8) + 2 - 2 * (r // 8)
    return nb, g, word, bit


def pack_dense(t):
    """Pack ternary t[N, K] into codes[N/16, K/128, 128] (uint32), format above."""
    t = np.asarray(t)
    n, k = t.shape
    if n % 16 or k % GROUP:
        raise ValueError("N must be a multiple of 16 and K of 128")
    field = np.zeros(t.shape, dtype=np.uint64)
    field[t == 1] = FIELD_OF_T[1]
    field[t == -1] = FIELD_OF_T[-1]
    nn, kk = np.meshgrid(np.arange(n), np.arange(k), indexing="ij")
    nb, g, word, bit = dense_location(nn, kk)
    words = np.zeros((n // 16, k // GROUP, 128), dtype=np.uint64)
    # every (tile, word, bit) is hit by exactly one element, so add == or
    np.add.at(words, (nb, g, word), field << bit.astype(np.uint64))
    return words.astype(np.uint32)


def unpack_dense(codes, k):
    """Inverse of pack_dense; raises on the invalid field 0b10."""
    codes = np.asarray(codes, dtype=np.uint32).astype(np.uint64)
    if codes.ndim != 3 or codes.shape[1] * GROUP != k or codes.shape[2] != 128:
        raise ValueError("codes shape does not match K")
    n = codes.shape[0] * 16
    nn, kk = np.meshgrid(np.arange(n), np.arange(k), indexing="ij")
    nb, g, word, bit = dense_location(nn, kk)
    f = (codes[nb, g, word] >> bit.astype(np.uint64)) & np.uint64(3)
    if np.any(f == 0b10):
        raise ValueError("invalid 2-bit code 0b10")
    return np.where(f == 0b01, 1, np.where(f == 0b11, -1, 0)).astype(np.int8)


def tile_scales(s16):
    """Scale bits by row, [N, G], into the dense storage order [N/16, G, 16]:
    the scale of row n and group g goes to [n // 16, g, n % 16]."""
    s16 = np.asarray(s16)
    n, g = s16.shape
    if n % 16:
        raise ValueError("N must be a multiple of 16")
    return np.ascontiguousarray(s16.reshape(n // 16, 16, g).transpose(0, 2, 1))


def untile_scales(t):
    """Inverse of tile_scales: [N/16, G, 16] -> [N, G]."""
    t = np.asarray(t)
    if t.ndim != 3 or t.shape[2] != 16:
        raise ValueError("dense scales must be [N/16, G, 16]")
    return np.ascontiguousarray(t.transpose(0, 2, 1).reshape(t.shape[0] * 16, t.shape[1]))


def quantize_dense(w):
    """Rotate 128x128 blocks, take absmean group scales, ternarise, pack.

    Returns a dict with codes (uint32 [N/16, K/128, 128]), scales (fp16 bits
    uint16 [N/16, K/128, 16], tile_scales) and the float64 intermediates wr
    (W'), s (unrounded scales, [N, K/128]) and t (int8 ternary values)."""
    w = _check_w(w)
    wr = rotate_blocks(w)
    s = absmean_scales(wr)
    t = ternarize(wr, s)
    return {"codes": pack_dense(t), "scales": tile_scales(f64_to_f16_bits(s)), "wr": wr, "s": s, "t": t}


# ---------------------------------------------------------------- error-minimising variant

def mse_threshold(a):
    """For magnitudes a[..., n] (float64, >= 0) of groups along the last axis:
    the threshold theta (one of the group's magnitudes) maximising S^2 / j over
    the kept sets {k : a_k >= theta}, j = their count and S their sum; among
    equal objectives the larger theta.  Returns (theta, j, S)."""
    a = np.asarray(a, dtype=np.float64)
    d = -np.sort(-a, axis=-1)                     # descending magnitudes
    n = d.shape[-1]
    S = np.cumsum(d, axis=-1)                     # S[j-1]: sum of the j largest
    j = np.arange(1, n + 1, dtype=np.float64)
    obj = S * S / j
    # a kept set {a >= theta} holds every copy of theta: only the last of a
    # run of equal magnitudes is a candidate
    last = np.ones(d.shape, dtype=bool)
    last[..., :-1] = d[..., :-1] > d[..., 1:]
    obj = np.where(last, obj, -np.inf)
    # argmax takes the first maximum, i.e. the smallest j: the larger theta
    best = np.argmax(obj, axis=-1)
    take = lambda arr: np.take_along_axis(arr, best[..., None], axis=-1)[..., 0]
    return take(d), best + 1, take(S)


def mse_objective_gap(a):
    """Relative gap between the best and the second-best objective S^2 / j over
    distinct thresholds of each group.  A group with a single candidate (one
    distinct magnitude) or an all-zero group gets inf: no other threshold can
    come close, so float rounding cannot change its choice."""
    a = np.asarray(a, dtype=np.float64)
    d = -np.sort(-a, axis=-1)
    n = d.shape[-1]
    S = np.cumsum(d, axis=-1)
    obj = S * S / np.arange(1, n + 1, dtype=np.float64)
    last = np.ones(d.shape, dtype=bool)
    last[..., :-1] = d[..., :-1] > d[..., 1:]
    obj = np.sort(np.where(last, obj, -np.inf), axis=-1)
    top, second = obj[..., -1], obj[..., -2]
    gap = np.where(np.isfinite(second), (top - second) / np.maximum(top, 1e-300), np.inf)
    return np.where(top > 0, gap, np.inf)


def quantize_dense_mse(w):
    """Rotate 128x128 blocks; per group the error-minimising threshold and scale
    (mse_threshold); t = sign(W') [|W'| >= theta]; pack as the dense format.

    Returns codes, scales (fp16 bits), and wr, s (unrounded scales), theta, t."""
    w = _check_w(w)
    wr = rotate_blocks(w)
    n, k = wr.shape
    a = np.abs(wr).reshape(n, k // GROUP, GROUP)
    theta, j, S = mse_threshold(a)
    s = S / j
    keep = a >= theta[..., None]
    t = (np.sign(wr) * keep.reshape(n, k)).astype(np.int8)
    return {"codes": pack_dense(t), "scales": tile_scales(f64_to_f16_bits(s)), "wr": wr, "s": s, "theta": theta,
            "t": t}


def near_threshold_mse(wr, theta, rel=NEAR_REL):
    """Elements whose |W'| is within rel * theta of their group's threshold."""
    thr = np.repeat(theta, GROUP, axis=1)
    return np.abs(np.abs(wr) - thr) <= rel * thr


def near_tie_mse(wr, rel=NEAR_REL):
    """Groups [N, K/128] whose best and second-best objective differ by at most
    rel (relative): float rounding may pick either threshold."""
    n, k = wr.shape
    return mse_objective_gap(np.abs(wr).reshape(n, k // GROUP, GROUP)) <= rel


# ---------------------------------------------------------------- residual second plane

def interleave_planes(a, b):
    """Per-group interleave of two planes along the group axis (axis 1): the
    result's group 2 g is a's group g and group 2 g + 1 is b's.  Works for
    codes [N/16, G, 128] and for scales [N/16, G, 16] (or [N, G])."""
    a = np.asarray(a)
    b = np.asarray(b)
    if a.shape != b.shape:
        raise ValueError("planes differ in shape")
    return np.stack([a, b], axis=2).reshape(a.shape[0], 2 * a.shape[1], *a.shape[2:])


def split_planes(x):
    """Inverse of interleave_planes: (plane 1, plane 2)."""
    x = np.asarray(x)
    return x[:, 0::2], x[:, 1::2]


def quantize_dense_residual(w):
    """Two ternary planes, W' ~ f16(s1) t1 + f16(s2) t2: the residual
    calibration of xxqk.cn/news/652513 §3, which stores the difference between
    the rotated coefficients and their ternary approximation and ternarises it
    once more.

    Plane 1 is quantize_dense's absmean rule.  The residual is taken against
    what the product will apply, the stored fp16 scale:
        d = W' - f16(s1) t1,
    and stays in the rotated basis, so both planes multiply the same rotated
    activations.  Plane 2 is the absmean rule applied to d: s2 = mean |d| per
    group, t2 = +-1 where |d| > s2 / 2, fp16 scale.

    Storage (interleave_planes): codes [N/16][2 K/128][128] and scales
    [N/16][2 K/128][16], where group 2 g + p holds plane p's group g (p = 0
    first).

    Returns codes, scales, and wr, s1, t1, d, s2, t2 (float64 / int8)."""
    w = _check_w(w)
    wr = rotate_blocks(w)
    s1 = absmean_scales(wr)
    t1 = ternarize(wr, s1)
    sc1 = f64_to_f16_bits(s1)
    d = wr - t1 * np.repeat(f16_bits_to_f64(sc1), GROUP, axis=1)
    s2 = absmean_scales(d)
    t2 = ternarize(d, s2)
    sc2 = f64_to_f16_bits(s2)
    return {"codes": interleave_planes(pack_dense(t1), pack_dense(t2)),
            "scales": interleave_planes(tile_scales(sc1), tile_scales(sc2)),
            "wr": wr, "s1": s1, "t1": t1, "d": d, "s2": s2, "t2": t2}


# ---------------------------------------------------------------- 2:4 variant

def select_24(wr):
    """For every quad of 4 along K, the positions of the two largest |W'|
    (ties go to the lower position); returns idx0 < idx1, each [N, K/4]."""
    n, k = wr.shape
    a = np.abs(wr).reshape(n, k // 4, 4)
    order = np.argsort(-a, axis=2, kind="stable")
    top = np.sort(order[:, :, :2], axis=2)
    return top[:, :, 0].astype(np.int64), top[:, :, 1].astype(np.int64)


def near_tie_24(wr, s, rel=NEAR_REL):
    """Quads whose selection or signs are ambiguous at float rounding level:
    the 2nd and 3rd largest |W'| are within rel of each other, or a kept
    element has |W'| <= rel * s (its sign is then ill-defined)."""
    n, k = wr.shape
    a = np.sort(np.abs(wr).reshape(n, k // 4, 4), axis=2)[:, :, ::-1]
    tie = np.abs(a[:, :, 1] - a[:, :, 2]) <= rel * np.maximum(a[:, :, 1], 1e-300)
    sq = np.repeat(s, GROUP // 4, axis=1)
    small = a[:, :, 1] <= rel * sq
    return tie | small


def quantize_24(w):
    """Rotate, keep 2 of every 4 along K, absmean over the kept elements, pack.

    Returns meta, signs, scales (stored, lane-major) plus wr, s, idx0, idx1,
    neg0, neg1 and the dense ternary equivalent t."""
    w = _check_w(w)
    wr = rotate_blocks(w)
    n, k = wr.shape
    idx0, idx1 = select_24(wr)
    quads = wr.reshape(n, k // 4, 4)
    v0 = np.take_along_axis(quads, idx0[:, :, None], axis=2)[:, :, 0]
    v1 = np.take_along_axis(quads, idx1[:, :, None], axis=2)[:, :, 0]
    kept_abs = (np.abs(v0) + np.abs(v1)).reshape(n, k // GROUP, GROUP // 4)
    s = kept_abs.sum(axis=2) / (GROUP // 2)
    neg0 = v0 < 0
    neg1 = v1 < 0
    meta, signs, scales = store_24(*pack_24(idx0, idx1, neg0, neg1), f64_to_f16_bits(s))
    t = dense_from_24(idx0, idx1, neg0, neg1)
    return {"meta": meta, "signs": signs, "scales": scales, "wr": wr, "s": s,
            "idx0": idx0, "idx1": idx1, "neg0": neg0, "neg1": neg1, "t": t}


def pack_24(idx0, idx1, neg0, neg1):
    idx0 = np.asarray(idx0, dtype=np.uint64)
    idx1 = np.asarray(idx1, dtype=np.uint64)
    n, nq = idx0.shape
    if nq % 16:
        raise ValueError("K/4 must be a multiple of 16")
    if np.any(idx0 >= idx1) or np.any(idx1 > 3):
        raise ValueError("need 0 <= idx0 < idx1 <= 3")
    nib = idx0 | (idx1 << np.uint64(2))
    meta = np.zeros((n, nq // 8), dtype=np.uint64)
    for j in range(8):
        meta |= nib[:, j::8] << np.uint64(4 * j)
    n0 = np.asarray(neg0).astype(np.uint64)
    n1 = np.asarray(neg1).astype(np.uint64)
    signs = np.zeros((n, nq // 16), dtype=np.uint64)
    for j in range(16):
        signs |= n0[:, j::16] << np.uint64(j)
        signs |= n1[:, j::16] << np.uint64(16 + j)
    return meta.astype(np.uint32), signs.astype(np.uint32)


def store_24(meta, signs, scales):
    """Row words and scales ([N, K/32], [N, K/64], [N, K/128]) into the stored
    lane-major arrays (module docstring): meta [N/16, G4, 64, 4], signs
    [N/16, G4, 64, 2], scales [N/16, G4, 4, 4, 4], groups past G zero."""
    meta = np.asarray(meta, dtype=np.uint32)
    signs = np.asarray(signs, dtype=np.uint32)
    scales = np.asarray(scales, dtype=np.uint16)
    n, nw = meta.shape
    if n % 16 or nw % 4 or signs.shape != (n, nw // 2) or scales.shape != (n, nw // 4):
        raise ValueError("2:4 rows must be [N, K/32], [N, K/64], [N, K/128] with N a multiple of 16")
    g = nw // 4
    g4 = -(-g // 4)
    # per row, group and lane column q: the meta word 4 g + q
    mw = np.zeros((n, 4 * g4, 4), dtype=np.uint32)
    mw[:, :g, :] = meta.reshape(n, g, 4)
    # the 16-bit sign field of (row, g, q) from sign word 2 g + q // 2
    sw = signs.reshape(n, g, 2).astype(np.uint64)
    field = np.zeros((n, 4 * g4, 4), dtype=np.uint64)
    for q in range(4):
        word = sw[:, :, q // 2]
        sh = np.uint64(8 * (q % 2))
        field[:, :g, q] = ((word >> sh) & np.uint64(0xFF)) | (((word >> (np.uint64(16) + sh)) & np.uint64(0xFF)) << np.uint64(8))
    sc = np.zeros((n, 4 * g4), dtype=np.uint16)
    sc[:, :g] = scales
    nb = n // 16
    # meta: (nb, i, b, j, q) -> (nb, b, q, i, j)
    m = mw.reshape(nb, 16, g4, 4, 4).transpose(0, 2, 4, 1, 3).reshape(nb, g4, 64, 4)
    # signs: pairs of groups in one word, (nb, i, b, p, e, q) -> (nb, b, q, i, p)
    f = field.reshape(nb, 16, g4, 2, 2, 4)
    pair = f[:, :, :, :, 0, :] | (f[:, :, :, :, 1, :] << np.uint64(16))
    sg = pair.transpose(0, 2, 4, 1, 3).reshape(nb, g4, 64, 2).astype(np.uint32)
    # scales: row 16 nb + 4 q + r, group 4 b + j -> [nb, b, q, j, r]
    st = sc.reshape(nb, 4, 4, g4, 4).transpose(0, 3, 1, 4, 2)
    return np.ascontiguousarray(m), np.ascontiguousarray(sg), np.ascontiguousarray(st)


def load_24(meta, signs, scales, k):
    """Inverse of store_24 for K-long rows: the row words [N, K/32],
    [N, K/64] and the scales [N, K/128]."""
    meta = np.asarray(meta, dtype=np.uint32)
    signs = np.asarray(signs, dtype=np.uint32)
    scales = np.asarray(scales, dtype=np.uint16)
    g = k // GROUP
    g4 = -(-g // 4)
    if k % GROUP or meta.ndim != 4 or meta.shape[1:] != (g4, 64, 4) or signs.shape != meta.shape[:2] + (64, 2) \
            or scales.shape != meta.shape[:2] + (4, 4, 4):
        raise ValueError("stored 2:4 planes must be [N/16, G4, 64, 4], [N/16, G4, 64, 2] and [N/16, G4, 4, 4, 4]")
    nb = meta.shape[0]
    n = 16 * nb
    m = meta.reshape(nb, g4, 4, 16, 4).transpose(0, 3, 1, 4, 2).reshape(n, 4 * g4, 4)[:, :g, :]
    pair = signs.reshape(nb, g4, 4, 16, 2).astype(np.uint64)
    field = np.stack([pair & np.uint64(0xFFFF), pair >> np.uint64(16)], axis=-1)  # (nb, b, q, i, p, e)
    field = field.transpose(0, 3, 1, 4, 5, 2).reshape(n, 4 * g4, 4)[:, :g, :]  # (row, g, q)
    sw = np.zeros((n, g, 2), dtype=np.uint64)
    for q in range(4):
        sh = np.uint64(8 * (q % 2))
        lo = field[:, :, q] & np.uint64(0xFF)
        hi = field[:, :, q] >> np.uint64(8)
        sw[:, :, q // 2] |= (lo << sh) | (hi << (np.uint64(16) + sh))
    sc = scales.transpose(0, 2, 4, 1, 3).reshape(n, 4 * g4)[:, :g]
    return (np.ascontiguousarray(m.reshape(n, 4 * g)), np.ascontiguousarray(sw.reshape(n, 2 * g).astype(np.uint32)),
            np.ascontiguousarray(sc))


def unpack_24(meta, signs, k):
    meta = np.asarray(meta, dtype=np.uint32).astype(np.uint64)
    signs = np.asarray(signs, dtype=np.uint32).astype(np.uint64)
    n = meta.shape[0]
    nq = k // 4
    if meta.shape[1] * 8 != nq or signs.shape[1] * 16 != nq:
        raise ValueError("meta/signs shape does not match K")
    idx0 = np.zeros((n, nq), dtype=np.int64)
    idx1 = np.zeros((n, nq), dtype=np.int64)
    for j in range(8):
        nib = (meta >> np.uint64(4 * j)) & np.uint64(0xF)
        idx0[:, j::8] = (nib & np.uint64(3)).astype(np.int64)
        idx1[:, j::8] = (nib >> np.uint64(2)).astype(np.int64)
    if np.any(idx0 >= idx1):
        raise ValueError("invalid 2:4 index nibble (need idx0 < idx1)")
    neg0 = np.zeros((n, nq), dtype=bool)
    neg1 = np.zeros((n, nq), dtype=bool)
    for j in range(16):
        neg0[:, j::16] = ((signs >> np.uint64(j)) & np.uint64(1)) == 1
        neg1[:, j::16] = ((signs >> np.uint64(16 + j)) & np.uint64(1)) == 1
    return idx0, idx1, neg0, neg1


def dense_from_24(idx0, idx1, neg0, neg1):
    """The ternary matrix a 2:4 encoding stands for (+-1 at kept positions)."""
    n, nq = np.asarray(idx0).shape
    t = np.zeros((n, nq, 4), dtype=np.int8)
    np.put_along_axis(t, np.asarray(idx0)[:, :, None], np.where(neg0, -1, 1)[:, :, None].astype(np.int8), axis=2)
    np.put_along_axis(t, np.asarray(idx1)[:, :, None], np.where(neg1, -1, 1)[:, :, None].astype(np.int8), axis=2)
    return t.reshape(n, nq * 4)
