"""Seeded synthetic inputs shared by the tests and the benchmark.

This module draws random numbers and formats them into the input buffers the
library takes (fp32 weights, bf16 activation bits, packed code words drawn
i.i.d. per field, fp16 scales).  It performs none of the method's arithmetic:
no transform, no scale, no ternarisation.

Workload shapes are those of a 27B-class layer: d_model = 5120, d_ff = 17408;
Q, K, V, O are 5120 x 5120, up and gate 17408 x 5120, down 5120 x 17408 (rows x
columns = out x in).
"""

import numpy as np

D_MODEL = 5120
D_FF = 17408

# (name, N rows = out features, K columns = in features)
LAYER_MATRICES = (
    ("q", D_MODEL, D_MODEL),
    ("k", D_MODEL, D_MODEL),
    ("v", D_MODEL, D_MODEL),
    ("o", D_MODEL, D_MODEL),
    ("up", D_FF, D_MODEL),
    ("gate", D_FF, D_MODEL),
    ("down", D_MODEL, D_FF),
)

# 2-bit field values of the dense code format: 0 -> 0b00, +1 -> 0b01, -1 -> 0b11
FIELD_ZERO, FIELD_POS, FIELD_NEG = 0b00, 0b01, 0b11
# the six valid 2:4 index nibbles idx0 | idx1 << 2 with idx0 < idx1
NIBBLES_24 = tuple(i0 | (i1 << 2) for i0 in range(4) for i1 in range(4) if i0 < i1)


def f32_to_bf16_bits(x):
    """float32 -> bf16 bit patterns, round to nearest even (NaN kept quiet)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    nan = np.isnan(x)
    out = rounded.astype(np.uint16)
    out[nan] = ((u[nan] >> np.uint64(16)) | np.uint64(0x40)).astype(np.uint16)
    return out


def gaussian_bf16(shape, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(scale))


def single_layer_weights(n=1024, k=1024, seed=0, sigma=0.02, outlier_frac=0.001, outlier_mult=20.0):
    """W ~ N(0, sigma^2) fp32 with round(outlier_frac * n * k) entries x outlier_mult."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((n, k)).astype(np.float32) * np.float32(sigma)
    count = int(round(outlier_frac * n * k))
    idx = rng.choice(n * k, count, replace=False)
    w.reshape(-1)[idx] *= np.float32(outlier_mult)
    return w


def stack_weights(n, k, seed, sigma=0.02, outlier_col_frac=0.01, nu=3.0):
    """W ~ N(0, sigma^2) fp32 with heavy-tailed outlier input channels: a fraction
    of the columns is replaced by sigma * Student-t(nu) draws."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((n, k)).astype(np.float32) * np.float32(sigma)
    ncol = max(1, int(round(outlier_col_frac * k)))
    cols = rng.choice(k, ncol, replace=False)
    w[:, cols] = (rng.standard_t(nu, size=(n, ncol)) * sigma).astype(np.float32)
    return w


def random_code_words(n, k, seed, p=(0.35, 0.30, 0.35)):
    """Dense code words [n/16, k/128, 128] uint32 (the tiled shape of the dense
    format) whose 2-bit fields are drawn i.i.d. with P(-1, 0, +1) = p.  Every
    field is independent, so no assignment of fields to elements is assumed."""
    rng = np.random.default_rng(seed)
    fields = rng.choice(np.array([FIELD_NEG, FIELD_ZERO, FIELD_POS], dtype=np.uint32),
                        size=(n * k // 16, 16), p=np.asarray(p) / np.sum(p))
    shifts = (2 * np.arange(16, dtype=np.uint32))
    words = np.bitwise_or.reduce(fields << shifts, axis=1).astype(np.uint32)
    return words.reshape(n // 16, k // 128, 128)


def random_scales_f16(n, k, seed, lo=0.005, hi=0.05):
    """fp16 bit patterns of U(lo, hi) draws in the dense storage shape
    [n/16, k/128, 16] (one scale per row and 128-group, tile-major; the draws
    are i.i.d., so no assignment of draws to rows is assumed)."""
    rng = np.random.default_rng(seed)
    return rng.uniform(lo, hi, size=(n // 16, k // 128, 16)).astype(np.float16).view(np.uint16)


def _blocks24(k):
    """Blocks of four 128-groups per 16-row tile in the stored 2:4 format, and
    the [blocks, 4] mask of the groups that exist (the last block of a K that
    is not a multiple of 512 is padded with zero groups)."""
    g = k // 128
    g4 = -(-g // 4)
    return g4, (np.arange(4 * g4).reshape(g4, 4) < g)


def random_scales24_f16(n, k, seed, lo=0.005, hi=0.05):
    """fp16 bit patterns of U(lo, hi) draws in the 2:4 format's stored scale
    shape [n/16, G4, 4, 4, 4] (G4 = ceil(k/512); [.., b, q, j, r] is group
    4 b + j; padded groups zero).  Independent draws, so any order is the
    same distribution."""
    rng = np.random.default_rng(seed)
    g4, valid = _blocks24(k)
    s = rng.uniform(lo, hi, size=(n // 16, g4, 4, 4, 4)).astype(np.float16).view(np.uint16)
    return s * valid[None, :, None, :, None].astype(np.uint16)


def random_24(n, k, seed):
    """2:4 planes in the stored shapes, meta [n/16, G4, 64, 4] (word [.., b, l, j]
    of group 4 b + j) with a uniform choice of the 6 index pairs per quad, and
    signs [n/16, G4, 64, 2] (two 16-bit fields per word, group 4 b + 2 p in
    the low half of word p) with fair random bits.  Padded groups are zero."""
    rng = np.random.default_rng(seed)
    g4, valid = _blocks24(k)
    nib = rng.choice(np.array(NIBBLES_24, dtype=np.uint32), size=(n // 16, g4, 64, 4, 8))
    meta = np.bitwise_or.reduce(nib << (4 * np.arange(8, dtype=np.uint32)), axis=4).astype(np.uint32)
    meta *= valid[None, :, None, :].astype(np.uint32)
    signs = rng.integers(0, 2 ** 32, size=(n // 16, g4, 64, 2), dtype=np.uint64).astype(np.uint32)
    half = valid.reshape(g4, 2, 2)  # [b, p, half]
    keep = (half[:, :, 0] * np.uint32(0xFFFF)) | (half[:, :, 1] * np.uint32(0xFFFF0000))
    signs &= keep[None, :, None, :].astype(np.uint32)
    return meta, signs


def small_int_bf16(shape, seed, lim=8):
    """bf16 bit patterns of integers in [-lim, lim] (exact in bf16)."""
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits(rng.integers(-lim, lim + 1, size=shape).astype(np.float32))


# ---------------------------------------------------------------- device-side
# Generators for benchmark-sized inputs, drawn on the GPU with torch (same
# distributions as above; not bit-identical to the numpy streams).

def torch_code_words(n, k, gen, device, p=(0.35, 0.30, 0.35)):
    """[n/16, k/128, 128] int32 code words, 2-bit fields i.i.d. with P(-1, 0, +1) = p."""
    import torch

    u = torch.rand((n // 16, k // 128, 128, 16), generator=gen, device=device)
    f = torch.where(u < p[0], FIELD_NEG, torch.where(u < p[0] + p[1], FIELD_ZERO, FIELD_POS)).to(torch.int64)
    del u
    shifts = 2 * torch.arange(16, device=device, dtype=torch.int64)
    w = (f << shifts).sum(dim=-1)
    return w.to(torch.int32)


def torch_scales_f16(n, k, gen, device, lo=0.005, hi=0.05):
    """U(lo, hi) fp16 scales in the dense storage shape [n/16, k/128, 16]."""
    import torch

    return (lo + (hi - lo) * torch.rand((n // 16, k // 128, 16), generator=gen, device=device)).to(torch.float16)


def torch_scales24_f16(n, k, gen, device, lo=0.005, hi=0.05):
    """U(lo, hi) fp16 scales in the 2:4 stored shape [n/16, G4, 4, 4, 4]
    (padded groups zero, as random_scales24_f16)."""
    import torch

    g4, valid = _blocks24(k)
    s = lo + (hi - lo) * torch.rand((n // 16, g4, 4, 4, 4), generator=gen, device=device)
    mask = torch.as_tensor(valid, device=device).view(1, g4, 1, 4, 1)
    return (s * mask).to(torch.float16)


def torch_gaussian_bf16(shape, gen, device, scale=1.0):
    import torch

    return (torch.randn(shape, generator=gen, device=device) * scale).to(torch.bfloat16)


def torch_stack_weights(n, k, gen, device, sigma=0.02, outlier_col_frac=0.01, nu=3):
    """The stack recipe of stack_weights drawn on the device: W ~ N(0, sigma^2)
    fp32 [n, k], with round(outlier_col_frac * k) input columns replaced by
    sigma * Student-t(nu) draws (a standard normal over the root of the mean of
    nu squared standard normals; nu a positive integer)."""
    import torch

    w = torch.randn((n, k), generator=gen, device=device) * sigma
    ncol = max(1, int(round(outlier_col_frac * k)))
    cols = torch.randperm(k, generator=gen, device=device)[:ncol]
    z = torch.randn((n, ncol), generator=gen, device=device)
    chi2 = torch.randn((nu, n, ncol), generator=gen, device=device).square().sum(dim=0)
    w[:, cols] = z / torch.sqrt(chi2 / nu) * sigma
    return w


def torch_24(n, k, gen, device):
    """2:4 planes in the stored shapes (meta [n/16, G4, 64, 4], signs
    [n/16, G4, 64, 2]) as int32, uniform index pairs and signs, padded groups
    zero (as random_24)."""
    import torch

    g4, valid = _blocks24(k)
    nib = torch.tensor(NIBBLES_24, dtype=torch.int64, device=device)
    sel = torch.randint(0, 6, (n // 16, g4, 64, 4, 8), generator=gen, device=device)
    meta = (nib[sel] << (4 * torch.arange(8, device=device, dtype=torch.int64))).sum(-1)
    meta = meta * torch.as_tensor(valid, device=device).view(1, g4, 1, 4)
    signs = torch.randint(0, 2 ** 32, (n // 16, g4, 64, 2), generator=gen, device=device, dtype=torch.int64)
    half = valid.reshape(g4, 2, 2).astype(np.int64)
    keep = torch.as_tensor(half[:, :, 0] * 0xFFFF | half[:, :, 1] * 0xFFFF0000, device=device).view(1, g4, 1, 2)
    signs = signs & keep
    # two's complement view of the uint32 words
    return (torch.where(meta >= 2 ** 31, meta - 2 ** 32, meta).to(torch.int32),
            torch.where(signs >= 2 ** 31, signs - 2 ** 32, signs).to(torch.int32))
