"""Helpers for the GPU parity tests: move numpy bit patterns to the device and
compare results with the oracle to the stated bars."""

import sys

import numpy as np
import torch

import oracle

DEV = torch.device("cuda:0")
FLOAT_TOL = 2e-3  # max |got - ref| <= FLOAT_TOL * max |ref|  (fp64 reference)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def f16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.float16)


def u32_dev(words):
    return torch.from_numpy(np.ascontiguousarray(words).view(np.int32)).to(DEV)


def f32_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def host_u32(t):
    return t.cpu().numpy().view(np.uint32)


def host_u16(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def host_f64(t):
    if t.dtype == torch.bfloat16:
        return oracle.numerics.bf16_bits_to_f64(host_u16(t))
    return t.cpu().double().numpy()


def bf16_half_ulp(v):
    """Half the bf16 spacing at |v| (8 significant bits): the rounding a bf16 output adds."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - 8), 0.0)


def assert_close(got, ref, what, tol=FLOAT_TOL, out_bf16=False):
    """max |got - ref| <= tol * max|ref| against the float64 reference.  For a bf16
    output the per-element bar also allows the half-ulp rounding of the output
    itself (the entry points round bf16 results to nearest even)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    if not ref.size:
        return 0.0
    bound = tol * float(np.max(np.abs(ref)))
    excess = np.abs(got - ref) - (bf16_half_ulp(ref) if out_bf16 else 0.0)
    err = float(np.max(np.abs(got - ref)))
    worst = float(np.max(excess))
    say(f"  {what}: max abs err {err:.3e}, bound {bound:.3e}" + (" + bf16 output rounding" if out_bf16 else ""))
    assert worst <= bound, f"{what}: error beyond the bar by {worst - bound:.3e} (bound {bound:.3e})"
    return err


def check_dense_codes(codes_gpu, scales_gpu, ref, k, what):
    """Codes bit-exact except near-threshold elements, where the code must be 0
    or sign(W'); fp16 scales equal or 1 ulp."""
    t_gpu = oracle.quant.unpack_dense(host_u32(codes_gpu), k)  # raises on an invalid field
    near = oracle.quant.near_threshold(ref["wr"], ref["s"])
    mism = t_gpu != ref["t"]
    outside = mism & ~near
    # at the threshold the two valid answers are 0 and sign(W'): never the opposite sign
    wrong_side = mism & near & (t_gpu != 0) & (t_gpu != np.sign(ref["wr"]))
    assert not wrong_side.any(), f"{what}: {int(wrong_side.sum())} near-threshold codes of the wrong sign"
    sg = host_u16(scales_gpu).astype(np.int64)
    sr = ref["scales"].astype(np.int64)
    ulp = np.abs(sg - sr)
    say(f"  {what}: {int(near.sum())} near-threshold elements, {int((mism & near).sum())} of them differ; "
        f"{int(outside.sum())} mismatches outside the band; scale 1-ulp diffs {int((ulp == 1).sum())}")
    assert not outside.any(), f"{what}: {int(outside.sum())} code mismatches outside the threshold band"
    assert ulp.max(initial=0) <= 1, f"{what}: scale differs by {ulp.max()} ulp"
    return int(near.sum()), int((mism & near).sum())


# ---------------------------------------------------------------- act8 operand
# Test-side reading of the act8 format (the activation operand of the dense
# GEMV, defined in include/tb.h): four e4m3 sub-rows with E8M0 block scales.

def e4m3_to_f64(b):
    b = np.asarray(b, dtype=np.int64)
    s, e, m = b >> 7, (b >> 3) & 15, b & 7
    v = np.where(e > 0, np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64)), np.ldexp(m / 8.0, -6))
    v = np.where((b & 0x7F) == 0x7F, np.nan, v)
    return np.where(s > 0, -v, v)


def act8_decode(buf, b, k):
    """x[b, k] as the sum of the four sub-rows of an act8 buffer (float64)."""
    buf = np.asarray(buf, dtype=np.uint8)
    g = k // 128
    vals = buf[:4 * b * k].reshape(b, g, 2, 4, 4, 16).astype(np.int64)  # [b][g][half][sub][q][byte]
    scl = buf[4 * b * k:4 * b * k + b * k // 8].reshape(b, g, 4, 4).astype(np.int64)  # [b][g][sub][block]
    x = np.zeros((b, k))
    for q in range(4):
        for half in range(2):
            kl = 64 * half + 16 * q + np.arange(16)           # K within the group
            v = e4m3_to_f64(vals[:, :, half, :, q, :])         # [b][g][sub][16]
            sc = scl[:, :, :, (kl // 32)]                       # [b][g][sub][16]
            fac = np.where(sc == 0xFF, np.nan, np.ldexp(1.0, (sc - 127)))
            part = np.sum(v * fac, axis=2)                      # [b][g][16]
            cols = (128 * np.arange(g)[:, None] + kl[None, :])  # [g][16]
            x[:, cols] += part
    return x


def act8_kept(x_bits):
    """bf16 bits of what act8 represents: the element itself when its exponent is
    within 10 of its 32-block's largest (level 0) or within 10 of the largest of
    the rest (level 1), else 0; bf16 subnormals become 0."""
    x = np.asarray(x_bits, dtype=np.uint16)
    out = x.copy()
    b, k = x.shape
    e = ((x >> 7) & 0xFF).astype(np.int64).reshape(b, k // 32, 32)
    fin = (e > 0) & (e < 255)
    m0 = np.max(np.where(e < 255, e, 0), axis=2, keepdims=True)
    rest = fin & (e + 10 < m0)
    m1 = np.max(np.where(rest, e, 0), axis=2, keepdims=True)
    keep = fin & ((e + 10 >= m0) | (rest & (e + 10 >= m1) & (m1 > 0)))
    keep = keep | (e == 255)
    out[~keep.reshape(b, k)] = 0
    return out


def check_24_planes(meta_gpu, signs_gpu, scales_gpu, ref, k, what):
    """2:4 planes against the oracle (oracle.quant.quantize_24 output `ref`).
    Outside near-tie quads (oracle.quant.near_tie_24) the kept pair and both
    signs are bit-exact.  In a near-tie quad the GPU may keep another pair,
    but each kept magnitude must be at least the quad's second largest (within
    1e-5 relative), and each kept element's sign must be that of W' wherever
    |W'| > 1e-5 s.  fp16 scales equal or 1 ulp.  Returns (near-tie quads,
    near-tie quads where the GPU differs)."""
    meta_r, signs_r, _ = oracle.quant.load_24(host_u32(meta_gpu), host_u32(signs_gpu), host_u16(scales_gpu), k)
    i0, i1, n0, n1 = oracle.quant.unpack_24(meta_r, signs_r, k)
    wr = ref["wr"]
    n = wr.shape[0]
    quads = wr.reshape(n, k // 4, 4)
    mag = np.abs(quads)
    second = np.sort(mag, axis=2)[:, :, 2]
    tie = oracle.quant.near_tie_24(wr, ref["s"])
    differ = (i0 != ref["idx0"]) | (i1 != ref["idx1"]) | (n0 != ref["neg0"]) | (n1 != ref["neg1"])
    outside = differ & ~tie
    pick = lambda arr, idx: np.take_along_axis(arr, idx[:, :, None], axis=2)[:, :, 0]
    w0, w1 = pick(quads, i0), pick(quads, i1)
    top2 = (np.abs(w0) >= second * (1 - 1e-5)) & (np.abs(w1) >= second * (1 - 1e-5))
    sq = np.repeat(ref["s"], 32, axis=1)
    sign0 = (np.abs(w0) <= 1e-5 * sq) | (n0 == (w0 < 0))
    sign1 = (np.abs(w1) <= 1e-5 * sq) | (n1 == (w1 < 0))
    valid = top2 & sign0 & sign1
    ulp = np.abs(host_u16(scales_gpu).astype(np.int64) - ref["scales"].astype(np.int64))
    say(f"  {what}: {int(tie.sum())} near-tie quads, {int((differ & tie).sum())} of them differ; "
        f"{int(outside.sum())} mismatches outside them; scale 1-ulp diffs {int((ulp == 1).sum())}")
    assert not outside.any(), f"{what}: {int(outside.sum())} 2:4 mismatches outside the near-tie quads"
    assert valid[tie].all(), f"{what}: {int((~valid & tie).sum())} near-tie quads with an invalid pick"
    assert ulp.max(initial=0) <= 1, f"{what}: scale differs by {ulp.max()} ulp"
    return int(tie.sum()), int((differ & tie).sum())
