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
    """Codes bit-exact except near-threshold elements; fp16 scales equal or 1 ulp."""
    t_gpu = oracle.quant.unpack_dense(host_u32(codes_gpu), k)  # raises on an invalid field
    near = oracle.quant.near_threshold(ref["wr"], ref["s"])
    mism = t_gpu != ref["t"]
    outside = mism & ~near
    sg = host_u16(scales_gpu).astype(np.int64)
    sr = ref["scales"].astype(np.int64)
    ulp = np.abs(sg - sr)
    say(f"  {what}: {int(near.sum())} near-threshold elements, {int((mism & near).sum())} of them differ; "
        f"{int(outside.sum())} mismatches outside the band; scale 1-ulp diffs {int((ulp == 1).sum())}")
    assert not outside.any(), f"{what}: {int(outside.sum())} code mismatches outside the threshold band"
    assert ulp.max(initial=0) <= 1, f"{what}: scale differs by {ulp.max()} ulp"
    return int(near.sum()), int((mism & near).sum())
