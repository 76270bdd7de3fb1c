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


def assert_close(got, ref, what, tol=FLOAT_TOL):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    bound = tol * float(np.max(np.abs(ref))) if ref.size else 0.0
    say(f"  {what}: max abs err {err:.3e}, bound {bound:.3e}")
    assert err <= bound, f"{what}: max abs err {err:.3e} > {bound:.3e}"
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
