"""GPU parity of tb_ternary_gemv and tb_ternary24_gemv against the oracle."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import DEV, assert_close, bf16_dev, f16_dev, say, u32_dev
from ternary_weights_hadamard_amd import synth, tb

pytestmark = pytest.mark.gpu


def _dense_inputs(n, k, b, seed):
    codes = synth.random_code_words(n, k, seed=seed)
    scales = synth.random_scales_f16(n, k, seed=seed + 1)
    x = synth.gaussian_bf16((b, k), seed=seed + 2)
    return codes, scales, x


@pytest.mark.parametrize("n,k", [(128, 128), (256, 384), (1024, 1024), (384, 2176)])
@pytest.mark.parametrize("b", [1, 2, 5, 8, 16])
def test_gemv_small_matches_oracle(n, k, b):
    say(f"gemv N={n} K={k} B={b}")
    codes, scales, x = _dense_inputs(n, k, b, seed=n + k + b)
    y = tb.tb_ternary_gemv(bf16_dev(x), u32_dev(codes), f16_dev(scales))
    torch.cuda.synchronize()
    ref = oracle.matvec.gemv(x, codes, scales, k)
    assert_close(y.cpu().numpy(), ref, f"gemv {n}x{k} B={b}")
    # fp32 accumulation of exact products: far inside the bar
    assert np.max(np.abs(y.cpu().numpy() - ref)) <= 1e-5 * np.max(np.abs(ref))


@pytest.mark.parametrize("n,k", [(5120, 5120), (17408, 5120), (5120, 17408)])
@pytest.mark.parametrize("b", [1, 8])
def test_gemv_full_size_sampled_rows(n, k, b):
    say(f"gemv full N={n} K={k} B={b}")
    codes, scales, x = _dense_inputs(n, k, b, seed=20 + b)
    y = tb.tb_ternary_gemv(bf16_dev(x), u32_dev(codes), f16_dev(scales)).cpu().numpy()
    rows = np.sort(np.random.default_rng(1).choice(n, 256, replace=False))
    ref = oracle.matvec.gemv(x, codes[rows], scales[rows], k)
    assert_close(y[:, rows], ref, f"gemv {n}x{k} B={b} (256 sampled rows)")


@pytest.mark.parametrize("b", [1, 3, 16])
def test_gemv_exact_small_integers(b):
    # integer activations and power-of-two scales: the exact result is an fp32 value
    n, k = 256, 1280
    codes = synth.random_code_words(n, k, seed=5)
    x = synth.small_int_bf16((b, k), seed=6)
    sc = (2.0 ** np.random.default_rng(7).integers(-6, 2, size=(n, k // 128))).astype(np.float16).view(np.uint16)
    y = tb.tb_ternary_gemv(bf16_dev(x), u32_dev(codes), f16_dev(sc))
    torch.cuda.synchronize()
    ref = oracle.matvec.gemv(x, codes, sc, k)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), ref)


def test_gemv_special_patterns():
    n, k = 128, 256
    x = synth.gaussian_bf16((1, k), seed=9)
    xv = oracle.numerics.bf16_bits_to_f64(x)
    ones_scale = np.full((n, k // 128), np.float16(1.0).view(np.uint16), dtype=np.uint16)
    t = np.ones((n, k), dtype=np.int8)
    y = tb.tb_ternary_gemv(bf16_dev(x), u32_dev(oracle.quant.pack_dense(t)), f16_dev(ones_scale))
    torch.cuda.synchronize()
    assert np.allclose(y.cpu().numpy(), xv.sum(), rtol=1e-5)
    cols = np.random.default_rng(2).integers(0, k, size=n)
    t = np.zeros((n, k), dtype=np.int8)
    t[np.arange(n), cols] = -1
    y = tb.tb_ternary_gemv(bf16_dev(x), u32_dev(oracle.quant.pack_dense(t)), f16_dev(ones_scale))
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy()[0], -xv[0, cols])
    t = np.zeros((n, k), dtype=np.int8)
    y = tb.tb_ternary_gemv(bf16_dev(x), u32_dev(oracle.quant.pack_dense(t)), f16_dev(ones_scale))
    torch.cuda.synchronize()
    assert np.all(y.cpu().numpy() == 0)


def test_gemv_canaries_and_empty_batch():
    n, k, b = 384, 640, 3
    codes, scales, x = _dense_inputs(n, k, b, seed=31)
    buf = torch.full((b * n + 128,), 12345.0, dtype=torch.float32, device=DEV)
    y = buf[64:64 + b * n].view(b, n)
    tb.tb_ternary_gemv(bf16_dev(x), u32_dev(codes), f16_dev(scales), y=y)
    torch.cuda.synchronize()
    assert torch.all(buf[:64] == 12345.0) and torch.all(buf[64 + b * n:] == 12345.0)
    assert_close(y.cpu().numpy(), oracle.matvec.gemv(x, codes, scales, k), "gemv canary run")
    e = torch.empty((0, k), dtype=torch.bfloat16, device=DEV)
    out = tb.tb_ternary_gemv(e, u32_dev(codes), f16_dev(scales))
    assert out.shape == (0, n)


# ------------------------------------------------------------------ 2:4

@pytest.mark.parametrize("n,k,b", [(128, 128, 1), (256, 384, 1), (1024, 1024, 1), (256, 640, 4), (128, 256, 16)])
def test_gemv24_small_matches_oracle(n, k, b):
    say(f"gemv24 N={n} K={k} B={b}")
    meta, signs = synth.random_24(n, k, seed=n + k)
    scales = synth.random_scales_f16(n, k, seed=3)
    x = synth.gaussian_bf16((b, k), seed=4)
    y = tb.tb_ternary24_gemv(bf16_dev(x), u32_dev(meta), u32_dev(signs), f16_dev(scales))
    torch.cuda.synchronize()
    ref = oracle.matvec.gemv24(x, meta, signs, scales, k)
    assert_close(y.cpu().numpy(), ref, f"gemv24 {n}x{k} B={b}")
    assert np.max(np.abs(y.cpu().numpy() - ref)) <= 1e-5 * np.max(np.abs(ref))


def test_gemv24_full_size_sampled():
    n, k = 17408, 5120
    say("gemv24 full 17408x5120 B=1")
    meta, signs = synth.random_24(n, k, seed=30)
    scales = synth.random_scales_f16(n, k, seed=31)
    x = synth.gaussian_bf16((1, k), seed=32)
    y = tb.tb_ternary24_gemv(bf16_dev(x), u32_dev(meta), u32_dev(signs), f16_dev(scales)).cpu().numpy()
    rows = np.sort(np.random.default_rng(3).choice(n, 256, replace=False))
    ref = oracle.matvec.gemv24(x, meta[rows], signs[rows], scales[rows], k)
    assert_close(y[:, rows], ref, "gemv24 17408x5120 (256 sampled rows)")


def test_gemv24_exact_and_dense_equivalence():
    n, k = 256, 1024
    meta, signs = synth.random_24(n, k, seed=40)
    x = synth.small_int_bf16((2, k), seed=41)
    sc = (2.0 ** np.random.default_rng(42).integers(-5, 2, size=(n, k // 128))).astype(np.float16).view(np.uint16)
    y24 = tb.tb_ternary24_gemv(bf16_dev(x), u32_dev(meta), u32_dev(signs), f16_dev(sc))
    i0, i1, n0, n1 = oracle.quant.unpack_24(meta, signs, k)
    dense = oracle.quant.pack_dense(oracle.quant.dense_from_24(i0, i1, n0, n1))
    yd = tb.tb_ternary_gemv(bf16_dev(x), u32_dev(dense), f16_dev(sc))
    torch.cuda.synchronize()
    ref = oracle.matvec.gemv24(x, meta, signs, sc, k)
    assert np.array_equal(y24.cpu().numpy().astype(np.float64), ref)
    assert np.array_equal(yd.cpu().numpy(), y24.cpu().numpy())
