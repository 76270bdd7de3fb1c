"""GPU parity of tb_ternary_gemm against the oracle (and against the GEMV)."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import DEV, assert_close, bf16_dev, f16_dev, host_f64, say, u32_dev
from ternary_weights_hadamard_amd import synth, tb

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("m,n,k", [(1, 128, 128), (7, 256, 384), (128, 128, 1024), (300, 384, 640), (257, 256, 256)])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_gemm_small_matches_oracle(m, n, k, out):
    say(f"gemm M={m} N={n} K={k} {out}")
    codes = synth.random_code_words(n, k, seed=m + n)
    scales = synth.random_scales_f16(n, k, seed=k)
    x = synth.gaussian_bf16((m, k), seed=m)
    y = tb.tb_ternary_gemm(bf16_dev(x), u32_dev(codes), f16_dev(scales),
                           out_dtype=torch.bfloat16 if out == "bf16" else torch.float32)
    torch.cuda.synchronize()
    ref = oracle.matvec.gemm(x, codes, scales, k)
    assert_close(host_f64(y), ref, f"gemm {m}x{n}x{k} {out}", out_bf16=out == "bf16")


@pytest.mark.parametrize("k,n", [(5120, 17408), (17408, 5120)])
def test_gemm_full_size_sampled(k, n):
    m = 2048
    say(f"gemm full M={m} K={k} N={n}")
    codes = synth.random_code_words(n, k, seed=40 if k == 5120 else 41)
    scales = synth.random_scales_f16(n, k, seed=43)
    x = synth.gaussian_bf16((m, k), seed=42)
    for out in (torch.bfloat16, torch.float32):
        y = host_f64(tb.tb_ternary_gemm(bf16_dev(x), u32_dev(codes), f16_dev(scales), out_dtype=out))
        rs = np.sort(np.random.default_rng(5).choice(m, 64, replace=False))
        tiles = np.sort(np.random.default_rng(6).choice(n // 16, 6, replace=False))
        cs = (16 * tiles[:, None] + np.arange(16)[None, :]).ravel()
        ref = oracle.matvec.gemm(x[rs], codes[tiles], scales[tiles], k)
        assert_close(y[np.ix_(rs, cs)], ref, f"gemm {m}x{n}x{k} {out} (64 rows x 6 tiles sampled)",
                     out_bf16=out == torch.bfloat16)
        del y


def test_gemm_exact_small_integers_and_gemv_agreement():
    m, n, k = 33, 256, 1024
    codes = synth.random_code_words(n, k, seed=50)
    x = synth.small_int_bf16((m, k), seed=51)
    sc = (2.0 ** np.random.default_rng(52).integers(-6, 2, size=(n // 16, k // 128, 16))).astype(np.float16).view(np.uint16)
    y = tb.tb_ternary_gemm(bf16_dev(x), u32_dev(codes), f16_dev(sc), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().astype(np.float64), oracle.matvec.gemm(x, codes, sc, k))
    # rows 0..7 through the GEMV give the same exact values
    yv = tb.tb_ternary_gemv(tb.tb_act8_prep(bf16_dev(x[:8])), u32_dev(codes), f16_dev(sc), 8)
    torch.cuda.synchronize()
    assert np.array_equal(yv.cpu().numpy(), y.cpu().numpy()[:8])


def test_gemm_tiny_and_wide_range_activations_exact():
    # bf16 activations far below the fp16 range (down to 2^-100) and up to
    # 2^20, times power-of-two scales: every product and every sum here is an
    # exact fp32 value, so the result must equal the oracle's exactly
    m, n, k = 40, 128, 512
    rng = np.random.default_rng(61)
    codes = synth.random_code_words(n, k, seed=60)
    e = rng.integers(-100, 20, size=(m, 1))          # one binade per row keeps the sums exact
    mant = rng.integers(-8, 9, size=(m, k))
    xv = mant.astype(np.float64) * np.exp2(e.astype(np.float64))
    x = oracle.numerics.f64_to_bf16_bits(xv)
    assert np.array_equal(oracle.numerics.bf16_bits_to_f64(x), xv)
    sc = (2.0 ** rng.integers(-6, 2, size=(n // 16, k // 128, 16))).astype(np.float16).view(np.uint16)
    y = tb.tb_ternary_gemm(bf16_dev(x), u32_dev(codes), f16_dev(sc), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().astype(np.float64), oracle.matvec.gemm(x, codes, sc, k))


@pytest.mark.parametrize("split", [False, True])
def test_gemm_zero_scale_groups(split):
    # scale groups with a zero scale add nothing: about a third of them at
    # random, every group of some columns, and the first or the last group of
    # others; N = 384 (half of the last 256-column tile) and 9 groups (an odd
    # count); the oracle's values, and exact zeros where every scale is zero
    m, n, k = 70, 384, 1152
    codes = synth.random_code_words(n, k, seed=90)
    sc = synth.random_scales_f16(n, k, seed=91).copy()  # [n / 16][groups][16]
    rng = np.random.default_rng(92)
    sc[rng.random(sc.shape) < 0.33] = 0
    sc[3, :, 5] = 0                              # column 53: every group
    sc[20, 0, :] = 0                             # columns 320..335: the first group
    sc[21, -1, :] = 0                            # columns 336..351: the last group
    x = synth.gaussian_bf16((m, k), seed=93)
    if split:
        y = tb.tb_ternary_gemm_splitk(bf16_dev(x), u32_dev(codes), f16_dev(sc), out_dtype=torch.float32)
    else:
        y = tb.tb_ternary_gemm(bf16_dev(x), u32_dev(codes), f16_dev(sc), out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = host_f64(y)
    assert_close(got, oracle.matvec.gemm(x, codes, sc, k), f"gemm with zero-scale groups (split {split})")
    assert np.all(got[:, 53] == 0.0)


def test_gemm_canaries_and_empty():
    m, n, k = 130, 128, 256
    codes = synth.random_code_words(n, k, seed=60)
    scales = synth.random_scales_f16(n, k, seed=61)
    x = synth.gaussian_bf16((m, k), seed=62)
    buf = torch.full((m * n + 256,), -9.0, dtype=torch.bfloat16, device=DEV)
    y = buf[128:128 + m * n].view(m, n)
    tb.tb_ternary_gemm(bf16_dev(x), u32_dev(codes), f16_dev(scales), y=y)
    torch.cuda.synchronize()
    assert torch.all(buf[:128] == -9.0) and torch.all(buf[128 + m * n:] == -9.0)
    assert_close(host_f64(y), oracle.matvec.gemm(x, codes, scales, k), "gemm canary run", out_bf16=True)
    e = tb.tb_ternary_gemm(torch.empty((0, k), dtype=torch.bfloat16, device=DEV), u32_dev(codes), f16_dev(scales))
    assert e.shape == (0, n)


# ---------------------------------------------------------------- split K (few activation rows)

@pytest.mark.parametrize("m,n,k", [(1, 256, 384), (17, 256, 640), (100, 384, 1280), (200, 128, 2176), (256, 256, 128)])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_gemm_splitk_small_matches_oracle(m, n, k, out):
    say(f"split-K gemm M={m} N={n} K={k} {out}")
    codes = synth.random_code_words(n, k, seed=m + 3 * n)
    scales = synth.random_scales_f16(n, k, seed=k + 1)
    x = synth.gaussian_bf16((m, k), seed=m + 7)
    ws_bytes = tb.tb_ternary_gemm_splitk_workspace(m, n, k)
    assert ws_bytes % (m * n * 4) == 0 and ws_bytes // (m * n * 4) <= min(16, k // 128)
    y = tb.tb_ternary_gemm_splitk(bf16_dev(x), u32_dev(codes), f16_dev(scales),
                                  out_dtype=torch.bfloat16 if out == "bf16" else torch.float32)
    torch.cuda.synchronize()
    ref = oracle.matvec.gemm(x, codes, scales, k)
    assert_close(host_f64(y), ref, f"split-K gemm {m}x{n}x{k} {out}", out_bf16=out == "bf16")


@pytest.mark.parametrize("m", [8, 16, 32, 64, 128, 256])
@pytest.mark.parametrize("n,k", [(5120, 5120), (17408, 5120), (5120, 17408)])
def test_gemm_splitk_mid_batch_sampled(m, n, k):
    say(f"split-K gemm mid-batch M={m} N={n} K={k}")
    codes = synth.random_code_words(n, k, seed=60 + m)
    scales = synth.random_scales_f16(n, k, seed=61)
    x = synth.gaussian_bf16((m, k), seed=62 + m)
    parts = tb.tb_ternary_gemm_splitk_workspace(m, n, k) // (m * n * 4)
    y = host_f64(tb.tb_ternary_gemm_splitk(bf16_dev(x), u32_dev(codes), f16_dev(scales), out_dtype=torch.float32))
    tiles = np.sort(np.random.default_rng(7).choice(n // 16, 6, replace=False))
    cs = (16 * tiles[:, None] + np.arange(16)[None, :]).ravel()
    ref = oracle.matvec.gemm(x, codes[tiles], scales[tiles], k)
    assert_close(y[:, cs], ref, f"split-K gemm {m}x{n}x{k} ({parts} splits, 6 tiles sampled)")


def test_gemm_splitk_exact_and_fallbacks():
    # small integers, power-of-two scales: every split's sum is exact, so the
    # split result equals the oracle and the one-pass GEMM bit for bit
    m, n, k = 48, 384, 2048
    codes = u32_dev(synth.random_code_words(n, k, seed=63))
    x_bits = synth.small_int_bf16((m, k), seed=64)
    sc = (2.0 ** np.random.default_rng(65).integers(-6, 2, size=(n // 16, k // 128, 16))).astype(np.float16).view(np.uint16)
    x, scales = bf16_dev(x_bits), f16_dev(sc)
    ref = oracle.matvec.gemm(x_bits, synth.random_code_words(n, k, seed=63), sc, k)
    parts = tb.tb_ternary_gemm_splitk_workspace(m, n, k) // (m * n * 4)
    assert parts > 1
    for out in (torch.float32, torch.bfloat16):
        y1 = tb.tb_ternary_gemm(x, codes, scales, out_dtype=out)
        ys = tb.tb_ternary_gemm_splitk(x, codes, scales, out_dtype=out)
        # a workspace with room for one partial only, and none: one pass
        small = torch.empty(m * n, dtype=torch.float32, device=DEV)
        yf = tb.tb_ternary_gemm_splitk(x, codes, scales, out_dtype=out, workspace=small)
        torch.cuda.synchronize()
        assert torch.equal(ys, y1) and torch.equal(yf, y1)
        if out == torch.float32:
            assert np.array_equal(host_f64(ys), ref)
    # canaries around y and the workspace
    wsb = tb.tb_ternary_gemm_splitk_workspace(m, n, k)
    wbuf = torch.full((wsb // 4 + 64,), 7.0, dtype=torch.float32, device=DEV)
    ws = wbuf[32:32 + wsb // 4]
    ybuf = torch.full((m * n + 64,), -5.0, dtype=torch.float32, device=DEV)
    y = ybuf[32:32 + m * n].view(m, n)
    tb.tb_ternary_gemm_splitk(x, codes, scales, y=y, workspace=ws)
    torch.cuda.synchronize()
    assert torch.all(wbuf[:32] == 7.0) and torch.all(wbuf[32 + wsb // 4:] == 7.0)
    assert torch.all(ybuf[:32] == -5.0) and torch.all(ybuf[32 + m * n:] == -5.0)
    assert np.array_equal(host_f64(y), ref)


# ---------------------------------------------------------------- mid-batch kernel (M <= 16)

# (n, k) chosen so the kernel runs with 1, 2, 4 and 8 waves per workgroup
# (K = 128, 384 -> G = 1, 3; N = 8448 -> more than 256 workgroups)
MID_SHAPES = [(128, 128), (256, 384), (384, 1280), (8448, 512), (1024, 2176)]


@pytest.mark.parametrize("m", [1, 2, 5, 15, 16])
@pytest.mark.parametrize("n,k", MID_SHAPES)
def test_gemm_mid_batch_matches_oracle(m, n, k):
    say(f"mid-batch gemm M={m} N={n} K={k}")
    codes = synth.random_code_words(n, k, seed=m + n + k)
    scales = synth.random_scales_f16(n, k, seed=k + 5)
    x = synth.gaussian_bf16((m, k), seed=m + 11)
    ref = oracle.matvec.gemm(x, codes, scales, k)
    cd, sd, xd = u32_dev(codes), f16_dev(scales), bf16_dev(x)
    for out in (torch.float32, torch.bfloat16):
        y = tb.tb_ternary_gemm(xd, cd, sd, out_dtype=out)
        ys = tb.tb_ternary_gemm_splitk(xd, cd, sd, out_dtype=out)
        torch.cuda.synchronize()
        assert_close(host_f64(y), ref, f"mid-batch gemm {m}x{n}x{k} {out}", out_bf16=out == torch.bfloat16)
        # the split-K entry point takes the same one-pass kernel for M <= 16
        assert torch.equal(ys, y)


def test_gemm_mid_batch_rows_independent_and_exact():
    # a row's result does not depend on how many rows share the launch, and
    # with small-integer activations and power-of-two scales every partial sum
    # is exact, so the result equals the oracle bit for bit
    n, k = 1024, 2176
    codes = synth.random_code_words(n, k, seed=70)
    sc = (2.0 ** np.random.default_rng(71).integers(-6, 2, size=(n // 16, k // 128, 16))).astype(np.float16).view(np.uint16)
    cd, sd = u32_dev(codes), f16_dev(sc)
    xi = synth.small_int_bf16((16, k), seed=72)
    y16 = tb.tb_ternary_gemm(bf16_dev(xi), cd, sd, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(host_f64(y16), oracle.matvec.gemm(xi, codes, sc, k))
    xg = synth.gaussian_bf16((16, k), seed=73)
    yg = tb.tb_ternary_gemm(bf16_dev(xg), cd, sd, out_dtype=torch.float32)
    for m, r0 in ((1, 0), (3, 5), (9, 7)):
        ym = tb.tb_ternary_gemm(bf16_dev(xg[r0:r0 + m]), cd, sd, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(ym, yg[r0:r0 + m]), (m, r0)


def test_gemm_mid_batch_wide_range_exact_and_canaries():
    # activations from 2^-100 to 2^20 (one binade per row keeps every sum exact)
    m, n, k = 16, 256, 1024
    rng = np.random.default_rng(74)
    codes = synth.random_code_words(n, k, seed=75)
    e = rng.integers(-100, 20, size=(m, 1))
    xv = rng.integers(-8, 9, size=(m, k)).astype(np.float64) * np.exp2(e.astype(np.float64))
    x = oracle.numerics.f64_to_bf16_bits(xv)
    sc = (2.0 ** rng.integers(-6, 2, size=(n // 16, k // 128, 16))).astype(np.float16).view(np.uint16)
    ybuf = torch.full((m * n + 256,), -7.0, dtype=torch.float32, device=DEV)
    y = ybuf[128:128 + m * n].view(m, n)
    tb.tb_ternary_gemm(bf16_dev(x), u32_dev(codes), f16_dev(sc), y=y)
    torch.cuda.synchronize()
    assert torch.all(ybuf[:128] == -7.0) and torch.all(ybuf[128 + m * n:] == -7.0)
    assert np.array_equal(host_f64(y), oracle.matvec.gemm(x, codes, sc, k))
    # M = 5 into a bf16 buffer: rows past M are never written
    m5 = 5
    bbuf = torch.full((16 * n + 256,), -3.0, dtype=torch.bfloat16, device=DEV)
    yb = bbuf[128:128 + m5 * n].view(m5, n)
    tb.tb_ternary_gemm(bf16_dev(x[:m5]), u32_dev(codes), f16_dev(sc), y=yb)
    torch.cuda.synchronize()
    assert torch.all(bbuf[:128] == -3.0) and torch.all(bbuf[128 + m5 * n:] == -3.0)
    assert_close(host_f64(yb), oracle.matvec.gemm(x[:m5], codes, sc, k), "mid-batch M=5 bf16", out_bf16=True)


# ---------------------------------------------------------------- output rotation fused

def _rotate_rows(y):
    return oracle.hadamard.fwht_dense(y)


@pytest.mark.parametrize("m,n,k", [(1, 128, 128), (7, 256, 384), (300, 384, 640), (64, 512, 2176)])
@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("split", [False, True])
def test_gemm_rotated_matches_oracle(m, n, k, out, split):
    say(f"rotated gemm M={m} N={n} K={k} {out} split={split}")
    codes = synth.random_code_words(n, k, seed=m + 5 * n)
    scales = synth.random_scales_f16(n, k, seed=k + 3)
    x = synth.gaussian_bf16((m, k), seed=m + 11)
    ws = None
    if split:
        wsb = tb.tb_ternary_gemm_splitk_workspace(m, n, k)
        ws = torch.empty(max(wsb // 4, 4), dtype=torch.float32, device=DEV)
    y = tb.tb_ternary_gemm_rotated(bf16_dev(x), u32_dev(codes), f16_dev(scales),
                                   out_dtype=torch.bfloat16 if out == "bf16" else torch.float32, workspace=ws)
    torch.cuda.synchronize()
    ref = _rotate_rows(oracle.matvec.gemm(x, codes, scales, k))
    assert_close(host_f64(y), ref, f"rotated gemm {m}x{n}x{k} {out}", out_bf16=out == "bf16")


@pytest.mark.parametrize("m,n,k", [(40, 384, 1280), (256, 5120, 5120)])
def test_gemm_rotated_equals_product_then_rotation(m, n, k):
    # the fused rotation is the same fp32 product and the same butterflies,
    # rounded once: bit for bit the two-call composition
    codes = u32_dev(synth.random_code_words(n, k, seed=71))
    scales = f16_dev(synth.random_scales_f16(n, k, seed=72))
    x = bf16_dev(synth.gaussian_bf16((m, k), seed=73))
    wsb = tb.tb_ternary_gemm_splitk_workspace(m, n, k)
    ws = torch.empty(max(wsb // 4, 4), dtype=torch.float32, device=DEV)
    for out in (torch.float32, torch.bfloat16):
        y1 = tb.tb_fwht128(tb.tb_ternary_gemm(x, codes, scales, out_dtype=torch.float32), out_dtype=out)
        yr = tb.tb_ternary_gemm_rotated(x, codes, scales, out_dtype=out)
        y2 = tb.tb_fwht128(tb.tb_ternary_gemm_splitk(x, codes, scales, out_dtype=torch.float32, workspace=ws),
                           out_dtype=out)
        yrs = tb.tb_ternary_gemm_rotated(x, codes, scales, out_dtype=out, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(yr, y1), f"one pass, {out}"
        assert torch.equal(yrs, y2), f"split K, {out}"


def test_gemm_rotated_full_size_sampled():
    m, k, n = 2048, 5120, 17408
    say(f"rotated gemm full M={m} K={k} N={n}")
    codes = synth.random_code_words(n, k, seed=74)
    scales = synth.random_scales_f16(n, k, seed=75)
    x = synth.gaussian_bf16((m, k), seed=76)
    y = host_f64(tb.tb_ternary_gemm_rotated(bf16_dev(x), u32_dev(codes), f16_dev(scales)))
    rs = np.sort(np.random.default_rng(8).choice(m, 48, replace=False))
    blocks = np.sort(np.random.default_rng(9).choice(n // 128, 2, replace=False))
    tiles = (8 * blocks[:, None] + np.arange(8)[None, :]).ravel()
    cs = (128 * blocks[:, None] + np.arange(128)[None, :]).ravel()
    ref = _rotate_rows(oracle.matvec.gemm(x[rs], codes[tiles], scales[tiles], k))
    assert_close(y[np.ix_(rs, cs)], ref, "rotated gemm (48 rows x 2 column blocks sampled)", out_bf16=True)


# ---------------------------------------------------------------- grouped products (tb_ternary_gemm_multi)

@pytest.mark.parametrize("ms", [(16, 16, 16, 16), (1, 7, 16, 3), (16, 40, 2, 5)])
def test_gemm_multi_matches_oracle(ms):
    # products of different K (G = 40, 5, 17, 136 groups) and row counts in one
    # call, bf16 and fp32 outputs; an M past 16 makes the call launch each
    # product on its own
    shapes = [(1920, 5120), (640, 640), (768, 2176), (256, 17408)]
    say(f"gemm multi, M = {ms}")
    segs, refs = [], []
    for c, ((n, k), m) in enumerate(zip(shapes, ms)):
        codes = synth.random_code_words(n, k, seed=500 + c)
        scales = synth.random_scales_f16(n, k, seed=510 + c)
        x = synth.gaussian_bf16((m, k), seed=520 + c)
        out = torch.bfloat16 if c % 2 else torch.float32
        y = torch.full((m, n), float("nan"), dtype=out, device=DEV)
        segs.append((bf16_dev(x), u32_dev(codes), f16_dev(scales), y))
        refs.append(oracle.matvec.gemm(x, codes, scales, k))
    tb.tb_ternary_gemm_multi(segs)
    torch.cuda.synchronize()
    for c, ((*_, y), ref) in enumerate(zip(segs, refs)):
        assert_close(host_f64(y), ref, f"gemm multi segment {c}", out_bf16=y.dtype == torch.bfloat16)


def test_gemm_multi_single_segment_and_exact_sums():
    # integer activations and power-of-two scales make every sum exact, so a
    # grouped launch (four tiles per workgroup, its own K slices and starting
    # groups) equals the single calls and the oracle bit for bit
    shapes = [(1536, 5120), (512, 5120), (3456, 5120), (512, 17408)]
    segs, host = [], []
    for c, (n, k) in enumerate(shapes):
        codes = synth.random_code_words(n, k, seed=530 + c)
        sc = (2.0 ** np.random.default_rng(540 + c).integers(-6, 2, size=(n // 16, k // 128, 16))).astype(np.float16)
        sc = sc.view(np.uint16)
        x = synth.small_int_bf16((16, k), seed=550 + c)
        segs.append((bf16_dev(x), u32_dev(codes), f16_dev(sc), torch.empty((16, n), dtype=torch.float32, device=DEV)))
        host.append((x, codes, sc, k))
    say("gemm multi, single segment and exact sums")
    # a single segment is the single call bit for bit, whatever the sums
    xg = bf16_dev(synth.gaussian_bf16((16, 5120), seed=536))
    cg = u32_dev(synth.random_code_words(1024, 5120, seed=537))
    sg_ = f16_dev(synth.random_scales_f16(1024, 5120, seed=538))
    ya = torch.empty((16, 1024), dtype=torch.float32, device=DEV)
    tb.tb_ternary_gemm_multi([(xg, cg, sg_, ya)])
    assert torch.equal(ya, tb.tb_ternary_gemm(xg, cg, sg_, out_dtype=torch.float32))
    tb.tb_ternary_gemm_multi(segs)
    torch.cuda.synchronize()
    for c, ((xd, cd, sd, y), (x, codes, sc, k)) in enumerate(zip(segs, host)):
        y1 = tb.tb_ternary_gemm(xd, cd, sd, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(y, y1), f"segment {c}: grouped differs from the single call"
        assert np.array_equal(y.cpu().numpy().astype(np.float64), oracle.matvec.gemm(x, codes, sc, k))


def test_gemm_multi_27b_layer_m16_sampled():
    # a 27B layer's four products at M = 16 in one launch (QKV 15360, O 5120,
    # gate/up 34816 rows on K = 5120; down 5120 rows on K = 17408), as the
    # batch-16 decode step runs them; 6 sampled tiles per product
    shapes = [(15360, 5120), (5120, 5120), (34816, 5120), (5120, 17408)]
    say("gemm multi, 27B layer at M = 16")
    segs, host = [], []
    for c, (n, k) in enumerate(shapes):
        codes = synth.random_code_words(n, k, seed=560 + c)
        scales = synth.random_scales_f16(n, k, seed=570 + c)
        x = synth.gaussian_bf16((16, k), seed=580 + c)
        segs.append((bf16_dev(x), u32_dev(codes), f16_dev(scales),
                     torch.empty((16, n), dtype=torch.float32, device=DEV)))
        host.append((x, codes, scales, k))
    tb.tb_ternary_gemm_multi(segs)
    torch.cuda.synchronize()
    for c, ((*_, y), (x, codes, scales, k)) in enumerate(zip(segs, host)):
        n = codes.shape[0] * 16
        tiles = np.sort(np.random.default_rng(590 + c).choice(n // 16, 6, replace=False))
        cols = (16 * tiles[:, None] + np.arange(16)[None, :]).ravel()
        ref = oracle.matvec.gemm(x, codes[tiles], scales[tiles], k)
        assert_close(host_f64(y)[:, cols], ref, f"27B layer product {c} at M = 16 (6 sampled tiles)")
