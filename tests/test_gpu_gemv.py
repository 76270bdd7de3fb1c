"""GPU parity of tb_act8_prep + tb_ternary_gemv and of tb_ternary24_gemv
against the oracle."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import (DEV, act8_decode, act8_kept, assert_close, bf16_dev, f16_dev, say, u32_dev)
from ternary_weights_hadamard_amd import synth, tb

pytestmark = pytest.mark.gpu


def _dense_inputs(n, k, b, seed):
    codes = synth.random_code_words(n, k, seed=seed)
    scales = synth.random_scales_f16(n, k, seed=seed + 1)
    x = synth.gaussian_bf16((b, k), seed=seed + 2)
    return codes, scales, x


def _gemv(x_bits, codes, scales):
    act = tb.tb_act8_prep(bf16_dev(x_bits))
    y = tb.tb_ternary_gemv(act, u32_dev(codes), f16_dev(scales), x_bits.shape[0])
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("n,k", [(128, 128), (256, 384), (1024, 1024), (384, 2176)])
@pytest.mark.parametrize("b", [1, 2, 5, 8, 16])
def test_gemv_small_matches_oracle(n, k, b):
    say(f"gemv N={n} K={k} B={b}")
    codes, scales, x = _dense_inputs(n, k, b, seed=n + k + b)
    y = _gemv(x, codes, scales)
    ref = oracle.matvec.gemv(x, codes, scales, k)
    assert_close(y, ref, f"gemv {n}x{k} B={b}")
    # exact products, fp32 accumulation: far inside the bar
    assert np.max(np.abs(y - ref)) <= 1e-5 * np.max(np.abs(ref))


@pytest.mark.parametrize("n,k", [(5120, 5120), (17408, 5120), (5120, 17408), (15360, 5120)])
@pytest.mark.parametrize("b", [1, 4, 8, 16])
def test_gemv_full_size_sampled_tiles(n, k, b):
    say(f"gemv full N={n} K={k} B={b}")
    codes, scales, x = _dense_inputs(n, k, b, seed=20 + b)
    y = _gemv(x, codes, scales)
    tiles = np.sort(np.random.default_rng(1).choice(n // 16, 16, replace=False))
    rows = (16 * tiles[:, None] + np.arange(16)[None, :]).ravel()
    ref = oracle.matvec.gemv(x, codes[tiles], scales[tiles], k)
    assert_close(y[:, rows], ref, f"gemv {n}x{k} B={b} (16 sampled tiles)")
    assert np.max(np.abs(y[:, rows] - ref)) <= 1e-5 * np.max(np.abs(ref))


@pytest.mark.parametrize("n,k,b", [(128, 128, 1), (384, 2176, 3), (1024, 5120, 16), (512, 17408, 2), (256, 1152, 7)])
def test_gemv_bf16_entry_matches_oracle_and_the_act8_route(n, k, b):
    # the rotated activations as bf16: the call encodes them into the caller's
    # workspace and multiplies; the result is the act8 route's bit for bit
    say(f"gemv bf16 entry N={n} K={k} B={b}")
    codes, scales, x = _dense_inputs(n, k, b, seed=300 + n + b)
    xd, cd, sc = bf16_dev(x), u32_dev(codes), f16_dev(scales)
    ws = torch.full((tb.tb_act8_bytes(b, k) + 64,), 0x5A, dtype=torch.uint8, device=DEV)
    y = tb.tb_ternary_gemv(xd, cd, sc, workspace=ws[:tb.tb_act8_bytes(b, k)])
    act = tb.tb_act8_prep(xd)
    y_act = tb.tb_ternary_gemv(act, cd, sc, b)
    torch.cuda.synchronize()
    assert torch.equal(y, y_act), "bf16 entry differs from the act8 route"
    assert torch.equal(ws[:act.numel()], act), "workspace does not hold the encoded operand"
    assert torch.all(ws[act.numel():] == 0x5A), "encoding wrote past the workspace it needs"
    ref = oracle.matvec.gemv(x, codes, scales, k)
    got = y.cpu().numpy().astype(np.float64)
    assert_close(got, ref, f"gemv bf16 entry {n}x{k} B={b}")
    assert np.max(np.abs(got - ref)) <= 1e-5 * np.max(np.abs(ref))


def test_gemv_resid_bf16_entry_equals_the_act8_route():
    n, k, b = 768, 2176, 4
    codes = synth.random_code_words(n, 2 * k, seed=321)
    scales = synth.random_scales_f16(n, 2 * k, seed=322)
    x = synth.gaussian_bf16((b, k), seed=323)
    xd, cd, sc = bf16_dev(x), u32_dev(codes), f16_dev(scales)
    y = tb.tb_ternary_gemv_resid(xd, cd, sc)
    y_act = tb.tb_ternary_gemv_resid(tb.tb_act8_prep(xd), cd, sc, b)
    torch.cuda.synchronize()
    assert torch.equal(y, y_act)
    assert_close(y.cpu().numpy(), oracle.matvec.gemv_residual(x, codes, scales, k), "two-plane bf16 entry")


@pytest.mark.parametrize("b", [1, 3, 16])
def test_gemv_exact_small_integers(b):
    # integer activations and power-of-two scales: the exact result is an fp32 value
    n, k = 256, 1280
    codes = synth.random_code_words(n, k, seed=5)
    x = synth.small_int_bf16((b, k), seed=6)
    sc = (2.0 ** np.random.default_rng(7).integers(-6, 2, size=(n // 16, k // 128, 16))).astype(np.float16).view(np.uint16)
    y = _gemv(x, codes, sc)
    ref = oracle.matvec.gemv(x, codes, sc, k)
    assert np.array_equal(y, ref)


def test_gemv_special_patterns():
    n, k = 128, 256
    x = synth.gaussian_bf16((1, k), seed=9)
    xv = oracle.numerics.bf16_bits_to_f64(x)
    ones_scale = np.full((n // 16, k // 128, 16), np.float16(1.0).view(np.uint16), dtype=np.uint16)
    t = np.ones((n, k), dtype=np.int8)
    y = _gemv(x, oracle.quant.pack_dense(t), ones_scale)
    assert np.allclose(y, xv.sum(), rtol=1e-5)
    cols = np.random.default_rng(2).integers(0, k, size=n)
    t = np.zeros((n, k), dtype=np.int8)
    t[np.arange(n), cols] = -1
    y = _gemv(x, oracle.quant.pack_dense(t), ones_scale)
    assert np.array_equal(y[0], -xv[0, cols])
    t = np.zeros((n, k), dtype=np.int8)
    y = _gemv(x, oracle.quant.pack_dense(t), ones_scale)
    assert np.all(y == 0)


def test_gemv_canaries_and_empty_batch():
    n, k, b = 384, 640, 3
    codes, scales, x = _dense_inputs(n, k, b, seed=31)
    act = tb.tb_act8_prep(bf16_dev(x))
    y = torch.full((b + 1, n), 7.0, dtype=torch.float32, device=DEV)
    tb.tb_ternary_gemv(act, u32_dev(codes), f16_dev(scales), b, y=y[:b])
    torch.cuda.synchronize()
    assert torch.all(y[b] == 7.0), "GEMV wrote past its output"
    assert_close(y[:b].cpu().numpy(), oracle.matvec.gemv(x, codes, scales, k), "gemv canary run")
    out = tb.tb_ternary_gemv(act, u32_dev(codes), f16_dev(scales), 0)
    assert out.shape == (0, n)


# ---------------------------------------------------------------- act8 operand

def _act8_host(x_bits):
    b, k = x_bits.shape
    act = tb.tb_act8_prep(bf16_dev(x_bits))
    torch.cuda.synchronize()
    buf = act.cpu().numpy()
    assert buf.size == tb.tb_act8_bytes(b, k)
    return buf


@pytest.mark.parametrize("b,k", [(1, 128), (3, 640), (16, 5120)])
def test_act8_reconstructs_gaussian_activations_exactly(b, k):
    x = synth.gaussian_bf16((b, k), seed=b + k)
    rec = act8_decode(_act8_host(x), b, k)
    assert np.array_equal(rec, oracle.numerics.bf16_bits_to_f64(x))


def _wide_range_bf16(b, k, seed, span=60):
    """bf16 values with exponents spread uniformly over `span` binades, random
    signs, some exact zeros and subnormals."""
    rng = np.random.default_rng(seed)
    e = rng.integers(127 - span // 2, 127 + span // 2, size=(b, k))
    m = rng.integers(0, 128, size=(b, k))
    s = rng.integers(0, 2, size=(b, k))
    bits = ((s << 15) | (e << 7) | m).astype(np.uint16)
    bits[rng.random((b, k)) < 0.02] = 0
    sub = rng.random((b, k)) < 0.01
    bits[sub] = rng.integers(1, 128, size=int(sub.sum())).astype(np.uint16)  # subnormals
    return bits


def test_act8_wide_range_keeps_what_the_format_promises():
    b, k = 2, 2048
    x = _wide_range_bf16(b, k, seed=3)
    rec = act8_decode(_act8_host(x), b, k)
    kept = act8_kept(x)
    assert np.array_equal(rec, oracle.numerics.bf16_bits_to_f64(kept))
    # what is dropped is below 2^-20 of its block's largest magnitude
    xv = np.abs(oracle.numerics.bf16_bits_to_f64(x)).reshape(b, k // 32, 32)
    dropped = (kept != x).reshape(b, k // 32, 32)
    blockmax = xv.max(axis=2, keepdims=True)
    assert np.all(np.where(dropped, xv, 0.0) < 2.0 ** -20 * blockmax)
    say(f"  act8 wide range: {int(dropped.sum())} of {b * k} elements below the kept range")


def test_gemv_wide_range_activations_exact_on_kept_values():
    n, k, b = 512, 2048, 3
    codes = synth.random_code_words(n, k, seed=41)
    scales = synth.random_scales_f16(n, k, seed=42)
    x = _wide_range_bf16(b, k, seed=43, span=40)
    y = _gemv(x, codes, scales)
    # the product of the activations as given, at the float bar
    assert_close(y, oracle.matvec.gemv(x, codes, scales, k), "gemv wide-range activations")
    # and, tighter, the exact product of what the operand format represents
    ref = oracle.matvec.gemv(act8_kept(x), codes, scales, k)
    assert_close(y, ref, "gemv wide-range activations (oracle on kept values)")
    assert np.max(np.abs(y - ref)) <= 1e-5 * np.max(np.abs(ref))


def test_gemv_nonfinite_activation_poisons_only_its_batch_row():
    n, k, b = 256, 512, 3
    codes, scales, x = _dense_inputs(n, k, b, seed=51)
    x = x.copy()
    x[1, 200] = 0x7F80  # +inf
    y = _gemv(x, codes, scales)
    assert np.all(np.isnan(y[1])), "a non-finite activation must make its output row non-finite"
    ref = oracle.matvec.gemv(x[[0, 2]], codes, scales, k)
    assert_close(y[[0, 2]], ref, "gemv rows next to a non-finite row")


def test_act8_from_fwht_equals_prep_of_rotated_bf16():
    b, k = 5, 1152
    x = synth.gaussian_bf16((b, k), seed=61)
    xd = bf16_dev(x)
    fused = tb.tb_fwht128(xd, out_dtype=torch.uint8)
    rotated = tb.tb_fwht128(xd)
    prep = tb.tb_act8_prep(rotated)
    torch.cuda.synchronize()
    assert torch.equal(fused, prep)


# ---------------------------------------------------------------- 2:4

@pytest.mark.parametrize("n,k,b", [(128, 128, 1), (256, 384, 1), (1024, 1024, 1), (256, 640, 4), (128, 256, 16),
                                   (384, 2176, 2), (512, 17408, 1), (256, 1152, 3), (640, 5120, 4), (128, 5120, 6)])
def test_gemv24_small_matches_oracle(n, k, b):
    say(f"gemv24 N={n} K={k} B={b}")
    meta, signs = synth.random_24(n, k, seed=n + k)
    scales = synth.random_scales24_f16(n, k, seed=3)
    x = synth.gaussian_bf16((b, k), seed=4)
    y = tb.tb_ternary24_gemv(bf16_dev(x), u32_dev(meta), u32_dev(signs), f16_dev(scales))
    torch.cuda.synchronize()
    ref = oracle.matvec.gemv24(x, meta, signs, scales, k)
    assert_close(y.cpu().numpy(), ref, f"gemv24 {n}x{k} B={b}")
    assert np.max(np.abs(y.cpu().numpy() - ref)) <= 1e-5 * np.max(np.abs(ref))


@pytest.mark.parametrize("n,k", [(17408, 5120), (5120, 17408)])
def test_gemv24_full_size_sampled(n, k):
    say(f"gemv24 full {n}x{k} B=1")
    meta, signs = synth.random_24(n, k, seed=30)
    scales = synth.random_scales24_f16(n, k, seed=31)
    x = synth.gaussian_bf16((1, k), seed=32)
    y = tb.tb_ternary24_gemv(bf16_dev(x), u32_dev(meta), u32_dev(signs), f16_dev(scales)).cpu().numpy()
    tiles = np.sort(np.random.default_rng(3).choice(n // 16, 16, replace=False))
    rows = (16 * tiles[:, None] + np.arange(16)[None, :]).ravel()
    ref = oracle.matvec.gemv24(x, meta[tiles], signs[tiles], scales[tiles], k)
    assert_close(y[:, rows], ref, f"gemv24 {n}x{k} (16 sampled tiles)")


def test_gemv24_exact_and_dense_equivalence():
    n, k = 256, 1024
    meta, signs = synth.random_24(n, k, seed=40)
    x = synth.small_int_bf16((2, k), seed=41)
    # power-of-two scales by row and group, in each format's stored order
    sc_rows = (2.0 ** np.random.default_rng(42).integers(-5, 2, size=(n, k // 128))).astype(np.float16).view(np.uint16)
    meta_r, signs_r, _ = oracle.quant.load_24(meta, signs, synth.random_scales24_f16(n, k, seed=43), k)
    meta, signs, sc = oracle.quant.store_24(meta_r, signs_r, sc_rows)
    y24 = tb.tb_ternary24_gemv(bf16_dev(x), u32_dev(meta), u32_dev(signs), f16_dev(sc))
    i0, i1, n0, n1 = oracle.quant.unpack_24(meta_r, signs_r, k)
    dense = oracle.quant.pack_dense(oracle.quant.dense_from_24(i0, i1, n0, n1))
    yd = tb.tb_ternary_gemv(tb.tb_act8_prep(bf16_dev(x)), u32_dev(dense), f16_dev(oracle.quant.tile_scales(sc_rows)),
                            x.shape[0])
    torch.cuda.synchronize()
    ref = oracle.matvec.gemv24(x, meta, signs, sc, k)
    assert np.array_equal(y24.cpu().numpy().astype(np.float64), ref)
    assert np.array_equal(yd.cpu().numpy(), y24.cpu().numpy())


# ---------------------------------------------------------------- grouped launches

@pytest.mark.parametrize("b", [1, 3, 8])
def test_grouped_fwht_and_gemv_equal_single_calls(b):
    # shapes with different K-slice counts in one launch (G = 40, 5, 17, 136)
    shapes = [(1920, 5120), (640, 640), (768, 2176), (128, 17408)]
    say(f"grouped fwht + gemv, B={b}")
    xs, segs, singles = [], [], []
    for c, (n, k) in enumerate(shapes):
        codes = synth.random_code_words(n, k, seed=70 + c)
        scales = synth.random_scales_f16(n, k, seed=80 + c)
        x = synth.gaussian_bf16((b, k), seed=90 + c)
        xs.append((bf16_dev(x), u32_dev(codes), f16_dev(scales), x, codes, scales))
    acts = [torch.empty(tb.tb_act8_bytes(b, x.shape[1]), dtype=torch.uint8, device=DEV) for _, _, _, x, _, _ in xs]
    tb.tb_fwht128_multi([(xd, a) for (xd, *_), a in zip(xs, acts)])
    ys = [torch.empty((b, n), dtype=torch.float32, device=DEV) for n, _ in shapes]
    tb.tb_ternary_gemv_multi([(a, cd, sc, b, y) for a, (_, cd, sc, *_), y in zip(acts, xs, ys)])
    torch.cuda.synchronize()
    for c, ((xd, cd, sc, x, codes, scales), a, y) in enumerate(zip(xs, acts, ys)):
        a1 = tb.tb_fwht128(xd, out_dtype=torch.uint8)
        y1 = tb.tb_ternary_gemv(a1, cd, sc, b)
        torch.cuda.synchronize()
        assert torch.equal(a, a1), f"segment {c}: grouped rotation differs from the single call"
        assert torch.equal(y, y1), f"segment {c}: grouped GEMV differs from the single call"
        k = x.shape[1]
        xr = oracle.numerics.f64_to_bf16_bits(oracle.hadamard.fwht_dense(oracle.numerics.bf16_bits_to_f64(x)))
        assert_close(y.cpu().numpy(), oracle.matvec.gemv(xr, codes, scales, k), f"grouped segment {c} vs oracle")


@pytest.mark.parametrize("batches", [(2, 5, 8, 16), (1, 2, 5, 8)])
def test_grouped_mixed_batches_equal_single_calls(batches):
    # segments of different batch sizes in one call: one wide launch sized for
    # the largest batch (tiles per wave chosen for the whole launch), or, with a
    # batch-1 segment among them, one launch per segment; either way every
    # segment equals its single call bit for bit and matches the oracle
    shapes = [(1920, 5120), (640, 640), (768, 2176), (256, 17408)]
    say(f"grouped gemv, batches {batches}")
    segs, singles = [], []
    for c, ((n, k), b) in enumerate(zip(shapes, batches)):
        codes = synth.random_code_words(n, k, seed=270 + c)
        scales = synth.random_scales_f16(n, k, seed=280 + c)
        x = synth.gaussian_bf16((b, k), seed=290 + c)
        act = tb.tb_act8_prep(bf16_dev(x))
        cd, sc = u32_dev(codes), f16_dev(scales)
        y = torch.empty((b, n), dtype=torch.float32, device=DEV)
        segs.append((act, cd, sc, b, y))
        singles.append((x, codes, scales, k))
    tb.tb_ternary_gemv_multi(segs)
    torch.cuda.synchronize()
    for c, ((act, cd, sc, b, y), (x, codes, scales, k)) in enumerate(zip(segs, singles)):
        y1 = tb.tb_ternary_gemv(act, cd, sc, b)
        torch.cuda.synchronize()
        assert torch.equal(y, y1), f"segment {c} (B={b}): grouped differs from the single call"
        ref = oracle.matvec.gemv(x, codes, scales, k)
        assert_close(y.cpu().numpy(), ref, f"mixed-batch segment {c} (B={b}) vs oracle")
        assert np.max(np.abs(y.cpu().numpy() - ref)) <= 1e-5 * np.max(np.abs(ref))


@pytest.mark.parametrize("b", [8, 12])
def test_grouped_27b_layer_wide_batch(b):
    # the d_model-input projections of a 27B layer in one launch (QKV 15360,
    # O 5120, up 17408 rows; K = 5120): enough tiles that the launch takes
    # the most tiles per wave (8 at batch 8, 4 at batch 12); each single call
    # takes fewer.  Grouped and single results are equal bit for bit, and 16
    # sampled tiles of each match the oracle.
    shapes = [(15360, 5120), (5120, 5120), (17408, 5120)]
    say(f"grouped 27B layer, B={b}")
    rng = np.random.default_rng(b)
    segs, singles = [], []
    for c, (n, k) in enumerate(shapes):
        codes = synth.random_code_words(n, k, seed=370 + c)
        scales = synth.random_scales_f16(n, k, seed=380 + c)
        x = synth.gaussian_bf16((b, k), seed=390 + c)
        act = tb.tb_act8_prep(bf16_dev(x))
        cd, sc = u32_dev(codes), f16_dev(scales)
        y = torch.empty((b, n), dtype=torch.float32, device=DEV)
        segs.append((act, cd, sc, b, y))
        singles.append((x, codes, scales, k))
    tb.tb_ternary_gemv_multi(segs)
    torch.cuda.synchronize()
    for c, ((act, cd, sc, _, y), (x, codes, scales, k)) in enumerate(zip(segs, singles)):
        y1 = tb.tb_ternary_gemv(act, cd, sc, b)
        torch.cuda.synchronize()
        assert torch.equal(y, y1), f"segment {c}: grouped differs from the single call"
        n = codes.shape[0] * 16
        tiles = np.sort(rng.choice(n // 16, 16, replace=False))
        rows = (16 * tiles[:, None] + np.arange(16)[None, :]).ravel()
        ref = oracle.matvec.gemv(x, codes[tiles], scales[tiles], k)
        got = y.cpu().numpy().astype(np.float64)[:, rows]
        assert_close(got, ref, f"27B segment {c} B={b} (16 sampled tiles)")
        assert np.max(np.abs(got - ref)) <= 1e-5 * np.max(np.abs(ref))


@pytest.mark.parametrize("b,parts", [(1, (4, 4, 4, 4)), (8, (4, 4, 4, 8)), (3, (2, 1, 8, 4))])
def test_grouped_layer_with_parts_in_any_order(b, parts):
    # a layer's four products (K = 5120 three times, then 17408) in one launch,
    # each split into K parts, the way the decode step groups them: the launch
    # schedules the long-K product first, so the order of the segments must
    # change nothing; each segment equals its own single-segment call bit for
    # bit, and its parts add up to the oracle's product
    shapes = [(1920, 5120), (640, 5120), (2176, 5120), (640, 17408)]
    say(f"grouped layer with parts {parts}, B={b}")
    ins = []
    for c, (n, k) in enumerate(shapes):
        codes = synth.random_code_words(n, k, seed=470 + c)
        scales = synth.random_scales_f16(n, k, seed=480 + c)
        x = synth.gaussian_bf16((b, k), seed=490 + c)
        ins.append((tb.tb_act8_prep(bf16_dev(x)), u32_dev(codes), f16_dev(scales), x, codes, scales))

    def run(order):
        ys = [torch.full((p, b, n), float("nan"), dtype=torch.float32, device=DEV) for p, (n, _) in zip(parts, shapes)]
        tb.tb_ternary_gemv_multi([(ins[j][0], ins[j][1], ins[j][2], b, ys[j], 1, parts[j]) for j in order])
        torch.cuda.synchronize()
        return ys

    base = run([0, 1, 2, 3])
    for order in ([3, 2, 1, 0], [1, 3, 0, 2]):
        for c, (y0, y1) in enumerate(zip(base, run(order))):
            assert torch.equal(y0, y1), f"segment {c}: result depends on the segment order {order}"
    for c, ((act, cd, sc, x, codes, scales), p, (n, k)) in enumerate(zip(ins, parts, shapes)):
        y1 = torch.empty((p, b, n), dtype=torch.float32, device=DEV)
        tb.tb_ternary_gemv_multi([(act, cd, sc, b, y1, 1, p)])
        torch.cuda.synchronize()
        assert torch.equal(base[c], y1), f"segment {c}: grouped differs from the single call"
        got = base[c].cpu().numpy().astype(np.float64).sum(axis=0)
        assert_close(got, oracle.matvec.gemv(x, codes, scales, k), f"segment {c} parts summed vs oracle")


def test_grouped_output_rotation_f32():
    shapes = [(2, 384), (2, 17408), (2, 1024)]
    xs = [torch.randn(s, dtype=torch.float32, device=DEV) for s in shapes]
    ys = [torch.empty_like(x) for x in xs]
    tb.tb_fwht128_multi(list(zip(xs, ys)))
    torch.cuda.synchronize()
    for x, y in zip(xs, ys):
        assert torch.equal(y, tb.tb_fwht128(x))


# ---------------------------------------------------------------- K split into parts

def _parts_of(g, parts):
    # scale groups [floor(G p / parts), floor(G (p + 1) / parts)) of part p
    return [(g * p // parts, g * (p + 1) // parts) for p in range(parts)]


@pytest.mark.parametrize("n,k,parts", [(128, 1024, 2), (256, 17408, 4), (384, 5120, 8), (1024, 2176, 4),
                                       (128, 512, 4), (512, 20480, 8),
                                       # 272 groups: 32 short slices, 16 or 4 waves per part
                                       (256, 34816, 2), (128, 34816, 8),
                                       # 320 groups: past the batch-1 kernel's slices (batched kernel)
                                       (128, 40960, 4)])
def test_gemv_parts_are_the_oracle_over_their_k_ranges(n, k, parts):
    say(f"gemv parts N={n} K={k} parts={parts}")
    codes, scales, x = _dense_inputs(n, k, 1, seed=n + k + parts)
    act = tb.tb_act8_prep(bf16_dev(x))
    cd, sd = u32_dev(codes), f16_dev(scales)
    yp = torch.full((parts, 1, n), float("nan"), dtype=torch.float32, device=DEV)
    tb.tb_ternary_gemv_multi([(act, cd, sd, 1, yp, 1, parts)])
    torch.cuda.synchronize()
    got = yp.cpu().numpy().astype(np.float64)
    for p, (g0, g1) in enumerate(_parts_of(k // 128, parts)):
        ref = oracle.matvec.gemv(x[:, 128 * g0:128 * g1], codes[:, g0:g1], scales[:, g0:g1], 128 * (g1 - g0))
        assert_close(got[p], ref, f"part {p} of {parts} (groups {g0}..{g1})")
        assert np.max(np.abs(got[p] - ref)) <= 1e-5 * np.max(np.abs(ref))
    full = oracle.matvec.gemv(x, codes, scales, k)
    assert_close(got.sum(axis=0), full, f"sum of {parts} parts")
    # grouped with an unsplit product, each is bit for bit what it is alone
    codes2, scales2, x2 = _dense_inputs(256, 1024, 1, seed=5)
    act2 = tb.tb_act8_prep(bf16_dev(x2))
    y2 = torch.empty((1, 256), dtype=torch.float32, device=DEV)
    yp_g = torch.empty_like(yp)
    tb.tb_ternary_gemv_multi([(act2, u32_dev(codes2), f16_dev(scales2), 1, y2, 1), (act, cd, sd, 1, yp_g, 1, parts)])
    y2_alone = tb.tb_ternary_gemv(act2, u32_dev(codes2), f16_dev(scales2), 1)
    torch.cuda.synchronize()
    assert torch.equal(yp_g, yp) and torch.equal(y2, y2_alone)


@pytest.mark.parametrize("n,k,b,parts", [(256, 1024, 2, 2), (384, 5120, 8, 4), (128, 17408, 5, 8), (1024, 2176, 16, 4),
                                         (256, 768, 8, 4), (128, 1024, 3, 8)])
def test_gemv_parts_batched_are_the_oracle_over_their_k_ranges(n, k, b, parts):
    say(f"gemv parts N={n} K={k} B={b} parts={parts}")
    codes, scales, x = _dense_inputs(n, k, b, seed=n + k + b + parts)
    act = tb.tb_act8_prep(bf16_dev(x))
    yp = torch.full((parts, b, n), float("nan"), dtype=torch.float32, device=DEV)
    tb.tb_ternary_gemv_multi([(act, u32_dev(codes), f16_dev(scales), b, yp, 1, parts)])
    torch.cuda.synchronize()
    got = yp.cpu().numpy().astype(np.float64)
    for p, (g0, g1) in enumerate(_parts_of(k // 128, parts)):
        ref = oracle.matvec.gemv(x[:, 128 * g0:128 * g1], codes[:, g0:g1], scales[:, g0:g1], 128 * (g1 - g0))
        assert_close(got[p], ref, f"part {p} of {parts} (groups {g0}..{g1}), batch {b}")
        assert np.max(np.abs(got[p] - ref)) <= 1e-5 * np.max(np.abs(ref))


@pytest.mark.parametrize("parts", [2, 4, 8])
def test_gemv_parts_two_plane_down_projection(parts):
    # a 27B down projection's two planes at batch 1 (K = 17408: 272 code
    # groups, more than one workgroup's short slices): its parts add up to
    # the oracle's product
    n, k = 640, 17408
    say(f"two-plane gemv parts N={n} K={k} parts={parts}")
    codes = synth.random_code_words(n, 2 * k, seed=95 + parts)
    scales = synth.random_scales_f16(n, 2 * k, seed=96 + parts)
    x = synth.gaussian_bf16((1, k), seed=97 + parts)
    act = tb.tb_act8_prep(bf16_dev(x))
    yp = torch.full((parts, 1, n), float("nan"), dtype=torch.float32, device=DEV)
    tb.tb_ternary_gemv_multi([(act, u32_dev(codes), f16_dev(scales), 1, yp, 2, parts)])
    torch.cuda.synchronize()
    ref = oracle.matvec.gemv_residual(x, codes, scales, k)
    got = yp.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    assert_close(got.sum(axis=0), ref, f"two-plane down projection, {parts} parts summed")


def test_gemv_parts_two_planes_and_explicit_one():
    n, k, parts = 256, 5120, 4
    codes = synth.random_code_words(n, 2 * k, seed=91)
    scales = synth.random_scales_f16(n, 2 * k, seed=92)
    x = synth.gaussian_bf16((1, k), seed=93)
    act = tb.tb_act8_prep(bf16_dev(x))
    cd, sd = u32_dev(codes), f16_dev(scales)
    yp = torch.empty((parts, 1, n), dtype=torch.float32, device=DEV)
    tb.tb_ternary_gemv_multi([(act, cd, sd, 1, yp, 2, parts)])
    torch.cuda.synchronize()
    ref = oracle.matvec.gemv_residual(x, codes, scales, k)
    assert_close(yp.cpu().numpy().astype(np.float64).sum(axis=0), ref, "two-plane parts summed")
    # parts = 1 given explicitly is the unsplit product
    codes1, scales1, x1 = _dense_inputs(256, 17408, 1, seed=94)
    act1 = tb.tb_act8_prep(bf16_dev(x1))
    y1 = torch.empty((1, 256), dtype=torch.float32, device=DEV)
    tb.tb_ternary_gemv_multi([(act1, u32_dev(codes1), f16_dev(scales1), 1, y1, 1, 1)])
    y0 = tb.tb_ternary_gemv(act1, u32_dev(codes1), f16_dev(scales1), 1)
    torch.cuda.synchronize()
    assert torch.equal(y1, y0)


@pytest.mark.parametrize("parts", [2, 4, 8])
def test_rotation_sums_partial_inputs_in_order(parts):
    rows, k = 3, 5120
    xs = torch.randn((parts, rows, k), dtype=torch.float32, device=DEV)
    y = torch.empty((rows, k), dtype=torch.float32, device=DEV)
    yb = torch.empty((rows, k), dtype=torch.bfloat16, device=DEV)
    other = torch.randn((2, 1024), dtype=torch.float32, device=DEV)
    other_y = torch.empty_like(other)
    tb.tb_fwht128_multi([(xs, y, parts), (other, other_y), (xs, yb, parts)])
    # the parts added in part order in fp32, then the plain transform
    s = xs[0].clone()
    for p in range(1, parts):
        s = s + xs[p]
    torch.cuda.synchronize()
    assert torch.equal(y, tb.tb_fwht128(s))
    assert torch.equal(yb, tb.tb_fwht128(s, out_dtype=torch.bfloat16))
    assert torch.equal(other_y, tb.tb_fwht128(other))
    ref = oracle.hadamard.fwht_dense(xs.double().sum(dim=0).cpu().numpy())
    assert_close(y.cpu().numpy().astype(np.float64), ref, f"rotation of {parts} parts")


def test_split_down_projection_fused_with_its_rotation():
    # the decode step's use: the down projection split into 4 parts, its output
    # rotated back while the parts are added; against the oracle's product
    # followed by the transform
    n, k, parts = 5120, 17408, 4
    codes, scales, x = _dense_inputs(n, k, 1, seed=77)
    act = tb.tb_act8_prep(bf16_dev(x))
    yp = torch.empty((parts, 1, n), dtype=torch.float32, device=DEV)
    y = torch.empty((1, n), dtype=torch.float32, device=DEV)
    tb.tb_ternary_gemv_multi([(act, u32_dev(codes), f16_dev(scales), 1, yp, 1, parts)])
    tb.tb_fwht128_multi([(yp, y, parts)])
    torch.cuda.synchronize()
    tiles = np.sort(np.random.default_rng(78).choice(n // 16, 16, replace=False))
    blocks = np.unique(tiles // 8)  # the 128-blocks of N these tiles fall in
    cs = (128 * blocks[:, None] + np.arange(128)[None, :]).ravel()
    ts = np.unique(cs // 16)
    yprime = oracle.matvec.gemv(x, codes[ts], scales[ts], k)
    ref = oracle.hadamard.fwht_dense(yprime)
    assert_close(y.cpu().numpy().astype(np.float64)[:, cs], ref, "split down projection + rotation (sampled blocks)")


# ---------------------------------------------------------------- two-plane weights

def _gemv_resid(x_bits, codes, scales):
    act = tb.tb_act8_prep(bf16_dev(x_bits))
    y = tb.tb_ternary_gemv_resid(act, u32_dev(codes), f16_dev(scales), x_bits.shape[0])
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def _resid_inputs(n, k, b, seed):
    # both planes' codes and scales, groups interleaved: the dense format of [n, 2k]
    codes = synth.random_code_words(n, 2 * k, seed=seed)
    scales = synth.random_scales_f16(n, 2 * k, seed=seed + 1)
    x = synth.gaussian_bf16((b, k), seed=seed + 2)
    return codes, scales, x


@pytest.mark.parametrize("n,k", [(128, 128), (256, 384), (1024, 1024), (384, 2176)])
@pytest.mark.parametrize("b", [1, 3, 5, 16])
def test_gemv_resid_small_matches_oracle(n, k, b):
    say(f"two-plane gemv N={n} K={k} B={b}")
    codes, scales, x = _resid_inputs(n, k, b, seed=3 * n + k + b)
    y = _gemv_resid(x, codes, scales)
    ref = oracle.matvec.gemv_residual(x, codes, scales, k)
    assert_close(y, ref, f"two-plane gemv {n}x{k} B={b}")
    assert np.max(np.abs(y - ref)) <= 1e-5 * np.max(np.abs(ref))


@pytest.mark.parametrize("n,k", [(5120, 5120), (17408, 5120), (5120, 17408)])
@pytest.mark.parametrize("b", [1, 8])
def test_gemv_resid_full_size_sampled_tiles(n, k, b):
    say(f"two-plane gemv full N={n} K={k} B={b}")
    codes, scales, x = _resid_inputs(n, k, b, seed=40 + b)
    y = _gemv_resid(x, codes, scales)
    tiles = np.sort(np.random.default_rng(2).choice(n // 16, 12, replace=False))
    rows = (16 * tiles[:, None] + np.arange(16)[None, :]).ravel()
    ref = oracle.matvec.gemv_residual(x, codes[tiles], scales[tiles], k)
    assert_close(y[:, rows], ref, f"two-plane gemv {n}x{k} B={b} (12 sampled tiles)")
    assert np.max(np.abs(y[:, rows] - ref)) <= 1e-5 * np.max(np.abs(ref))


@pytest.mark.parametrize("b", [1, 4, 9])
def test_gemv_resid_exact_small_integers(b):
    n, k = 256, 1280
    codes = synth.random_code_words(n, 2 * k, seed=15)
    x = synth.small_int_bf16((b, k), seed=16)
    sc = (2.0 ** np.random.default_rng(17).integers(-6, 2, size=(n // 16, 2 * k // 128, 16))).astype(np.float16).view(np.uint16)
    y = _gemv_resid(x, codes, sc)
    assert np.array_equal(y, oracle.matvec.gemv_residual(x, codes, sc, k))


def test_gemv_resid_of_quantised_weights():
    # quantiser -> two-plane GEMV: closer to W' x' than the one-plane product
    n, k = 512, 1024
    w = synth.stack_weights(n, k, seed=44)
    x = synth.gaussian_bf16((2, k), seed=45)
    c2, _, s2 = tb.tb_quantize_pack(torch.from_numpy(w).to(DEV), fmt=tb.TB_FMT_DENSE_RESID)
    c1, _, s1 = tb.tb_quantize_pack(torch.from_numpy(w).to(DEV))
    act = tb.tb_act8_prep(bf16_dev(x))
    y2 = tb.tb_ternary_gemv_resid(act, c2, s2, 2)
    y1 = tb.tb_ternary_gemv(act, c1, s1, 2)
    torch.cuda.synchronize()
    exact = oracle.numerics.bf16_bits_to_f64(x) @ oracle.hadamard.rotate_blocks(w.astype(np.float64)).T
    e1 = np.linalg.norm(y1.cpu().numpy() - exact)
    e2 = np.linalg.norm(y2.cpu().numpy() - exact)
    say(f"  |y - W'x|: one plane {e1:.4e}, two planes {e2:.4e}")
    assert e2 < 0.75 * e1
    # and it is the oracle's product over the GPU's own planes
    assert_close(y2.cpu().numpy(), oracle.matvec.gemv_residual(x, c2.cpu().numpy().view(np.uint32),
                                                               s2.cpu().numpy().view(np.uint16), k), "quantised two-plane")


@pytest.mark.parametrize("b", [1, 3, 6])
def test_grouped_two_plane_and_mixed_equal_single_calls(b):
    # all two-plane, then one- and two-plane segments mixed in one call
    shapes = [(1920, 5120, 2), (640, 640, 2), (768, 2176, 2), (256, 17408, 2)]
    mixed = [(1920, 5120, 1), (640, 640, 2), (768, 2176, 1), (256, 17408, 2)]
    for case, spec in (("two-plane", shapes), ("mixed", mixed)):
        say(f"grouped {case} gemv, B={b}")
        segs, singles = [], []
        for c, (n, k, p) in enumerate(spec):
            codes = synth.random_code_words(n, p * k, seed=170 + c)
            scales = synth.random_scales_f16(n, p * k, seed=180 + c)
            x = synth.gaussian_bf16((b, k), seed=190 + c)
            act = tb.tb_act8_prep(bf16_dev(x))
            cd, sc = u32_dev(codes), f16_dev(scales)
            y = torch.empty((b, n), dtype=torch.float32, device=DEV)
            segs.append((act, cd, sc, b, y, p))
            singles.append((x, codes, scales, k, p))
        tb.tb_ternary_gemv_multi(segs)
        torch.cuda.synchronize()
        for c, ((act, cd, sc, _, y, p), (x, codes, scales, k, _)) in enumerate(zip(segs, singles)):
            y1 = tb.tb_ternary_gemv_resid(act, cd, sc, b) if p == 2 else tb.tb_ternary_gemv(act, cd, sc, b)
            torch.cuda.synchronize()
            assert torch.equal(y, y1), f"{case} segment {c}: grouped differs from the single call"
            ref = (oracle.matvec.gemv_residual if p == 2 else oracle.matvec.gemv)(x, codes, scales, k)
            assert_close(y.cpu().numpy(), ref, f"{case} segment {c} vs oracle")


# ---------------------------------------------------------------- grouped 2:4

@pytest.mark.parametrize("batches", [(1, 1, 1, 1), (2, 1, 4, 3), (1, 6, 2, 1)])
def test_grouped_24_matches_oracle(batches):
    # products of different K (G = 40, 5, 17, 3 and 136 groups: ragged blocks
    # included) and batches in one call; a batch past 4 makes the call launch
    # each product on its own
    shapes = [(1920, 5120), (640, 640), (768, 2176), (256, 17408)]
    if batches == (1, 1, 1, 1):
        shapes[1] = (512, 384)
    say(f"grouped gemv24, batches {batches}")
    segs, refs = [], []
    for c, ((n, k), b) in enumerate(zip(shapes, batches)):
        meta, signs = synth.random_24(n, k, seed=300 + c)
        scales = synth.random_scales24_f16(n, k, seed=310 + c)
        x = synth.gaussian_bf16((b, k), seed=320 + c)
        y = torch.full((b, n), float("nan"), dtype=torch.float32, device=DEV)
        segs.append((bf16_dev(x), u32_dev(meta), u32_dev(signs), f16_dev(scales), y))
        refs.append(oracle.matvec.gemv24(x, meta, signs, scales, k))
    tb.tb_ternary24_gemv_multi(segs)
    torch.cuda.synchronize()
    for c, ((*_, y), ref) in enumerate(zip(segs, refs)):
        assert_close(y.cpu().numpy(), ref, f"grouped 2:4 segment {c} vs oracle")
        assert np.max(np.abs(y.cpu().numpy() - ref)) <= 1e-5 * np.max(np.abs(ref))


def test_grouped_24_exact_equals_single_calls():
    # integer activations and power-of-two scales make every sum exact, so the
    # grouped launch (whatever K split it picks) equals the single calls and
    # the oracle bit for bit
    shapes = [(896, 5120), (384, 5120), (1152, 5120), (256, 17408)]
    segs, singles = [], []
    for c, (n, k) in enumerate(shapes):
        meta, signs = synth.random_24(n, k, seed=330 + c)
        rows = (2.0 ** np.random.default_rng(340 + c).integers(-6, 2, size=(n, k // 128))).astype(np.float16)
        m_r, s_r, _ = oracle.quant.load_24(meta, signs, synth.random_scales24_f16(n, k, seed=1), k)
        meta, signs, sc = oracle.quant.store_24(m_r, s_r, rows.view(np.uint16))
        x = synth.small_int_bf16((1, k), seed=350 + c)
        y = torch.empty((1, n), dtype=torch.float32, device=DEV)
        segs.append((bf16_dev(x), u32_dev(meta), u32_dev(signs), f16_dev(sc), y))
        singles.append((x, meta, signs, sc, k))
    say("grouped gemv24, exact sums")
    # a single segment is the single call bit for bit, whatever the sums
    xg = bf16_dev(synth.gaussian_bf16((1, 5120), seed=333))
    mg, sg_ = (u32_dev(a) for a in synth.random_24(896, 5120, seed=334))
    cg = f16_dev(synth.random_scales24_f16(896, 5120, seed=335))
    ya = torch.empty((1, 896), dtype=torch.float32, device=DEV)
    tb.tb_ternary24_gemv_multi([(xg, mg, sg_, cg, ya)])
    assert torch.equal(ya, tb.tb_ternary24_gemv(xg, mg, sg_, cg))
    tb.tb_ternary24_gemv_multi(segs)
    torch.cuda.synchronize()
    for c, ((xd, md, sd, cd, y), (x, meta, signs, sc, k)) in enumerate(zip(segs, singles)):
        y1 = tb.tb_ternary24_gemv(xd, md, sd, cd)
        torch.cuda.synchronize()
        assert torch.equal(y, y1), f"segment {c}: grouped differs from the single call"
        assert np.array_equal(y.cpu().numpy().astype(np.float64), oracle.matvec.gemv24(x, meta, signs, sc, k))


def test_grouped_24_27b_layer_sampled():
    # a 27B layer's four products (QKV 15360, O 5120, gate/up 34816 rows on
    # K = 5120; down 5120 rows on K = 17408) in one launch, batch 1, as the
    # 2:4 decode step runs them; 8 sampled tiles per product against the oracle
    shapes = [(15360, 5120), (5120, 5120), (34816, 5120), (5120, 17408)]
    say("grouped gemv24, 27B layer")
    segs, host = [], []
    for c, (n, k) in enumerate(shapes):
        meta, signs = synth.random_24(n, k, seed=360 + c)
        scales = synth.random_scales24_f16(n, k, seed=370 + c)
        x = synth.gaussian_bf16((1, k), seed=380 + c)
        segs.append((bf16_dev(x), u32_dev(meta), u32_dev(signs), f16_dev(scales),
                     torch.empty((1, n), dtype=torch.float32, device=DEV)))
        host.append((x, meta, signs, scales, k))
    tb.tb_ternary24_gemv_multi(segs)
    torch.cuda.synchronize()
    for c, ((*_, y), (x, meta, signs, scales, k)) in enumerate(zip(segs, host)):
        n = meta.shape[0] * 16
        tiles = np.sort(np.random.default_rng(390 + c).choice(n // 16, 8, replace=False))
        rows = (16 * tiles[:, None] + np.arange(16)[None, :]).ravel()
        ref = oracle.matvec.gemv24(x, meta[tiles], signs[tiles], scales[tiles], k)
        assert_close(y.cpu().numpy()[:, rows], ref, f"27B layer product {c} (8 sampled tiles)")
