"""GPU parity of tb_quantize_pack (dense and 2:4) against the oracle."""

import numpy as np
import pytest
import scipy.linalg
import torch

import oracle
from gpu_util import DEV, check_24_planes, check_dense_codes, f32_dev, host_u16, host_u32, say
from ternary_weights_hadamard_amd import synth, tb

pytestmark = pytest.mark.gpu

H = scipy.linalg.hadamard(128).astype(np.float64)


def _quant(w, fmt=tb.TB_FMT_DENSE, flag=None):
    codes, meta, scales = tb.tb_quantize_pack(f32_dev(w), fmt=fmt, err_flag=flag)
    torch.cuda.synchronize()
    return codes, meta, scales


def test_single_layer_1024_seed0():
    # 1024 x 1024, N(0, 0.02^2) with 0.1 % outliers x20, seed 0
    w = synth.single_layer_weights(1024, 1024, seed=0)
    say("quantize 1024x1024 seed 0")
    codes, _, scales = _quant(w)
    ref = oracle.quant.quantize_dense(w.astype(np.float64))
    check_dense_codes(codes, scales, ref, 1024, "1024^2")


@pytest.mark.parametrize("n,k,seed", [(128, 128, 1), (256, 384, 2), (384, 1280, 3), (640, 256, 4)])
def test_ragged_block_grids(n, k, seed):
    w = synth.stack_weights(n, k, seed=seed)
    say(f"quantize {n}x{k} seed {seed}")
    codes, _, scales = _quant(w)
    check_dense_codes(codes, scales, oracle.quant.quantize_dense(w.astype(np.float64)), k, f"{n}x{k}")


def test_full_layer_sampled_blocks():
    # a 27B down projection, 5120 x 17408, with heavy-tailed outlier input
    # channels (the stack recipe), quantised in one launch as the stack
    # benchmark does; 16 sampled 128 x 128 blocks checked against the oracle
    # run on each block alone (blocks are independent)
    n, k = 5120, 17408
    w = synth.stack_weights(n, k, seed=21)
    say(f"quantize full layer {n}x{k}")
    codes, _, scales = _quant(w)
    rng = np.random.default_rng(22)
    picks = list(zip(rng.integers(0, n // 128, 16), rng.integers(0, k // 128, 16)))
    # an outlier column's block is among them
    cols = np.nonzero(np.max(np.abs(w), axis=0) > 0.2)[0]
    picks[0] = (0, int(cols[0]) // 128)
    for a, b in picks:
        wb = w[128 * a:128 * (a + 1), 128 * b:128 * (b + 1)]
        ref = oracle.quant.quantize_dense(wb.astype(np.float64))
        cb = codes[8 * a:8 * (a + 1), b:b + 1, :].contiguous()
        sb = scales[8 * a:8 * (a + 1), b:b + 1].contiguous()
        check_dense_codes(cb, sb, ref, 128, f"block ({a}, {b})")


def test_closed_form_blocks():
    w = np.zeros((256, 512), dtype=np.float32)
    w[3, 9] = 4.0                    # spike in block (0,0): lossless, all codes +-1
    w[128:256, 128:256] = np.eye(128, dtype=np.float32)  # identity block
    w[:128, 256:384] = 0.375         # constant block
    # block (1, 3) stays zero
    codes, _, scales = _quant(w)
    ref = oracle.quant.quantize_dense(w.astype(np.float64))
    check_dense_codes(codes, scales, ref, 512, "closed forms")
    t = oracle.quant.unpack_dense(host_u32(codes), 512)
    assert np.array_equal(t, ref["t"])
    s = oracle.quant.untile_scales(host_u16(scales))
    assert np.all(s[:128, 0] == np.float16(4.0 / 128).view(np.uint16))
    assert np.all(s[128:, 1] == np.float16(1.0 / 128).view(np.uint16))
    assert s[0, 2] == np.float16(0.375).view(np.uint16) and np.all(s[1:128, 2] == 0)
    assert np.all(s[128:, 3] == 0) and np.all(host_u32(codes)[128:, 24:32] == 0)


def test_tie_at_half_scale():
    wr = np.zeros((128, 128))
    wr[0, :48] = 1.0
    wr[0, 48:112] = 0.25
    w = (H @ wr @ H / 128).astype(np.float32)
    codes, _, scales = _quant(w)
    t = oracle.quant.unpack_dense(host_u32(codes), 128)
    assert np.all(t[0, :48] == 1) and np.all(t[0, 48:] == 0)
    assert host_u16(scales)[0, 0, 0] == np.float16(0.5).view(np.uint16)


def test_error_flags():
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    w = np.zeros((128, 256), dtype=np.float32)
    w[5, 200] = np.nan
    _quant(w, flag=flag)
    assert int(flag.item()) & tb.TB_EFLAG_NONFINITE
    # every rule, NaN and both infinities, in a block of otherwise ordinary weights
    for fmt in (tb.TB_FMT_DENSE, tb.TB_FMT_24, tb.TB_FMT_DENSE_MINERR, tb.TB_FMT_DENSE_RESID):
        for bad in (np.nan, np.inf, -np.inf):
            w = synth.stack_weights(128, 256, seed=7)
            w[77, 3] = bad
            flag.zero_()
            _quant(w, fmt=fmt, flag=flag)
            assert int(flag.item()) & tb.TB_EFLAG_NONFINITE, (fmt, bad)
    flag.zero_()
    w = np.full((128, 128), 1.0e5, dtype=np.float32)  # row 0 scale = 1e5 > fp16 max
    _quant(w, flag=flag)
    assert int(flag.item()) & tb.TB_EFLAG_SCALE_OVF
    flag.zero_()
    _quant(synth.stack_weights(128, 128, seed=5), flag=flag)
    assert int(flag.item()) == 0


def test_output_canaries():
    n, k = 256, 256
    w = synth.stack_weights(n, k, seed=6)
    cb = torch.full((n * k // 16 + 8,), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    sb = torch.full((n * k // 128 + 16,), -3.0, dtype=torch.float16, device=DEV)
    codes = cb[4:4 + n * k // 16].view(n // 16, k // 128, 128)
    scales = sb[8:8 + n * k // 128].view(n // 16, k // 128, 16)
    tb.tb_quantize_pack(f32_dev(w), codes=codes, scales=scales)
    torch.cuda.synchronize()
    assert torch.all(cb[:4] == 0x5A5A5A5A) and torch.all(cb[4 + n * k // 16:] == 0x5A5A5A5A)
    assert torch.all(sb[:8] == -3.0) and torch.all(sb[8 + n * k // 128:] == -3.0)
    check_dense_codes(codes, scales, oracle.quant.quantize_dense(w.astype(np.float64)), k, "canary run")


@pytest.mark.parametrize("n,k,seed", [(128, 128, 11), (256, 512, 12), (1024, 1024, 0), (256, 384, 13),
                                      (128, 1664, 14)])
def test_24_matches_oracle(n, k, seed):
    # K = 128, 384 and 1664 leave the last block of four groups 3, 1 and 3
    # groups short: those stored groups must come back zero (the buffers start
    # filled with another pattern)
    w = synth.single_layer_weights(n, k, seed=seed) if seed == 0 else synth.stack_weights(n, k, seed=seed)
    say(f"quantize 2:4 {n}x{k}")
    g4 = -(-k // 512)
    signs = torch.full((n // 16, g4, 64, 2), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    meta = torch.full((n // 16, g4, 64, 4), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    scales = torch.full((n // 16, g4, 4, 4, 4), -3.0, dtype=torch.float16, device=DEV)
    tb.tb_quantize_pack(f32_dev(w), fmt=tb.TB_FMT_24, codes=signs, meta=meta, scales=scales)
    torch.cuda.synchronize()
    ref = oracle.quant.quantize_24(w.astype(np.float64))
    check_24_planes(meta, signs, scales, ref, k, f"2:4 {n}x{k}")
    pad = 4 * g4 - k // 128
    if pad:
        first = 4 - pad  # first padded group of the last block
        assert torch.all(meta[:, -1, :, first:] == 0)
        assert np.all(host_u16(scales[:, -1, :, first:, :]) == 0)
        halves = torch.from_numpy(host_u32(signs[:, -1]).astype(np.int64)).view(n // 16, 64, 2)
        fields = torch.stack([halves & 0xFFFF, halves >> 16], dim=-1).view(n // 16, 64, 4)
        assert torch.all(fields[:, :, first:] == 0)


def test_24_full_layer_sampled_blocks():
    # the 2:4 shape of the 27B up projection, 17408 x 5120, stack recipe, one
    # launch; 16 sampled 128 x 128 blocks against the oracle run on each block
    n, k = 17408, 5120
    w = synth.stack_weights(n, k, seed=23)
    say(f"quantize 2:4 full layer {n}x{k}")
    signs, meta, scales = _quant(w, fmt=tb.TB_FMT_24)
    rng = np.random.default_rng(24)
    for a, b in zip(rng.integers(0, n // 128, 16), rng.integers(0, k // 128, 16)):
        rows = slice(128 * a, 128 * (a + 1))
        ref = oracle.quant.quantize_24(w[rows, 128 * b:128 * (b + 1)].astype(np.float64))
        tiles = slice(8 * a, 8 * (a + 1))  # the block's eight 16-row tiles
        # group b of those tiles as the stored planes of a K = 128 matrix (through the oracle's layout)
        m_r, s_r, sc_r = oracle.quant.load_24(host_u32(meta[tiles]), host_u32(signs[tiles]), host_u16(scales[tiles]), k)
        mb, gb, sb = oracle.quant.store_24(m_r[:, 4 * b:4 * b + 4], s_r[:, 2 * b:2 * b + 2], sc_r[:, b:b + 1])
        check_24_planes(torch.from_numpy(mb.view(np.int32)), torch.from_numpy(gb.view(np.int32)),
                        torch.from_numpy(sb.view(np.int16)).view(torch.float16), ref, 128, f"block ({a}, {b})")


# ---------------------------------------------------------------- error-minimising rule

def _check_minerr(codes, scales, w, what):
    """Codes and scales of TB_FMT_DENSE_MINERR against the oracle.  Groups whose
    best and second-best thresholds are within float rounding (near ties) may
    take either: for them the GPU's kept set must be threshold-shaped and its
    float64 objective within 1e-5 of the best.  Elsewhere codes are bit-exact
    except elements within 1e-5 of the threshold; scales equal or 1 ulp."""
    ref = oracle.quant.quantize_dense_mse(w.astype(np.float64))
    n, k = w.shape
    wr = ref["wr"]
    t_gpu = oracle.quant.unpack_dense(host_u32(codes), k)
    tie = oracle.quant.near_tie_mse(wr)                                # [n, k/128]
    near = oracle.quant.near_threshold_mse(wr, ref["theta"])           # [n, k]
    tie_el = np.repeat(tie, 128, axis=1)
    bad = (t_gpu != ref["t"]) & ~near & ~tie_el
    # every kept element's sign agrees with W'
    assert np.all((t_gpu == 0) | (np.sign(wr) == t_gpu) | (np.abs(wr) <= 1e-12)), f"{what}: sign of a kept element"
    # near-tie groups: threshold-shaped and near-optimal
    a = np.abs(wr).reshape(n, k // 128, 128)
    kept = (t_gpu != 0).reshape(n, k // 128, 128)
    j = kept.sum(axis=2)
    S = np.where(kept, a, 0).sum(axis=2)
    obj = np.where(j > 0, S * S / np.maximum(j, 1), 0.0)
    _, jb, Sb = oracle.quant.mse_threshold(a)
    best = Sb * Sb / jb
    lo_kept = np.where(kept, a, np.inf).min(axis=2)
    hi_drop = np.where(~kept & (a > 0), a, 0).max(axis=2)
    shaped = lo_kept >= hi_drop * (1 - 1e-5)
    near_opt = obj >= best * (1 - 1e-5)
    sg = oracle.quant.untile_scales(host_u16(scales)).astype(np.int64)
    sr = oracle.quant.untile_scales(ref["scales"]).astype(np.int64)
    s_ok = np.abs(sg - sr) <= 1
    # in near-tie groups the scale belongs to the GPU's own kept set
    own = oracle.numerics.f64_to_f16_bits(np.where(j > 0, S / np.maximum(j, 1), 0.0)).astype(np.int64)
    s_ok_tie = np.abs(sg - own) <= 1
    say(f"  {what}: {int(tie.sum())} near-tie groups of {tie.size}, {int(near.sum())} near-threshold elements, "
        f"{int(bad.sum())} mismatches elsewhere")
    assert not bad.any(), f"{what}: {int(bad.sum())} code mismatches outside near ties and the threshold band"
    assert np.all(shaped | (j == 0)), f"{what}: a kept set that is not threshold-shaped"
    assert np.all(near_opt[tie]), f"{what}: a near-tie group more than 1e-5 from the best objective"
    assert np.all(s_ok[~tie]) and np.all(s_ok_tie[tie]), f"{what}: scale beyond 1 ulp"
    return ref


@pytest.mark.parametrize("n,k,seed", [(128, 128, 11), (256, 384, 12), (1024, 1024, 0), (384, 1280, 13)])
def test_minerr_matches_oracle(n, k, seed):
    w = synth.single_layer_weights(n, k, seed=seed) if seed == 0 else synth.stack_weights(n, k, seed=seed)
    say(f"quantize min-error {n}x{k} seed {seed}")
    codes, meta, scales = _quant(w, fmt=tb.TB_FMT_DENSE_MINERR)
    assert meta is None
    _check_minerr(codes, scales, w, f"min-error {n}x{k}")


def test_minerr_closed_forms_and_lower_error_than_absmean():
    w = synth.stack_weights(256, 512, seed=21)
    w[:128, :128] = 0.0                                   # all-zero block: codes 0, scale 0
    w[5, 130] = 3.0                                       # a spike: lossless
    codes, _, scales = _quant(w, fmt=tb.TB_FMT_DENSE_MINERR)
    ref = _check_minerr(codes, scales, w, "min-error closed forms")
    s = oracle.quant.untile_scales(host_u16(scales))
    assert np.all(s[:128, 0] == 0) and np.all(host_u32(codes)[:8, 0] == 0)
    # reconstruction error in the rotated domain: never above the absmean rule's
    ca, _, sa = _quant(w)
    wr = ref["wr"]
    f16 = lambda b: b.view(np.float16).astype(np.float64)
    err = lambda t, sc: np.sum((wr - np.repeat(f16(oracle.quant.untile_scales(host_u16(sc))), 128, axis=1) * t) ** 2)
    e_min = err(oracle.quant.unpack_dense(host_u32(codes), 512), scales)
    e_abs = err(oracle.quant.unpack_dense(host_u32(ca), 512), sa)
    say(f"  squared error: min-error rule {e_min:.4e}, absmean rule {e_abs:.4e}")
    assert e_min < e_abs


# ---------------------------------------------------------------- residual second plane

def _f16(b):
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float64)


def _check_resid(codes, scales, w, what):
    """Codes and scales of TB_FMT_DENSE_RESID against the oracle.  Plane 1 as the
    one-plane rule.  Plane 2 is bit-exact (outside its own threshold band) in
    groups where the GPU's plane 1 equals the oracle's; where plane 1 took the
    other side of a near-threshold element or the other fp16 rounding of s1,
    plane 2 must be the absmean rule applied to the GPU's own residual."""
    ref = oracle.quant.quantize_dense_residual(w.astype(np.float64))
    n, k = w.shape
    g = k // 128
    c1, c2 = oracle.quant.split_planes(host_u32(codes))
    sc1, sc2 = (oracle.quant.untile_scales(p).astype(np.int64) for p in oracle.quant.split_planes(host_u16(scales)))
    r1, r2 = (oracle.quant.untile_scales(p).astype(np.int64) for p in oracle.quant.split_planes(ref["scales"]))
    t1 = oracle.quant.unpack_dense(c1, k)
    t2 = oracle.quant.unpack_dense(c2, k)
    wr = ref["wr"]
    near1 = oracle.quant.near_threshold(wr, ref["s1"])
    assert not ((t1 != ref["t1"]) & ~near1).any(), f"{what}: plane-1 code mismatch outside the band"
    assert np.abs(sc1 - r1).max(initial=0) <= 1, f"{what}: plane-1 scale beyond 1 ulp"
    same = (t1 == ref["t1"]).reshape(n, g, 128).all(axis=2) & (sc1 == r1)
    same_el = np.repeat(same, 128, axis=1)
    near2 = oracle.quant.near_threshold(ref["d"], ref["s2"])
    bad2 = (t2 != ref["t2"]) & ~near2 & same_el
    assert not bad2.any(), f"{what}: {int(bad2.sum())} plane-2 code mismatches outside the band"
    assert np.abs(sc2 - r2)[same].max(initial=0) <= 1, f"{what}: plane-2 scale beyond 1 ulp"
    # the other groups: the absmean rule on the GPU's own residual (test-side)
    d_own = wr - np.repeat(_f16(sc1), 128, axis=1) * t1
    s2_own = np.abs(d_own).reshape(n, g, 128).mean(axis=2)
    thr = np.repeat(s2_own / 2, 128, axis=1)
    t2_own = np.where(d_own > thr, 1, np.where(d_own < -thr, -1, 0))
    band = np.abs(np.abs(d_own) - thr) <= 1e-5 * thr
    other = ~same_el
    assert not ((t2 != t2_own) & ~band & other).any(), f"{what}: plane 2 is not the rule on the GPU's own residual"
    own16 = oracle.numerics.f64_to_f16_bits(s2_own).astype(np.int64)
    assert np.abs(sc2 - own16)[~same].max(initial=0) <= 1
    say(f"  {what}: {int(near1.sum())} plane-1 near-threshold elements, {int((~same).sum())} of {same.size} "
        f"groups with another plane 1, {int((near2 & same_el).sum())} plane-2 near-threshold elements")
    return ref, t1, t2, sc1, sc2


@pytest.mark.parametrize("n,k,seed", [(128, 128, 31), (256, 384, 32), (1024, 1024, 0), (384, 1280, 33)])
def test_resid_matches_oracle(n, k, seed):
    w = synth.single_layer_weights(n, k, seed=seed) if seed == 0 else synth.stack_weights(n, k, seed=seed)
    say(f"quantize two-plane {n}x{k} seed {seed}")
    codes, meta, scales = _quant(w, fmt=tb.TB_FMT_DENSE_RESID)
    assert meta is None and tuple(codes.shape) == (n // 16, 2 * k // 128, 128) and tuple(scales.shape) == (n // 16, 2 * k // 128, 16)
    _, t1, t2, sc1, sc2 = _check_resid(codes, scales, w, f"two-plane {n}x{k}")
    # plane 1 is the one-plane format, word for word
    c_one, _, s_one = _quant(w)
    assert np.array_equal(oracle.quant.split_planes(host_u32(codes))[0], host_u32(c_one))
    assert np.array_equal(oracle.quant.split_planes(host_u16(scales))[0], host_u16(s_one))


def test_resid_closed_forms_and_error():
    # the hand-worked rows of the oracle's residual fixture, as a rotated block
    wr = np.zeros((256, 256))
    wr[0, :64], wr[0, 64:128] = 1.0, 0.5            # exact two-level row: lossless
    wr[1, :64], wr[1, 64:128] = 1.0, 0.25           # s1 0.625, s2 0.3125
    wr[2, :32], wr[2, 32:128] = -0.5, 0.5           # already ternary: plane 2 zero
    wr[3, :128] = 1.0006103515625                   # fp16 rounding of s1 decides plane 2
    wr[128:, 128:] = np.random.default_rng(5).standard_normal((128, 128)) * 0.02 * 128
    w = np.zeros_like(wr)
    for a in (0, 128):
        for b in (0, 128):
            w[a:a + 128, b:b + 128] = H @ wr[a:a + 128, b:b + 128] @ H / 128
    codes, _, scales = _quant(w.astype(np.float32), fmt=tb.TB_FMT_DENSE_RESID)
    ref, t1, t2, sc1, sc2 = _check_resid(codes, scales, w.astype(np.float32), "two-plane closed forms")
    s1, s2 = _f16(sc1), _f16(sc2)
    assert s1[0, 0] == 0.75 and s2[0, 0] == 0.25 and np.all(t2[0, :64] == 1) and np.all(t2[0, 64:128] == -1)
    assert s1[1, 0] == 0.625 and s2[1, 0] == 0.3125 and np.all(t2[1, :128] == 1)
    assert s2[2, 0] == 0 and np.all(t2[2, :128] == 0)
    assert s1[3, 0] == 1.0009765625 and s2[3, 0] == 0.0003662109375 and np.all(t2[3, :128] == -1)
    assert np.all(sc1[4:128, 0] == 0) and np.all(sc2[4:128, 0] == 0) and np.all(t2[4:128, :128] == 0)
    # the second plane lowers the error of every Gaussian group
    rec1 = np.repeat(s1, 128, axis=1) * t1
    rec2 = rec1 + np.repeat(s2, 128, axis=1) * t2
    e1 = ((ref["wr"] - rec1) ** 2).reshape(256, 2, 128).sum(axis=2)[128:, 1]
    e2 = ((ref["wr"] - rec2) ** 2).reshape(256, 2, 128).sum(axis=2)[128:, 1]
    say(f"  squared error of the Gaussian block: one plane {e1.sum():.4e}, two planes {e2.sum():.4e}")
    assert np.all(e2 < e1)
