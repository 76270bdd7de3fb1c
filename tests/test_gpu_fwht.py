"""GPU parity of tb_fwht128 against the oracle's blockwise transform."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import DEV, assert_close, bf16_dev, f32_dev, host_f64, host_u16, say
from ternary_weights_hadamard_amd import synth, tb

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rows,k", [(1, 128), (3, 384), (17, 1024), (64, 5120), (5, 17408)])
@pytest.mark.parametrize("din,dout", [("bf16", "bf16"), ("bf16", "f32"), ("f32", "f32"), ("f32", "bf16")])
def test_fwht_matches_oracle(rows, k, din, dout):
    say(f"fwht rows={rows} K={k} {din}->{dout}")
    xb = synth.gaussian_bf16((rows, k), seed=rows * 7 + k)
    if din == "bf16":
        xin = bf16_dev(xb)
        xv = oracle.numerics.bf16_bits_to_f64(xb)
    else:
        xf = np.random.default_rng(k).standard_normal((rows, k)).astype(np.float32)
        xin = f32_dev(xf)
        xv = xf.astype(np.float64)
    y = tb.tb_fwht128(xin, out_dtype=torch.bfloat16 if dout == "bf16" else torch.float32)
    torch.cuda.synchronize()
    ref = oracle.hadamard.fwht_dense(xv)
    assert_close(host_f64(y), ref, f"fwht {din}->{dout}", out_bf16=dout == "bf16")
    if dout == "f32":
        # fp32 arithmetic: far inside the bar
        assert np.max(np.abs(host_f64(y) - ref)) <= 1e-5 * np.max(np.abs(ref))
    else:
        # bf16 output: within one bf16 rounding of the exact value
        err = np.abs(host_f64(y) - ref)
        assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 1e-30 + 1e-6 * np.max(np.abs(ref)))


def test_fwht_in_place_and_special_vectors():
    k = 256
    x = np.zeros((4, k), dtype=np.float32)
    x[0, 0] = 1.0        # spike -> every output +-1/sqrt(128)
    x[1, 200] = -3.0
    x[2, :128] = 0.5     # constant block -> DC only
    x[3] = np.arange(k, dtype=np.float32)
    t = f32_dev(x)
    ptr = t.data_ptr()
    out = tb.tb_fwht128(t, y=t)
    torch.cuda.synchronize()
    assert out.data_ptr() == ptr
    ref = oracle.hadamard.fwht_dense(x.astype(np.float64))
    got = host_f64(t)
    assert np.max(np.abs(got - ref)) <= 1e-5 * np.max(np.abs(ref))
    assert np.allclose(np.abs(got[0, :128]), 1 / np.sqrt(128), rtol=1e-6)
    assert np.all(got[0, 128:] == 0)
    assert abs(got[2, 0] - 0.5 * np.sqrt(128)) < 1e-5 and np.max(np.abs(got[2, 1:])) < 1e-6
    # applying the transform twice gives the input back (it is its own inverse)
    tb.tb_fwht128(t, y=t)
    torch.cuda.synchronize()
    assert np.max(np.abs(host_f64(t) - x)) <= 1e-5 * np.max(np.abs(x))


def test_fwht_bf16_in_place_and_canaries():
    k = 384
    xb = synth.gaussian_bf16((9, k), seed=3)
    buf = torch.full((9 * k + 64,), -7.0, dtype=torch.bfloat16, device=DEV)
    view = buf[32:32 + 9 * k].view(9, k)
    view.copy_(bf16_dev(xb))
    tb.tb_fwht128(view, y=view)
    torch.cuda.synchronize()
    assert torch.all(buf[:32] == -7.0) and torch.all(buf[32 + 9 * k:] == -7.0)
    ref = oracle.hadamard.fwht_dense(oracle.numerics.bf16_bits_to_f64(xb))
    assert_close(host_f64(view), ref, "fwht bf16 in place", out_bf16=True)


def test_fwht_empty_batch_is_noop():
    t = torch.zeros((0, 128), dtype=torch.bfloat16, device=DEV)
    tb.tb_fwht128(t)
    torch.cuda.synchronize()


@pytest.mark.parametrize("din,dout", [("bf16", "bf16"), ("bf16", "f32"), ("f32", "f32"), ("f32", "bf16"),
                                      ("bf16", "act8"), ("f32", "act8")])
def test_grouped_fwht_ragged_segments_equal_single_calls(din, dout):
    # eight segments of 1-17 blocks: in a grouped launch each segment starts on a
    # four-block boundary, so the lanes past a segment's end must write nothing
    shapes = [(1, 128), (1, 256), (3, 128), (1, 640), (7, 128), (3, 384), (1, 1664), (1, 2176)]
    say(f"grouped fwht {din}->{dout}, blocks {[r * k // 128 for r, k in shapes]}")
    canary = 64  # bytes after each output
    xs, ys, outs = [], [], []
    for c, (rows, k) in enumerate(shapes):
        if din == "bf16":
            x = bf16_dev(synth.gaussian_bf16((rows, k), seed=300 + c))
        else:
            x = f32_dev(np.random.default_rng(300 + c).standard_normal((rows, k)).astype(np.float32))
        nbytes = tb.tb_act8_bytes(rows, k) if dout == "act8" else rows * k * (2 if dout == "bf16" else 4)
        buf = torch.full((nbytes + canary,), 0xA5, dtype=torch.uint8, device=DEV)
        if dout == "act8":
            y = buf[:nbytes]
        else:
            y = buf[:nbytes].view(torch.bfloat16 if dout == "bf16" else torch.float32).view(rows, k)
        xs.append(x)
        ys.append(y)
        outs.append(buf)
    tb.tb_fwht128_multi(list(zip(xs, ys)))
    torch.cuda.synchronize()
    for c, (x, y, buf) in enumerate(zip(xs, ys, outs)):
        if dout == "act8":
            single = tb.tb_fwht128(x, out_dtype=torch.uint8)
        else:
            single = tb.tb_fwht128(x, out_dtype=torch.bfloat16 if dout == "bf16" else torch.float32)
        torch.cuda.synchronize()
        nbytes = buf.numel() - canary
        assert torch.equal(buf[:nbytes], single.contiguous().view(-1).view(torch.uint8)), f"segment {c} differs"
        assert bool((buf[nbytes:] == 0xA5).all()), f"segment {c}: write past its end"


def test_grouped_fwht_mixed_dtypes_equal_single_calls():
    # one launch whose segments differ in dtypes (a layer's fp32 outputs rotated
    # back next to the following layer's bf16 inputs rotated into act8), ragged
    # block counts, canaries after each output; each segment equals its single call
    specs = [("f32", "f32", 1, 15360), ("bf16", "act8", 1, 5120), ("f32", "f32", 3, 640), ("bf16", "act8", 2, 17408),
             ("bf16", "bf16", 1, 384), ("f32", "bf16", 1, 1152), ("f32", "act8", 5, 128), ("bf16", "f32", 1, 2176)]
    canary = 64
    pairs, outs = [], []
    for c, (din, dout, rows, k) in enumerate(specs):
        if din == "bf16":
            x = bf16_dev(synth.gaussian_bf16((rows, k), seed=500 + c))
        else:
            x = f32_dev(np.random.default_rng(500 + c).standard_normal((rows, k)).astype(np.float32))
        nbytes = tb.tb_act8_bytes(rows, k) if dout == "act8" else rows * k * (2 if dout == "bf16" else 4)
        buf = torch.full((nbytes + canary,), 0xA5, dtype=torch.uint8, device=DEV)
        y = buf[:nbytes] if dout == "act8" else buf[:nbytes].view(torch.bfloat16 if dout == "bf16" else torch.float32).view(rows, k)
        pairs.append((x, y))
        outs.append((buf, dout))
    say(f"grouped fwht, mixed dtypes: {[(a, b, r * k // 128) for a, b, r, k in specs]}")
    tb.tb_fwht128_multi(pairs)
    torch.cuda.synchronize()
    for c, ((x, _), (buf, dout)) in enumerate(zip(pairs, outs)):
        od = {"act8": torch.uint8, "bf16": torch.bfloat16, "f32": torch.float32}[dout]
        single = tb.tb_fwht128(x, out_dtype=od)
        torch.cuda.synchronize()
        nbytes = buf.numel() - canary
        assert torch.equal(buf[:nbytes], single.contiguous().view(-1).view(torch.uint8)), f"segment {c} differs"
        assert bool((buf[nbytes:] == 0xA5).all()), f"segment {c}: write past its end"
