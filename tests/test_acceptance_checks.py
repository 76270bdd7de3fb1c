"""CPU checks of the GPU tests' acceptance rules (tests/gpu_util.py): fed the
oracle's own output they pass, and fed the oracle's output with one planted
mistake they fail.  This is what keeps a band that forgives too much from
passing silently."""

import numpy as np
import pytest
import scipy.linalg
import torch

import oracle
from gpu_util import check_24_planes, check_dense_codes

H = scipy.linalg.hadamard(128).astype(np.float64)


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int32 if a.dtype == np.uint32 else np.int16))


def _from_rotated(wr):
    w = np.empty_like(wr)
    for a in range(0, wr.shape[0], 128):
        for b in range(0, wr.shape[1], 128):
            w[a:a + 128, b:b + 128] = H @ wr[a:a + 128, b:b + 128] @ H / 128
    return w


def test_dense_check_accepts_the_oracle_and_the_other_side_of_the_threshold():
    # row 0: 48 x 1.0, 64 x 0.25, 16 x 0 -> s = 0.5, the 0.25 entries sit exactly on s/2
    wr = np.zeros((128, 128))
    wr[0, :48], wr[0, 48:112] = 1.0, 0.25
    wr[1:] = np.random.default_rng(1).standard_normal((127, 128))
    ref = oracle.quant.quantize_dense(_from_rotated(wr))
    check_dense_codes(_t(ref["codes"]), _t(ref["scales"]), ref, 128, "oracle itself")
    t = ref["t"].copy()
    t[0, 50] = 1  # sign(W') at the threshold: valid
    check_dense_codes(_t(oracle.quant.pack_dense(t)), _t(ref["scales"]), ref, 128, "other side")


@pytest.mark.parametrize("where", ["wrong sign at the threshold", "flip outside the band", "scale 2 ulp"])
def test_dense_check_rejects_planted_mistakes(where):
    wr = np.zeros((128, 128))
    wr[0, :48], wr[0, 48:112] = 1.0, 0.25
    wr[1:] = np.random.default_rng(1).standard_normal((127, 128))
    ref = oracle.quant.quantize_dense(_from_rotated(wr))
    t, sc = ref["t"].copy(), ref["scales"].copy()
    if where == "wrong sign at the threshold":
        t[0, 50] = -1
    elif where == "flip outside the band":
        t[0, 3] = 0
    else:
        sc[5, 0] += 2
    with pytest.raises(AssertionError):
        check_dense_codes(_t(oracle.quant.pack_dense(t)), _t(sc), ref, 128, where)


def _24_case():
    # quad 0 of row 0 is a near tie (2nd and 3rd magnitude equal); the rest Gaussian
    wr = np.random.default_rng(2).standard_normal((128, 128))
    wr[0, :4] = [3.0, 2.0, -2.0, 0.5]
    return oracle.quant.quantize_24(_from_rotated(wr))


def _planes(ref, idx0, idx1, neg0, neg1):
    rows_scales = oracle.quant.load_24(ref["meta"], ref["signs"], ref["scales"], 128)[2]
    meta, signs, scales = oracle.quant.store_24(*oracle.quant.pack_24(idx0, idx1, neg0, neg1), rows_scales)
    return _t(meta), _t(signs), _t(scales)


def test_24_check_accepts_the_oracle_and_the_other_tied_pair():
    ref = _24_case()
    i0, i1, n0, n1 = (ref[k].copy() for k in ("idx0", "idx1", "neg0", "neg1"))
    check_24_planes(*_planes(ref, i0, i1, n0, n1), ref, 128, "oracle itself")
    # rounding in the rotation decides which of 2.0 and -2.0 the oracle keeps; keep the other
    assert (i0[0, 0], i1[0, 0]) in ((0, 1), (0, 2))
    i1[0, 0], n1[0, 0] = (2, True) if i1[0, 0] == 1 else (1, False)
    check_24_planes(*_planes(ref, i0, i1, n0, n1), ref, 128, "other tied pair")


@pytest.mark.parametrize("where", ["tie quad keeps the smallest", "tie quad wrong sign", "sign flip elsewhere",
                                   "pair change elsewhere"])
def test_24_check_rejects_planted_mistakes(where):
    ref = _24_case()
    i0, i1, n0, n1 = (ref[k].copy() for k in ("idx0", "idx1", "neg0", "neg1"))
    if where == "tie quad keeps the smallest":
        i0[0, 0], i1[0, 0], n0[0, 0], n1[0, 0] = 0, 3, False, False
    elif where == "tie quad wrong sign":
        n1[0, 0] = ~n1[0, 0]  # the kept +-2.0 with the other sign
    elif where == "sign flip elsewhere":
        n0[5, 7] = ~n0[5, 7]
    else:
        i0[9, 3], i1[9, 3] = (0, 1) if (i0[9, 3], i1[9, 3]) != (0, 1) else (2, 3)
    with pytest.raises(AssertionError):
        check_24_planes(*_planes(ref, i0, i1, n0, n1), ref, 128, where)
