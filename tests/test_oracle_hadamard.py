"""Pins of the oracle's Hadamard code against things other than itself:
hand-written small matrices, scipy's Hadamard routine, the algebraic
identities the pages state, and closed forms of the transform."""

import os

import numpy as np
import pytest
import scipy.linalg

from oracle import hadamard as hd


def _golden_mats(path):
    mats, name, rows = {}, None, []
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line[0].isalpha():
            if name:
                mats[name] = np.array(rows, dtype=float)
            name, rows = line, []
        else:
            rows.append([float(v) for v in line.split()])
    mats[name] = np.array(rows, dtype=float)
    return mats


def test_small_matrices_match_hand_written(golden_dir):
    mats = _golden_mats(os.path.join(golden_dir, "hadamard_small.txt"))
    for name, n in (("H2", 2), ("H4", 4), ("H8", 8)):
        assert np.array_equal(hd.hadamard_bitrule(n), mats[name])
        assert np.array_equal(hd.hadamard_sylvester(n), mats[name])


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64, 128])
def test_bitrule_equals_sylvester_and_scipy(n):
    h = hd.hadamard_bitrule(n)
    assert np.array_equal(h, hd.hadamard_sylvester(n))
    assert np.array_equal(h, scipy.linalg.hadamard(n).astype(float))


@pytest.mark.parametrize("n", [2, 16, 128])
def test_identities(n):
    # H H^T = H H = n I, H = H^T (xxqk.cn/news/652513 §2; mhpq.cn/news/1159370 §2.2)
    h = hd.hadamard_bitrule(n)
    assert np.array_equal(h, h.T)
    assert np.array_equal(h @ h.T, n * np.eye(n))
    assert np.array_equal(h @ h, n * np.eye(n))
    assert np.all(h[0] == 1) and np.all(h[:, 0] == 1)


def test_forward_inverse_pair():
    # y = H x, x = (1/n) H y (zwxr.cn/news/303439 §2.1), n = 32 as on that page
    rng = np.random.default_rng(3)
    x = rng.standard_normal(32)
    h = hd.hadamard_bitrule(32)
    assert np.allclose(h @ (h @ x) / 32, x, rtol=0, atol=1e-13)


def test_2d_dc_component():
    # In Y = H W H^T the (0, 0) entry is the block's DC term, the sum of all of W
    # (zwxr.cn/news/303439 §2.1); rotate_blocks divides by 128.
    rng = np.random.default_rng(4)
    w = rng.standard_normal((128, 128))
    assert np.isclose(hd.rotate_blocks(w)[0, 0], w.sum() / 128, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64, 128])
def test_fwht_dense_equals_butterfly_tiny_n(n):
    rng = np.random.default_rng(n)
    x = rng.standard_normal((3, 4 * n))
    a = hd.fwht_dense(x, n)
    b = hd.fwht_butterfly(x, n)
    assert np.max(np.abs(a - b)) <= 1e-12 * max(1.0, np.max(np.abs(a)))
    # and against an explicit per-block product with scipy's matrix
    ref = (x.reshape(3, 4, n) @ (scipy.linalg.hadamard(n) / np.sqrt(n)).T).reshape(3, 4 * n)
    assert np.max(np.abs(a - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_fwht_properties():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((5, 512))
    y = hd.fwht_butterfly(x)
    # involution: the normalised transform is its own inverse
    assert np.max(np.abs(hd.fwht_butterfly(y) - x)) < 1e-13
    # Parseval per 128-block (energy preserved, mhpq.cn §2.2)
    assert np.allclose((y.reshape(5, 4, 128) ** 2).sum(-1), (x.reshape(5, 4, 128) ** 2).sum(-1), rtol=1e-13)
    # constant block -> all energy in the DC term: c * sqrt(128) * e0
    c = np.full((1, 128), 0.75)
    dc = np.zeros((1, 128))
    dc[0, 0] = 0.75 * np.sqrt(128)
    assert np.allclose(hd.fwht_dense(c), dc, atol=1e-14)
    # a spike is spread evenly: every output is +-1/sqrt(128) (outlier spreading, mhpq.cn §2.3)
    for j in (0, 1, 77, 127):
        e = np.zeros((1, 128))
        e[0, j] = 1.0
        out = hd.fwht_dense(e)[0]
        assert np.allclose(np.abs(out), 1 / np.sqrt(128), atol=1e-15)
        assert np.allclose(out * np.sqrt(128), scipy.linalg.hadamard(128)[:, j])


def test_fwht_blocks_are_independent():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((2, 384))
    y = hd.fwht_dense(x)
    x2 = x.copy()
    x2[:, 128:256] += 5.0
    y2 = hd.fwht_dense(x2)
    assert np.array_equal(y[:, :128], y2[:, :128]) and np.array_equal(y[:, 256:], y2[:, 256:])


def test_rotation_identity_without_quantisation():
    # With no quantisation, R_N (W' (R_K x)) = W x (R = blockwise orthonormal FWHT)
    rng = np.random.default_rng(9)
    w = rng.standard_normal((256, 384))
    x = rng.standard_normal(384)
    wr = hd.rotate_blocks(w)
    y = hd.fwht_dense((wr @ hd.fwht_dense(x[None, :])[0])[None, :])[0]
    assert np.max(np.abs(y - w @ x)) < 1e-11


def test_rotate_blocks_matches_kron_form():
    # the blockwise 2D rotation equals blockdiag(H) W blockdiag(H) / 128
    rng = np.random.default_rng(10)
    w = rng.standard_normal((256, 256))
    big = np.kron(np.eye(2), scipy.linalg.hadamard(128))
    assert np.allclose(hd.rotate_blocks(w), big @ w @ big / 128, atol=1e-12)


def test_shape_errors():
    with pytest.raises(ValueError):
        hd.rotate_blocks(np.zeros((128, 100)))
    with pytest.raises(ValueError):
        hd.fwht_dense(np.zeros((1, 130)))
    with pytest.raises(ValueError):
        hd.hadamard_bitrule(12)
