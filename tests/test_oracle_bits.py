"""Pins of the bit ledger against the numbers the pages print."""

import json
import math
import os

import numpy as np
import pytest

from oracle import bits, quant as q
from ternary_weights_hadamard_amd import synth


def _ledger(golden_dir):
    return json.load(open(os.path.join(golden_dir, "bit_ledger.json")))


def test_ledger_matches_printed_numbers(golden_dir):
    g = _ledger(golden_dir)
    assert round(math.log2(3), 3) == g["ternary_code_bits"]["value"]
    assert 16 / 128 == g["scale_bits_per_weight"]["value"]
    assert round(bits.information_bound_bits(), 2) == g["ledger_total_bits"]["value"]
    assert round(2 - math.log2(3), 3) == g["two_bit_waste_bits"]["value"]
    assert round(27e9 * 1.72 / 8 / 1e9, 1) == g["weights_gb_at_1p72_bits_27b"]["value"]
    assert 27e9 * 2 / 1e9 == g["fp16_gb_27b"]["value"]


def test_storage_bits():
    assert bits.information_bound_bits() == pytest.approx(1.7099625, abs=1e-7)
    assert bits.dense_storage_bits() == 2.125
    assert bits.storage24_bits() == 1.625


@pytest.mark.parametrize("n,k", [(128, 128), (1024, 1024), (5120, 17408), (17408, 5120)])
def test_packed_bytes_formula(n, k):
    c, m, s = bits.packed_bytes("dense", n, k)
    assert (c * 8 + s * 8) / (n * k) == bits.dense_storage_bits()
    c, m, s = bits.packed_bytes("24", n, k)
    kp = -(-k // 512) * 512  # the 2:4 format pads K to whole blocks of four groups
    assert ((c + m + s) * 8) / (n * kp) == bits.storage24_bits()
    assert (kp == k) == (k % 512 == 0)


def test_buffers_have_formula_sizes():
    rng = np.random.default_rng(0)
    r = q.quantize_dense(rng.standard_normal((256, 384)))
    c, _, s = bits.packed_bytes("dense", 256, 384)
    assert r["codes"].nbytes == c and r["scales"].nbytes == s
    r = q.quantize_24(rng.standard_normal((256, 384)))
    c, m, s = bits.packed_bytes("24", 256, 384)
    assert r["signs"].nbytes == c and r["meta"].nbytes == m and r["scales"].nbytes == s


def test_entropy_of_uniform_and_config_distribution():
    t = np.array([-1, 0, 1] * 1000)
    assert bits.entropy_bits(t) == pytest.approx(math.log2(3), abs=1e-12)
    p = (0.35, 0.30, 0.35)
    expect = -sum(v * math.log2(v) for v in p)
    t = q.unpack_dense(synth.random_code_words(512, 1024, seed=3), 1024)
    assert bits.entropy_bits(t) == pytest.approx(expect, abs=0.003)
    with pytest.raises(ValueError):
        bits.packed_bytes("dense", 100, 128)
