"""Pins of the oracle's fp16 / bf16 rounding: exhaustive round trips,
numpy's float16 cast, torch's bfloat16 cast and hand-worked ties."""

import numpy as np

from oracle import numerics as nu


def test_f16_exhaustive_round_trip_and_numpy_decode():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = nu.f16_bits_to_f64(bits)
    ok = ~np.isnan(v)
    assert np.array_equal(nu.f64_to_f16_bits(v[ok]), bits[ok])
    assert np.array_equal(v[ok], bits[ok].view(np.float16).astype(np.float64))
    assert np.all(np.isnan(bits[~ok].view(np.float16)))


def test_bf16_exhaustive_round_trip_and_float32_decode():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = nu.bf16_bits_to_f64(bits)
    ok = ~np.isnan(v)
    assert np.array_equal(nu.f64_to_bf16_bits(v[ok]), bits[ok])
    # a bf16 pattern is the top half of a float32 pattern
    as_f32 = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(v[ok], as_f32[ok])


def test_f16_rounding_matches_numpy():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(200000) * np.exp(rng.uniform(-30, 13, 200000))
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(nu.f64_to_f16_bits(x), ref)


def test_bf16_rounding_matches_torch_on_float32_values():
    import torch

    rng = np.random.default_rng(1)
    x32 = (rng.standard_normal(200000) * np.exp(rng.uniform(-60, 60, 200000))).astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(nu.f64_to_bf16_bits(x32.astype(np.float64)), ref)


def test_hand_worked_ties_and_limits():
    # bf16 keeps 7 mantissa bits: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> even (1.0)
    assert nu.f64_to_bf16_bits(1 + 2.0 ** -8) == 0x3F80
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even) -> 1 + 2^-6
    assert nu.f64_to_bf16_bits(1 + 3 * 2.0 ** -8) == 0x3F82
    # just above the tie rounds up
    assert nu.f64_to_bf16_bits(1 + 2.0 ** -8 + 2.0 ** -30) == 0x3F81
    # fp16: largest finite 65504 = 0x7BFF; 65520 is the tie with "65536" -> inf
    assert nu.f64_to_f16_bits(65504.0) == 0x7BFF
    assert nu.f64_to_f16_bits(65519.99) == 0x7BFF
    assert nu.f64_to_f16_bits(65520.0) == 0x7C00
    # smallest subnormal 2^-24; 2^-25 is the tie with 0 -> 0; a hair above -> 2^-24
    assert nu.f64_to_f16_bits(2.0 ** -24) == 0x0001
    assert nu.f64_to_f16_bits(2.0 ** -25) == 0x0000
    assert nu.f64_to_f16_bits(2.0 ** -25 * 1.001) == 0x0001
    assert nu.f64_to_f16_bits(-2.0) == 0xC000
    assert nu.f64_to_f16_bits(np.inf) == 0x7C00
    assert nu.f64_to_bf16_bits(-np.inf) == 0xFF80
    assert nu.f16_bits_to_f64(0x3555) == np.float64(np.float16(0.333251953125))
