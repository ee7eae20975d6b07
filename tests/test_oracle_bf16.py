"""Pins for oracle.bf16: RNE rounding checked against torch's float32->bfloat16
conversion (a library routine that rounds to nearest even) and hand cases."""
import numpy as np
import pytest
import torch

from oracle import bf16


def test_matches_torch_conversion_on_float32_values():
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(20000) * 1e30).astype(np.float32),
        (rng.standard_normal(20000) * 1e-30).astype(np.float32),
        (rng.standard_normal(20000) * 1e-39).astype(np.float32),   # binary32 subnormals
    ])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = bf16.round_bf16(x.astype(np.float64))
    np.testing.assert_array_equal(got, want)


def test_ties_round_to_even():
    one = 1.0
    # 1 + 2^-8 lies half way between 1 and 1 + 2^-7: even neighbour is 1.
    assert bf16.round_bf16(one + 2.0 ** -8) == 1.0
    # 1 + 3*2^-8 lies half way between 1 + 2^-7 (odd) and 1 + 2^-6 (even).
    assert bf16.round_bf16(one + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    # just above the tie rounds up
    assert bf16.round_bf16(one + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7
    assert bf16.round_bf16(-(one + 2.0 ** -8)) == -1.0


def test_no_double_rounding_from_float64():
    # Half-way in bf16 after a float32 rounding, but below the tie in float64:
    # x = 1 + 2^-8 - 2^-40 must round down to 1 (a float32 step would give the tie).
    x = 1.0 + 2.0 ** -8 - 2.0 ** -40
    assert bf16.round_bf16(x) == 1.0


def test_overflow_nan_zero_and_idempotence():
    assert np.isinf(bf16.round_bf16(3.5e38))
    assert bf16.round_bf16(bf16.BF16_MAX) == bf16.BF16_MAX
    assert np.isnan(bf16.round_bf16(np.nan))
    assert bf16.round_bf16(0.0) == 0.0
    rng = np.random.default_rng(1)
    x = bf16.round_bf16(rng.standard_normal(1000) * 10)
    np.testing.assert_array_equal(bf16.round_bf16(x), x)


def test_bits_round_trip_and_ulp():
    rng = np.random.default_rng(2)
    x = bf16.round_bf16(rng.standard_normal(1000))
    np.testing.assert_array_equal(bf16.bits_to_f64(bf16.f64_to_bits(x)), x)
    assert bf16.bf16_ulp(1.0) == 2.0 ** -7
    assert bf16.bf16_ulp(1.5) == 2.0 ** -7
    assert bf16.bf16_ulp(2.0) == 2.0 ** -6
    a = np.array([1.0, 1.0, -1.0])
    b = np.array([1.0 + 2 ** -7, 1.0 + 2 ** -6, 1.0])
    np.testing.assert_array_equal(bf16.ulp_distance(a, b), [1, 2, 2 * 0x3F80])
    with pytest.raises(ValueError):
        bf16.f64_to_bits(np.array([1.0 + 2 ** -9]))
