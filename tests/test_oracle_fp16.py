"""Pins for oracle.fp16: RNE rounding to binary16 checked against numpy's
float64 -> float16 conversion (a library routine that rounds the float64 bits
directly, to nearest even) on normal, subnormal, tie and overflow values, and
hand cases."""
import numpy as np

from oracle import fp16


def test_matches_numpy_conversion_from_float64():
    rng = np.random.default_rng(6)
    x = np.concatenate([
        rng.standard_normal(200000),
        rng.standard_normal(20000) * 3e4,                 # near and beyond 65504
        rng.standard_normal(20000) * 1e-5,                # subnormal range (< 2^-14)
        rng.standard_normal(20000) * 1e-8,                # below half the smallest subnormal
        # exact ties between neighbours, and values one float64 step either side
        (np.arange(1, 20001) + 0.5) * 2.0 ** -10,
        np.nextafter((np.arange(1, 20001) + 0.5) * 2.0 ** -10, 0),
        np.nextafter((np.arange(1, 20001) + 0.5) * 2.0 ** -10, 10),
    ])
    want = x.astype(np.float16).astype(np.float64)
    got = fp16.round_f16(x)
    np.testing.assert_array_equal(got, want)


def test_hand_cases():
    # 1 + 2^-11 is half way between 1 and 1 + 2^-10: the even neighbour is 1
    assert fp16.round_f16(1.0 + 2.0 ** -11) == 1.0
    assert fp16.round_f16(1.0 + 3 * 2.0 ** -11) == 1.0 + 2.0 ** -9
    # no double rounding: just below the tie in float64
    assert fp16.round_f16(1.0 + 2.0 ** -11 - 2.0 ** -40) == 1.0
    # largest finite, the overflow threshold (65520 ties to the even 2^16 -> inf)
    assert fp16.round_f16(65504.0) == 65504.0
    assert fp16.round_f16(65519.9) == 65504.0
    assert np.isinf(fp16.round_f16(65520.0))
    # smallest subnormal 2^-24; half of it ties to even zero
    assert fp16.round_f16(2.0 ** -24) == 2.0 ** -24
    assert fp16.round_f16(2.0 ** -25) == 0.0
    assert fp16.round_f16(1.5 * 2.0 ** -24) == 2.0 ** -23
    assert np.isnan(fp16.round_f16(np.nan))


def test_bits_round_trip_and_ulp():
    rng = np.random.default_rng(3)
    x = fp16.round_f16(rng.standard_normal(1000))
    np.testing.assert_array_equal(fp16.bits_to_f64(fp16.f64_to_bits(x)), x)
    assert fp16.f16_ulp(1.0) == 2.0 ** -10
    assert fp16.f16_ulp(2.0) == 2.0 ** -9
    assert fp16.f16_ulp(1e-6) == 2.0 ** -24
    a = np.array([1.0, -1.0])
    b = np.array([1.0 + 2 ** -9, 1.0])
    np.testing.assert_array_equal(fp16.ulp_distance(a, b), [2, 2 * 0x3C00])
