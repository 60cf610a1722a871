"""Pins for the oracle's hand-written IEEE binary16 codec.

The Buddy-MLIR walkthrough (sec. 6.4.7) shows an f16 decode done with a bf16-style
16-bit shift; the oracle's codec is therefore written by hand and checked here against
numpy's float16, an independent implementation, on every bit pattern.
"""
import numpy as np
import pytest


def test_decode_every_bit_pattern(ora):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = ora.f16_to_f64(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.signbit(mine[0x8000]) and not np.signbit(mine[0])


def test_encode_roundtrips_every_finite_value(ora):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16).astype(np.float64)
    fin = np.isfinite(vals)
    back = ora.f64_to_f16(vals[fin])
    assert np.array_equal(back, bits[fin])


def test_encode_midpoints_ties_to_even(ora):
    # every pair of adjacent positive finite f16 values; the midpoint is exact in fp64
    lo = np.arange(0, 0x7bff, dtype=np.uint16)
    a = lo.view(np.float16).astype(np.float64)
    b = (lo + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    mid = (a + b) / 2
    got = ora.f64_to_f16(mid)
    even = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint16)
    assert np.array_equal(got, even)
    # just above / below the midpoint go to the nearer neighbour
    up = ora.f64_to_f16(np.nextafter(mid, np.inf))
    dn = ora.f64_to_f16(np.nextafter(mid, -np.inf))
    assert np.array_equal(up, lo + 1)
    assert np.array_equal(dn, lo)


def test_encode_random_doubles_match_numpy(ora):
    rng = np.random.default_rng(1234)
    x = np.concatenate([
        rng.standard_normal(200_000),
        rng.standard_normal(100_000) * 1e-5,          # subnormal range
        rng.standard_normal(100_000) * 3e4,           # near overflow
        rng.uniform(-1e-7, 1e-7, 50_000),
    ])
    got = ora.f64_to_f16(x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("x,expect", [
    (65504.0, 0x7BFF), (65519.99, 0x7BFF), (65520.0, 0x7C00), (1e9, 0x7C00),
    (-65520.0, 0xFC00), (2.0 ** -24, 0x0001), (2.0 ** -25, 0x0000),
    (np.nextafter(2.0 ** -25, 1.0), 0x0001), (3 * 2.0 ** -25, 0x0002),
    (-0.0, 0x8000), (float("inf"), 0x7C00), (2.0 ** -14, 0x0400),
    (2.0 ** -14 - 2.0 ** -25, 0x0400),
])
def test_encode_edge_cases(ora, x, expect):
    assert int(ora.f64_to_f16(np.array([x]))[0]) == expect


def test_encode_nan(ora):
    out = int(ora.f64_to_f16(np.array([np.nan]))[0])
    assert (out & 0x7C00) == 0x7C00 and (out & 0x3FF) != 0
