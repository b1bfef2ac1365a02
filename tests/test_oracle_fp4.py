"""Pins of the oracle's FP4 (E2M1) block encoding (oracle/fp4.py): every code's value
from the bit fields written out by hand, round-to-nearest-even on every tie and between
them, saturation, and the block scale's defining property."""

import math

import numpy as np
import pytest

from oracle import fp4


def test_every_code_value():
    # sign | exponent (bias 1) | mantissa, written out: 0, 0.5 (subnormal), then 1.m * 2^(e-1)
    expect = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    np.testing.assert_array_equal(fp4.e2m1_values()[:8], expect)
    np.testing.assert_array_equal(fp4.e2m1_values()[8:], [-v for v in expect])
    # encoding every value returns its code (both zeros keep their sign bit)
    np.testing.assert_array_equal(fp4.e2m1_encode(fp4.e2m1_values()), np.arange(16))


def test_round_to_nearest_even_on_every_tie():
    pos = fp4.e2m1_values()[:8]
    mids = (pos[1:] + pos[:-1]) / 2  # 0.25 0.75 1.25 1.75 2.5 3.5 5
    got = fp4.e2m1_encode(mids)
    # the tie goes to the code with mantissa bit 0: 0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0
    np.testing.assert_array_equal(fp4.e2m1_values()[got], [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0])
    assert all(c % 2 == 0 for c in got)
    # just off a tie: nearest, either way
    np.testing.assert_array_equal(fp4.e2m1_encode(mids * (1 + 1e-9)), np.arange(1, 8))
    np.testing.assert_array_equal(fp4.e2m1_encode(mids * (1 - 1e-9)), np.arange(0, 7))
    np.testing.assert_array_equal(fp4.e2m1_encode(-mids * (1 + 1e-9)), np.arange(1, 8) | 8)


def test_nearest_by_brute_force_and_saturation():
    rng = np.random.default_rng(1)
    x = rng.uniform(-8, 8, 100000)
    codes = fp4.e2m1_encode(x)
    vals = fp4.e2m1_values()
    err = np.abs(vals[codes] - np.clip(x, -6, 6))
    best = np.abs(vals[None, :] - np.clip(x, -6, 6)[:, None]).min(axis=1)
    np.testing.assert_allclose(err, best, rtol=0, atol=1e-15)
    assert (vals[fp4.e2m1_encode(np.array([7.0, 100.0, -9.0]))] == [6, 6, -6]).all()


@pytest.mark.parametrize("amax", [6.0, 6.0000001, 3.0, 3.1, 1.0, 1e-30, 255.9, 256.0, 0.0])
def test_block_exponent_is_the_smallest_that_fits(amax):
    e = fp4.block_exponent(amax)
    if amax == 0:
        assert e == -127
        return
    assert amax <= 6 * 2.0 ** e
    assert e == -127 or amax > 6 * 2.0 ** (e - 1)


def test_encode_blocks_round_trip_and_error_bound():
    rng = np.random.default_rng(2)
    x = np.exp2(rng.uniform(-20, 8, (3, 128))) * rng.choice([-1, 1], (3, 128))
    x[1, 32:64] = 0.0
    codes, e = fp4.encode_blocks(x)
    assert codes.shape == x.shape and e.shape == (3, 4)
    assert e[1, 1] == -127 and (codes[1, 32:64] & 7 == 0).all()
    y = fp4.decode_blocks(codes, e)
    # each value is within half a step of its block's grid: <= 1 * 2^e (step 2 at 4..6),
    # and the largest magnitude of a block is never clipped
    step_bound = np.repeat(np.exp2(e.astype(float)), 32, axis=1)
    assert np.all(np.abs(y - x) <= step_bound * (1 + 1e-12))
    for b in range(3):
        for k in range(4):
            blk = x[b, 32 * k:32 * (k + 1)]
            if np.any(blk):
                i = np.argmax(np.abs(blk))
                assert abs(y[b, 32 * k + i]) >= abs(blk[i]) * 0.75  # 4 of (3, 6] at worst
    # block scaling commutes with powers of two
    codes2, e2 = fp4.encode_blocks(x * 2.0 ** 5)
    np.testing.assert_array_equal(codes2, codes)
    np.testing.assert_array_equal(e2, np.where(e == -127, e2, e + 5))
    assert math.isclose(fp4.decode_blocks(codes2, e2)[0, 0], y[0, 0] * 32)
