"""Pins for the MXFP4 (E2M1 + E8M0) oracle codec, from the format definition."""

import itertools

import numpy as np
import pytest

from oracle import mxfp4


def value_from_bits(code):
    """E2M1 value straight from the bit fields: s.ee.m, bias 1."""
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = (m / 2.0) * 2.0 ** (1 - 1) if e == 0 else (1 + m / 2.0) * 2.0 ** (e - 1)
    return -mag if s else mag


def test_decode_all_codes():
    got = mxfp4.decode(np.arange(16))
    want = [value_from_bits(c) for c in range(16)]
    assert np.array_equal(got, np.array(want))
    assert list(got[:8]) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def test_encode_round_trips_every_value():
    vals = mxfp4.decode(np.arange(16))
    codes = mxfp4.encode(vals)
    assert np.array_equal(mxfp4.decode(codes), vals)
    assert codes[8] == 0                    # -0 is encoded as +0


@pytest.mark.parametrize("seed", range(3))
def test_encode_is_nearest_ties_to_even(seed):
    rng = np.random.default_rng(seed)
    grid = [value_from_bits(c) for c in range(8)]
    xs = np.concatenate([rng.uniform(-7, 7, 2000),
                         [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.75, -2.5, -5.0, 6.5, -100.0, 1e-9]])
    codes = mxfp4.encode(xs)
    for x, c in zip(xs, codes):
        a = min(abs(x), 6.0)
        d = [abs(a - g) for g in grid]
        best = min(d)
        ties = [i for i in range(8) if d[i] == best]
        mag = [t for t in ties if t % 2 == 0][0] if len(ties) > 1 else ties[0]
        want = mag | (8 if (x < 0 and mag > 0) else 0)
        assert c == want, (x, c, want)


def test_block_exponent_is_smallest_fitting_power():
    for amax in [1e-3, 0.3, 0.75, 1.0, 1.5, 3.0, 5.9, 6.0, 6.1, 12.0, 100.0, 2.0 ** -20]:
        e = int(mxfp4.block_exponent(np.array(amax)))
        assert amax * 2.0 ** -e <= 6.0
        assert amax * 2.0 ** -(e - 1) > 6.0
    assert int(mxfp4.block_exponent(np.array(0.0))) == 0
    assert int(mxfp4.block_exponent(np.array(2.0 ** -140))) == -127      # E8M0 floor


def test_quantize_blocks_bound_and_round_trip():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 5, 64)) * np.exp(rng.uniform(-4, 4, (3, 5, 1)))
    codes, e = mxfp4.quantize_blocks(x, axis=-1, block=32)
    assert e.shape == (3, 5, 2)
    y = mxfp4.dequantize_blocks(codes, e, axis=-1, block=32)
    # every element is within half a grid step of the scaled value: the E2M1
    # grid steps are 0.5 below 2, 1 in [2, 4) and 2 in [4, 6]
    scale = np.exp2(np.repeat(e, 32, axis=-1).astype(float))
    a = np.abs(x) / scale
    half = np.where(a < 2, 0.25, np.where(a < 4, 0.5, 1.0))
    assert np.all(np.abs(y - x) <= half * scale)
    # values already on the scaled grid come back exactly
    codes2, e2 = mxfp4.quantize_blocks(y, axis=-1, block=32)
    assert np.array_equal(mxfp4.dequantize_blocks(codes2, e2, axis=-1, block=32), y)


def test_quantize_blocks_along_other_axis():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((64, 3))
    c0, e0 = mxfp4.quantize_blocks(x, axis=0, block=32)
    c1, e1 = mxfp4.quantize_blocks(x.T, axis=-1, block=32)
    assert np.array_equal(c0, c1.T) and np.array_equal(e0, e1.T)
