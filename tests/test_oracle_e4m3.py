"""Pins for the e4m3 codec: every code, and torch's float8_e4m3fn casts."""

import numpy as np
import pytest
import torch

from oracle import e4m3


def torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8).copy()).view(torch.float8_e4m3fn).double().numpy()


def test_all_codes_decode_like_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours, ref = e4m3.decode(codes), torch_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}


def test_all_codes_round_trip():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    assert np.array_equal(e4m3.encode(e4m3.decode(codes)), codes)


def test_known_values():
    assert e4m3.decode(np.array([0x7E]))[0] == 448.0
    assert e4m3.decode(np.array([0x01]))[0] == 2.0 ** -9
    assert e4m3.decode(np.array([0x08]))[0] == 2.0 ** -6
    assert e4m3.decode(np.array([0x38]))[0] == 1.0
    # ties go to even: 1 + 1/16 lies halfway between 1 and 1.125
    assert e4m3.round_to_e4m3(np.array([1.0 + 1 / 16]))[0] == 1.0
    assert e4m3.round_to_e4m3(np.array([1.0 + 3 / 16]))[0] == 1.25
    # saturation
    assert e4m3.round_to_e4m3(np.array([1e9, -500.0]))[0] == 448.0
    assert e4m3.round_to_e4m3(np.array([-500.0]))[0] == -448.0


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_rounding_matches_torch_cast(seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(200000) * np.exp2(rng.integers(-14, 9, 200000))
    x = np.clip(x, -448.0, 448.0).astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3.encode(x), ref)


def test_block_exponent_is_smallest_fitting_power():
    rng = np.random.default_rng(7)
    amax = np.abs(rng.standard_normal(5000)) * np.exp2(rng.integers(-20, 20, 5000))
    amax = np.concatenate([amax, [448.0, 224.0, 449.0, 1.0, 0.875 * 2 ** 3, 0.0]])
    e = e4m3.block_exponent(amax)
    pos = amax > 0
    assert np.all(amax[pos] * np.exp2(-e[pos]) <= 448.0)
    assert np.all(amax[pos] * np.exp2(-(e[pos] - 1)) > 448.0)
    assert e[-1] == 0
