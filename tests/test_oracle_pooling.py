"""Pins for the pooling oracle: exact sums, closed forms, alternative formulas."""

import math

import numpy as np
import pytest

from oracle import pooling, e4m3
from workloads import round_to_bf16


def rand_inputs(seed, B=1, H=2, N=150, d=8, bf16=True):
    rng = np.random.default_rng(seed)
    Np = 64 * ((N + 63) // 64)
    x = np.zeros((B, H, Np, d), np.float32)
    x[:, :, :N] = rng.standard_normal((B, H, N, d)).astype(np.float32) * 3
    return round_to_bf16(x) if bf16 else x


def test_counts_closed_form():
    assert list(pooling.block_counts(150, 192)) == [64, 64, 22]
    assert list(pooling.block_counts(128, 128)) == [64, 64]
    assert list(pooling.block_counts(1, 64)) == [1]
    assert pooling.block_counts(0, 0).shape == (0,)


@pytest.mark.parametrize("bf16", [True, False])
def test_block_means_equal_correctly_rounded_sums(bf16):
    # bf16 sums of 64 values are exact in fp64, so the sequential sum must
    # equal math.fsum (the correctly rounded sum); the mean is sum/n then fp32.
    x = rand_inputs(3, bf16=bf16)
    N = 150
    mean32, mean64, n = pooling.block_means(x, N)
    B, H, Np, d = x.shape
    for b in range(B):
        for h in range(H):
            for j in range(Np // 64):
                toks = range(64 * j, min(N, 64 * j + 64))
                for i in range(d):
                    s = math.fsum(float(x[b, h, t, i]) for t in toks)
                    if bf16:
                        assert mean64[b, h, j, i] == s / len(toks)
                        assert mean32[b, h, j, i] == np.float32(s / len(toks))
                    else:
                        assert abs(mean64[b, h, j, i] - s / len(toks)) <= 1e-15 * max(1.0, abs(s))


def test_block_sums_are_sequential():
    # 1e16 + 1 + 1 - 1e16 in order gives 0; a pairwise or exact sum gives 2
    x = np.zeros((1, 1, 64, 1), np.float32)
    x[0, 0, :4, 0] = [np.float32(2.0 ** 53), 1.0, 1.0, -np.float32(2.0 ** 53)]
    assert pooling.block_sums(x, 4)[0, 0, 0, 0] == 0.0


def test_pad_rows_are_ignored():
    x = rand_inputs(5)
    y = x.copy()
    y[:, :, 150:] = 1e30
    a = pooling.pool(x, x, x, 150, moments=True, spreads=True, fp8=True)
    b = pooling.pool(y, y, y, 150, moments=True, spreads=True, fp8=True)
    for key in ("qbar", "kbar", "vbar", "kmom", "klam", "q8", "kexp"):
        assert np.array_equal(a[key], b[key]), key


def test_moments_alternative_formula():
    # sum (k - kbar) v^T == sum k v^T - n kbar vbar^T
    k, v = rand_inputs(11, N=170, d=6), rand_inputs(12, N=170, d=6)
    N = 170
    H = pooling.block_moments(k, v, N)
    _, kbar, n = pooling.block_means(k, N)
    _, vbar, _ = pooling.block_means(v, N)
    for j in range(H.shape[2]):
        t = slice(64 * j, min(N, 64 * j + 64))
        kv = np.einsum("bhni,bhno->bhio", k[:, :, t].astype(np.float64), v[:, :, t].astype(np.float64))
        alt = kv - n[j] * np.einsum("bhi,bho->bhio", kbar[:, :, j], vbar[:, :, j])
        np.testing.assert_allclose(H[:, :, j], alt, rtol=1e-10, atol=1e-9)


def test_moments_brute_force():
    k, v = rand_inputs(21, H=1, N=70, d=3), rand_inputs(22, H=1, N=70, d=3)
    H = pooling.block_moments(k, v, 70)
    for j, toks in enumerate([range(64), range(64, 70)]):
        kb = [sum(float(k[0, 0, t, i]) for t in toks) / len(toks) for i in range(3)]
        for i in range(3):
            for o in range(3):
                ref = sum((float(k[0, 0, t, i]) - kb[i]) * float(v[0, 0, t, o]) for t in toks)
                assert abs(H[0, 0, j, i, o] - ref) < 1e-9


def test_spreads_variance_identity():
    k, v = rand_inputs(31, N=130), rand_inputs(32, N=130)
    lam = pooling.block_spreads(k, v, 130)
    for j, n in enumerate([64, 64, 2]):
        t = slice(64 * j, 64 * j + n)
        r2 = []
        for x in (k, v):
            xx = x[:, :, t].astype(np.float64)
            r2.append((xx ** 2).sum(axis=(2, 3)) - n * (xx.mean(axis=2) ** 2).sum(axis=2))
        ref = 0.5 * np.log(r2[0]) + 0.5 * np.log(r2[1])
        np.testing.assert_allclose(lam[:, :, j], ref, rtol=1e-5)


def test_single_token_block_spread_is_minus_inf():
    k = rand_inputs(41, N=65)
    assert np.all(np.isneginf(pooling.block_spreads(k, k, 65)[:, :, 1]))


def test_e4m3_blocks_scale_and_error():
    x = rand_inputs(51, N=150, d=16)
    codes, e = pooling.e4m3_blocks(x, 150)
    back = e4m3.decode(codes) * np.exp2(e.repeat(64, axis=2))[..., None]
    for j in range(3):
        t = slice(64 * j, min(150, 64 * j + 64))
        amax = np.abs(x[:, :, t]).max(axis=(2, 3))
        assert np.all(amax * np.exp2(-e[:, :, j]) <= 448)
        assert np.all(amax * np.exp2(-e[:, :, j]) > 224)   # uses the top binade
        err = np.abs(back[:, :, t] - x[:, :, t])
        # relative half-ulp of e4m3 (2^-4) for normals, absolute 2^-10 * 2^e below
        tol = np.maximum(np.abs(x[:, :, t]) * 2.0 ** -4,
                         2.0 ** -10 * np.exp2(e[:, :, j])[:, :, None, None])
        assert np.all(err <= tol)
    assert np.all(codes[:, :, 150:] == 0)
