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


def test_covariance_norm_rank_one_closed_form():
    # block 0: keys move along one direction u, so H_0 = u w^T with
    # w = sum_n (c_n - c_mean) v_n; block 1: constant keys, H_1 = 0.
    # H_bar = H_0 / 2, so both deviations have norm |u| |w| / 2.
    rng = np.random.default_rng(61)
    d, blk = 5, 8
    u = rng.integers(-3, 4, d).astype(np.float64)
    c = rng.integers(-4, 5, blk).astype(np.float64)
    k = np.zeros((1, 1, 2 * blk, d), np.float32)
    k[0, 0, :blk] = 1.0 + c[:, None] * u[None, :]
    k[0, 0, blk:] = rng.integers(-2, 3, d)
    v = rng.integers(-3, 4, (1, 1, 2 * blk, d)).astype(np.float32)
    cm = sum(c) / blk
    w = [sum((c[n] - cm) * float(v[0, 0, n, o]) for n in range(blk)) for o in range(d)]
    ref = math.sqrt(sum(x * x for x in u)) * math.sqrt(sum(x * x for x in w)) / 2
    lnm = pooling.covariance_norms(k, v, 2 * blk, blk)
    np.testing.assert_allclose(np.exp(lnm[0, 0]), [ref, ref], rtol=1e-12)


def test_covariance_norm_diagonal_closed_form():
    # each block holds, per dimension i, a token pair k = base +- a e_i,
    # v = c +- b e_i: the keys average to base and H_j = diag(2 a b), so
    # M_j = max_i |2 a_ji b_ji - mean_j(2 a_ji b_ji)|.
    rng = np.random.default_rng(62)
    d, nb = 4, 3
    blk = 2 * d
    a = rng.integers(1, 5, (nb, d)).astype(np.float64)
    b = rng.integers(-4, 5, (nb, d)).astype(np.float64)
    k = np.zeros((1, 1, nb * blk, d), np.float32)
    v = np.zeros((1, 1, nb * blk, d), np.float32)
    for j in range(nb):
        base = rng.integers(-3, 4, d)
        for i in range(d):
            cvec = rng.integers(-3, 4, d)
            for s, t in ((1, 2 * i), (-1, 2 * i + 1)):
                k[0, 0, j * blk + t] = base
                k[0, 0, j * blk + t, i] += s * a[j, i]
                v[0, 0, j * blk + t] = cvec
                v[0, 0, j * blk + t, i] += s * b[j, i]
    h = 2 * a * b
    ref = [max(abs(h[j, i] - sum(h[:, i]) / nb) for i in range(d)) for j in range(nb)]
    lnm = pooling.covariance_norms(k, v, nb * blk, blk)
    np.testing.assert_allclose(np.exp(lnm[0, 0]), ref, rtol=1e-12)


def test_covariance_norm_invariances():
    k, v = rand_inputs(63, N=200, d=6), rand_inputs(64, N=200, d=6)
    base = pooling.covariance_norms(k, v, 200)
    # a constant shift of one block's keys leaves its centred moment unchanged
    k2 = k.copy()
    k2[:, :, 64:128] += np.float32(0.5)
    np.testing.assert_allclose(pooling.covariance_norms(k2, v, 200), base, rtol=1e-9)
    # scaling V by c scales every M_j by |c|
    np.testing.assert_allclose(pooling.covariance_norms(k, np.float32(-2.0) * v, 200), base + math.log(2.0),
                               rtol=1e-9)
    # identical blocks (a power-of-two count, so the mean is exact): M_j = 0
    blockv = v[:, :, :64]
    same = np.concatenate([k[:, :, :64]] * 4, axis=2), np.concatenate([blockv] * 4, axis=2)
    assert np.all(np.isneginf(pooling.covariance_norms(*same, 256)))


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
