"""Pins for the SparsePR probe-fitted residual oracle."""

import numpy as np

from oracle import attention, residual


def test_probe_rows_one_per_block_inside_the_valid_rows():
    N, nb = 150, 3                                   # blocks of 64, 64, 22 rows
    for phase in (0, 5, 63):
        rows = residual.probe_rows(N, nb, phase)
        assert len(rows) == nb
        for a, r in enumerate(rows):
            assert 64 * a <= r < min(N, 64 * a + 64)
    assert not np.array_equal(residual.probe_rows(N, nb, 0), residual.probe_rows(N, nb, 1))


def test_fit_recovers_an_exact_low_rank_affine_map():
    # R = b0 + X B0 with B0 = U V^T (rank r) and b0 in span(V): with no ridge
    # the fit and the subspace restriction give back B0 and b0 exactly
    rng = np.random.default_rng(30)
    M, d, r = 200, 16, 3
    X = rng.standard_normal((M, d))
    V, _ = np.linalg.qr(rng.standard_normal((d, r)))
    U = rng.standard_normal((d, r))
    B0 = U @ V.T
    b0 = V @ rng.standard_normal(r)
    R = b0 + X @ B0
    W, c = residual.fit_residual(X, R, 0.0, r)
    np.testing.assert_allclose(W, B0, atol=1e-10)
    np.testing.assert_allclose(c, b0, atol=1e-10)


def test_ridge_equals_augmented_least_squares():
    # the penalised normal equations against lstsq on [Xc; sqrt(lam) I]
    rng = np.random.default_rng(31)
    M, d = 60, 8
    X = rng.standard_normal((M, d))
    R = rng.standard_normal((M, d))
    ridge = 0.3
    W, c = residual.fit_residual(X, R, ridge, d)      # full rank: P = I
    Xc, Rc = X - X.mean(0), R - R.mean(0)
    lam = ridge * np.trace(Xc.T @ Xc) / d
    A = np.vstack([Xc, np.sqrt(lam) * np.eye(d)])
    Bls = np.linalg.lstsq(A, np.vstack([Rc, np.zeros((d, d))]), rcond=None)[0]
    np.testing.assert_allclose(W, Bls, atol=1e-10)
    np.testing.assert_allclose(c, R.mean(0) - X.mean(0) @ Bls, atol=1e-10)


def test_subspace_is_the_top_singular_directions():
    # residuals along two known directions with clearly separated energy
    rng = np.random.default_rng(32)
    M, d = 100, 10
    e = np.eye(d)
    R = np.outer(rng.standard_normal(M) * 5, e[2]) + np.outer(rng.standard_normal(M) * 3, e[7]) \
        + 1e-3 * rng.standard_normal((M, d))
    X = rng.standard_normal((M, d))
    W, c = residual.fit_residual(X, R, 0.1, 2)
    # every correction lies in span(e2, e7)
    mask = np.ones(d, bool); mask[[2, 7]] = False
    assert np.abs(W[:, mask]).max() < 1e-3 and np.abs(c[mask]).max() < 1e-3


def test_exact_sparse_output_is_left_unchanged():
    rng = np.random.default_rng(33)
    N, d = 150, 8
    q, k, v = (np.pad(rng.standard_normal((1, 1, N, d)) * 0.5, ((0, 0), (0, 0), (0, 42), (0, 0))) for _ in range(3))
    Od, _ = attention.dense_attention(q, k, v, N, 1.0)
    out, fits, dense = residual.probe_correct(q, k, v, N, 1.0, Od, 3, 1e-3, 4)
    np.testing.assert_allclose(out, Od, atol=1e-12)
    W, c = fits[(0, 0)]
    assert np.abs(W).max() < 1e-12 and np.abs(c).max() < 1e-12


def test_probe_dense_rows_match_dense_attention():
    rng = np.random.default_rng(34)
    N, d = 100, 8
    q, k, v = (np.pad(rng.standard_normal((1, 1, N, d)), ((0, 0), (0, 0), (0, 28), (0, 0))) for _ in range(3))
    Od, _ = attention.dense_attention(q, k, v, N, 0.7)
    rows = residual.probe_rows(N, 2, 9)
    np.testing.assert_allclose(residual.probe_dense(q[0, 0], k[0, 0], v[0, 0], N, 0.7, rows), Od[0, 0, rows],
                               atol=1e-12)


def test_quality_probe_correction_reduces_the_error():
    # report-only page claim (the probe fit recovers part of the residual),
    # asserted loosely on the reduced Wan-like layer with centroid compensation
    from oracle import pooling, routing
    from workloads import get_workload, make_qkv
    wl = get_workload(2, small=True)
    q, k, v, _ = make_qkv(wl)
    po = pooling.pool(q, k, v, wl.N)
    idx, cnt = routing.route_topk(po["qbar"], po["kbar"], wl.topk)
    Os, _ = attention.sparse_attention(q, k, v, wl.N, 1.0, 0, po, idx, cnt)
    Od, _ = attention.dense_attention(q, k, v, wl.N, 1.0)
    Oc, _, _ = residual.probe_correct(q, k, v, wl.N, 1.0, Os, 0, 1e-3, 8)
    assert np.linalg.norm(Oc - Od) < 0.95 * np.linalg.norm(Os - Od)
