"""Pins for the routing oracle: exact integer scores, exhaustive top-k,
LVSA rotation and window invariants, Triage tier structure."""

import itertools
import math

import numpy as np
import pytest

from oracle import routing
from workloads import get_workload, tile_major_coords, block_frame_ranges


def int_feats(rng, shape, lo=-3, hi=4):
    return rng.integers(lo, hi, shape).astype(np.float32)


def test_scores_exact_on_integers():
    rng = np.random.default_rng(0)
    q, k = int_feats(rng, (2, 3, 7, 5)), int_feats(rng, (2, 3, 9, 5))
    s = routing.block_scores(q, k)
    ref = np.einsum("bhai,bhji->bhaj", q.astype(np.int64), k.astype(np.int64))
    assert np.array_equal(s, ref.astype(np.float64))


def test_scores_fold_in_dimension_order():
    q = np.array([[1.0, 1.0, 1.0, 1.0]], np.float32)
    k = np.array([[2.0 ** 60, 1.0, 1.0, -(2.0 ** 60)]], np.float32)
    assert routing.block_scores(q, k)[0, 0] == 0.0


def brute_topk(scores, k):
    """Among all k-subsets, the max-sum one; ties -> lexicographically smallest."""
    best, best_sum = None, None
    for sub in itertools.combinations(range(len(scores)), k):
        s = sum(int(scores[j]) for j in sub)
        if best_sum is None or s > best_sum:
            best, best_sum = sub, s
    return list(best)


@pytest.mark.parametrize("seed", range(6))
def test_topk_exhaustive(seed):
    rng = np.random.default_rng(seed)
    nb = 9
    q, kb = int_feats(rng, (1, 1, nb, 3), -2, 3), int_feats(rng, (1, 1, nb, 3), -2, 3)
    s = routing.block_scores(q, kb)[0, 0]
    for k in (1, 3, 5, 9):
        idx, cnt = routing.route_topk(q, kb, k)
        for a in range(nb):
            assert list(idx[0, 0, a]) == brute_topk(s[a], k)
            assert cnt[0, 0, a] == k


def test_topk_monotone_and_ties_low_index():
    rng = np.random.default_rng(9)
    q = np.ones((1, 1, 1, 1), np.float32)
    kb = np.array([3, 1, 3, 2, 3, 0], np.float32).reshape(1, 1, 6, 1)
    idx, _ = routing.route_topk(q, kb, 2)
    assert list(idx[0, 0, 0]) == [0, 2]
    for _ in range(20):
        kb = rng.standard_normal((1, 1, 20, 4)).astype(np.float32)
        q = rng.standard_normal((1, 1, 3, 4)).astype(np.float32)
        idx, _ = routing.route_topk(q, kb, 5)
        j = int(idx[0, 0, 0, 2])
        kb2 = kb.copy()
        kb2[0, 0, j] *= 2.0 if float(q[0, 0, 0] @ kb[0, 0, j]) > 0 else 0.5
        idx2, _ = routing.route_topk(q, kb2, 5)
        assert j in idx2[0, 0, 0]


@pytest.mark.parametrize("seed", range(4))
def test_topk_cov_exhaustive(seed):
    # integer scores and integer log-norms: every key is an exact integer
    rng = np.random.default_rng(100 + seed)
    nb = 9
    q, kb = int_feats(rng, (1, 1, nb, 3), -2, 3), int_feats(rng, (1, 1, nb, 3), -2, 3)
    kcov = rng.integers(-3, 4, (1, 1, nb)).astype(np.float32)
    s = routing.block_scores(q, kb)[0, 0]
    for scale in (1.0, 2.0):
        for k in (1, 4, 9):
            idx, cnt = routing.route_topk_cov(q, kb, kcov, scale, k)
            for a in range(nb):
                key = [scale * s[a, j] + float(kcov[0, 0, j]) for j in range(nb)]
                assert list(idx[0, 0, a]) == brute_topk(key, k)
                assert cnt[0, 0, a] == k


def test_topk_cov_equal_norms_is_topk():
    rng = np.random.default_rng(110)
    q = rng.standard_normal((2, 2, 12, 8)).astype(np.float32)
    kb = rng.standard_normal((2, 2, 12, 8)).astype(np.float32)
    kcov = np.full((2, 2, 12), 1.25, np.float32)
    a, _ = routing.route_topk_cov(q, kb, kcov, 1.0, 5)
    b, _ = routing.route_topk(q, kb, 5)
    assert np.array_equal(a, b)


def test_topk_cov_zero_queries_rank_by_norm():
    # all scores 0: the key is ln M_j alone; -inf (M_j = 0) blocks come last
    kcov = np.array([0.5, -np.inf, 2.0, 0.5, -1.0, -np.inf, 3.0], np.float32).reshape(1, 1, 7)
    q = np.zeros((1, 1, 2, 3), np.float32)
    kb = np.ones((1, 1, 7, 3), np.float32)
    for k, want in ((3, [0, 2, 6]), (5, [0, 2, 3, 4, 6]), (6, [0, 1, 2, 3, 4, 6])):
        idx, _ = routing.route_topk_cov(q, kb, kcov, 1.0, k)
        assert list(idx[0, 0, 0]) == want and list(idx[0, 0, 1]) == want


def brute_error(q, kb_tokens, kbar_j, scale):
    """E = sum_n (exp(scale q.k_n) - exp(scale q.kbar_j))^2 straight from the definition."""
    c = math.exp(scale * sum(float(a) * float(b) for a, b in zip(q, kbar_j)))
    return sum((math.exp(scale * sum(float(a) * float(b) for a, b in zip(q, kn))) - c) ** 2 for kn in kb_tokens)


def test_error_logs_brute_force():
    rng = np.random.default_rng(120)
    blk, d, N = 4, 3, 11                      # blocks of 4, 4, 3 tokens
    k = rng.standard_normal((1, 2, 12, d)).astype(np.float32)
    q = rng.standard_normal((1, 2, 3, d)).astype(np.float32)
    kbar = np.stack([k[:, :, 4 * j:min(N, 4 * j + 4)].mean(axis=2) for j in range(3)], axis=2).astype(np.float32)
    for scale in (1.0, 0.7):
        L = routing.error_logs(q, k, kbar, N, scale, blk)
        for h in range(2):
            for a in range(3):
                for j in range(3):
                    toks = k[0, h, 4 * j:min(N, 4 * j + 4)]
                    E = brute_error(q[0, h, a], toks, kbar[0, h, j], float(np.float32(scale)))
                    c = float(np.float32(scale)) * sum(float(x) * float(y) for x, y in zip(q[0, h, a], kbar[0, h, j]))
                    assert abs(L[0, h, a, j] + 2 * c - math.log(E)) < 1e-9


def test_error_logs_two_token_closed_form():
    # keys kbar +- u: delta = +-t with t = q.u, and
    # expm1(t)^2 + expm1(-t)^2 = 2 cosh(2t) - 4 cosh(t) + 2
    q = np.array([[[[0.5, -1.0, 2.0]]]], np.float32)
    u = np.array([0.25, 0.5, -0.125], np.float32)
    base = np.array([1.0, 2.0, -1.0], np.float32)
    k = np.stack([base + u, base - u])[None, None].astype(np.float32)
    L = routing.error_logs(q, k, base[None, None, None, :], 2, 1.0, 2)
    t = float(q[0, 0, 0] @ u)
    assert abs(L[0, 0, 0, 0] - math.log(2 * math.cosh(2 * t) - 4 * math.cosh(t) + 2)) < 1e-12


def test_error_logs_degenerate_blocks_are_minus_inf():
    rng = np.random.default_rng(121)
    k = rng.standard_normal((1, 1, 8, 4)).astype(np.float32)
    k[0, 0, 4:8] = k[0, 0, 4]                 # block 1: four identical keys
    N = 8
    kbar = np.stack([k[:, :, 0:4].mean(axis=2), k[:, :, 4:5].mean(axis=2)], axis=2).astype(np.float32)
    q = rng.standard_normal((1, 1, 2, 4)).astype(np.float32)
    L = routing.error_logs(q, k, kbar, N, 1.0, 4)
    assert np.all(np.isfinite(L[..., 0])) and np.all(np.isneginf(L[..., 1]))
    # a one-token tail block
    L1 = routing.error_logs(q, k[:, :, :5], kbar, 5, 1.0, 4)
    assert np.all(np.isneginf(L1[..., 1]))


def test_route_error_follows_the_error_to_size_ratio():
    # brute-force E / n_j from the definition, then the first k by (-ratio, j)
    rng = np.random.default_rng(122)
    blk, d, N, nb = 4, 3, 22, 6                # last block holds 2 tokens
    for trial in range(4):
        k = rng.standard_normal((1, 1, nb * blk, d)).astype(np.float32)
        q = rng.standard_normal((1, 1, nb, d)).astype(np.float32)
        n = np.array([min(blk, N - blk * j) for j in range(nb)], np.int32)
        kbar = np.stack([k[:, :, blk * j:blk * j + n[j]].mean(axis=2) for j in range(nb)], axis=2).astype(np.float32)
        L = routing.error_logs(q, k, kbar, N, 1.0, blk)
        for kk in (1, 3, 5):
            idx, cnt = routing.route_error(q, kbar, n, L.astype(np.float32), 1.0, kk)
            for a in range(nb):
                ratio = [brute_error(q[0, 0, a], k[0, 0, blk * j:blk * j + n[j]], kbar[0, 0, j], 1.0) / n[j]
                         for j in range(nb)]
                want = sorted(sorted(range(nb), key=lambda j: (-ratio[j], j))[:kk])
                assert list(idx[0, 0, a]) == want and cnt[0, 0, a] == kk


def test_route_error_equal_logs_is_topk():
    rng = np.random.default_rng(123)
    q = rng.standard_normal((1, 2, 10, 8)).astype(np.float32)
    kb = rng.standard_normal((1, 2, 10, 8)).astype(np.float32)
    L = np.full((1, 2, 10, 10), -3.5, np.float32)
    a, _ = routing.route_error(q, kb, np.full(10, 64, np.int32), L, 1.0, 4)
    b, _ = routing.route_topk(q, kb, 4)
    assert np.array_equal(a, b)


def test_lvsa_anchor_rotation_covers_each_block_once():
    nb, anchors, phase = 1975, 8, 117
    P = nb // anchors
    seen = np.zeros(nb, int)
    for s in range(P):
        seen[routing.lvsa_anchor_set(nb, anchors, phase, s)] += 1
    assert np.all(seen[:anchors * P] == 1)
    assert np.all(seen[anchors * P:] == 0)


def test_lvsa_window_symmetric_and_contains_self():
    wl = get_workload(4, small=True)
    lo, hi = block_frame_ranges(tile_major_coords(wl.T, wl.Y, wl.X))
    idx, cnt = routing.route_lvsa(lo, hi, wl.window, 0, 0, 0)     # window only
    nb = wl.nb
    M = np.zeros((nb, nb), bool)
    for a in range(nb):
        M[a, idx[a, :cnt[a]]] = True
        assert M[a, a]
        assert np.all(np.diff(idx[a, :cnt[a]]) > 0)
        assert np.all(idx[a, cnt[a]:] == -1)
    assert np.array_equal(M, M.T)


def test_lvsa_window_closed_form_on_aligned_blocks():
    # 8 frames of 8x8: every block is one 4x4x4 tile inside a 4-frame group.
    lo, hi = block_frame_ranges(tile_major_coords(12, 8, 8))
    assert np.all(hi - lo == 3)
    idx, cnt = routing.route_lvsa(lo, hi, 2, 0, 0, 0)
    group = lo // 4
    for a in range(len(lo)):
        ref = np.nonzero(np.abs(group - group[a]) <= 1)[0]
        assert list(idx[a, :cnt[a]]) == list(ref)


def test_lvsa_anchors_added_to_every_row():
    wl = get_workload(4, small=True)
    lo, hi = block_frame_ranges(tile_major_coords(wl.T, wl.Y, wl.X))
    anc = routing.lvsa_anchor_set(wl.nb, wl.anchors, 1, 2)
    idx, cnt = routing.route_lvsa(lo, hi, wl.window, wl.anchors, 1, 2)
    for a in range(wl.nb):
        assert set(anc) <= set(idx[a, :cnt[a]])


def test_triage_tiers_partition_and_counts():
    rng = np.random.default_rng(4)
    nb = 40
    q, kb = rng.standard_normal((1, 2, nb, 8)).astype(np.float32), rng.standard_normal((1, 2, nb, 8)).astype(np.float32)
    lam = rng.standard_normal((1, 2, nb)).astype(np.float32)
    n = np.full(nb, 64, np.int32)
    n[-1] = 17
    ri, rc, si, sc = routing.route_triage(q, kb, lam, n, 1.0, 16, 6)
    assert np.all(rc == 6) and np.all(sc == 10)
    for b, h, a in itertools.product(range(1), range(2), range(nb)):
        r, s = set(ri[b, h, a]), set(si[b, h, a])
        assert not (r & s) and len(r) == 6 and len(s) == 10
        eskip = routing.block_scores(q, kb)[b, h, a] + lam[b, h].astype(np.float64)
        keep = np.lexsort((np.arange(nb), -eskip))[:16]
        assert r | s == set(keep.tolist())


def test_triage_equal_spreads_give_nested_topk():
    rng = np.random.default_rng(5)
    nb = 30
    q, kb = rng.standard_normal((1, 1, nb, 8)).astype(np.float32), rng.standard_normal((1, 1, nb, 8)).astype(np.float32)
    lam = np.full((1, 1, nb), 0.25, np.float32)
    n = np.full(nb, 64, np.int32)
    ri, _, si, _ = routing.route_triage(q, kb, lam, n, 1.0, 12, 5)
    top12, _ = routing.route_topk(q, kb, 12)
    top5, _ = routing.route_topk(q, kb, 5)
    for a in range(nb):
        assert list(ri[0, 0, a]) == list(top5[0, 0, a])
        assert sorted(set(ri[0, 0, a]) | set(si[0, 0, a])) == list(top12[0, 0, a])
