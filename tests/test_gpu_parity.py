"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Routing indices must match bit for bit; outputs within 1e-2 (bf16) and 1e-4
(fp32) max-abs.  Reduced grids are compared element by element; the full
workload sizes are compared on sampled query blocks and head subsets.
"""

import numpy as np
import pytest
import torch

from oracle import attention, pooling, routing
from workloads import get_workload, block_frame_ranges, lvsa_anchor_phase
from workloads.configs import WORKLOADS
import gpu_cases as gc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_present():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import free_block_sparse_attn_amd as fbsa
    assert fbsa.abi_version() == 9


def medium(wid):
    """Several 64-wide centroid tiles and a ragged tail, oracle-sized."""
    grids = {2: (9, 24, 41), 3: (9, 20, 45), 4: (29, 16, 19), 5: (9, 20, 45)}
    return WORKLOADS[wid].small(*grids[wid], H=2)


def check_pool(wl, pooled_o, res, v=None):
    assert np.array_equal(res["kcount"], pooled_o["kcount"])
    for n in ("qbar", "kbar", "vbar"):
        assert np.array_equal(res[n], pooled_o[n]), n          # bit-exact contract
    if "cent" in res:
        # fp16 high part and residual of the fp32 means (numpy's fp16 cast is
        # round-to-nearest-even); rows nb .. nbc-1 zero
        nb = pooled_o["kbar"].shape[2]
        for p, n in ((0, "kbar"), (2, "vbar")):
            m = pooled_o[n].astype(np.float32)
            hi = m.astype(np.float16)
            lo = (m - hi.astype(np.float32)).astype(np.float16)
            assert np.array_equal(res["cent"][:, :, p, :nb], hi), n
            assert np.array_equal(res["cent"][:, :, p + 1, :nb], lo), n
        assert not np.any(res["cent"][:, :, :, nb:]), "centroid pad rows"
    if "v16" in res and v is not None:
        # fp16 copy of the (bf16-exact) values, pad rows zero
        assert np.array_equal(res["v16"][:, :, :wl.N], v[:, :, :wl.N].astype(np.float16))
        assert not np.any(res["v16"][:, :, wl.N:]), "v16 pad rows"
    if "hbar" in res and "hbar" in pooled_o:
        # value-major mean moment; fp32 MFMA sums of bf16 products against fp64
        ref = np.swapaxes(pooled_o["hbar"], -1, -2)
        err = np.abs(res["hbar"].astype(np.float64) - ref)
        assert err.max() <= 1e-4 * np.abs(ref).max(), err.max()
    if "kmom" in res:
        # fp16 copy of H_j 2^-e_j: the largest entry of each block in
        # [2^14, 2^15] (2^15 by rounding up), values within fp16 rounding
        # (2^-11 relative) plus the fp32 MFMA sums' error of the hi + lo bf16
        # centred keys
        ex = res["kmom_exp"].astype(np.int64)
        amax = np.abs(res["kmom"]).max(axis=(-1, -2)).astype(np.float64)
        assert np.all(((amax >= 2.0 ** 14) & (amax <= 2.0 ** 15)) | ((amax == 0) & (ex == 0))), (amax.min(), amax.max())
        ref = np.swapaxes(pooled_o["kmom"], -1, -2)               # value-major layout
        got = res["kmom"].astype(np.float64) * np.exp2(ex)[..., None, None]
        err = np.abs(got - ref)
        assert np.all(err <= 2.0 ** -11 * np.abs(ref) + 1e-4 * np.abs(ref).max()), err.max()
    if "kcov" in res and "kcov" in pooled_o:
        # ln M_j: the block moment rebuilt in fp32 MFMA sums, H_bar subtracted,
        # up to 32 fp32 Lanczos steps and Sturm multisection of the tridiagonal (a
        # Ritz value, from below) against the fp64 singular value
        ref = pooled_o["kcov"]
        assert np.array_equal(np.isneginf(res["kcov"]), np.isneginf(ref))
        fin = np.isfinite(ref)
        err = np.abs(res["kcov"][fin].astype(np.float64) - ref[fin])
        assert err.max() <= 1e-3, err.max()
    if "klam" in res:
        np.testing.assert_allclose(res["klam"], pooled_o["klam"], rtol=1e-5, atol=1e-5)
    if "q4" in res and "q4" in pooled_o:
        # MXFP4 codes and scale exponents: bit-exact
        for n in ("q4", "qs4", "k4", "ks4", "v4", "vs4"):
            assert np.array_equal(res[n], pooled_o[n]), n
    if "q8" in res:
        for i, n in enumerate(("q", "k", "v")):
            assert np.array_equal(res[n + "8"], pooled_o[n + "8"]), n
            assert np.array_equal(res["exp8"][..., i], pooled_o[n + "exp"]), n


def check_route(wl, pooled_o, res, coords, step=0, scale=1.0):
    """Stage-wise (the GPU's pooled features) and end-to-end (the oracle's)."""
    for feats in (res, pooled_o):
        if wl.rule == "topk":
            idx, cnt = routing.route_topk(feats["qbar"], feats["kbar"], wl.topk)
            assert np.array_equal(res["idx"], idx)
            assert np.array_equal(res["cnt"], cnt)
        elif wl.rule == "error":
            # GPU error logs L(a, j) (stored key-block-major) against the fp64
            # definition; selection bit-exact on the GPU's logs
            elog = np.swapaxes(res["ekey"], -1, -2)
            idx, cnt = routing.route_error(res["qbar"], res["kbar"], res["kcount"], elog, scale, wl.topk)
            assert np.array_equal(res["idx"], idx)
            assert np.array_equal(res["cnt"], cnt)
            break          # the logs are not bit-reproducible: stage-wise only
        elif wl.rule == "topk_cov":
            idx, cnt = routing.route_topk_cov(feats["qbar"], feats["kbar"], feats["kcov"], scale, wl.topk)
            assert np.array_equal(res["idx"], idx)
            assert np.array_equal(res["cnt"], cnt)
            break          # ln M_j is not bit-reproducible: stage-wise only
        elif wl.rule == "lvsa":
            lo, hi = block_frame_ranges(coords)
            idx, cnt = routing.route_lvsa(lo, hi, wl.window, wl.anchors,
                                          lvsa_anchor_phase(wl.wid, wl.anchor_period), step)
            B, H = res["cnt"].shape[:2]
            for b in range(B):
                for h in range(H):
                    assert np.array_equal(res["cnt"][b, h], cnt)
                    assert np.array_equal(res["idx"][b, h, :, :idx.shape[1]], idx)
                    assert np.all(res["idx"][b, h, :, idx.shape[1]:] == -1)
            break
        else:
            ri, rc, si, sc = routing.route_triage(feats["qbar"], feats["kbar"], feats["klam"],
                                                  feats["kcount"], scale, wl.n_keep, wl.n_refine)
            assert np.array_equal(res["idx"][..., :ri.shape[-1]], ri)
            assert np.array_equal(res["cnt"], rc)
            assert np.array_equal(res["idx2"], si)
            assert np.array_equal(res["cnt2"], sc)
            break          # klam is not bit-reproducible: stage-wise only


ELOG_TOL = 1e-3   # |L_gpu - L| : three bf16 hi/lo MFMA passes (~16 bits per factor), fp32 sums


def check_error_logs(wl, res, elog, k, rows=None, scale=1.0):
    """L(a, j) of the query blocks `rows` (all when None) against the oracle's fp64 value."""
    sel = np.arange(wl.nb) if rows is None else np.asarray(rows)
    ref = routing.error_logs(res["qbar"][:, :, sel], k, res["kbar"], wl.N, scale)
    got = elog[:, :, sel]
    assert np.array_equal(np.isneginf(got), np.isneginf(ref))
    fin = np.isfinite(ref)
    err = np.abs(got[fin].astype(np.float64) - ref[fin])
    assert err.max() <= ELOG_TOL, err.max()
    return err.max()


def check_out(wl, res, ref, rows):
    """Outputs row by row against gc.row_tol (plus the oracle's skim slack), lse."""
    worst = 0.0
    for (b, h, a), (o, l, slack) in ref.items():
        r0, r1 = 64 * a, min(wl.N, 64 * a + 64)
        err = np.abs(res["out"][b, h, r0:r1] - o).max(axis=1)
        bar = gc.row_tol(wl.dtype, o) + slack
        lerr = np.abs(res["lse"][b, h, r0:r1] - l)
        lbar = gc.LSE_TOL[wl.dtype] + gc.LSE_REL[wl.dtype] * np.abs(l)
        worst = max(worst, err.max())
        i = int(np.argmax(err - bar))
        assert err[i] <= bar[i], (b, h, a, i, err[i], bar[i])
        i = int(np.argmax(lerr - lbar))
        assert lerr[i] <= lbar[i], (b, h, a, i, lerr[i], lbar[i])
    return worst


def all_rows(wl):
    return [(b, h, a) for b in range(wl.B) for h in range(wl.H) for a in range(wl.nb)]


@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("size", ["small", "medium"])
def test_parity_reduced(wid, size):
    if size == "medium" and wid == 1:
        pytest.skip("the tiny workload is already full size")
    wl = get_workload(wid, small=True) if size == "small" else medium(wid)
    print(f"\n[case] {wl.name} size={size} N={wl.N} H={wl.H} nb={wl.nb}", flush=True)
    (q, k, v), dev, coords = gc.inputs(wl)
    steps = range(wl.steps) if wl.rule == "lvsa" else [0]
    pooled_o = gc.oracle_pool(wl, q, k, v)
    for step in steps:
        res = gc.run_gpu(wl, dev, coords, step=step)
        check_pool(wl, pooled_o, res, v)
        check_route(wl, pooled_o, res, coords, step)
        ref = gc.oracle_rows(wl, q, k, v, pooled_o, res, all_rows(wl))
        worst = check_out(wl, res, ref, all_rows(wl))
        # pad rows are written as zero
        assert np.all(res["out"][:, :, wl.N:] == 0)
        print(f"[ok] step={step} max|err|={worst:.3e}", flush=True)


@pytest.mark.parametrize("grid,rem", [((5, 11, 11), 2), ((6, 12, 14), 0)])
def test_parity_order1_workgroup_tails(grid, rem):
    """The block first-order form runs four query blocks of a head per
    workgroup and streams the union of their compensated blocks' moments;
    these heads leave 2 and 0 query blocks over in the last group (the small,
    medium and full-size cases leave 1 and 3), and three heads put groups of
    consecutive heads side by side."""
    wl = WORKLOADS[3].small(*grid, H=3)
    assert wl.nb % 4 == rem
    print(f"\n[case] {wl.name} N={wl.N} H={wl.H} nb={wl.nb}", flush=True)
    (q, k, v), dev, coords = gc.inputs(wl)
    pooled_o = gc.oracle_pool(wl, q, k, v)
    res = gc.run_gpu(wl, dev, coords)
    check_pool(wl, pooled_o, res, v)
    check_route(wl, pooled_o, res, coords, 0)
    ref = gc.oracle_rows(wl, q, k, v, pooled_o, res, all_rows(wl))
    worst = check_out(wl, res, ref, all_rows(wl))
    assert np.all(res["out"][:, :, wl.N:] == 0)
    print(f"[ok] max|err|={worst:.3e}", flush=True)


@pytest.mark.parametrize("sc", [0.37, 4.0])
@pytest.mark.parametrize("kind", ["topk", "error", "cov", "triage", "order1", "global", "lvsa", "mxfp4"])
def test_parity_softmax_scale(kind, sc):
    """Softmax scales other than 1 through routing (the error pass, the
    covariance key, Triage's tiers), every compensation form, the skim tier
    and, for the top-k layer, the residual pass's dense probes.  At 4 the
    logits reach ~60: the running maximum's lazy rescale and overflow checks."""
    from dataclasses import replace
    wl = replace(_batch2_workload(kind), B=1)
    print(f"\n[case] {wl.name} scale={sc} N={wl.N} H={wl.H} nb={wl.nb}", flush=True)
    (q, k, v), dev, coords = gc.inputs(wl)
    pooled_o = gc.oracle_pool(wl, q, k, v)
    res = gc.run_gpu(wl, dev, coords, scale=sc)
    check_route(wl, pooled_o, res, coords, 0, scale=sc)
    if kind == "error":
        check_error_logs(wl, res, np.swapaxes(res["ekey"], -1, -2), k, scale=sc)
    ref = gc.oracle_rows(wl, q, k, v, pooled_o, res, all_rows(wl), scale=sc)
    worst = check_out(wl, res, ref, all_rows(wl))
    if kind == "topk":
        res, corr, fit = run_residual(wl, dev, coords, scale=sc)
        heads = {(0, h): np.arange(wl.N_pad) for h in range(wl.H)}
        worst = max(worst, check_residual(wl, q, k, v, res, corr, fit, heads, scale=sc))
    print(f"[ok] max|err|={worst:.3e}", flush=True)


@pytest.mark.parametrize("kind", ["topk", "lvsa", "triage", "order1", "global", "cov", "error", "mxfp4"])
def test_parity_single_head(kind):
    """H = 1 (and B = 1): no kernel may assume more than one head."""
    from dataclasses import replace
    wl = replace(_batch2_workload(kind), B=1, H=1)
    print(f"\n[case] {wl.name} H=1 N={wl.N} nb={wl.nb}", flush=True)
    (q, k, v), dev, coords = gc.inputs(wl)
    pooled_o = gc.oracle_pool(wl, q, k, v)
    res = gc.run_gpu(wl, dev, coords)
    check_pool(wl, pooled_o, res, v)
    check_route(wl, pooled_o, res, coords, 0)
    ref = gc.oracle_rows(wl, q, k, v, pooled_o, res, all_rows(wl))
    worst = check_out(wl, res, ref, all_rows(wl))
    assert np.all(res["out"][:, :, wl.N:] == 0)
    if kind == "topk":
        res, corr, fit = run_residual(wl, dev, coords)
        worst = max(worst, check_residual(wl, q, k, v, res, corr, fit, {(0, 0): np.arange(wl.N_pad)}))
    print(f"[ok] max|err|={worst:.3e}", flush=True)


@pytest.mark.parametrize("kind", ["topk", "triage", "error", "global", "mxfp4"])
def test_parity_no_ragged_tail(kind):
    """N a multiple of 64 (4 x 16 x 16 = 1024 tokens): the last block is full."""
    from dataclasses import replace
    wl = replace(_batch2_workload(kind), B=1, T=4, Y=16, X=16)
    assert wl.N % 64 == 0 and wl.N == wl.N_pad
    print(f"\n[case] {wl.name} N={wl.N} nb={wl.nb}", flush=True)
    (q, k, v), dev, coords = gc.inputs(wl)
    pooled_o = gc.oracle_pool(wl, q, k, v)
    res = gc.run_gpu(wl, dev, coords)
    check_pool(wl, pooled_o, res, v)
    check_route(wl, pooled_o, res, coords, 0)
    ref = gc.oracle_rows(wl, q, k, v, pooled_o, res, all_rows(wl))
    worst = check_out(wl, res, ref, all_rows(wl))
    if kind == "topk":
        res, corr, fit = run_residual(wl, dev, coords)
        heads = {(0, h): np.arange(wl.N_pad) for h in range(wl.H)}
        worst = max(worst, check_residual(wl, q, k, v, res, corr, fit, heads))
    print(f"[ok] max|err|={worst:.3e}", flush=True)


@pytest.mark.parametrize("kind", ["topk", "error", "order1", "global"])
def test_parity_one_kept_block(kind):
    """top-k = 1: capacity-1 lists, every other block compensated."""
    from dataclasses import replace
    wl = replace(_batch2_workload(kind), B=1, keep_pct=1)
    assert wl.topk == 1
    print(f"\n[case] {wl.name} topk=1 N={wl.N} nb={wl.nb}", flush=True)
    (q, k, v), dev, coords = gc.inputs(wl)
    pooled_o = gc.oracle_pool(wl, q, k, v)
    res = gc.run_gpu(wl, dev, coords)
    check_route(wl, pooled_o, res, coords, 0)
    assert np.all(res["cnt"] == 1)
    ref = gc.oracle_rows(wl, q, k, v, pooled_o, res, all_rows(wl))
    worst = check_out(wl, res, ref, all_rows(wl))
    if kind == "topk":
        res, corr, fit = run_residual(wl, dev, coords)
        heads = {(0, h): np.arange(wl.N_pad) for h in range(wl.H)}
        worst = max(worst, check_residual(wl, q, k, v, res, corr, fit, heads))
    print(f"[ok] max|err|={worst:.3e}", flush=True)


def _far_skim_lists(J, full):
    """List edit: block J moves to every query block's skim list (from its
    exact list, or in place of the last skim entry); the query blocks in
    `full` get no exact tile and every block skimmed."""
    def edit(idx, cnt, idx2, cnt2):
        idx, cnt, idx2, cnt2 = (t.cpu().numpy().copy() for t in (idx, cnt, idx2, cnt2))
        B, H, nq, _ = idx.shape
        new2 = np.zeros((B, H, nq, nq), np.int32)
        for b in range(B):
            for h in range(H):
                for a in range(nq):
                    ex = [int(x) for x in idx[b, h, a, :cnt[b, h, a]]]
                    sk = [int(x) for x in idx2[b, h, a, :cnt2[b, h, a]]]
                    if (b, h, a) in full:
                        ex, sk = [], list(range(nq))
                    elif J in ex:
                        ex.remove(J)
                        sk.append(J)
                    elif J not in sk:
                        sk = sk[:-1] + [J]
                    idx[b, h, a, :len(ex)] = sorted(ex)
                    cnt[b, h, a] = len(ex)
                    new2[b, h, a, :len(sk)] = sorted(sk)
                    cnt2[b, h, a] = len(sk)
        return tuple(torch.from_numpy(x).cuda() for x in (idx, cnt, new2, cnt2))
    return edit


def test_skim_far_above_reference():
    """Skim tiles whose logits lie ~100 binades above every logit a row saw
    before them (the skim tier's lazy rescale by ~2^-100), and query blocks
    with no exact tile and every block skimmed (no centroids: a skim tile
    sets those rows' first reference)."""
    from dataclasses import replace
    wl = replace(_batch2_workload("triage"), B=1)
    q, k, v, coords = gc.make_qkv(wl)
    J = wl.nb // 2
    # head 0: one shared direction lowers every row's logits against all
    # blocks but J by ~72 (~100 binades), so J's ordinary-sized logits lie far
    # above everything else (large logits would instead measure the
    # block-scaled MFMA's sums, whose error grows with their magnitude);
    # head 1 unchanged
    inJ = np.zeros(wl.N_pad, bool)
    inJ[64 * J:64 * J + 64] = True
    valid = np.arange(wl.N_pad) < wl.N
    q[0, 0, :wl.N, 0] += 6.0
    k[0, 0, valid & ~inJ, 0] -= 12.0
    q, k = (torch.from_numpy(x).to(torch.bfloat16).float().numpy() for x in (q, k))
    c2 = 1.4426950408889634
    s = np.einsum("nd,md->nm", q[0, 0, :wl.N].astype(np.float64), k[0, 0, :wl.N].astype(np.float64)) * c2
    iJ = inJ[:wl.N]
    assert np.min(s[:, iJ].max(axis=1) - s[:, ~iJ].max(axis=1)) > 40.0
    assert np.abs(s[:, iJ]).max() < 32.0
    dev = gc.to_device(wl, q, k, v)
    full = {(0, 0, 0), (0, 1, 0), (0, 1, wl.nb - 1)}
    print(f"\n[case] {wl.name} far skim block {J} N={wl.N} H={wl.H} nb={wl.nb}", flush=True)
    pooled_o = gc.oracle_pool(wl, q, k, v)
    res = gc.run_gpu(wl, dev, coords, edit=_far_skim_lists(J, full))
    assert all(J in gc.lists_of(res["idx2"], res["cnt2"], 0, h, a) for h in range(wl.H) for a in range(wl.nb))
    assert all(res["cnt"][0, h, a] == 0 and res["cnt2"][0, h, a] == wl.nb for (_, h, a) in full)
    ref = gc.oracle_rows(wl, q, k, v, pooled_o, res, all_rows(wl))
    worst = check_out(wl, res, ref, all_rows(wl))
    assert np.all(res["out"][:, :, wl.N:] == 0)
    print(f"[ok] max|err|={worst:.3e}", flush=True)


def _skim_length_lists(edit_len):
    """List edit: query block a keeps only edit_len(a) of its skim blocks,
    the lowest ones for even a and the highest (which hold the ragged last
    block when it is skimmed) for odd a; the dropped blocks are compensated."""
    def edit(idx, cnt, idx2, cnt2):
        idx2, cnt2 = (t.cpu().numpy().copy() for t in (idx2, cnt2))
        B, H, nq = cnt2.shape
        for b in range(B):
            for h in range(H):
                for a in range(nq):
                    sk = sorted(int(x) for x in idx2[b, h, a, :cnt2[b, h, a]])
                    n = min(edit_len(a), len(sk))
                    sk = sk[:n] if a % 2 == 0 else sk[len(sk) - n:]
                    idx2[b, h, a, :] = 0
                    idx2[b, h, a, :n] = sk
                    cnt2[b, h, a] = n
        return idx, cnt, torch.from_numpy(idx2).cuda(), torch.from_numpy(cnt2).cuda()
    return edit


@pytest.mark.parametrize("kind", ["triage", "mxfp4"])
def test_skim_list_lengths(kind):
    """Skim lists of every length from 0 to 5 (the skim loop pads odd lengths
    with a masked null tile and runs its row-block pipeline two tiles deep),
    with and without the ragged last block."""
    from dataclasses import replace
    wl = replace(_batch2_workload(kind), B=1)
    (q, k, v), dev, coords = gc.inputs(wl)
    print(f"\n[case] {wl.name} skim lists of length a % 6 N={wl.N} H={wl.H} nb={wl.nb}", flush=True)
    pooled_o = gc.oracle_pool(wl, q, k, v)
    res = gc.run_gpu(wl, dev, coords, edit=_skim_length_lists(lambda a: a % 6))
    assert sorted(set(int(c) for c in res["cnt2"].ravel())) == list(range(6))
    assert any(wl.nb - 1 in gc.lists_of(res["idx2"], res["cnt2"], 0, h, a)
               for h in range(wl.H) for a in range(1, wl.nb, 2))
    ref = gc.oracle_rows(wl, q, k, v, pooled_o, res, all_rows(wl))
    worst = check_out(wl, res, ref, all_rows(wl))
    print(f"[ok] max|err|={worst:.3e}", flush=True)


def _batch2_workload(kind):
    from dataclasses import replace
    from workloads import configs as C
    base = {"topk": C.SMALL[2], "lvsa": C.SMALL[4], "triage": C.SMALL[5], "order1": C.SMALL[3],
            "global": C.GLOBAL_ORDER1_SMALL, "cov": C.GLOBAL_COV_SMALL, "error": C.ERROR_ROUTED_SMALL,
            "mxfp4": C.TRIAGE_FP4_SMALL}[kind]
    return replace(base, B=2)


@pytest.mark.parametrize("kind", ["topk", "lvsa", "triage", "order1", "global", "cov", "error", "mxfp4"])
def test_parity_batch_of_two(kind):
    """B = 2: the (batch, head) indexing of pooling (moments, H-bar, covariance
    norms, fp8 / MXFP4 copies), routing (LVSA writes its shared lists for every
    batch and head; the error pass), the forward and, for the top-k layer, the
    residual pass."""
    wl = _batch2_workload(kind)
    wid = 2 if kind == "topk" else 0
    print(f"\n[case] {wl.name} B={wl.B} N={wl.N} H={wl.H} nb={wl.nb}", flush=True)
    (q, k, v), dev, coords = gc.inputs(wl)
    assert q.shape[0] == 2 and not np.array_equal(q[0], q[1])
    pooled_o = gc.oracle_pool(wl, q, k, v)
    res = gc.run_gpu(wl, dev, coords)
    check_pool(wl, pooled_o, res, v)
    check_route(wl, pooled_o, res, coords, 0)
    if kind == "error":
        check_error_logs(wl, res, np.swapaxes(res["ekey"], -1, -2), k)
    ref = gc.oracle_rows(wl, q, k, v, pooled_o, res, all_rows(wl))
    worst = check_out(wl, res, ref, all_rows(wl))
    assert np.all(res["out"][:, :, wl.N:] == 0)
    if wid == 2:
        res, corr, fit = run_residual(wl, dev, coords)
        heads = {(b, h): np.arange(wl.N_pad) for b in range(wl.B) for h in range(wl.H)}
        worst = max(worst, check_residual(wl, q, k, v, res, corr, fit, heads))
    print(f"[ok] max|err|={worst:.3e}", flush=True)


@pytest.mark.parametrize("wid", [2, 3, 4, 5])
def test_parity_full_size_sampled(wid):
    """Full workload shape in the benchmark's launch configuration; the
    oracle checks head subsets (pool, route) and sampled query blocks."""
    wl = WORKLOADS[wid]
    print(f"\n[case] full {wl.name} N={wl.N} H={wl.H} nb={wl.nb}", flush=True)
    (q, k, v), dev, coords = gc.inputs(wl)
    rng = np.random.default_rng(wid)
    heads = sorted(rng.choice(wl.H, 2, replace=False).tolist())
    steps = [0, wl.steps - 1] if wl.rule == "lvsa" else [0]
    for step in steps:
        res = gc.run_gpu(wl, dev, coords, step=step)
        sub = lambda x: x[:, heads]
        qs, ks, vs = sub(q), sub(k), sub(v)
        pooled_o = pooling.pool(qs, ks, vs, wl.N, spreads=wl.rule == "triage", fp8=wl.rule == "triage")
        rsub = {n: (x[:, heads] if n not in ("kcount",) else x) for n, x in res.items()}
        check_pool(wl, pooled_o, {n: rsub[n] for n in ("qbar", "kbar", "vbar", "kcount")})
        if wl.rule == "triage":
            check_pool(wl, pooled_o, {n: rsub[n] for n in ("klam", "q8", "k8", "v8", "exp8", "kcount",
                                                           "qbar", "kbar", "vbar")})
        check_route(wl, pooled_o, rsub, coords, step)
        rows = [(0, hi, int(a)) for hi in range(len(heads)) for a in rng.choice(wl.nb, 3, replace=False)]
        rows.append((0, 0, wl.nb - 1))                                  # ragged tail block
        if wl.comp == 1:
            mom = {}
            for hi in range(len(heads)):
                mom[hi] = pooling.block_moments(ks[:, hi:hi + 1], vs[:, hi:hi + 1], wl.N)[0, 0]
            pooled_o["kmom"] = np.stack([mom[i] for i in range(len(heads))])[None]
        ref = gc.oracle_rows(wl, qs, ks, vs, pooled_o, rsub, rows)
        worst = check_out(wl, rsub, ref, rows)
        print(f"[ok] step={step} max|err|={worst:.3e}", flush=True)


@pytest.mark.parametrize("wid", [2, 3, 4, 5])
def test_parity_full_head(wid):
    """One whole head at the full workload shape, element by element: every
    query block of the last head (the Triage layer: every fourth, its oracle
    costs ~1.4 s per query block), in the benchmark's launch configuration,
    against the oracle computed in parallel worker processes on the GPU's
    lists (routing is checked bit-exact on the same head).  Covers the long
    LVSA rows (at step 1; the sampled test takes steps 0 and 3) and the full
    kept-block bitmask."""
    wl = WORKLOADS[wid]
    step = 1 if wl.rule == "lvsa" else 0
    print(f"\n[case] full head {wl.name} N={wl.N} H={wl.H} nb={wl.nb} step={step}", flush=True)
    (q, k, v), dev, coords = gc.inputs(wl)
    res = gc.run_gpu(wl, dev, coords, step=step)
    h = wl.H - 1
    one = lambda x: x[:, h:h + 1]
    qs, ks, vs = one(q), one(k), one(v)
    pooled_o = gc.oracle_pool(wl, qs, ks, vs)
    rsub = {n: (x if n == "kcount" else x[:, h:h + 1]) for n, x in res.items()}
    check_pool(wl, pooled_o, {n: rsub[n] for n in rsub if n not in ("out", "lse", "idx", "cnt", "idx2", "cnt2")}, vs)
    check_route(wl, pooled_o, rsub, coords, step)
    rows = list(range(0, wl.nb, 4 if wl.rule == "triage" else 1))
    if rows[-1] != wl.nb - 1:
        rows.append(wl.nb - 1)                                     # the ragged tail block
    ref = gc.oracle_rows_parallel(wl, qs, ks, vs, pooled_o, rsub, rows)
    worst = check_out(wl, rsub, ref, rows)
    assert np.all(rsub["out"][:, :, wl.N:] == 0)
    print(f"[ok] {len(rows)} query blocks, max|err|={worst:.3e}", flush=True)


def test_full_tiny_is_elementwise():
    # the tiny workload at its full size is oracle-cheap: compare everything
    test_parity_reduced(1, "small")


@pytest.mark.parametrize("opts", [
    dict(moments=True, spreads=True, fp8=True),          # the general pooling kernel's moment phase
    dict(global_moment=True, spreads=True),              # streaming means, then the H_bar partial-sum pass
    dict(moments=True, global_moment=True, fp4=True),    # both moment forms at once
])
def test_pool_option_combinations(opts):
    """Pooling options requested together, which take the kernels no
    configured layer uses: every output against the oracle's pooling."""
    import free_block_sparse_attn_amd as fbsa
    from dataclasses import replace
    wl = replace(WORKLOADS[3].small(9, 20, 45), H=2)
    print(f"\n[case] pool {sorted(opts)} N={wl.N} nb={wl.nb}", flush=True)
    (q, k, v), (dq, dk, dv), _ = gc.inputs(wl)
    pooled = fbsa.sparse_attn_pool(dq, dk, dv, wl.N, **opts)
    torch.cuda.synchronize()
    res = gc.pool_results(pooled, wl.N_pad)
    pooled_o = pooling.pool(q, k, v, wl.N, moments=opts.get("moments", False), spreads=opts.get("spreads", False),
                            fp8=opts.get("fp8", False), hbar=opts.get("global_moment", False),
                            fp4=opts.get("fp4", False))
    for n in ("kmom", "hbar", "klam", "q8", "q4"):
        assert (n in res) == (n in pooled_o), n
    check_pool(wl, pooled_o, res, v)
    print("[ok]", flush=True)


@pytest.mark.parametrize("comp,sc", [(0, 1.0), (-1, 1.0), (0, 0.37), (0, 4.0)])
def test_parity_fp32_ragged(comp, sc):
    """The fp32 path (d = 64) on a grid with a ragged tail (1200 tokens: 19
    blocks, the last 48 long), with and without the centroid terms, at
    softmax scales through 4 (logits up to ~40 in log2 units)."""
    from dataclasses import replace
    wl = replace(WORKLOADS[1], T=5, Y=12, X=20, comp=comp)
    assert wl.dtype == "f32" and wl.N % 64 != 0
    print(f"\n[case] {wl.name} comp={comp} scale={sc} N={wl.N} nb={wl.nb}", flush=True)
    (q, k, v), dev, coords = gc.inputs(wl)
    pooled_o = gc.oracle_pool(wl, q, k, v)
    res = gc.run_gpu(wl, dev, coords, scale=sc)
    check_pool(wl, pooled_o, res, v)
    check_route(wl, pooled_o, res, coords, 0, scale=sc)
    ref = gc.oracle_rows(wl, q, k, v, pooled_o, res, all_rows(wl), scale=sc)
    worst = check_out(wl, res, ref, all_rows(wl))
    assert np.all(res["out"][:, :, wl.N:] == 0) and np.all(res["lse"][:, :, wl.N:] == 0)
    print(f"[ok] max|err|={worst:.3e}", flush=True)


@pytest.mark.parametrize("wid", [2, 3])
def test_deterministic(wid):
    wl = medium(wid)
    (q, k, v), dev, coords = gc.inputs(wl)
    r1 = gc.run_gpu(wl, dev, coords)
    r2 = gc.run_gpu(wl, dev, coords)
    for n in r1:
        assert np.array_equal(r1[n], r2[n]), n


def test_empty_and_single_token():
    import free_block_sparse_attn_amd as fbsa
    q = torch.zeros(1, 2, 0, 128, dtype=torch.bfloat16, device="cuda")
    pooled = fbsa.sparse_attn_pool(q, q, q, 0)
    assert pooled["qbar"].numel() == 0
    # one valid token: the output is that token's value.  The matrix core
    # multiplies fp16(v) = v (exact) by the weight p rounded to fp16 and the
    # denominator is the same rounded weight, so o = v fp16(p) / fp16(p) is v
    # up to fp32 rounding (2^-23 relative), which the bf16 store of the bf16
    # value v removes: o == v exactly.  lse = ln fp16(p) + the reference: the
    # token's logit within -ln(1 - 2^-11) (fp16 unit roundoff of the weight).
    x = torch.randn(1, 2, 64, 128, device="cuda").to(torch.bfloat16)
    x[:, :, 1:] = 7.0                                     # pad rows must not leak
    pooled = fbsa.sparse_attn_pool(x, x, x, 1)
    idx, cnt, _, _ = fbsa.sparse_attn_route(pooled, 1, fbsa.SA_ROUTE_TOPK, topk=1)
    for comp in (-1, 0):
        out, lse = fbsa.sparse_attn_fwd(x, x, x, 1, 1.0, comp, pooled, idx, cnt)
        torch.cuda.synchronize()
        v0 = x[:, :, 0].float()
        assert torch.equal(out[:, :, 0].float(), v0)
        logit = (v0 * v0).sum(-1)
        assert torch.all((lse[:, :, 0] - logit).abs() <= gc.LSE_TOL["bf16"])
        assert torch.all(out[:, :, 1:] == 0)


def test_topk_ties_at_the_cut():
    """Top-k with whole groups of equal scores straddling the k-th place: key
    blocks repeat five token patterns, so every row's 48 scores take five
    values about ten times each.  For every k the GPU lists must equal the
    oracle's (first k in the order (-score, j): the lower index wins a tie)."""
    import free_block_sparse_attn_amd as fbsa
    rng = np.random.default_rng(7)
    B, H, nb, d = 1, 2, 48, 128
    N = 64 * nb
    base = rng.standard_normal((5, 64, d)).astype(np.float32)
    k_np = np.stack([base[j % 5] for j in range(nb)], axis=0).reshape(1, 1, N, d).repeat(H, axis=1)
    q_np = rng.standard_normal((B, H, N, d)).astype(np.float32)
    to = lambda x: torch.from_numpy(x).to(torch.bfloat16).cuda()
    q, k = to(q_np), to(k_np)
    pooled = fbsa.sparse_attn_pool(q, k, k, N)
    qbar, kbar = pooled["qbar"].cpu().numpy(), pooled["kbar"].cpu().numpy()
    for kk in (1, 9, 10, 11, 13, 19, 20, 21, 29, 38, 40, 47, 48):
        idx, cnt, _, _ = fbsa.sparse_attn_route(pooled, N, fbsa.SA_ROUTE_TOPK, topk=kk)
        ri, rc = routing.route_topk(qbar, kbar, kk)
        assert np.array_equal(cnt.cpu().numpy(), rc), kk
        assert np.array_equal(idx.cpu().numpy()[..., :kk], ri), kk


@pytest.mark.parametrize("nb", [19, 300, 1100, 2100])
def test_route_one_sign_rows(nb):
    """Query blocks whose scores against every key block are all positive, all
    negative, or mixed (a third each), for top-k and for Triage's two
    selections.  All-positive rows have order keys that share the sign bit, so
    the threshold search's first interval reaches 2^64.  The block counts take
    the search's gathered-interval path at once (19), after some passes (300,
    1100), and the long-row kernel past 2048 blocks (2100)."""
    import free_block_sparse_attn_amd as fbsa
    rng = np.random.default_rng(11)
    d = 128
    N = 64 * nb
    u = rng.standard_normal(d).astype(np.float32)
    u /= np.linalg.norm(u)
    blk = np.arange(N) // 64
    sign = np.where(blk % 3 == 0, 1.0, np.where(blk % 3 == 1, -1.0, 0.0)).astype(np.float32)
    k_np = (rng.standard_normal((1, 1, N, d)) * 0.3 + 2.0 * u).astype(np.float32)
    q_np = (rng.standard_normal((1, 1, N, d)) * 0.3 + (2.0 * sign)[None, None, :, None] * u).astype(np.float32)
    to = lambda x: torch.from_numpy(x).to(torch.bfloat16).cuda()
    q, k = to(q_np), to(k_np)
    pooled = fbsa.sparse_attn_pool(q, k, k, N, spreads=True)
    f = {x: pooled[x].cpu().numpy() for x in ("qbar", "kbar", "klam", "kcount")}
    print(f"\n[case] one-sign rows nb={nb}", flush=True)
    kk = max(2, nb // 5)
    idx, cnt, _, _ = fbsa.sparse_attn_route(pooled, N, fbsa.SA_ROUTE_TOPK, topk=kk)
    ri, rc = routing.route_topk(f["qbar"], f["kbar"], kk)
    assert np.array_equal(cnt.cpu().numpy(), rc)
    assert np.array_equal(idx.cpu().numpy()[..., :kk], ri)
    scale = d ** -0.5
    n_keep, n_refine = max(1, 2 * nb // 5), 3 * nb // 20
    idx, cnt, idx2, cnt2 = fbsa.sparse_attn_route(pooled, N, fbsa.SA_ROUTE_TRIAGE, n_keep=n_keep,
                                                  n_refine=n_refine, scale=scale)
    ri, rc, si, sc = routing.route_triage(f["qbar"], f["kbar"], f["klam"], f["kcount"], scale, n_keep, n_refine)
    assert np.array_equal(idx.cpu().numpy()[..., :ri.shape[-1]], ri)
    assert np.array_equal(cnt.cpu().numpy(), rc)
    assert np.array_equal(idx2.cpu().numpy(), si)
    assert np.array_equal(cnt2.cpu().numpy(), sc)


def test_topk_all_blocks_matches_dense():
    wl = get_workload(2, small=True)
    (q, k, v), dev, coords = gc.inputs(wl)
    import free_block_sparse_attn_amd as fbsa
    pooled = fbsa.sparse_attn_pool(*dev, wl.N)
    idx, cnt, _, _ = fbsa.sparse_attn_route(pooled, wl.N, fbsa.SA_ROUTE_TOPK, topk=wl.nb)
    out, lse = fbsa.sparse_attn_fwd(*dev, wl.N, 1.0, 0, pooled, idx, cnt)
    Od, lsed = attention.dense_attention(q, k, v, wl.N, 1.0)
    assert np.abs(out.float().cpu().numpy() - Od).max() <= gc.BF16_TOL
    assert np.abs(lse.cpu().numpy()[:, :, :wl.N] - lsed[:, :, :wl.N]).max() <= gc.LSE_TOL["bf16"]


@pytest.mark.parametrize("rule", ["topk", "topk_cov"])
@pytest.mark.parametrize("size", ["small", "medium"])
def test_parity_global_first_order(size, rule):
    """PISA's global first-order term (comp 2) on the HunyuanVideo-like layer,
    routed by plain or covariance-aware top-k."""
    from workloads.configs import GLOBAL_ORDER1_SMALL, GLOBAL_COV_SMALL
    from dataclasses import replace
    if size == "small":
        wl = GLOBAL_ORDER1_SMALL if rule == "topk" else GLOBAL_COV_SMALL
    else:
        wl = replace(medium(3), comp=2, rule=rule)
    print(f"\n[case] {wl.name} size={size} N={wl.N} H={wl.H} nb={wl.nb}", flush=True)
    (q, k, v), dev, coords = gc.inputs(wl)
    pooled_o = gc.oracle_pool(wl, q, k, v)
    res = gc.run_gpu(wl, dev, coords)
    check_pool(wl, pooled_o, res, v)
    check_route(wl, pooled_o, res, coords)
    ref = gc.oracle_rows(wl, q, k, v, pooled_o, res, all_rows(wl))
    worst = check_out(wl, res, ref, all_rows(wl))
    assert np.all(res["out"][:, :, wl.N:] == 0)
    print(f"[ok] max|err|={worst:.3e}", flush=True)


@pytest.mark.parametrize("rule", ["topk", "topk_cov"])
def test_parity_global_first_order_full_size_sampled(rule):
    from workloads.configs import GLOBAL_ORDER1, GLOBAL_COV
    wl = GLOBAL_ORDER1 if rule == "topk" else GLOBAL_COV
    print(f"\n[case] full {wl.name} N={wl.N} H={wl.H} nb={wl.nb}", flush=True)
    (q, k, v), dev, coords = gc.inputs(wl)
    rng = np.random.default_rng(7)
    heads = sorted(rng.choice(wl.H, 2, replace=False).tolist())
    res = gc.run_gpu(wl, dev, coords)
    qs, ks, vs = (x[:, heads] for x in (q, k, v))
    pooled_o = pooling.pool(qs, ks, vs, wl.N, hbar=True, cov=rule == "topk_cov")
    rsub = {n: (x[:, heads] if n not in ("kcount",) else x) for n, x in res.items()}
    check_pool(wl, pooled_o, {n: rsub[n] for n in ("qbar", "kbar", "vbar", "kcount", "hbar", "kcov") if n in rsub})
    check_route(wl, pooled_o, rsub, coords)
    rows = [(0, hi, int(a)) for hi in range(len(heads)) for a in rng.choice(wl.nb, 3, replace=False)]
    rows.append((0, 0, wl.nb - 1))
    ref = gc.oracle_rows(wl, qs, ks, vs, pooled_o, rsub, rows)
    worst = check_out(wl, rsub, ref, rows)
    print(f"[ok] max|err|={worst:.3e}", flush=True)


@pytest.mark.parametrize("size", ["small", "medium"])
def test_parity_error_routed(size):
    """SVG-EAR error-aware routing on the Wan-like layer, centroid compensation."""
    from dataclasses import replace
    from workloads.configs import ERROR_ROUTED_SMALL
    wl = ERROR_ROUTED_SMALL if size == "small" else replace(medium(2), rule="error")
    print(f"\n[case] {wl.name} size={size} N={wl.N} H={wl.H} nb={wl.nb}", flush=True)
    (q, k, v), dev, coords = gc.inputs(wl)
    pooled_o = gc.oracle_pool(wl, q, k, v)
    res = gc.run_gpu(wl, dev, coords)
    check_pool(wl, pooled_o, res, v)
    check_route(wl, pooled_o, res, coords)
    lerr = check_error_logs(wl, res, np.swapaxes(res["ekey"], -1, -2), k)
    ref = gc.oracle_rows(wl, q, k, v, pooled_o, res, all_rows(wl))
    worst = check_out(wl, res, ref, all_rows(wl))
    assert np.all(res["out"][:, :, wl.N:] == 0)
    print(f"[ok] max|dL|={lerr:.2e} max|err|={worst:.3e}", flush=True)


def test_parity_error_routed_full_size_sampled():
    from workloads.configs import ERROR_ROUTED
    wl = ERROR_ROUTED
    print(f"\n[case] full {wl.name} N={wl.N} H={wl.H} nb={wl.nb}", flush=True)
    (q, k, v), dev, coords = gc.inputs(wl)
    rng = np.random.default_rng(8)
    heads = sorted(rng.choice(wl.H, 2, replace=False).tolist())
    res = gc.run_gpu(wl, dev, coords)
    qs, ks, vs = (x[:, heads] for x in (q, k, v))
    pooled_o = pooling.pool(qs, ks, vs, wl.N)
    rsub = {n: (x[:, heads] if n not in ("kcount",) else x) for n, x in res.items()}
    check_pool(wl, pooled_o, {n: rsub[n] for n in ("qbar", "kbar", "vbar", "kcount")})
    check_route(wl, pooled_o, rsub, coords)
    sample = sorted(rng.choice(wl.nb, 6, replace=False).tolist()) + [wl.nb - 1]
    lerr = check_error_logs(wl, rsub, np.swapaxes(rsub["ekey"], -1, -2), ks, rows=sample)
    rows = [(0, hi, int(a)) for hi in range(len(heads)) for a in sample[:3]] + [(0, 0, wl.nb - 1)]
    ref = gc.oracle_rows(wl, qs, ks, vs, pooled_o, rsub, rows)
    worst = check_out(wl, rsub, ref, rows)
    print(f"[ok] max|dL|={lerr:.2e} max|err|={worst:.3e}", flush=True)


@pytest.mark.parametrize("size", ["small", "medium"])
def test_parity_triage_mxfp4(size):
    """Triage with the skim tier in MXFP4 (the page's 4 bits)."""
    from dataclasses import replace
    from workloads.configs import TRIAGE_FP4_SMALL
    wl = TRIAGE_FP4_SMALL if size == "small" else replace(medium(5), skim_fmt="mxfp4")
    print(f"\n[case] {wl.name} size={size} N={wl.N} H={wl.H} nb={wl.nb}", flush=True)
    (q, k, v), dev, coords = gc.inputs(wl)
    pooled_o = gc.oracle_pool(wl, q, k, v)
    res = gc.run_gpu(wl, dev, coords)
    check_pool(wl, pooled_o, res, v)
    check_route(wl, pooled_o, res, coords)
    ref = gc.oracle_rows(wl, q, k, v, pooled_o, res, all_rows(wl))
    worst = check_out(wl, res, ref, all_rows(wl))
    assert np.all(res["out"][:, :, wl.N:] == 0)
    print(f"[ok] max|err|={worst:.3e}", flush=True)


def test_parity_triage_mxfp4_full_size_sampled():
    from workloads.configs import TRIAGE_FP4
    wl = TRIAGE_FP4
    print(f"\n[case] full {wl.name} N={wl.N} H={wl.H} nb={wl.nb}", flush=True)
    (q, k, v), dev, coords = gc.inputs(wl)
    rng = np.random.default_rng(9)
    heads = sorted(rng.choice(wl.H, 2, replace=False).tolist())
    res = gc.run_gpu(wl, dev, coords)
    qs, ks, vs = (x[:, heads] for x in (q, k, v))
    pooled_o = pooling.pool(qs, ks, vs, wl.N, spreads=True, fp4=True)
    rsub = {n: (x[:, heads] if n not in ("kcount",) else x) for n, x in res.items()}
    check_pool(wl, pooled_o, {n: rsub[n] for n in ("qbar", "kbar", "vbar", "kcount", "q4", "qs4", "k4", "ks4",
                                                  "v4", "vs4")})
    check_route(wl, pooled_o, rsub, coords)
    rows = [(0, hi, int(a)) for hi in range(len(heads)) for a in rng.choice(wl.nb, 3, replace=False)]
    rows.append((0, 0, wl.nb - 1))
    ref = gc.oracle_rows(wl, qs, ks, vs, pooled_o, rsub, rows)
    worst = check_out(wl, rsub, ref, rows)
    print(f"[ok] max|err|={worst:.3e}", flush=True)


RES_PHASE, RES_RIDGE, RES_RANK = 3, 1e-3, 8


def run_residual(wl, dev, coords, phase=RES_PHASE, ridge=RES_RIDGE, rank=RES_RANK, scale=1.0):
    """GPU sparse forward, then the probe-fitted residual pass on its output."""
    import free_block_sparse_attn_amd as fbsa
    res = gc.run_gpu(wl, dev, coords, scale=scale)
    q, k, v = dev
    out = torch.from_numpy(res["out"]).to(torch.bfloat16).cuda()
    r = fbsa.sparse_attn_residual(q, k, v, out, wl.N, scale, phase, ridge, rank)
    torch.cuda.synchronize()
    fit = {n: r[n].cpu().numpy() for n in ("xp", "od", "W", "c")}
    return res, out.float().cpu().numpy(), fit


def check_residual(wl, q, k, v, res, corr, fit, heads_rows, phase=RES_PHASE, ridge=RES_RIDGE, rank=RES_RANK,
                   scale=1.0):
    """Dense probe rows, the fit on the GPU's probe data, and the corrected rows."""
    from oracle import residual
    nb = wl.nb
    rows = residual.probe_rows(wl.N, nb, phase)
    worst = 0.0
    for (b, h), check_rows in heads_rows.items():
        od = residual.probe_dense(q[b, h], k[b, h], v[b, h], wl.N, scale, rows)
        perr = np.abs(fit["od"][b, h, :nb] - od).max(axis=1)
        assert perr.max() <= gc.BF16_TOL, (b, h, np.round(perr, 4))
        assert np.array_equal(fit["xp"][b, h, :nb], res["out"][b, h, rows])
        # stage-wise: the oracle's fit on the GPU's probe outputs
        X = fit["xp"][b, h, :nb].astype(np.float64)
        W, c = residual.fit_residual(X, fit["od"][b, h, :nb] - X, ridge, rank)
        wscale = max(np.abs(W).max(), np.abs(c).max(), 1e-12)
        assert np.abs(fit["W"][b, h] - W).max() <= 1e-3 * wscale, np.abs(fit["W"][b, h] - W).max()
        assert np.abs(fit["c"][b, h] - c).max() <= 1e-3 * wscale
        # end to end: o + c + o W on the GPU's sparse output, dense rows at the probes
        O = res["out"][b, h].astype(np.float64)
        ref = O + c + O @ W
        ref[rows] = od
        ref[wl.N:] = 0.0
        err = np.abs(corr[b, h, check_rows] - ref[check_rows]).max(axis=1)
        bar = gc.row_tol("bf16", ref[check_rows])
        worst = max(worst, err.max())
        assert np.all(err <= bar), (b, h, err.max())
    return worst


@pytest.mark.parametrize("size", ["small", "medium"])
def test_parity_probe_residual(size):
    """SparsePR's probe-fitted residual on the Wan-like layer's sparse output."""
    wl = get_workload(2, small=True) if size == "small" else medium(2)
    print(f"\n[case] residual {wl.name} size={size} N={wl.N} H={wl.H} nb={wl.nb}", flush=True)
    (q, k, v), dev, coords = gc.inputs(wl)
    res, corr, fit = run_residual(wl, dev, coords)
    heads = {(0, h): np.arange(wl.N_pad) for h in range(wl.H)}
    worst = check_residual(wl, q, k, v, res, corr, fit, heads)
    assert np.all(corr[:, :, wl.N:] == 0)
    print(f"[ok] max|err|={worst:.3e}", flush=True)


def test_parity_probe_residual_odd_rank():
    """Rank 3 (two of the four solve waves idle, one zero right-hand side in
    the last pair), another probe phase and a larger ridge."""
    wl = get_workload(2, small=True)
    phase, ridge, rank = 11, 1e-2, 3
    print(f"\n[case] residual {wl.name} rank={rank} phase={phase} ridge={ridge} N={wl.N} nb={wl.nb}", flush=True)
    (q, k, v), dev, coords = gc.inputs(wl)
    res, corr, fit = run_residual(wl, dev, coords, phase, ridge, rank)
    heads = {(0, h): np.arange(wl.N_pad) for h in range(wl.H)}
    worst = check_residual(wl, q, k, v, res, corr, fit, heads, phase, ridge, rank)
    assert np.all(corr[:, :, wl.N:] == 0)
    print(f"[ok] max|err|={worst:.3e}", flush=True)


def test_parity_probe_residual_full_size_sampled():
    wl = WORKLOADS[2]
    print(f"\n[case] residual full {wl.name} N={wl.N} H={wl.H} nb={wl.nb}", flush=True)
    (q, k, v), dev, coords = gc.inputs(wl)
    res, corr, fit = run_residual(wl, dev, coords)
    rng = np.random.default_rng(10)
    heads = sorted(rng.choice(wl.H, 2, replace=False).tolist())
    sample = {(0, h): np.sort(rng.choice(wl.N, 512, replace=False)) for h in heads}
    worst = check_residual(wl, q, k, v, res, corr, fit, sample)
    print(f"[ok] max|err|={worst:.3e}", flush=True)
