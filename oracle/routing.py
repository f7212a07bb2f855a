"""Block routing: which key blocks each query block computes exactly.

All selections are returned as ascending index lists padded with -1 plus a
count per query block.  Orderings are total: ties on the score go to the lower
block index.
"""

import numpy as np


def block_scores(qbar: np.ndarray, kbar: np.ndarray) -> np.ndarray:
    """s(a, j) = sum_i qbar[a, i] * kbar[j, i] in fp64, accumulated in i order.

    qbar, kbar: fp32 [..., nq, d] and [..., nk, d].  Each fp32 x fp32 product
    is exact in fp64, so a fused or an unfused multiply-add gives the same
    bits; the sum runs over i = 0 .. d-1 in order from +0.0.
    Pages: pooled block scores drive PISA's top-k selection (section 2,
    "Routage Sensible a la Covariance") and SVG-EAR's critique of score
    routing (section 1).
    """
    q = np.asarray(qbar, np.float32).astype(np.float64)
    k = np.asarray(kbar, np.float32).astype(np.float64)
    acc = np.zeros(q.shape[:-1] + (k.shape[-2],), np.float64)
    for i in range(q.shape[-1]):
        acc = acc + q[..., :, None, i] * k[..., None, :, i]
    return acc


def _select_first(keys: np.ndarray, count: int) -> np.ndarray:
    """Indices of the first `count` entries in the order (-key, index), ascending."""
    order = np.lexsort((np.arange(keys.shape[0]), -keys))
    return np.sort(order[:count])


def _pack(lists, cap: int):
    idx = np.full((len(lists), cap), -1, np.int32)
    cnt = np.zeros(len(lists), np.int32)
    for a, sel in enumerate(lists):
        idx[a, :len(sel)] = sel
        cnt[a] = len(sel)
    return idx, cnt


def route_topk(qbar: np.ndarray, kbar: np.ndarray, k: int):
    """Top-k key blocks per query block on pooled scores.

    qbar, kbar fp32 [B,H,nb,d] -> (idx int32 [B,H,nb,k], cnt int32 [B,H,nb]).
    PISA selects the critical set S_i per query block by top-k on block
    scores (section 2, "Algorithme Central" / "Routage Sensible a la
    Covariance"); ties go to the lower index.
    """
    B, H, nq, _ = qbar.shape
    nk = kbar.shape[2]
    kk = min(k, nk)
    idx = np.full((B, H, nq, kk), -1, np.int32)
    cnt = np.full((B, H, nq), kk, np.int32)
    for b in range(B):
        for h in range(H):
            s = block_scores(qbar[b, h], kbar[b, h])
            for a in range(nq):
                idx[b, h, a] = _select_first(s[a], kk)
    return idx, cnt


def route_topk_cov(qbar: np.ndarray, kbar: np.ndarray, kcov: np.ndarray, scale: float, k: int):
    """PISA's covariance-aware top-k ("PISA ...", section 2, "Routage Sensible
    a la Covariance"): the selection key combines the block's attention score
    with the norm M_j = ||H_j - H_bar||_2 of its deviation from the global
    first-order statistic.

    Reading used: after the global term, block j's remaining first-order
    error at query t is alpha_{t,j} q_t (H_j - H_bar), at most
    exp(scale q_t.k_bar_j) |q_t| M_j; at the pooled query the row factor |q|
    is common to all j, so blocks are ranked by its log
      key(a, j) = fl(fl(scale * s(a, j)) + ln M_j)      (fp64, ln M_j from fp32)
    High-score blocks and strongly heterogeneous blocks both rank high.  The
    first k in the order (-key, j) are computed exactly.
    kcov: fp32 [B,H,nb] = ln M_j.  Returns (idx int32 [B,H,nb,k], cnt).
    """
    B, H, nq, _ = qbar.shape
    nk = kbar.shape[2]
    kk = min(k, nk)
    sc = np.float64(np.float32(scale))
    idx = np.full((B, H, nq, kk), -1, np.int32)
    cnt = np.full((B, H, nq), kk, np.int32)
    for b in range(B):
        for h in range(H):
            key = sc * block_scores(qbar[b, h], kbar[b, h]) + \
                np.asarray(kcov[b, h], np.float32).astype(np.float64)[None, :]
            for a in range(nq):
                idx[b, h, a] = _select_first(key[a], kk)
    return idx, cnt


def error_logs(qbar: np.ndarray, k: np.ndarray, kbar: np.ndarray, N: int, scale: float,
               blk: int = 64) -> np.ndarray:
    """SVG-EAR's per-block approximation error ("SVG-EAR ...", section 2B,
    error estimation with query centroids as proxies), as a log.

    For query-block centroid q_a and key block j (valid keys k_n, centroid
    k_bar_j), the proxy query's attention weights to the block are
    e^{x_n}, x_n = scale q_a.k_n; replacing the keys by their centroid gives
    e^{c} to each, c = scale q_a.k_bar_j.  The squared error of the weights is
      E(a, j) = sum_n (e^{x_n} - e^{c})^2 = e^{2c} sum_n expm1(delta_n)^2,
      delta_n = scale q_a.(k_n - k_bar_j).
    Returns L(a, j) = ln sum_n expm1(delta_n)^2 (the factor e^{2c} is added by
    the router, from the pooled score), fp64 [B,H,nq,nb]; -inf where every
    delta is 0 (e.g. one-token blocks).  qbar, kbar: the pooled fp32 means;
    k: the input token keys [B,H,N_pad,d].
    """
    B, H, nq, d = qbar.shape
    nb = kbar.shape[2]
    sc = np.float64(np.float32(scale))
    out = np.empty((B, H, nq, nb), np.float64)
    for b in range(B):
        for h in range(H):
            qa = np.asarray(qbar[b, h], np.float32).astype(np.float64)
            for j in range(nb):
                n = min(blk, N - blk * j)
                kc = np.asarray(k[b, h, blk * j: blk * j + n], np.float64) - \
                    np.asarray(kbar[b, h, j], np.float32).astype(np.float64)[None, :]
                delta = sc * (qa @ kc.T)                                  # [nq, n]
                with np.errstate(divide="ignore"):
                    out[b, h, :, j] = np.log(np.sum(np.expm1(delta) ** 2, axis=1))
    return out


def route_error(qbar: np.ndarray, kbar: np.ndarray, kcount: np.ndarray, elog: np.ndarray,
                scale: float, k: int):
    """SVG-EAR error-aware routing ("SVG-EAR ...", section 2B): under the
    block budget, greedily take the blocks with the largest error-to-cost
    ratio E(a, j) / n_j (error normalised by the block's size).  With every
    block costing one tile, the greedy choice is the first k in the order
    (-key, j) of
      key(a, j) = fl(fl(2 fl(scale s(a, j)) + L(a, j)) - ln n_j)     (fp64)
    = ln(E / n_j), where L = error_logs(...) (given as fp32, the router's input).
    elog: [B,H,nq,nb].  Returns (idx int32 [B,H,nq,k], cnt).
    """
    B, H, nq, _ = qbar.shape
    nk = kbar.shape[2]
    kk = min(k, nk)
    sc = np.float64(np.float32(scale))
    logn = np.log(np.asarray(kcount, np.float64))
    idx = np.full((B, H, nq, kk), -1, np.int32)
    cnt = np.full((B, H, nq), kk, np.int32)
    for b in range(B):
        for h in range(H):
            ss = sc * block_scores(qbar[b, h], kbar[b, h])
            key = (2.0 * ss + np.asarray(elog[b, h], np.float32).astype(np.float64)) - logn[None, :]
            for a in range(nq):
                idx[b, h, a] = _select_first(key[a], kk)
    return idx, cnt


def lvsa_anchor_set(nb: int, anchors: int, phase: int, step: int) -> np.ndarray:
    """Rotating global anchor key blocks G_s at denoising step s.

    LVSA ("LVSA: Training-Free Sparse Attention for Long Video Diffusion",
    section 2, "Mecanisme Central"): the global set shifts by s mod T_per at
    each step, so over T_per steps every position is an anchor exactly once.
    Here the grid is `anchors` key blocks at stride P = nb // anchors with
    offset (phase + s) mod P.  No anchors when `anchors` is 0; `anchors`
    may not exceed nb.
    """
    if anchors == 0:
        return np.zeros(0, np.int64)
    assert anchors <= nb
    P = nb // anchors
    off = (phase + step) % P
    return off + P * np.arange(anchors)


def route_lvsa(frame_lo: np.ndarray, frame_hi: np.ndarray, window: int,
               anchors: int, phase: int, step: int):
    """LVSA block mask A(t) = G_s  U  W(t) on 64-token blocks.

    Query block a attends to key block j when their latent-frame ranges come
    within `window` frames of each other ([lo_j, hi_j] meets
    [lo_a - w, hi_a + w]), or when j is one of the step's anchors.  Page:
    LVSA section 2, "Mecanisme Central" (A(t) = G U W(t)).
    Returns (idx int32 [nb, cap], cnt int32 [nb]) with cap = the row maximum.
    """
    lo = np.asarray(frame_lo, np.int64)
    hi = np.asarray(frame_hi, np.int64)
    nb = lo.shape[0]
    anc = np.zeros(nb, bool)
    anc[lvsa_anchor_set(nb, anchors, phase, step)] = True
    lists = []
    for a in range(nb):
        near = (lo <= hi[a] + window) & (hi >= lo[a] - window)
        lists.append(np.nonzero(near | anc)[0])
    cap = max(len(x) for x in lists)
    return _pack(lists, cap)


def route_triage(qbar: np.ndarray, kbar: np.ndarray, klam: np.ndarray, kcount: np.ndarray,
                 scale: float, n_keep: int, n_refine: int):
    """Triage tiers per (query block, key block) tile: refine / skim / skip.

    Page: "Triage: Skip, Skim, or Refine Attention Tiles in Video Diffusion
    Transformers" ("Un routage fonde sur l'erreur estimee"): from block
    statistics the router estimates each tile's weight and the error of
    omitting it, and spends more compute where the estimated error drop
    justifies it.  Reading used here, in log space with fp64 keys:
      e_skip(a, j) = fl(fl(scale * s(a, j)) + lambda_j)   omission error
      w(a, j)      = fl(fl(scale * s(a, j)) + ln n_j)     tile weight
    The first n_keep blocks in the order (-e_skip, j) are not skipped; of
    those, the first n_refine in the order (-w, j) are refined (exact bf16)
    and the rest skimmed (fp8).  Everything else is skipped and compensated.
    Returns (ref_idx, ref_cnt, skim_idx, skim_cnt) with caps n_refine and
    n_keep - n_refine.
    """
    B, H, nq, _ = qbar.shape
    nk = kbar.shape[2]
    n_keep = min(n_keep, nk)
    n_refine = min(n_refine, n_keep)
    sc = np.float64(np.float32(scale))
    logn = np.log(np.asarray(kcount, np.float64))
    ref_idx = np.full((B, H, nq, n_refine), -1, np.int32)
    skim_idx = np.full((B, H, nq, n_keep - n_refine), -1, np.int32)
    for b in range(B):
        for h in range(H):
            s = block_scores(qbar[b, h], kbar[b, h])
            ss = sc * s
            eskip = ss + np.asarray(klam[b, h], np.float32).astype(np.float64)[None, :]
            w = ss + logn[None, :]
            for a in range(nq):
                keep = _select_first(eskip[a], n_keep)
                ref = keep[_select_first(w[a, keep], n_refine)]
                ref = np.sort(ref)
                skim = np.setdiff1d(keep, ref)
                ref_idx[b, h, a] = ref
                skim_idx[b, h, a] = skim
    ref_cnt = np.full((B, H, nq), n_refine, np.int32)
    skim_cnt = np.full((B, H, nq), n_keep - n_refine, np.int32)
    return ref_idx, ref_cnt, skim_idx, skim_cnt
