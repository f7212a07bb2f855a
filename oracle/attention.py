"""Dense attention and the compensated block-sparse rule, fp64.

The rule follows PISA ("PISA: Piecewise Sparse Attention Is Wiser for
Efficient Diffusion Transformers", section 2, "Algorithme Central"): for a
query t of query block a,

    o_t = N_t / D_t
    D_t = sum_{j in E} sum_n e^{s q.k_n}                      exact blocks
        + sum_{j in M} sum_n e^{s l~_tn}                      skim blocks
        + [c >= 0] sum_{j in U} n_j e^{s q.k_bar_j}           zeroth order
    N_t = sum_{j in E} sum_n e^{s q.k_n} v_n
        + sum_{j in M} sum_n p~_tn v~_n 2^{e_v(j)}
        + [c >= 0] sum_{j in U} n_j e^{s q.k_bar_j} v_bar_j
        + [c == 1] sum_{j in U} e^{s q.k_bar_j} s (q^T H_j)
        + [c == 2] s (sum_{j in U} e^{s q.k_bar_j}) (q^T H_bar)

with s the softmax scale, E the exactly computed key blocks, M the fp8 skim
blocks (Triage's low-precision tier), U every other block, n_j the block's
valid key count, k_bar_j / v_bar_j its exact means and H_j = sum_n
(k_n - k_bar_j) v_n^T.  The zeroth-order term is PISA's alpha_{t,j} times the
block's value sum (alpha_{t,j} = exp(q_t k_bar_j^T)), which equals SVG-EAR's
centroid replacement ("SVG-EAR ...", section 2A) of all n_j keys and values
by their means.  The first-order term is PISA's with the per-block matrix
H_j in place of the global mean H_bar; c == 2 is PISA's own hybrid-order
form, with H_bar = mean_j H_j over all blocks of the head shared by every
skipped block.  Either first-order term has no denominator share because
sum_n (k_n - k_bar_j) = 0 for the exact mean.  Every approximation sits
inside the one normalisation D_t, as PISA's "Coherence de Normalisation"
asks.

Skim tile (a, j) emulation (Triage's fast tier), in one of two formats:
  e4m3   q~, k~, v~ are the per-block scaled e4m3 copies with exponents
         e_q(a), e_k(j), e_v(j): l~_tn = (q~_t . k~_n) 2^{e_q(a) + e_k(j)}
  mxfp4  the page's 4 bits: q~, k~ carry one E8M0 scale per token and 32
         dimensions, v~ one per block and dimension; l~ = q~ . k~ and v~ are
         the dequantised values (exact in fp64)
With L_tn = s l~_tn log2(e) and c_t = ceil(max_n L_tn) for the tile,
p~_tn = 2^{c_t - 8} e4m3(2^{8 + L_tn - c_t}) in both formats (the weights
stay 8-bit).  The denominator takes the unquantised weights.
"""

import math

import numpy as np

from . import e4m3, mxfp4

BLK = 64
LOG2E = 1.0 / math.log(2.0)


def dense_attention(q, k, v, N: int, scale: float):
    """softmax(scale * q k^T) v over the N valid tokens, fp64.

    Returns (O [B,H,N_pad,d], lse [B,H,N_pad]); pad rows are 0.
    """
    B, H, Np, d = q.shape
    O = np.zeros((B, H, Np, d))
    lse = np.zeros((B, H, Np))
    for b in range(B):
        for h in range(H):
            Q = np.asarray(q[b, h, :N], np.float64)
            K = np.asarray(k[b, h, :N], np.float64)
            V = np.asarray(v[b, h, :N], np.float64)
            S = scale * (Q @ K.T)
            m = S.max(axis=1, keepdims=True)
            P = np.exp(S - m)
            D = P.sum(axis=1, keepdims=True)
            O[b, h, :N] = (P @ V) / D
            lse[b, h, :N] = (m + np.log(D))[:, 0]
    return O, lse


def _tokens(blocks, N: int, blk: int) -> np.ndarray:
    blocks = np.asarray(blocks, np.int64)
    t = (blocks[:, None] * blk + np.arange(blk)[None, :]).ravel()
    return t[t < N]


def skim_weights(L: np.ndarray) -> np.ndarray:
    """Quantised weights p~ for one skim tile, given L = s * l~ * log2(e).

    L: [rows, keys] (one key block).  Returns p~ in absolute units (as the
    weights 2^L they stand for), each row scaled by its own power-of-two
    reference c_t = ceil(max L_t).
    """
    c = np.ceil(L.max(axis=1, keepdims=True))
    return np.exp2(c - 8.0) * e4m3.round_to_e4m3(np.exp2(8.0 + L - c))


def skim_weight_slack(L: np.ndarray, eps: float) -> np.ndarray:
    """Largest change of each quantised weight of skim_weights(L) over the
    decisions that an evaluation of L off by at most eps (log2 units) can take
    differently: each weight's e4m3 code (rounding is monotone, so the codes
    reachable from [L - eps, L + eps] are those of its ends) and the row's
    reference c_t = ceil(max L_t) (ceil(max L_t -+ eps)).  Zero wherever every
    such evaluation gives the same weight.  [rows, keys], absolute units.
    """
    base = skim_weights(L)
    mx = L.max(axis=1, keepdims=True)
    c = np.ceil(mx)
    lo, hi = np.ceil(mx - eps), np.ceil(mx + eps)
    d = np.zeros_like(base)
    for cc in (c - 1.0, c, c + 1.0):
        reach = (lo <= cc) & (cc <= hi)
        for dl in (-eps, 0.0, eps):
            alt = np.exp2(cc - 8.0) * e4m3.round_to_e4m3(np.exp2(8.0 + L + dl - cc))
            d = np.maximum(d, np.where(reach, np.abs(alt - base), 0.0))
    return d


def rule_block(Qa, k, v, N: int, scale: float, comp: int, kbar, vbar, kcount,
               exact, skim=(), kmom=None, fp8=None, a: int = 0, blk: int = BLK, hbar=None,
               slack_eps=None, skim_dlog2=None):
    """Compensated rule for the valid rows Qa [r, d] of query block a, one head.

    k, v: [N_pad, d]; kbar, vbar: exact fp64 means [nb, d]; kcount [nb];
    exact / skim: key block index lists; kmom [nb, d, d] for comp == 1;
    hbar [d, d] (the head's mean first-order matrix) for comp == 2;
    fp8: the skim tier's copies: dict(q8, k8, v8 codes [N_pad, d], qexp, kexp,
    vexp [nb]) for e4m3, or dict(q4, qs4, k4, ks4, v4, vs4) for mxfp4.
    Returns (o [r, d], lse [r]); with slack_eps, also a per-row bound [r] on
    max_i |o'_i - o_i| over every evaluation o' whose skim logits (log2 units)
    are off by at most slack_eps each: with S_N a bound on the numerator's
    change per component (the weights' code decisions, skim_weight_slack,
    and their continuous change, times max_i |v~_i| of each key) and S_D on
    the denominator's, o' - o = (N' - N) / D' + o (D - D') / D', so
    |o' - o| <= (S_N + |o|_inf S_D) / (D - S_D).
    skim_dlog2: optional list (one per skim block, in ascending block order)
    of [r, n_j] offsets added to that tile's logits in log2 units before
    anything else (a perturbed evaluation, for testing the bound).
    """
    Qa = np.asarray(Qa, np.float64)
    nb = kbar.shape[0]
    exact = np.asarray(sorted(exact), np.int64)
    skim = np.asarray(sorted(skim), np.int64)
    U = np.setdiff1d(np.arange(nb), np.concatenate([exact, skim]))

    # ordinary softmax terms: exact keys, then centroid pseudo-keys
    te = _tokens(exact, N, blk)
    logits = [scale * (Qa @ np.asarray(k[te], np.float64).T)]
    values = [np.asarray(v[te], np.float64)]
    if comp >= 0 and U.size:
        cl = scale * (Qa @ kbar[U].T) + np.log(kcount[U].astype(np.float64))[None, :]
        logits.append(cl)
        values.append(vbar[U])

    skim_terms = []
    if skim.size and "q4" in fp8:
        rows = slice(a * blk, a * blk + Qa.shape[0])
        qa = mxfp4.dequantize_blocks(fp8["q4"][rows], fp8["qs4"][rows])
        for j in skim:
            tj = _tokens([j], N, blk)
            l = qa @ mxfp4.dequantize_blocks(fp8["k4"][tj], fp8["ks4"][tj]).T
            vt = mxfp4.decode(fp8["v4"][tj]) * np.exp2(np.asarray(fp8["vs4"][j], np.float64))[None, :]
            skim_terms.append((scale * l, vt))
    elif skim.size:
        qa = e4m3.decode(fp8["q8"][a * blk:a * blk + Qa.shape[0]])
        for j in skim:
            tj = _tokens([j], N, blk)
            l = (qa @ e4m3.decode(fp8["k8"][tj]).T) * 2.0 ** (int(fp8["qexp"][a]) + int(fp8["kexp"][j]))
            vt = e4m3.decode(fp8["v8"][tj]) * 2.0 ** int(fp8["vexp"][j])
            skim_terms.append((scale * l, vt))

    if skim_dlog2 is not None:
        skim_terms = [(lg + np.asarray(dl, np.float64) / LOG2E, vt)
                      for (lg, vt), dl in zip(skim_terms, skim_dlog2)]
    m = np.max(np.concatenate([x for x in logits] + [t[0] for t in skim_terms], axis=1), axis=1)
    D = np.zeros(Qa.shape[0])
    Nt = np.zeros_like(Qa)
    for lg, val in zip(logits, values):
        P = np.exp(lg - m[:, None])
        D += P.sum(axis=1)
        Nt += P @ val
    slack = np.zeros(Qa.shape[0])
    slack_den = np.zeros(Qa.shape[0])
    for lg, vt in skim_terms:
        D += np.exp(lg - m[:, None]).sum(axis=1)
        L = lg * LOG2E
        pq = skim_weights(L) * np.exp2(-m * LOG2E)[:, None]
        Nt += pq @ vt
        if slack_eps is not None:
            # code decisions, plus the continuous change of every weight (in
            # the numerator, and through the denominator on o)
            g = np.exp2(slack_eps) - 1.0
            sc = np.exp2(-m * LOG2E)[:, None]
            slack += ((skim_weight_slack(L, slack_eps) + g * skim_weights(L)) * sc) @ np.abs(vt).max(axis=1)
            slack_den += g * np.exp(lg - m[:, None]).sum(axis=1)
    if comp == 2 and U.size:
        alpha = np.exp(scale * (Qa @ kbar[U].T) - m[:, None])        # [r, |U|]
        Nt += scale * alpha.sum(axis=1)[:, None] * (Qa @ hbar)
    if comp == 1 and U.size:
        alpha = np.exp(scale * (Qa @ kbar[U].T) - m[:, None])        # [r, |U|]
        QH = np.matmul(Qa[None], kmom[U])                             # [|U|, r, d]: q^T H_j
        Nt += scale * np.einsum("ru,uro->ro", alpha, QH)
    if slack_eps is not None:
        o = Nt / D[:, None]
        assert np.all(slack_den < D), "skim logit slack too large for a bound"
        return o, m + np.log(D), (slack + slack_den * np.abs(o).max(axis=1)) / (D - slack_den)
    return Nt / D[:, None], m + np.log(D)


def sparse_attention(q, k, v, N: int, scale: float, comp: int, pooled: dict,
                     exact_idx, exact_cnt, skim_idx=None, skim_cnt=None, blk: int = BLK,
                     lowp: str = "e4m3"):
    """The rule on every query block of every (b, h); fp64 (O, lse), pad rows 0.

    `pooled` is oracle.pooling.pool(...) output (kbar64, vbar64, kcount and,
    when needed, kmom and the skim copies: fp8 for lowp "e4m3", fp4 for "mxfp4").
    """
    B, H, Np, d = q.shape
    nb = Np // blk
    O = np.zeros((B, H, Np, d))
    lse = np.zeros((B, H, Np))
    for b in range(B):
        for h in range(H):
            fp8 = None
            if skim_idx is not None:
                names = ("q4", "qs4", "k4", "ks4", "v4", "vs4") if lowp == "mxfp4" else \
                    ("q8", "k8", "v8", "qexp", "kexp", "vexp")
                fp8 = {n: pooled[n][b, h] for n in names}
            kmom = pooled["kmom"][b, h] if comp == 1 else None
            hbar = pooled["hbar"][b, h] if comp == 2 else None
            for a in range(nb):
                r0, r1 = a * blk, min(N, (a + 1) * blk)
                if r1 <= r0:
                    continue
                ex = exact_idx[b, h, a, :exact_cnt[b, h, a]]
                sk = () if skim_idx is None else skim_idx[b, h, a, :skim_cnt[b, h, a]]
                o, l = rule_block(q[b, h, r0:r1], k[b, h], v[b, h], N, scale, comp,
                                  pooled["kbar64"][b, h], pooled["vbar64"][b, h], pooled["kcount"],
                                  ex, sk, kmom, fp8, a, blk, hbar)
                O[b, h, r0:r1] = o
                lse[b, h, r0:r1] = l
    return O, lse
