"""Per-block statistics of Q, K, V (fp64, sequential sums).

Pages: PISA ("PISA: Piecewise Sparse Attention Is Wiser for Efficient
Diffusion Transformers", section 2, "Algorithme Central" and "Implementation
Materielle") approximates each non-critical key block through its centroid
k_bar_j and its value sum, and precomputes centroids, value sums and the
per-block first-order matrices before the attention pass.  SVG-EAR ("SVG-EAR:
Parameter-Free Linear Compensation for Sparse Video Generation via
Error-aware Routing", section 2A) replaces skipped keys and values by their
means.  Here a block is the geometric run of 64 consecutive tokens.

Arithmetic contract (so that routing can be compared bit for bit): block sums
are fp64, over valid tokens in increasing order, starting from +0.0; the mean
is the fp64 quotient sum / n_j, then rounded to fp32.
"""

import numpy as np

from . import e4m3, mxfp4

BLK = 64


def block_counts(N: int, N_pad: int, blk: int = BLK) -> np.ndarray:
    """Valid tokens per block: n_j = min(blk, N - blk*j), int32 [N_pad/blk]."""
    nb = N_pad // blk
    j = np.arange(nb)
    return np.clip(N - blk * j, 0, blk).astype(np.int32)


def _blocked(x: np.ndarray, blk: int) -> np.ndarray:
    B, H, Np, d = x.shape
    return x.reshape(B, H, Np // blk, blk, d)


def block_sums(x: np.ndarray, N: int, blk: int = BLK) -> np.ndarray:
    """fp64 sums of the valid tokens of each block, accumulated in token order."""
    xb = _blocked(np.asarray(x), blk)
    nb = xb.shape[2]
    valid = (np.arange(nb)[:, None] * blk + np.arange(blk)[None, :]) < N   # [nb, blk]
    acc = np.zeros(xb.shape[:3] + (xb.shape[4],), np.float64)
    for t in range(blk):
        term = np.where(valid[:, t][None, None, :, None], xb[:, :, :, t, :].astype(np.float64), 0.0)
        acc = acc + term
    return acc


def block_means(x: np.ndarray, N: int, blk: int = BLK):
    """(fp32 means [B,H,nb,d], fp64 exact-order means, int32 counts [nb])."""
    n = block_counts(N, x.shape[2], blk)
    s = block_sums(x, N, blk)
    m64 = s / np.maximum(n, 1)[None, None, :, None].astype(np.float64)
    return m64.astype(np.float32), m64, n


def block_moments(k: np.ndarray, v: np.ndarray, N: int, blk: int = BLK) -> np.ndarray:
    """First-order block matrices H_j = sum_n (k_n - k_bar_j) v_n^T, fp64 [B,H,nb,d,d].

    H_j[i, o] pairs key dimension i with value dimension o, so q^T H_j is a
    value-space vector (PISA, "Algorithme Central": the per-block first-order
    matrices whose mean is H_bar).
    """
    _, kbar, n = block_means(k, N, blk)
    kb = _blocked(np.asarray(k, np.float64), blk)
    vb = _blocked(np.asarray(v, np.float64), blk)
    nb = kb.shape[2]
    valid = ((np.arange(nb)[:, None] * blk + np.arange(blk)[None, :]) < N).astype(np.float64)
    kc = (kb - kbar[:, :, :, None, :]) * valid[None, None, :, :, None]
    return np.einsum("bhjni,bhjno->bhjio", kc, vb * valid[None, None, :, :, None])


def global_moment(k: np.ndarray, v: np.ndarray, N: int, blk: int = BLK) -> np.ndarray:
    """PISA's global first-order statistic H_bar, fp64 [B,H,d,d]: the mean of
    the per-block first-order matrices H_j over all nb blocks of the head
    (PISA, section 2, "Algorithme Central", global first-order correction;
    precomputed before the attention pass per "Implementation Materielle").
    """
    return block_moments(k, v, N, blk).mean(axis=2)


def covariance_norms(k: np.ndarray, v: np.ndarray, N: int, blk: int = BLK) -> np.ndarray:
    """ln M_j with M_j = ||H_j - H_bar||_2, the largest singular value of the
    block's deviation from the head's mean moment, fp64 [B,H,nb].

    PISA's covariance-aware top-k ("PISA ...", section 2, "Routage Sensible a
    la Covariance") weighs each block by this norm: a block whose moment is
    far from H_bar is badly served by the global first-order term.  The
    spectral norm is taken from the singular values (numpy's matrix 2-norm);
    a block whose moment equals H_bar gets ln 0 = -inf.
    """
    H = block_moments(k, v, N, blk)
    D = H - H.mean(axis=2)[:, :, None]
    M = np.linalg.norm(D, ord=2, axis=(3, 4))
    with np.errstate(divide="ignore"):
        return np.log(M)


def block_spreads(k: np.ndarray, v: np.ndarray, N: int, blk: int = BLK) -> np.ndarray:
    """lambda_j = ln(r_k * r_v) with r_x^2 = sum_n ||x_n - x_bar_j||^2, as fp32 [B,H,nb].

    Triage's router ("Triage ...", "Un routage fonde sur l'erreur estimee")
    estimates each tile's omission error from block statistics; the spread of
    keys and values around their centroids bounds the first-order error of the
    centroid term (|q^T H_j| <= |q| r_k r_v).  A block with one token has
    spread 0 and lambda = -inf.
    """
    out = []
    for x in (k, v):
        _, xbar, _ = block_means(x, N, blk)
        xb = _blocked(np.asarray(x, np.float64), blk)
        nb = xb.shape[2]
        valid = ((np.arange(nb)[:, None] * blk + np.arange(blk)[None, :]) < N)
        dev = (xb - xbar[:, :, :, None, :]) * valid[None, None, :, :, None]
        out.append(np.sum(dev * dev, axis=(3, 4)))
    with np.errstate(divide="ignore"):
        lam = 0.5 * np.log(out[0]) + 0.5 * np.log(out[1])
    return lam.astype(np.float32)


def e4m3_blocks(x: np.ndarray, N: int, blk: int = BLK):
    """Per-block power-of-two scaled e4m3 copy of x.

    Returns (codes uint8 [B,H,N_pad,d], exponents int [B,H,nb]) with
    codes = e4m3(x * 2^-e_j) and e_j the smallest integer with
    amax_j * 2^-e_j <= 448 (amax over the block's valid tokens).  Pad rows
    get code 0.
    """
    xb = _blocked(np.asarray(x, np.float64), blk)
    B, H, nb, _, d = xb.shape
    valid = ((np.arange(nb)[:, None] * blk + np.arange(blk)[None, :]) < N)
    amax = np.max(np.where(valid[None, None, :, :, None], np.abs(xb), 0.0), axis=(3, 4))
    e = e4m3.block_exponent(amax)
    scaled = xb * np.exp2(-e.astype(np.float64))[:, :, :, None, None]
    codes = e4m3.encode(scaled)
    codes = np.where(valid[None, None, :, :, None], codes, 0).astype(np.uint8)
    return codes.reshape(B, H, nb * blk, d), e


def mxfp4_copies(q, k, v, N: int, blk: int = BLK) -> dict:
    """MXFP4 copies for the 4-bit skim tier (Triage's fast tier in the page's
    own 4 bits).  Q and K: one E8M0 scale per token and 32 consecutive
    dimensions (the reduction axis of Q K^T); V: one scale per key block and
    dimension over the block's valid keys (the reduction axis of P V is the
    key).  Codes are one per element (0..15); pad tokens are code 0 with
    exponent 0.  Returns q4, qs4 [B,H,N_pad,d/32], k4, ks4, v4 [B,H,N_pad,d],
    vs4 [B,H,nb,d].
    """
    out = {}
    for name, x in (("q", q), ("k", k)):
        xx = np.array(x, np.float64)
        xx[:, :, N:] = 0.0
        c, e = mxfp4.quantize_blocks(xx, axis=-1, block=32)
        out[name + "4"], out[name + "s4"] = c, e
    vb = _blocked(np.array(v, np.float64), blk)
    nb = vb.shape[2]
    valid = ((np.arange(nb)[:, None] * blk + np.arange(blk)[None, :]) < N)
    vb = np.where(valid[None, None, :, :, None], vb, 0.0)
    e = mxfp4.block_exponent(np.abs(vb).max(axis=3))                     # [B,H,nb,d]
    codes = mxfp4.encode(vb * np.exp2(-e.astype(np.float64))[:, :, :, None, :])
    out["v4"] = codes.reshape(np.shape(v))
    out["vs4"] = e
    return out


def pool(q, k, v, N, blk: int = BLK, moments=False, spreads=False, fp8=False, hbar=False, cov=False,
         fp4=False):
    """Everything the router and the fused forward read, in one dict."""
    qbar, qbar64, n = block_means(q, N, blk)
    kbar, kbar64, _ = block_means(k, N, blk)
    vbar, vbar64, _ = block_means(v, N, blk)
    out = dict(qbar=qbar, kbar=kbar, vbar=vbar, kcount=n,
               qbar64=qbar64, kbar64=kbar64, vbar64=vbar64)
    if moments:
        out["kmom"] = block_moments(k, v, N, blk)
    if hbar:
        out["hbar"] = global_moment(k, v, N, blk)
    if cov:
        out["kcov"] = covariance_norms(k, v, N, blk)
    if spreads:
        out["klam"] = block_spreads(k, v, N, blk)
    if fp4:
        out.update(mxfp4_copies(q, k, v, N, blk))
    if fp8:
        for name, x in (("q", q), ("k", k), ("v", v)):
            c, e = e4m3_blocks(x, N, blk)
            out[name + "8"] = c
            out[name + "exp"] = e
    return out
