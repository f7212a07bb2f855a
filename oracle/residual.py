"""SparsePR's probe-fitted residual reconstruction ("Partition the Support,
Reconstruct the Residual...", section 2B), fp64.

A few query rows are computed densely; on them the residual of the sparse
output, R = O_dense - O_sparse, is modelled as an affine map of the sparse
output, R ~ b + x B, fitted by ridge regression; the fitted correction is
restricted to the span of the leading right singular vectors of the probe
residuals and added to every other row.

Readings (the page leaves M, lambda and r open):
  probes   one row per query block (stratified over the blocks, which are
           this build's query groups): row 64 a + ((phase + 37 a) mod n_a),
           n_a the block's valid rows
  ridge    lambda = ridge * tr(Xc^T Xc) / d on the centred probe outputs Xc;
           the intercept b is not penalised
  subspace the top `rank` right singular vectors V_r of R (uncentred);
           correction (b + x B) V_r V_r^T, i.e. W = B P, c = b P, P = V_r V_r^T
  rows     probe rows take their dense output; every other valid row gets
           o_t + c + o_t W
"""

import numpy as np

from .attention import dense_attention

BLK = 64


def probe_rows(N: int, nb: int, phase: int, blk: int = BLK) -> np.ndarray:
    """Probe row of every query block a: 64 a + ((phase + 37 a) mod n_a)."""
    a = np.arange(nb)
    n = np.minimum(blk, N - blk * a)
    return blk * a + (phase + 37 * a) % n


def fit_residual(X: np.ndarray, R: np.ndarray, ridge: float, rank: int):
    """Affine ridge fit R ~ b + X B restricted to the top-`rank` right singular
    subspace of R.  X, R: [M, d].  Returns (W = B P [d, d], c = b P [d])."""
    X = np.asarray(X, np.float64)
    R = np.asarray(R, np.float64)
    d = X.shape[1]
    xm, rm = X.mean(axis=0), R.mean(axis=0)
    Xc, Rc = X - xm, R - rm
    G = Xc.T @ Xc
    lam = ridge * np.trace(G) / d
    B = np.linalg.solve(G + lam * np.eye(d), Xc.T @ Rc)
    b = rm - xm @ B
    _, _, Vt = np.linalg.svd(R, full_matrices=False)
    Vr = Vt[:rank].T
    P = Vr @ Vr.T
    return B @ P, b @ P


def probe_correct(q, k, v, N: int, scale: float, O_sparse, phase: int, ridge: float, rank: int,
                  blk: int = BLK):
    """The corrected output for every (b, h): [B,H,N_pad,d] fp64 (pad rows 0).

    Also returns the per-head fits {(b, h): (W, c)} and the dense probe rows."""
    B_, H, Np, d = q.shape
    nb = Np // blk
    rows = probe_rows(N, nb, phase, blk)
    out = np.array(O_sparse, np.float64)
    fits, dense = {}, {}
    for b in range(B_):
        for h in range(H):
            Od = probe_dense(q[b, h], k[b, h], v[b, h], N, scale, rows)
            X = out[b, h, rows]
            W, c = fit_residual(X, Od - X, ridge, rank)
            fits[(b, h)] = (W, c)
            dense[(b, h)] = Od
            corr = out[b, h, :N] + c + out[b, h, :N] @ W
            out[b, h, :N] = corr
            out[b, h, rows] = Od
            out[b, h, N:] = 0.0
    return out, fits, dense


def probe_dense(qh, kh, vh, N: int, scale: float, rows) -> np.ndarray:
    """Dense softmax attention of the given query rows of one head, fp64 [len(rows), d]."""
    Q = np.asarray(qh, np.float64)[np.asarray(rows)]
    S = scale * (Q @ np.asarray(kh[:N], np.float64).T)
    S -= S.max(axis=1, keepdims=True)
    P = np.exp(S)
    return (P @ np.asarray(vh[:N], np.float64)) / P.sum(axis=1, keepdims=True)
