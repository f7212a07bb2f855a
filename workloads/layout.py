"""Tile-major token order and per-block frame ranges (integer index work only)."""

import numpy as np

BLOCK = 64
TILE = 4


def padded_len(n_tokens: int, blk: int = BLOCK) -> int:
    """Smallest multiple of `blk` that holds `n_tokens` tokens."""
    return blk * ((n_tokens + blk - 1) // blk)


def tile_major_coords(T: int, Y: int, X: int, tile: int = TILE) -> np.ndarray:
    """(t, y, x) coordinates of the T*Y*X tokens in tile-major sequence order.

    Returns int32 [T*Y*X, 3].  Tiles are visited in (t, y, x) row-major order
    over the ceil(T/4) x ceil(Y/4) x ceil(X/4) grid; inside a tile the tokens
    are (t, y, x) row-major.  Edge tiles hold fewer tokens.
    """
    t, y, x = np.meshgrid(np.arange(T), np.arange(Y), np.arange(X), indexing="ij")
    t, y, x = t.ravel(), y.ravel(), x.ravel()
    # lexsort: last key is the primary one
    order = np.lexsort((x % tile, y % tile, t % tile, x // tile, y // tile, t // tile))
    return np.stack([t[order], y[order], x[order]], axis=1).astype(np.int32)


def block_frame_ranges(coords: np.ndarray, blk: int = BLOCK):
    """First and last latent frame (t) covered by each block of `blk` tokens.

    Returns two int32 arrays of length ceil(N/blk).  Only valid tokens count,
    so the tail block's range covers its valid tokens only.
    """
    n = coords.shape[0]
    nb = (n + blk - 1) // blk
    tt = coords[:, 0]
    lo = np.empty(nb, np.int32)
    hi = np.empty(nb, np.int32)
    for j in range(nb):
        seg = tt[j * blk:min(n, (j + 1) * blk)]
        lo[j] = seg.min()
        hi[j] = seg.max()
    return lo, hi
