"""OCP MXFP4: fp4 E2M1 elements with an E8M0 power-of-two scale per block,
written from the format definition.

E2M1 bit layout s.ee.m, exponent bias 1, no infinities or NaN: exponent
field 0 holds the subnormal 0.5 m, so the eight magnitudes are
0, 0.5, 1, 1.5, 2, 3, 4, 6.  E8M0 holds 2^(byte - 127).

Triage's fast tier ("Triage: Skip, Skim, or Refine Attention Tiles in Video
Diffusion Transformers") computes tiles in 4 bits; CDNA4's block-scaled
matrix instructions take this format natively.  Scales here are chosen so no
element saturates: the block exponent is the smallest e with
amax * 2^-e <= 6.  Zero magnitudes are encoded as +0.
"""

import numpy as np

MAX_FINITE = 6.0
SCALE_BIAS = 127


def decode(codes: np.ndarray) -> np.ndarray:
    """Values (float64) of 4-bit codes (one code per array element, 0..15)."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    sign = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = c & 0x1
    val = np.where(e == 0, 0.5 * m, (1.0 + 0.5 * m) * np.exp2(e - 1.0))
    return sign * val


def encode(x: np.ndarray) -> np.ndarray:
    """Round float64 values to E2M1 codes: nearest, ties to the even code,
    saturating at 6; a result of magnitude 0 is +0."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), MAX_FINITE)
    grid = decode(np.arange(8))                       # 0, 0.5, ..., 6 in code order
    dist = np.abs(a[..., None] - grid)
    best = dist.min(axis=-1, keepdims=True)
    cand = dist == best                               # one code, or two on a tie
    # among tied codes take the even one (the codes of a tie differ by one)
    mag = np.where(cand[..., ::2].any(axis=-1),
                   2 * np.argmax(cand[..., ::2], axis=-1),
                   2 * np.argmax(cand[..., 1::2], axis=-1) + 1)
    sign = (x < 0) & (mag > 0)
    return (mag | (sign.astype(np.int64) << 3)).astype(np.uint8)


def block_exponent(amax: np.ndarray) -> np.ndarray:
    """Smallest integer e with amax * 2^-e <= 6 (0 where amax == 0), but at
    least -127, the smallest E8M0 scale.

    With amax = f * 2^k, f in [0.5, 1): 6 = 0.75 * 2^3, so e = k - 3 when
    f <= 0.75 and k - 2 otherwise.
    """
    amax = np.asarray(amax, dtype=np.float64)
    f, k = np.frexp(amax)
    e = np.maximum(np.where(f <= 0.75, k - 3, k - 2), -127)
    return np.where(amax > 0, e, 0).astype(np.int64)


def quantize_blocks(x: np.ndarray, axis: int = -1, block: int = 32):
    """MXFP4 copy of x with one scale per `block` consecutive elements along
    `axis` (whose length must be a multiple of `block`).

    Returns (codes uint8 with x's shape, exponents int64 with that axis
    divided by `block`); x ~= decode(codes) * 2^exponent of its block.
    """
    x = np.moveaxis(np.asarray(x, np.float64), axis, -1)
    shp = x.shape
    xb = x.reshape(shp[:-1] + (shp[-1] // block, block))
    e = block_exponent(np.abs(xb).max(axis=-1))
    codes = encode(xb * np.exp2(-e.astype(np.float64))[..., None])
    return np.moveaxis(codes.reshape(shp), -1, axis), np.moveaxis(e, -1, axis)


def dequantize_blocks(codes: np.ndarray, e: np.ndarray, axis: int = -1, block: int = 32) -> np.ndarray:
    """Inverse of quantize_blocks (exact in float64)."""
    c = np.moveaxis(np.asarray(codes), axis, -1)
    ee = np.moveaxis(np.asarray(e, np.int64), axis, -1)
    vals = decode(c) * np.exp2(np.repeat(ee, block, axis=-1).astype(np.float64))
    return np.moveaxis(vals, -1, axis)
