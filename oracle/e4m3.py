"""OCP fp8 E4M3 ("e4m3fn") codec written from the format definition.

Bit layout s.eeee.mmm, exponent bias 7, no infinities, S.1111.111 is NaN, so
the largest finite magnitude is 1.110b * 2^8 = 448.  Exponent field 0 holds
subnormals m * 2^-9.  Triage's low-precision tier (page "Triage: Skip, Skim,
or Refine Attention Tiles in Video Diffusion Transformers", plain-language
summary) is a fast low-precision tile; the 8-bit e4m3 format is this build's
stated reading of it.
"""

import numpy as np

MAX_FINITE = 448.0
MIN_NORMAL = 2.0 ** -6
SUBNORMAL_QUANTUM = 2.0 ** -9


def decode(codes: np.ndarray) -> np.ndarray:
    """Values (float64) of uint8 e4m3 codes; NaN codes decode to NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m * SUBNORMAL_QUANTUM, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


def encode(x: np.ndarray) -> np.ndarray:
    """Round float64 values to e4m3 codes: nearest, ties to even, saturating at 448.

    NaN maps to 0x7F.  The sign of zero is kept.
    """
    x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x).astype(np.int64) << 7
    a = np.abs(x)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, MAX_FINITE))
    # exponent of the leading bit: a = f * 2^k with f in [0.5, 1)
    _, k = np.frexp(np.where(a > 0, a, 1.0))
    E = np.maximum(k - 1, -6)                       # subnormals share exponent -6
    quantum = np.exp2(E - 3.0)
    m = np.rint(a / quantum).astype(np.int64)       # exact scaling; rint = ties to even
    # mantissa overflow 16 -> next binade
    carry = m >= 16
    E = np.where(carry, E + 1, E)
    m = np.where(carry, m // 2, m)
    normal = m >= 8
    efield = np.where(normal, E + 7, 0)
    mfield = np.where(normal, m - 8, m)
    code = sign | (efield << 3) | mfield
    code = np.where(nan, 0x7F, code)
    return code.astype(np.uint8)


def round_to_e4m3(x: np.ndarray) -> np.ndarray:
    """x rounded to the nearest e4m3 value (float64), with the encode() rule."""
    return decode(encode(x))


def block_exponent(amax: np.ndarray) -> np.ndarray:
    """Smallest integer e with amax * 2^-e <= 448 (0 where amax == 0).

    With amax = f * 2^k, f in [0.5, 1): 448 * 2^(k-9) = 0.875 * 2^k, so
    e = k - 9 when f <= 0.875 and k - 8 otherwise.  Integer logic only.
    """
    amax = np.asarray(amax, dtype=np.float64)
    f, k = np.frexp(amax)
    e = np.where(f <= 0.875, k - 9, k - 8)
    return np.where(amax > 0, e, 0).astype(np.int64)
