"""Seeded Fourier-plus-noise token fields (input generation only)."""

import numpy as np

from .layout import padded_len, tile_major_coords

N_MODES = 8
MAX_FREQ = 1.0 / 16.0   # cycles per latent token: blocks of 4x4x4 stay coherent
NOISE_STD = 0.3


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are already bf16-representable."""
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def make_head(workload_id: int, b: int, h: int, tensor: int, coords: np.ndarray,
              d: int, n_pad: int, dtype: str) -> np.ndarray:
    """One [n_pad, d] float32 slab of Q (tensor 0), K (1) or V (2); pad rows are 0."""
    rng = np.random.default_rng(np.random.SeedSequence([workload_id, b, h, tensor]))
    omega = rng.uniform(-MAX_FREQ, MAX_FREQ, size=(N_MODES, 3))
    phase = rng.uniform(0.0, 2.0 * np.pi, size=N_MODES)
    amp = rng.standard_normal((N_MODES, d))
    noise = rng.standard_normal((coords.shape[0], d), dtype=np.float32)
    waves = np.cos(2.0 * np.pi * (coords.astype(np.float64) @ omega.T) + phase)
    x = (waves @ amp + NOISE_STD * noise) * d ** -0.25
    out = np.zeros((n_pad, d), np.float32)
    out[:coords.shape[0]] = x.astype(np.float32)
    if dtype == "bf16":
        out = round_to_bf16(out)
    return out


def _make_one(job):
    return make_head(*job)


def make_qkv(wl, heads=None, batches=None, workers: int = 1):
    """Q, K, V as float32 [B', H', N_pad, d] for the chosen batches and heads.

    `wl` is a Workload.  The values are exactly representable in the
    workload's dtype.  `workers` > 1 generates the (tensor, batch, head) slabs
    in that many processes (each slab has its own seed, so the values do not
    depend on it).  Returns (q, k, v, coords).
    """
    coords = tile_major_coords(wl.T, wl.Y, wl.X)
    n_pad = padded_len(coords.shape[0])
    heads = list(range(wl.H)) if heads is None else list(heads)
    batches = list(range(wl.B)) if batches is None else list(batches)
    jobs = [(wl.wid, b, h, tensor, coords, wl.d, n_pad, wl.dtype)
            for tensor in range(3) for b in batches for h in heads]
    if workers > 1 and len(jobs) > 1:
        import multiprocessing
        with multiprocessing.get_context("fork").Pool(min(workers, len(jobs))) as pool:
            slabs = pool.map(_make_one, jobs, chunksize=1)
    else:
        slabs = [_make_one(j) for j in jobs]
    out = []
    it = iter(slabs)
    for tensor in range(3):
        arr = np.zeros((len(batches), len(heads), n_pad, wl.d), np.float32)
        for bi in range(len(batches)):
            for hi in range(len(heads)):
                arr[bi, hi] = next(it)
        out.append(arr)
    return out[0], out[1], out[2], coords


def lvsa_anchor_phase(workload_id: int, period: int) -> int:
    """Seeded phase offset o in [0, period) of the rotating anchor grid."""
    rng = np.random.default_rng(np.random.SeedSequence([workload_id, 4]))
    return int(rng.integers(period))
