"""Seeded synthetic video-token workloads.

This package is the only code shared by the fp64 CPU oracle and the GPU path.
It holds no attention arithmetic: it lays tokens out, draws the random fields,
rounds them to the storage dtype and describes the five workload shapes.

Token layout. A latent video of T x Y x X tokens is cut into 4 x 4 x 4
(t, y, x) tiles.  Tokens are ordered tile-major: tiles in (t, y, x) row-major
order over the tile grid, and inside a tile (t, y, x) row-major, with partial
tiles at the edges.  The flat sequence is then cut into consecutive 64-token
blocks and tail-padded to a multiple of 64.  This is the geometric blocking on
which all five methods of the pages route (PISA's key blocks, SVG-EAR's
centroid blocks, Triage's tiles, LVSA's per-frame block sets).

Field generator. Every (workload, batch, head, tensor) draws its own stream
from numpy's SeedSequence([workload_id, b, h, tensor]) with tensor 0/1/2 for
Q/K/V: eight cosine modes over (t, y, x) with wave vectors uniform in
[-1/16, 1/16) cycles per token, phases uniform in [0, 2 pi) and N(0, I_d)
amplitude vectors, plus N(0, 0.3^2) noise, all scaled by d^-1/4 (so the
softmax scale is 1).  Values are rounded to fp32, then to bf16 (RNE) for the
bf16 workloads.
"""

from .layout import tile_major_coords, block_frame_ranges, padded_len
from .fields import make_qkv, round_to_bf16, bf16_bits, lvsa_anchor_phase
from .configs import WORKLOADS, Workload, get_workload

__all__ = [
    "tile_major_coords", "block_frame_ranges", "padded_len",
    "make_qkv", "round_to_bf16", "bf16_bits", "lvsa_anchor_phase",
    "WORKLOADS", "Workload", "get_workload",
]
