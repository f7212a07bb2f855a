"""The five video-attention workloads and their reduced test variants.

Sizes mirror the latent grids of the models the pages evaluate (Wan 480p,
HunyuanVideo 720p and a long Wan horizon).  Head counts and head_dim are the
usual ones of those models; the pages give none.
"""

from dataclasses import dataclass, replace

from .layout import padded_len, BLOCK


def _ceil_pct(pct: int, n: int) -> int:
    return (pct * n + 99) // 100


@dataclass(frozen=True)
class Workload:
    wid: int            # seed namespace
    name: str
    B: int
    H: int
    d: int
    T: int
    Y: int
    X: int
    dtype: str          # "f32" or "bf16"
    rule: str           # "topk", "topk_cov", "error", "lvsa" or "triage"
    comp: int           # compensation order of skipped blocks: -1 drop, 0 centroid, 1 block Taylor,
                        # 2 global Taylor (one mean moment per head)
    keep_pct: int = 0           # top-k: percent of key blocks kept per query block
    window: int = 0             # LVSA: +- latent frames around the query block's frames
    anchors: int = 0            # LVSA: number of rotating anchor key blocks
    steps: int = 1              # LVSA: denoising steps (anchor rotation index s)
    refine_pct: int = 0         # Triage: percent of tiles computed exactly in bf16
    skim_pct: int = 0           # Triage: percent of tiles computed in low precision
    skim_fmt: str = "e4m3"      # Triage: skim tier format, "e4m3" or "mxfp4"

    @property
    def N(self) -> int:
        return self.T * self.Y * self.X

    @property
    def N_pad(self) -> int:
        return padded_len(self.N)

    @property
    def nb(self) -> int:
        return self.N_pad // BLOCK

    @property
    def topk(self) -> int:
        return _ceil_pct(self.keep_pct, self.nb)

    @property
    def n_refine(self) -> int:
        return _ceil_pct(self.refine_pct, self.nb)

    @property
    def n_keep(self) -> int:
        """Triage: refine + skim tiles per query block (the rest are skipped)."""
        return self.n_refine + _ceil_pct(self.skim_pct, self.nb)

    @property
    def anchor_period(self) -> int:
        return self.nb // self.anchors if self.anchors else 0

    def small(self, T: int, Y: int, X: int, H: int = 2) -> "Workload":
        """Same rule and dtype on a reduced grid (for element-wise parity tests)."""
        return replace(self, name=f"{self.name}-small", T=T, Y=Y, X=X, H=H)


WORKLOADS = {
    1: Workload(1, "tiny", 1, 2, 64, 4, 16, 16, "f32", "topk", 0, keep_pct=25),
    2: Workload(2, "wan13b", 1, 12, 128, 21, 30, 52, "bf16", "topk", 0, keep_pct=20),
    3: Workload(3, "hunyuan720p", 1, 24, 128, 33, 45, 80, "bf16", "topk", 1, keep_pct=10),
    4: Workload(4, "lvsa-long", 1, 12, 128, 81, 30, 52, "bf16", "lvsa", 0,
                window=2, anchors=8, steps=4),
    5: Workload(5, "triage", 1, 24, 128, 33, 45, 80, "bf16", "triage", 0,
                refine_pct=15, skim_pct=25),
}

# Reduced grids for element-wise parity: several blocks and a ragged tail.
SMALL = {
    1: WORKLOADS[1],
    2: WORKLOADS[2].small(5, 12, 20),     # 1200 tokens -> 19 blocks, tail 48
    3: WORKLOADS[3].small(6, 10, 18),     # 1080 tokens -> 17 blocks, tail 56
    4: WORKLOADS[4].small(21, 8, 9),      # 1512 tokens -> 24 blocks, tail 40
    5: WORKLOADS[5].small(6, 12, 15),     # 1080 tokens -> 17 blocks, tail 56
}


# The HunyuanVideo-like layer with PISA's global first-order term (same seeds
# and shapes as workload 3, so the two first-order forms see the same inputs).
GLOBAL_ORDER1 = replace(WORKLOADS[3], name="hunyuan720p-global", comp=2)
GLOBAL_ORDER1_SMALL = replace(SMALL[3], name="hunyuan720p-global-small", comp=2)
# ... routed by PISA's covariance-aware top-k (attention score and the norm of
# each block's moment deviation from H_bar) at the same 10% budget.
GLOBAL_COV = replace(GLOBAL_ORDER1, name="hunyuan720p-global-cov", rule="topk_cov")
GLOBAL_COV_SMALL = replace(GLOBAL_ORDER1_SMALL, name="hunyuan720p-global-cov-small", rule="topk_cov")

# The Wan-1.3B-like layer routed by SVG-EAR's error-aware rule at the same
# 20% block budget, centroid compensation of the rest.
ERROR_ROUTED = replace(WORKLOADS[2], name="wan13b-ear", rule="error")
ERROR_ROUTED_SMALL = replace(SMALL[2], name="wan13b-ear-small", rule="error")


# The Triage layer with its skim tier in the page's own 4 bits (MXFP4).
TRIAGE_FP4 = replace(WORKLOADS[5], name="triage-mxfp4", skim_fmt="mxfp4")
TRIAGE_FP4_SMALL = replace(SMALL[5], name="triage-mxfp4-small", skim_fmt="mxfp4")


def get_workload(wid: int, small: bool = False) -> Workload:
    return (SMALL if small else WORKLOADS)[wid]
