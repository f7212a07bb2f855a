#!/usr/bin/env python3
"""Benchmark of compensated block-sparse video attention layers on one MI355X.

Headline workload (the largest single-GPU layer): the HunyuanVideo-720p-like
layer with Triage's three tiers - B=1, H=24, head_dim=128, bf16,
33x45x80 = 118800 latent tokens (padded to 118848) in 4x4x4 tile-major
64-token blocks, seeded Fourier-plus-noise Q/K/V; per query block 15% of the
key blocks (279) are refined exactly in bf16, 25% (465) skimmed in fp8 e4m3,
the remaining 1113 compensated by their centroids.

One step = pool -> route -> fused forward on inputs already resident in HBM.
After the timed headline steps, every other configured workload runs the same
step (tiny fp32, Wan-480p top-k, Hunyuan-720p per-block first order, LVSA
with its anchors rotating over 4 denoising steps) and reports under
"configs".  --layer runs another layer as the headline (the pages' other
workloads: covariance / error-aware routing, the global first-order term,
the SparsePR residual pass, the MXFP4 skim tier).

The JSON line reports:
  value          kept-tile work of the layer / step time (TFLOP/s); a kept
                 tile (refine or skim) is 4*64*64*d flop
  roofline       the fused forward kernel (the dominant one), mean launch time
                 from HIP events on the launch stream; bf16 layers: kept flop /
                 time against 2.5 PFLOP/s; with a skim tier the bound is the
                 MFMA time at each dtype's peak (refine at 2.5, fp8 / fp4 skim
                 at 5.0 PFLOP/s), reported as the bf16-equivalent rate
                 (refine + skim / 2) / time.  traffic = HBM bytes per launch
                 from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary
                 when it matches the current kernel source, else null
  cpu_baseline   the fp64 numpy oracle (test infrastructure) on a bounded
                 sample of the headline layer, timed on this host's cores and
                 scaled to the whole layer
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0
MFMA_FP8_PEAK_TFLOPS = 5000.0
FP32_PEAK_TFLOPS = 157.3
HBM_PEAK_GBS = 8000.0
FP64_PEAK_TFLOPS = 78.6
# the forward kernel's source and the headers it includes: counters taken on
# other sources are stale
FWD_SOURCES = [os.path.join(ROOT, "free_block_sparse_attn_amd", "csrc", f)
               for f in ("fwd_bf16.hip", "fwd_bf16_skim.hip", "lds_tile.h", "common.h", "launch.h")]
HEADLINE = "triage-e4m3"

LAYERS = {
    # name: (workload key, description)
    "tiny": ("tiny", "tiny-layer: B=1 H=2 d=64 fp32 T*Y*X=4*16*16 (N=1024), top-k 25% (k=4/16), "
                     "centroid compensation"),
    "wan13b": ("wan13b", "wan13b-480p-layer: B=1 H=12 d=128 T*Y*X=21*30*52 (N=32760), "
                         "64-token 4x4x4 tile-major blocks, top-k 20% (k=103/512), centroid compensation"),
    "wan13b-error": ("wan13b-ear", "wan13b-480p-layer, SVG-EAR error-aware routing (k=103/512), "
                                   "centroid compensation"),
    "wan13b-residual": ("wan13b", "wan13b-480p-layer as wan13b, then the SparsePR probe-fitted "
                                  "residual pass (rank 8)"),
    "hunyuan-order1": ("hunyuan720p", "hunyuan720p-layer: B=1 H=24 d=128 T*Y*X=33*45*80 (N=118800), "
                                      "top-k 10% (k=186/1857), per-block first-order (H_j) compensation"),
    "hunyuan-global": ("hunyuan720p-global", "hunyuan720p-layer, top-k 10%, PISA global first-order "
                                             "(H_bar) compensation"),
    "hunyuan-global-cov": ("hunyuan720p-global-cov", "hunyuan720p-layer, covariance-aware top-k 10%, "
                                                     "global first-order compensation"),
    "lvsa": ("lvsa-long", "lvsa-long-layer: B=1 H=12 d=128 T*Y*X=81*30*52 (N=126360), +-2-frame window "
                          "+ 8 anchors rotating over 4 denoising steps, centroid compensation"),
    "triage-e4m3": ("triage", "hunyuan720p-triage-layer: B=1 H=24 d=128 T*Y*X=33*45*80 (N=118800), "
                              "64-token 4x4x4 tile-major blocks, Triage tiers per query block: refine 15% "
                              "(279 bf16 tiles), skim 25% (465 fp8 e4m3 tiles), skip 60% (centroid compensation)"),
    "triage-mxfp4": ("triage-mxfp4", "hunyuan720p-triage-layer as triage-e4m3 with the skim tier in MXFP4"),
}
# the other configured workloads, reported under "configs" after the headline
CONFIG_LAYERS = (("1-tiny", "tiny"), ("2-wan13b", "wan13b"), ("3-hunyuan720p-order1", "hunyuan-order1"),
                 ("4-lvsa-long", "lvsa"), ("5-triage", "triage-e4m3"))


def layer_workload(name):
    from workloads import WORKLOADS
    from workloads.configs import GLOBAL_ORDER1, GLOBAL_COV, ERROR_ROUTED, TRIAGE_FP4
    key = LAYERS[name][0]
    table = {"tiny": WORKLOADS[1], "wan13b": WORKLOADS[2], "hunyuan720p": WORKLOADS[3],
             "lvsa-long": WORKLOADS[4], "triage": WORKLOADS[5], "hunyuan720p-global": GLOBAL_ORDER1,
             "hunyuan720p-global-cov": GLOBAL_COV, "wan13b-ear": ERROR_ROUTED, "triage-mxfp4": TRIAGE_FP4}
    return table[key]


def fwd_source_sha256():
    """sha256 over the forward kernel's source files, in FWD_SOURCES order."""
    h = hashlib.sha256()
    for path in FWD_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_record(layer):
    """HBM bytes per forward launch from the committed counter summary of this
    layer, if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"fwd_bf16_{layer}_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
        src = fwd_source_sha256()
        if rec.get("source_sha256") != src:
            return None
        return rec["bytes_per_launch"]
    except (OSError, ValueError, KeyError):
        return None


def nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


class Layer:
    """Device inputs and the pool -> route -> fwd step of one layer."""

    def __init__(self, name, host_qkv):
        import torch
        import free_block_sparse_attn_amd as fbsa
        from workloads import block_frame_ranges, lvsa_anchor_phase
        self.name, self.fbsa = name, fbsa
        wl = self.wl = layer_workload(name)
        dev = torch.device("cuda:0")
        q, k, v, coords = host_qkv
        dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
        self.q, self.k, self.v = (torch.from_numpy(x).to(dev).to(dt) for x in (q, k, v))
        self.N = N = wl.N
        f4 = wl.skim_fmt == "mxfp4"
        self.triage = wl.rule == "triage"
        self.pool_kw = dict(moments=wl.comp == 1, global_moment=wl.comp == 2, cov=wl.rule == "topk_cov",
                            spreads=self.triage, fp8=self.triage and not f4, fp4=self.triage and f4)
        self.skim_fmt = fbsa.SA_SKIM_MXFP4 if f4 else fbsa.SA_SKIM_E4M3
        self.scale = 1.0
        self.pooled = fbsa.sparse_attn_pool(self.q, self.k, self.v, N, **self.pool_kw)
        self.nsteps_route = 1
        if wl.rule == "topk":
            kw = dict(mode=fbsa.SA_ROUTE_TOPK, topk=wl.topk)
        elif wl.rule == "topk_cov":
            kw = dict(mode=fbsa.SA_ROUTE_TOPK_COV, topk=wl.topk, scale=self.scale)
        elif wl.rule == "error":
            ekey = torch.empty(wl.B, wl.H, wl.nb, wl.nb, dtype=torch.float32, device=dev)
            kw = dict(mode=fbsa.SA_ROUTE_ERROR, topk=wl.topk, scale=self.scale, keys=self.k, ekey=ekey)
        elif wl.rule == "lvsa":
            lo, hi = block_frame_ranges(coords)
            cap = fbsa.sparse_attn_lvsa_capacity(lo, hi, wl.window, wl.anchors)
            kw = dict(mode=fbsa.SA_ROUTE_LVSA, frame_lo=torch.from_numpy(lo).to(dev),
                      frame_hi=torch.from_numpy(hi).to(dev), window=wl.window, anchors=wl.anchors,
                      anchor_phase=lvsa_anchor_phase(wl.wid, wl.anchor_period), step=0, cap=cap)
            self.nsteps_route = wl.steps            # the anchors rotate with the denoising step
        else:
            kw = dict(mode=fbsa.SA_ROUTE_TRIAGE, n_keep=wl.n_keep, n_refine=wl.n_refine, scale=self.scale)
        self.mode = kw.pop("mode")
        self.route_kw = kw
        self.route_out = fbsa.sparse_attn_route(self.pooled, N, self.mode, **kw)
        self.out, self.lse = fbsa.sparse_attn_fwd(self.q, self.k, self.v, N, self.scale, wl.comp, self.pooled,
                                                  *self.route_out, skim_fmt=self.skim_fmt)
        self.residual = name == "wan13b-residual"
        self.ws = None
        if self.residual:
            self.ws = fbsa.sparse_attn_residual(self.q, self.k, self.v, self.out, N, self.scale)["workspace"]
        self.names = ("pool", "route", "fwd") + (("residual",) if self.residual else ())
        self.tiles = []            # (kept, skim) tile counts of each timed step
        torch.cuda.synchronize()

    def step(self, i, evs=None):
        fbsa, N, wl = self.fbsa, self.N, self.wl

        def run(name, fn):
            if evs is None:
                fn()
                return
            s, e = evs[name][i]
            s.record()
            fn()
            e.record()
        kw = dict(self.route_kw)
        if self.nsteps_route > 1:
            kw["step"] = i % self.nsteps_route
        run("pool", lambda: fbsa.sparse_attn_pool(self.q, self.k, self.v, N, out=self.pooled))
        run("route", lambda: fbsa.sparse_attn_route(self.pooled, N, self.mode, out=self.route_out, **kw))
        run("fwd", lambda: fbsa.sparse_attn_fwd(self.q, self.k, self.v, N, self.scale, wl.comp, self.pooled,
                                                *self.route_out, out=self.out, lse=self.lse,
                                                skim_fmt=self.skim_fmt))
        if self.residual:
            run("residual", lambda: fbsa.sparse_attn_residual(self.q, self.k, self.v, self.out, N, self.scale,
                                                              workspace=self.ws))

    def timed(self, steps, warmup):
        """warmup untimed steps, then `steps` timed ones; HIP events bracket
        each kernel on the current stream (the stream the binding launches on).
        Returns (ms per step by wall clock, {kernel: mean ms})."""
        import torch
        evs = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(steps)] for n in self.names}
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(i, evs)
        torch.cuda.synchronize()
        ms_step = (time.perf_counter() - t0) * 1e3 / steps
        ms = {n: sum(s.elapsed_time(e) for s, e in evs[n]) / steps for n in self.names}
        # tile counts of the lists each route step produced (LVSA: per step)
        for s in range(self.nsteps_route):
            if self.nsteps_route > 1:
                kw = dict(self.route_kw, step=s)
                self.fbsa.sparse_attn_route(self.pooled, self.N, self.mode, out=self.route_out, **kw)
            cnt = int(self.route_out[1].sum().item())
            skim = int(self.route_out[3].sum().item()) if self.triage else 0
            self.tiles.append((cnt, skim))
        return ms_step, ms

    def metrics(self, ms_step, ms):
        wl = self.wl
        tile_flop = 4.0 * 64 * 64 * wl.d
        kept = sum(t[0] for t in self.tiles) / len(self.tiles)
        skim = sum(t[1] for t in self.tiles) / len(self.tiles)
        kept_flop = (kept + skim) * tile_flop
        t_fwd = ms["fwd"] * 1e-3
        if wl.dtype == "f32":
            peak, eq = FP32_PEAK_TFLOPS, kept_flop
        else:
            peak, eq = MFMA_BF16_PEAK_TFLOPS, (kept + skim * MFMA_BF16_PEAK_TFLOPS / MFMA_FP8_PEAK_TFLOPS) * tile_flop
        pool_in = nbytes(self.q) + nbytes(self.k) + nbytes(self.v)
        pool_out = sum(nbytes(t) for n, t in self.pooled.items() if n != "hbar_ws")
        pool_bytes = pool_in + pool_out
        route_in = nbytes(self.pooled["qbar"]) + nbytes(self.pooled["kbar"])
        if self.triage:
            route_in += nbytes(self.pooled["klam"]) + nbytes(self.pooled["kcount"])
        elif wl.rule == "topk_cov":
            route_in += nbytes(self.pooled["kcov"])
        elif wl.rule == "error":
            route_in += nbytes(self.k) + nbytes(self.pooled["kcount"])
        route_out = sum(nbytes(t) for t in self.route_out if t is not None)
        route_bytes = route_in + route_out
        m = {
            "ms": {**{n: round(t, 4) for n, t in ms.items()}, "step": round(ms_step, 4)},
            "kept_tiles": int(round(kept)),
            "kept_tflop": round(kept_flop / 1e12, 4),
            "value_tflops": round(kept_flop / (ms_step * 1e-3) / 1e12, 2),
            "fwd_kept_tflops": round(kept_flop / t_fwd / 1e12, 2),
            "fwd_frac": round(eq / t_fwd / 1e12 / peak, 4),
            "pool_GBps": round(pool_bytes / (ms["pool"] * 1e-3) / 1e9, 1),
            "pool_hbm_frac": round(pool_bytes / (ms["pool"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "route_GBps": round(route_bytes / (ms["route"] * 1e-3) / 1e9, 1),
            "route_hbm_frac": round(route_bytes / (ms["route"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        }
        if self.triage:
            m["skim_tiles"] = int(round(skim))
            m["fwd_bf16_equiv_tflops"] = round(eq / t_fwd / 1e12, 2)
        if wl.rule in ("topk", "topk_cov", "triage", "error"):
            route_flop = 2.0 * wl.B * wl.H * wl.nb * wl.nb * wl.d
            m["route_fp64_frac"] = round(route_flop / (ms["route"] * 1e-3) / 1e12 / FP64_PEAK_TFLOPS, 4)
        if wl.comp == 1:
            # every skipped tile also takes a Q H_j product (2 * 64 * d * d flop)
            nbq = wl.B * wl.H * wl.nb
            taylor = (nbq * wl.nb - kept) * 2.0 * 64 * wl.d * wl.d
            cent = nbq * ((wl.nb + 31) // 32) * 4.0 * 64 * 32 * wl.d * 2     # hi + lo planes
            m["fwd_all_mfma_tflops"] = round((kept * tile_flop + taylor + cent) / t_fwd / 1e12, 2)
        if self.nsteps_route > 1:
            m["steps_rotated"] = self.nsteps_route
            m["kept_tiles_per_step"] = [t[0] for t in self.tiles]
        return m, eq / t_fwd / 1e12, peak, kept_flop


def cpu_baseline(wl, q, k, v):
    """fp64 numpy oracle on a bounded sample of the Triage layer, scaled to the layer.

    Sample: pool (means, counts, spreads) of every head; the fp8 copies of
    SAMPLE_HEADS heads spread over the layer (every other head); Triage
    routing and the compensated rule (exact, skim and centroid terms) for one
    query block per sampled head, the blocks spread along the sequence.  Whole-layer time = pool of every head + fp8 copies per head x H +
    route and rule per query block x B*H*nb; value = the layer's kept flop /
    that time.
    """
    import numpy as np
    from oracle import pooling, routing, attention
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count()
    SAMPLE_HEADS = max(1, wl.H // 2)
    t0 = time.perf_counter()
    po = pooling.pool(q, k, v, wl.N, spreads=True)
    t_pool = time.perf_counter() - t0
    heads = list(range(0, wl.H, wl.H // SAMPLE_HEADS))[:SAMPLE_HEADS]
    t0 = time.perf_counter()
    fp8 = {}
    for h in heads:
        c = {}
        for name, x in (("q", q), ("k", k), ("v", v)):
            codes, e = pooling.e4m3_blocks(x[:, h:h + 1], wl.N)
            c[name + "8"], c[name + "exp"] = codes[0, 0], e[0, 0]
        fp8[h] = c
    t_fp8 = (time.perf_counter() - t0) / len(heads)
    rows = [(h, int((i + 0.5) * wl.nb / len(heads))) for i, h in enumerate(heads)]
    kept = 0
    t0 = time.perf_counter()
    for h, a in rows:
        sl = (slice(0, 1), slice(h, h + 1))
        ri, rc, si, sc = routing.route_triage(po["qbar"][sl][:, :, a:a + 1], po["kbar"][sl], po["klam"][sl],
                                              po["kcount"], 1.0, wl.n_keep, wl.n_refine)
        r0, r1 = 64 * a, min(wl.N, 64 * a + 64)
        attention.rule_block(q[0, h, r0:r1], k[0, h], v[0, h], wl.N, 1.0, wl.comp, po["kbar64"][0, h],
                             po["vbar64"][0, h], po["kcount"], ri[0, 0, 0, :rc[0, 0, 0]], si[0, 0, 0, :sc[0, 0, 0]],
                             None, fp8[h], a)
        kept += int(rc[0, 0, 0]) + int(sc[0, 0, 0])
    t_row = (time.perf_counter() - t0) / len(rows)
    n_rows = wl.B * wl.H * wl.nb
    t_layer = t_pool + t_fp8 * wl.B * wl.H + t_row * n_rows
    kept_flop = kept / len(rows) * n_rows * 4.0 * 64 * 64 * wl.d
    return {"value": kept_flop / t_layer / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": (f"fp64 numpy oracle: pool (means, counts, spreads) of all {wl.H} heads {t_pool:.1f} s; "
                       f"e4m3 copies of {len(heads)} heads {t_fp8:.1f} s/head; Triage route + compensated rule "
                       f"on {len(rows)} query blocks {t_row:.2f} s/block; scaled to {wl.H} heads x {wl.nb} "
                       f"query blocks = {t_layer / 3600:.2f} h per layer")}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layer", default=HEADLINE, choices=sorted(LAYERS),
                    help="headline layer (default: the Hunyuan-720p Triage layer, the largest configured one)")
    ap.add_argument("--no-configs", action="store_true", help="skip the other configured workloads")
    ap.add_argument("--config-steps", type=int, default=4, help="timed steps per other workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workers", type=int, default=max(1, min(16, os.cpu_count() or 1)),
                    help="processes generating the synthetic inputs (use 1 under a profiler)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="end with a 1 GiB device-to-device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported "
              "(one GPU runs the whole layer; heads are independent, so more GPUs would split them with no exchange)",
              file=sys.stderr)
        sys.exit(2)

    from workloads import make_qkv
    wl = layer_workload(args.layer)
    others = [] if args.no_configs else [(key, n) for key, n in CONFIG_LAYERS if n != args.layer]
    # every layer's inputs are generated before the GPU is touched (the
    # generator forks worker processes)
    t0 = time.perf_counter()
    host = {n: make_qkv(layer_workload(n), workers=args.workers) for n in [args.layer] + [n for _, n in others]}
    print(f"inputs of {len(host)} layer(s) generated in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)

    import torch
    torch.cuda.set_device(0)
    head = Layer(args.layer, host[args.layer])
    ms_step, ms = head.timed(args.steps, args.warmup)
    m, achieved, peak, kept_flop = head.metrics(ms_step, ms)
    del head
    torch.cuda.empty_cache()

    print(f"{args.layer}: {ms_step:.3f} ms per step", file=sys.stderr, flush=True)
    configs = {}
    if not args.no_configs:
        for key, name in CONFIG_LAYERS:
            if name == args.layer:
                configs[key] = dict(m, note="the headline run")
                continue
            lay = Layer(name, host.pop(name))
            s, k = lay.timed(max(args.config_steps, lay.nsteps_route), 1)
            configs[key] = lay.metrics(s, k)[0]
            print(f"{name}: {s:.3f} ms per step", file=sys.stderr, flush=True)
            del lay
            torch.cuda.empty_cache()

    line = {
        "metric": "effective TFLOP/s of sparse attn fwd (kept blocks) + % MFMA peak; ms/layer",
        "value": round(kept_flop / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16+e4m3" if wl.rule == "triage" and wl.skim_fmt == "e4m3" else
                 ("bf16+mxfp4" if wl.rule == "triage" else wl.dtype),
        "data": "synthetic (seeded Fourier-plus-noise video tokens)",
        "config": {"workload": LAYERS[args.layer][1],
                   "global_batch": wl.B, "seq_len": wl.N, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": traffic_record(args.layer)},
        "kernels_ms": m["ms"],
        "pool_GBps": m["pool_GBps"],
        "pool_hbm_frac": m["pool_hbm_frac"],
        "route_GBps": m["route_GBps"],
        "route_hbm_frac": m["route_hbm_frac"],
        "kept_tiles": m["kept_tiles"],
    }
    for n in ("skim_tiles", "route_fp64_frac", "fwd_all_mfma_tflops"):
        if n in m:
            line[n] = m[n]
    if configs:
        line["configs"] = configs
    if wl.rule == "triage" and wl.skim_fmt == "e4m3" and not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, *host[args.layer][:3])
    print(json.dumps(line), flush=True)
    if args.copy_calibration:
        x = torch.ones(1 << 29, dtype=torch.int16, device="cuda:0")       # 1 GiB
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        y.copy_(x)
        torch.cuda.synchronize()


if __name__ == "__main__":
    main()
