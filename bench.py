#!/usr/bin/env python3
"""Benchmark of one compensated block-sparse attention layer on one MI355X.

Workload: the Wan-1.3B-like 480p layer - B=1, H=12, head_dim=128, bf16,
21x30x52 = 32760 latent tokens (padded to 32768) in 4x4x4 tile-major 64-token
blocks, seeded Fourier-plus-noise Q/K/V, top-k keeping 20% of key blocks per
query block (103 of 512) with centroid (zeroth-order) compensation of the rest.

One step = pool -> route -> fused forward on inputs already resident in HBM.
The JSON line reports:
  value          kept-tile work of the layer / step time (TFLOP/s), where a
                 kept tile is 4*64*64*d flop (two 64x64xd products)
  roofline       the fused forward kernel (the dominant one): kept flop per
                 launch / its mean launch time measured with HIP events on the
                 launch stream, against the 2.5 PFLOP/s dense bf16 MFMA peak;
                 traffic = HBM bytes per launch from rocprofv3 FETCH_SIZE +
                 WRITE_SIZE when the committed counter summary matches the
                 current kernel source, else null
  cpu_baseline   the fp64 numpy oracle (test infrastructure) on one head of the
                 same layer, timed on this host's cores
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
HBM_PEAK_GBS = 8000.0
FP64_PEAK_TFLOPS = 78.6
FWD_SOURCE = os.path.join(ROOT, "free_block_sparse_attn_amd", "csrc", "fwd_bf16.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd_bf16_wan13b_traffic.json")


def kernel_traffic():
    """HBM bytes per forward launch from the committed counter summary, if current."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        src = hashlib.sha256(open(FWD_SOURCE, "rb").read()).hexdigest()
        if rec.get("source_sha256") != src:
            return None
        return rec["bytes_per_launch"]
    except (OSError, ValueError, KeyError):
        return None


CPU_HEADS = 6


def cpu_baseline(wl, q, k, v):
    """fp64 oracle on CPU_HEADS heads of the layer (pool, route, compensated rule)."""
    import numpy as np
    from oracle import pooling, routing, attention
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count()
    qh, kh, vh = (x[:, :CPU_HEADS] for x in (q, k, v))
    t0 = time.perf_counter()
    po = pooling.pool(qh, kh, vh, wl.N)
    idx, cnt = routing.route_topk(po["qbar"], po["kbar"], wl.topk)
    attention.sparse_attention(qh, kh, vh, wl.N, 1.0, wl.comp, po, idx, cnt)
    dt = time.perf_counter() - t0
    kept = float(cnt.sum()) * 4 * 64 * 64 * wl.d
    return {"value": kept / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{CPU_HEADS} of {wl.H} heads (all {wl.nb} query blocks each): pool + top-k "
                      f"route + compensated rule, fp64 numpy, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="end with a 1 GiB device-to-device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported "
              "(one GPU runs the whole layer; heads are independent, so more GPUs would split them with no exchange)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import free_block_sparse_attn_amd as fbsa
    from workloads import WORKLOADS, make_qkv

    wl = WORKLOADS[2]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v, _ = make_qkv(wl)
    dq, dk, dv = (torch.from_numpy(x).to(torch.bfloat16).to(dev) for x in (q, k, v))
    N = wl.N

    pooled = fbsa.sparse_attn_pool(dq, dk, dv, N)
    route_out = fbsa.sparse_attn_route(pooled, N, fbsa.SA_ROUTE_TOPK, topk=wl.topk)
    out, lse = fbsa.sparse_attn_fwd(dq, dk, dv, N, 1.0, wl.comp, pooled, route_out[0], route_out[1])
    torch.cuda.synchronize()

    # HIP events bracket each kernel of every timed step on the current
    # stream, which is the stream the binding launches on
    names = ("pool", "route", "fwd")
    evs = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)] for n in names}

    def step(i=None):
        def run(name, fn):
            if i is None:
                fn()
                return
            s, e = evs[name][i]
            s.record()
            fn()
            e.record()
        run("pool", lambda: fbsa.sparse_attn_pool(dq, dk, dv, N, out=pooled))
        run("route", lambda: fbsa.sparse_attn_route(pooled, N, fbsa.SA_ROUTE_TOPK, topk=wl.topk, out=route_out))
        run("fwd", lambda: fbsa.sparse_attn_fwd(dq, dk, dv, N, 1.0, wl.comp, pooled, route_out[0], route_out[1],
                                                out=out, lse=lse))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    # mean launch duration of each kernel over the timed steps
    ms_pool, ms_route, ms_fwd = (sum(s.elapsed_time(e) for s, e in evs[n]) / args.steps for n in names)

    cnt = route_out[1].cpu().numpy()
    kept_flop = float(cnt.sum()) * 4 * 64 * 64 * wl.d
    fwd_tflops = kept_flop / (ms_fwd * 1e-3) / 1e12
    pool_bytes = 3 * dq.numel() * 2 + 3 * pooled["qbar"].numel() * 4
    route_flop = 2.0 * wl.B * wl.H * wl.nb * wl.nb * wl.d
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
        "dtype": "bf16",
        "data": "synthetic (seeded Fourier-plus-noise video tokens)",
        "config": {"workload": "wan13b-480p-layer: B=1 H=12 d=128 T*Y*X=21*30*52 (N=32760), "
                               "64-token 4x4x4 tile-major blocks, top-k 20% (k=103/512), "
                               "centroid compensation",
                   "global_batch": wl.B, "seq_len": wl.N, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(fwd_tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(fwd_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": kernel_traffic()},
        "kernels_ms": {"pool": round(ms_pool, 4), "route": round(ms_route, 4), "fwd": round(ms_fwd, 4)},
        "pool_GBps": round(pool_bytes / (ms_pool * 1e-3) / 1e9, 1),
        "pool_hbm_frac": round(pool_bytes / (ms_pool * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "route_fp64_frac": round(route_flop / (ms_route * 1e-3) / 1e12 / FP64_PEAK_TFLOPS, 4),
        "kept_tiles": int(cnt.sum()),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, q, k, v)
    print(json.dumps(line), flush=True)
    if args.copy_calibration:
        x = torch.ones(1 << 29, dtype=torch.int16, device=dev)       # 1 GiB
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        y.copy_(x)
        torch.cuda.synchronize()


if __name__ == "__main__":
    main()
