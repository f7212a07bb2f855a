"""Shared helpers of the GPU parity tests: seeded inputs on the device, the
oracle on the same values, and the comparison bars."""

import numpy as np
import torch

from oracle import attention, pooling, routing
from workloads import make_qkv, block_frame_ranges, lvsa_anchor_phase

BF16_TOL = 1e-2      # max |out - oracle| for bf16 outputs (row_tol: plus the store's half-ulp above 4)
F32_TOL = 1e-4       # max |out - oracle| for fp32 outputs
# lse: the bf16 path normalises with the sum of the fp16-rounded weights the
# matrix core multiplies, each within 2^-11 (fp16 unit roundoff) relative of
# the exact weight, so |d lse| <= -ln(1 - 2^-11) = 4.9e-4; plus fp32 logit
# error (exact tiles: fp32 MFMA sums of exact products; centroids: means as
# fp16 high + low parts) and, on skim rows, the block-scaled MFMA's logit
# error (<= 1.4e-4): 1e-3.
LSE_TOL = {"bf16": 1e-3, "f32": 1e-5}
# fp32 lse: a logit s = scale q.k is a sum of d = 64 fp32 products, whose
# rounding grows with the terms' size (random-walk estimate sqrt(d) 2^-24 |s|
# = 4.8e-7 |s|), and lse follows the largest logits; so on top of 1e-5 the
# fp32 bar allows 1e-6 |lse| (at scale 4 the logits reach ~40).  The bf16
# bar above already covers its logits' error.
LSE_REL = {"bf16": 0.0, "f32": 1e-6}
# The fp8 / MXFP4 skim tier's logits come out of the block-scaled MFMA, whose
# sums differ from the exact dot products of the low-precision copies by up
# to ~2e-4 in log2 units on these workloads (row lse off by <= 1.4e-4 where a
# skim block dominates).  Skim rows are checked against the oracle's bound of
# how far the output moves when those logits are off by SKIM_EPS (both e4m3
# codes accepted for weights that close to a rounding boundary, plus the
# continuous change; oracle.attention.rule_block slack_eps).
SKIM_EPS = 5e-4


def row_tol(dtype, o):
    """Per-row output bar.  fp32: 1e-4.  bf16: max-abs 1e-2 for rows with
    |o|_inf < 4; above, 1e-2 plus the half-ulp of the bf16 store at the row's
    largest magnitude (2^(e - 8) for |o|_inf in [2^e, 2^(e+1))), because from
    4 up that rounding alone (>= 2^-6 = 0.0156) can exceed 1e-2."""
    if dtype != "bf16":
        return np.full(o.shape[0], F32_TOL)
    amax = np.abs(o).max(axis=1)
    e = np.floor(np.log2(np.maximum(amax, 4.0)))
    return np.where(amax < 4.0, BF16_TOL, BF16_TOL + np.exp2(e - 8.0))


def to_device(wl, q, k, v):
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    return [torch.from_numpy(x).to(dt).cuda() for x in (q, k, v)]


def inputs(wl, heads=None):
    """numpy fp32 (exact input values) and device tensors of a workload."""
    q, k, v, coords = make_qkv(wl, heads=heads)
    return (q, k, v), to_device(wl, q, k, v), coords


def pool_results(pooled, n_pad):
    """The pooling pass's device outputs as numpy, in the oracle's layouts."""
    res = {n: (t.cpu().float() if t.dtype == torch.bfloat16 else t.cpu()).numpy() for n, t in pooled.items()}
    if "v8" in res:
        res["v8"] = v8_row_major(res["v8"], n_pad)
    if "q4" in res:
        for n in ("q4", "k4"):
            res[n] = unpack_nibbles(res[n])
        for n in ("qs4", "ks4", "vs4"):
            res[n] = res[n].astype(np.int64) - 127
        res["v4"] = v8_row_major(unpack_nibbles(res["v4"]), n_pad)
    if "kmom" in res:
        res["kmom"] = kmom_value_major(res["kmom"])
    return res


def run_gpu(wl, dev_qkv, coords, step=0, scale=1.0, edit=None):
    """pool -> route -> fwd through the C ABI; returns dict of numpy results.

    `edit` may replace the route's lists: (idx, cnt, idx2, cnt2) -> new ones."""
    import free_block_sparse_attn_amd as fbsa
    q, k, v = dev_qkv
    N = wl.N
    pooled = fbsa.sparse_attn_pool(q, k, v, N, moments=wl.comp == 1, global_moment=wl.comp == 2,
                                   cov=wl.rule == "topk_cov", spreads=wl.rule == "triage",
                                   fp8=wl.rule == "triage" and wl.skim_fmt == "e4m3",
                                   fp4=wl.rule == "triage" and wl.skim_fmt == "mxfp4")
    idx2 = cnt2 = None
    if wl.rule == "topk":
        idx, cnt, _, _ = fbsa.sparse_attn_route(pooled, N, fbsa.SA_ROUTE_TOPK, topk=wl.topk)
    elif wl.rule == "topk_cov":
        idx, cnt, _, _ = fbsa.sparse_attn_route(pooled, N, fbsa.SA_ROUTE_TOPK_COV, topk=wl.topk, scale=scale)
    elif wl.rule == "error":
        B, H = q.shape[:2]
        ekey = torch.empty(B, H, wl.nb, wl.nb, dtype=torch.float32, device=q.device)
        idx, cnt, _, _ = fbsa.sparse_attn_route(pooled, N, fbsa.SA_ROUTE_ERROR, topk=wl.topk, scale=scale,
                                                keys=k, ekey=ekey)
        pooled = dict(pooled, ekey=ekey)
    elif wl.rule == "lvsa":
        lo, hi = block_frame_ranges(coords)
        cap = fbsa.sparse_attn_lvsa_capacity(lo, hi, wl.window, wl.anchors)
        idx, cnt, _, _ = fbsa.sparse_attn_route(
            pooled, N, fbsa.SA_ROUTE_LVSA, frame_lo=torch.from_numpy(lo).cuda(),
            frame_hi=torch.from_numpy(hi).cuda(), window=wl.window, anchors=wl.anchors,
            anchor_phase=lvsa_anchor_phase(wl.wid, wl.anchor_period), step=step, cap=cap)
    else:
        idx, cnt, idx2, cnt2 = fbsa.sparse_attn_route(
            pooled, N, fbsa.SA_ROUTE_TRIAGE, n_keep=wl.n_keep, n_refine=wl.n_refine, scale=scale)
    if edit is not None:
        idx, cnt, idx2, cnt2 = edit(idx, cnt, idx2, cnt2)
    out, lse = fbsa.sparse_attn_fwd(q, k, v, N, scale, wl.comp, pooled, idx, cnt, idx2, cnt2,
                                    skim_fmt=fbsa.SA_SKIM_MXFP4 if wl.skim_fmt == "mxfp4" else fbsa.SA_SKIM_E4M3)
    torch.cuda.synchronize()
    res = pool_results(pooled, wl.N_pad)
    res["idx"], res["cnt"] = idx.cpu().numpy(), cnt.cpu().numpy()
    if idx2 is not None:
        res["idx2"], res["cnt2"] = idx2.cpu().numpy(), cnt2.cpu().numpy()
    res["out"] = out.float().cpu().numpy()
    res["lse"] = lse.cpu().numpy()
    return res


def kappa(p):
    """Key held at position p of a block-transposed fp8 V block."""
    return 32 * ((p % 32) // 16) + 8 * ((p % 16) // 4) + 4 * (p // 32) + p % 4


def v8_row_major(v8t, n_pad):
    """[B,H,nb,d,64] block-transposed codes -> [B,H,N_pad,d] row-major codes."""
    B, H, nb, d, _ = v8t.shape
    out = np.empty((B, H, nb, 64, d), v8t.dtype)
    p = np.arange(64)
    out[:, :, :, kappa(p), :] = np.swapaxes(v8t, -1, -2)
    return out.reshape(B, H, n_pad, d)


def unpack_nibbles(x):
    """uint8 [..., n] with two 4-bit codes per byte (even element low) -> [..., 2n]."""
    lo, hi = x & 0xF, x >> 4
    return np.stack([lo, hi], axis=-1).reshape(x.shape[:-1] + (2 * x.shape[-1],))


def kmom_value_major(x):
    """[B,H,nb,d*d] moments in MFMA operand order -> [B,H,nb,d,d] value-major G[o][i]:
    element ((o/32*8 + i/16)*64 + o%32 + 32*((i/8)%2))*8 + i%8 holds G[o][i]."""
    B, H, nb, dd = x.shape
    d = int(round(dd ** 0.5))
    y = x.reshape(B, H, nb, d // 32, d // 16, 2, 32, 8)        # [db][ks][h][o32][e]
    y = y.transpose(0, 1, 2, 3, 6, 4, 5, 7)                    # [db][o32][ks][h][e]
    return y.reshape(B, H, nb, d, d)


def oracle_pool(wl, q, k, v):
    return pooling.pool(q, k, v, wl.N, moments=wl.comp == 1, spreads=wl.rule == "triage",
                        fp8=wl.rule == "triage" and wl.skim_fmt == "e4m3", hbar=wl.comp == 2,
                        cov=wl.rule == "topk_cov", fp4=wl.rule == "triage" and wl.skim_fmt == "mxfp4")


def lists_of(idx, cnt, b, h, a):
    return idx[b, h, a, :cnt[b, h, a]]


def oracle_rows(wl, q, k, v, pooled, res, rows, scale=1.0):
    """Oracle (o, lse) of the sampled (b, h, a) query blocks, with the GPU's lists."""
    out = {}
    for (b, h, a) in rows:
        r0, r1 = 64 * a, min(wl.N, 64 * a + 64)
        ex = lists_of(res["idx"], res["cnt"], b, h, a) if res["idx"].shape[-1] else []
        sk = lists_of(res["idx2"], res["cnt2"], b, h, a) if "idx2" in res else ()
        fp8 = None
        if len(sk):
            names = ("q4", "qs4", "k4", "ks4", "v4", "vs4") if wl.skim_fmt == "mxfp4" else \
                ("q8", "k8", "v8", "qexp", "kexp", "vexp")
            fp8 = {n: pooled[n][b, h] for n in names}
        kmom = pooled["kmom"][b, h] if wl.comp == 1 else None
        hbar = pooled["hbar"][b, h] if wl.comp == 2 else None
        r = attention.rule_block(
            q[b, h, r0:r1], k[b, h], v[b, h], wl.N, scale, wl.comp, pooled["kbar64"][b, h],
            pooled["vbar64"][b, h], pooled["kcount"], ex, sk, kmom, fp8, a, hbar=hbar,
            slack_eps=SKIM_EPS if len(sk) else None)
        out[(b, h, a)] = r if len(sk) else (r[0], r[1], np.zeros(r1 - r0))
    return out


def _rows_worker(job):
    """One chunk of oracle rows in a spawned worker (reads the arrays that
    oracle_rows_parallel saved; single-threaded BLAS)."""
    path, wl, scale, chunk = job
    import numpy as np_
    from oracle import attention as att
    z = np_.load(path, allow_pickle=False)
    d = {n: z[n] for n in z.files}
    out = []
    for a in chunk:
        r0, r1 = 64 * a, min(wl.N, 64 * a + 64)
        ex = d["idx"][a, :d["cnt"][a]]
        sk = d["idx2"][a, :d["cnt2"][a]] if "idx2" in d else ()
        fp8 = None
        if len(sk):
            names = ("q4", "qs4", "k4", "ks4", "v4", "vs4") if wl.skim_fmt == "mxfp4" else \
                ("q8", "k8", "v8", "qexp", "kexp", "vexp")
            fp8 = {n: d[n] for n in names}
        r = att.rule_block(d["q"][r0:r1], d["k"], d["v"], wl.N, scale, wl.comp, d["kbar64"], d["vbar64"],
                           d["kcount"], ex, sk, d.get("kmom"), fp8, a, hbar=d.get("hbar"),
                           slack_eps=SKIM_EPS if len(sk) else None)
        out.append((a, r if len(sk) else (r[0], r[1], np_.zeros(r1 - r0))))
    return out


def oracle_rows_parallel(wl, q, k, v, pooled, res, rows, scale=1.0, workers=16):
    """oracle_rows for the query blocks `rows` of one head (b = h = 0 of the
    given arrays) in spawned worker processes (fresh interpreters, no GPU
    state; one BLAS thread each).  Returns {(0, 0, a): (o, lse, slack)}."""
    import os
    import tempfile
    import multiprocessing
    from concurrent.futures import ProcessPoolExecutor
    arrs = {"q": q[0, 0], "k": k[0, 0], "v": v[0, 0], "kbar64": pooled["kbar64"][0, 0],
            "vbar64": pooled["vbar64"][0, 0], "kcount": pooled["kcount"],
            "idx": res["idx"][0, 0], "cnt": res["cnt"][0, 0]}
    if "idx2" in res:
        arrs["idx2"], arrs["cnt2"] = res["idx2"][0, 0], res["cnt2"][0, 0]
        names = ("q4", "qs4", "k4", "ks4", "v4", "vs4") if wl.skim_fmt == "mxfp4" else \
            ("q8", "k8", "v8", "qexp", "kexp", "vexp")
        for n in names:
            arrs[n] = pooled[n][0, 0]
    if wl.comp == 1:
        arrs["kmom"] = pooled["kmom"][0, 0]
    if wl.comp == 2:
        arrs["hbar"] = pooled["hbar"][0, 0]
    workers = max(1, min(workers, os.cpu_count() or 1))
    chunks = [list(rows[i::workers * 4]) for i in range(workers * 4)]
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, "head.npz")
        np.savez(path, **arrs)
        saved = {n: os.environ.get(n) for n in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
        for n in saved:
            os.environ[n] = "1"
        try:
            ctx = multiprocessing.get_context("spawn")
            with ProcessPoolExecutor(workers, mp_context=ctx) as ex:
                parts = list(ex.map(_rows_worker, [(path, wl, scale, c) for c in chunks if c]))
        finally:
            for n, val in saved.items():
                if val is None:
                    os.environ.pop(n, None)
                else:
                    os.environ[n] = val
    return {(0, 0, a): r for part in parts for a, r in part}
