"""Compensated block-sparse attention for video diffusion transformers on MI355X.

Python face of libsparse_attn.so.  The three calls mirror the C ABI
(include/sparse_attn.h) and take torch tensors that already live on the GPU;
outputs are allocated here with torch (plumbing) and filled by the HIP
kernels on the current stream:

    pooled = sparse_attn_pool(q, k, v, N, moments=..., spreads=..., fp8=...)
    idx, cnt, idx2, cnt2 = sparse_attn_route(pooled, N, mode=..., ...)
    out, lse = sparse_attn_fwd(q, k, v, N, scale, comp, pooled, idx, cnt, idx2, cnt2)
"""

import ctypes

import torch

from . import _lib
from ._lib import (SparseAttnError, SA_F32, SA_BF16, SA_COMP_DROP, SA_COMP_ORDER0,
                   SA_COMP_ORDER1_BLOCK, SA_COMP_ORDER1_GLOBAL, SA_ROUTE_TOPK, SA_ROUTE_LVSA,
                   SA_ROUTE_TRIAGE, SA_ROUTE_TOPK_COV, SA_ROUTE_ERROR, SA_SKIM_E4M3, SA_SKIM_MXFP4)

__all__ = [
    "sparse_attn_pool", "sparse_attn_pool_static", "sparse_attn_route", "sparse_attn_fwd",
    "sparse_attn_lvsa_capacity", "sparse_attn_residual",
    "abi_version", "SparseAttnError", "SA_COMP_DROP", "SA_COMP_ORDER0", "SA_COMP_ORDER1_BLOCK",
    "SA_COMP_ORDER1_GLOBAL",
    "SA_ROUTE_TOPK", "SA_ROUTE_LVSA", "SA_ROUTE_TRIAGE", "SA_ROUTE_TOPK_COV",
    "SA_ROUTE_ERROR", "SA_SKIM_E4M3", "SA_SKIM_MXFP4",
]

BLK = 64


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _shape(q, N):
    B, H, Np, d = q.shape
    return _lib.Shape(B, H, N, Np, d)


def _dtype(t):
    if t.dtype == torch.bfloat16:
        return SA_BF16
    if t.dtype == torch.float32:
        return SA_F32
    raise SparseAttnError(1, f"unsupported tensor dtype {t.dtype}")


def _contig(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise SparseAttnError(1, "tensors must be contiguous CUDA tensors")


def abi_version() -> int:
    return _lib.load().sparse_attn_abi_version()


def sparse_attn_pool(q, k, v, N: int, moments=False, spreads=False, fp8=False, cent=None,
                     global_moment=False, cov=False, fp4=False, out=None) -> dict:
    """Block means (fp32), counts and the optional centroid planes / moments /
    mean moment H_bar (with its 64-partial scratch) / covariance log-norms
    ln ||H_j - H_bar||_2 (`cov`, implies `global_moment`) / spreads / e4m3
    copies / MXFP4 copies (`fp4`).  What the bf16 forward reads - the fp16
    centroid planes and the fp16 copy of V - is produced by default for bf16
    inputs with d == 128.

    `out` may pass a dict returned by an earlier call to reuse its buffers.
    """
    return _pool(q, k, v, N, moments, spreads, fp8, cent, global_moment, cov, fp4, out, static=False)


def sparse_attn_pool_static(q, k, v, N: int, moments=False, spreads=False, fp8=False, cent=None,
                            global_moment=False, cov=False, fp4=False, out=None) -> dict:
    """sparse_attn_pool through the allocation-free entry point: the H_bar
    partial sums use the library's own device scratch (no hbar_ws buffer;
    B * H <= SPARSE_ATTN_POOL_STATIC_HEADS when H_bar is requested).  With
    `out`, nothing is allocated here either."""
    return _pool(q, k, v, N, moments, spreads, fp8, cent, global_moment, cov, fp4, out, static=True)


def _pool(q, k, v, N, moments, spreads, fp8, cent, global_moment, cov, fp4, out, static):
    lib = _lib.load()
    _contig(q, k, v)
    B, H, Np, d = q.shape
    nb = Np // BLK
    dev = q.device
    if out is None:
        out = {
            "qbar": torch.empty(B, H, nb, d, dtype=torch.float32, device=dev),
            "kbar": torch.empty(B, H, nb, d, dtype=torch.float32, device=dev),
            "vbar": torch.empty(B, H, nb, d, dtype=torch.float32, device=dev),
            "kcount": torch.empty(nb, dtype=torch.int32, device=dev),
        }
        if cent is None:
            cent = q.dtype == torch.bfloat16 and d == 128
        if cent:
            nbc = BLK * ((nb + BLK - 1) // BLK)
            out["cent"] = torch.empty(B, H, 4, nbc, d, dtype=torch.float16, device=dev)
            out["v16"] = torch.empty(B, H, Np, d, dtype=torch.float16, device=dev)
        if moments:
            out["kmom"] = torch.empty(B, H, nb, d * d, dtype=torch.float16, device=dev)    # MFMA operand order
            out["kmom_exp"] = torch.empty(B, H, nb, dtype=torch.int8, device=dev)
        if global_moment or cov:
            out["hbar"] = torch.empty(B, H, d, d, dtype=torch.float32, device=dev)          # value-major
            if not static:
                out["hbar_ws"] = torch.empty(B, H, 64, d, d, dtype=torch.float32, device=dev)   # scratch
        if cov:
            out["kcov"] = torch.empty(B, H, nb, dtype=torch.float32, device=dev)
        if spreads:
            out["klam"] = torch.empty(B, H, nb, dtype=torch.float32, device=dev)
        if fp8:
            for n in ("q8", "k8"):
                out[n] = torch.empty(B, H, Np, d, dtype=torch.uint8, device=dev)
            out["v8"] = torch.empty(B, H, nb, d, BLK, dtype=torch.uint8, device=dev)   # block-transposed
            out["exp8"] = torch.empty(B, H, nb, 3, dtype=torch.int8, device=dev)
        if fp4:
            for n in ("q4", "k4"):
                out[n] = torch.empty(B, H, Np, d // 2, dtype=torch.uint8, device=dev)
            for n in ("qs4", "ks4"):
                out[n] = torch.empty(B, H, Np, d // 32, dtype=torch.uint8, device=dev)
            out["v4"] = torch.empty(B, H, nb, d, BLK // 2, dtype=torch.uint8, device=dev)   # block-transposed
            out["vs4"] = torch.empty(B, H, nb, d, dtype=torch.uint8, device=dev)
    g = out.get
    head = [ctypes.byref(_shape(q, N)), _dtype(q), _ptr(q), _ptr(k), _ptr(v),
            _ptr(out["qbar"]), _ptr(out["kbar"]), _ptr(out["vbar"]), _ptr(out["kcount"]),
            _ptr(g("cent")), _ptr(g("v16")), _ptr(g("kmom")), _ptr(g("kmom_exp")), _ptr(g("hbar"))]
    tail = [_ptr(g("kcov")), _ptr(g("klam")), _ptr(g("q8")), _ptr(g("k8")), _ptr(g("v8")), _ptr(g("exp8")),
            *_fp4_ptrs(out), _stream(q)]
    if static:
        _lib.check(lib.sparse_attn_pool_static(*head, *tail))
    else:
        _lib.check(lib.sparse_attn_pool(*head, _ptr(g("hbar_ws")), *tail))
    return out


def _fp4_ptrs(pooled):
    return [_ptr(pooled.get(n)) for n in ("q4", "k4", "v4", "qs4", "ks4", "vs4")]


def sparse_attn_lvsa_capacity(frame_lo, frame_hi, window: int, anchors: int) -> int:
    """Row capacity that holds every LVSA row (host int32 arrays)."""
    import numpy as np
    lo = np.ascontiguousarray(frame_lo, np.int32)
    hi = np.ascontiguousarray(frame_hi, np.int32)
    return _lib.load().sparse_attn_lvsa_capacity(lo.ctypes.data_as(ctypes.c_void_p),
                                                 hi.ctypes.data_as(ctypes.c_void_p),
                                                 lo.shape[0], window, anchors)


def sparse_attn_route(pooled: dict, N: int, mode: int = SA_ROUTE_TOPK, topk: int = 0,
                      frame_lo=None, frame_hi=None, window: int = 0, anchors: int = 0,
                      anchor_phase: int = 0, step: int = 0, cap: int = 0,
                      n_keep: int = 0, n_refine: int = 0, scale: float = 1.0,
                      keys=None, ekey=None, out=None):
    """Key-block lists per query block: (idx, cnt, idx2, cnt2); idx2/cnt2 only for Triage.

    TOPK_COV reads pooled["kcov"] (sparse_attn_pool(..., cov=True)), Triage
    pooled["klam"] (spreads=True); ERROR reads the bf16 token `keys` and
    fills the fp32 [B,H,nb,nb] workspace `ekey` (allocated here when None;
    ekey[b,h,j,a] = L(a, j)).  All three use `scale` in their keys.

    `out` may pass preallocated (idx, cnt, idx2, cnt2) tensors.
    """
    lib = _lib.load()
    qbar, kbar = pooled["qbar"], pooled["kbar"]
    B, H, nb, d = qbar.shape
    dev = qbar.device
    shape = _lib.Shape(B, H, N, nb * BLK, d)
    spec = _lib.RouteSpec(mode, topk, None, None, window, anchors, anchor_phase, step,
                          n_keep, n_refine, scale)
    cap2 = 0
    kterm = pooled.get("kcov") if mode == SA_ROUTE_TOPK_COV else pooled.get("klam")
    if mode in (SA_ROUTE_TOPK, SA_ROUTE_TOPK_COV, SA_ROUTE_ERROR):
        cap = cap or topk
    if mode == SA_ROUTE_ERROR:
        _contig(keys)
        if ekey is None:
            ekey = torch.empty(B, H, nb, nb, dtype=torch.float32, device=dev)
        _contig(ekey)
        spec.keys = keys.data_ptr()
        spec.ekey = ekey.data_ptr()
    elif mode == SA_ROUTE_LVSA:
        _contig(frame_lo, frame_hi)
        spec.frame_lo = frame_lo.data_ptr()
        spec.frame_hi = frame_hi.data_ptr()
        if not cap:
            raise SparseAttnError(1, "LVSA routing needs cap (see sparse_attn_lvsa_capacity)")
    elif mode == SA_ROUTE_TRIAGE:
        cap = n_refine
        cap2 = n_keep - n_refine
    if out is None:
        idx = torch.empty(B, H, nb, max(cap, 1), dtype=torch.int32, device=dev)
        cnt = torch.empty(B, H, nb, dtype=torch.int32, device=dev)
        idx2 = cnt2 = None
        if mode == SA_ROUTE_TRIAGE:
            idx2 = torch.empty(B, H, nb, max(cap2, 1), dtype=torch.int32, device=dev)
            cnt2 = torch.empty(B, H, nb, dtype=torch.int32, device=dev)
    else:
        idx, cnt, idx2, cnt2 = out
    _lib.check(lib.sparse_attn_route(
        ctypes.byref(shape), ctypes.byref(spec), _ptr(qbar), _ptr(kbar), _ptr(pooled.get("kcount")),
        _ptr(kterm), _ptr(idx), _ptr(cnt), cap, _ptr(idx2), _ptr(cnt2), cap2, _stream(qbar)))
    return idx, cnt, idx2, cnt2


def sparse_attn_fwd(q, k, v, N: int, scale: float, comp: int, pooled: dict, idx, cnt,
                    idx2=None, cnt2=None, want_lse=True, out=None, lse=None, skim_fmt=SA_SKIM_E4M3):
    """Compensated block-sparse attention forward; returns (out, lse).

    The skim tier (idx2 / cnt2) reads the e4m3 copies (skim_fmt SA_SKIM_E4M3)
    or the MXFP4 copies (SA_SKIM_MXFP4) from `pooled`."""
    lib = _lib.load()
    _contig(q, k, v, idx, cnt, idx2, cnt2)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        B, H, Np, _ = q.shape
        lse = torch.empty(B, H, Np, dtype=torch.float32, device=q.device)
    g = pooled.get
    cap = idx.shape[-1] if idx is not None else 0
    cap2 = idx2.shape[-1] if idx2 is not None else 0
    _lib.check(lib.sparse_attn_fwd(
        ctypes.byref(_shape(q, N)), _dtype(q), comp, scale, _ptr(q), _ptr(k), _ptr(v),
        _ptr(g("kbar")), _ptr(g("vbar")), _ptr(g("cent")), _ptr(g("v16")), _ptr(g("kcount")), _ptr(g("kmom")),
        _ptr(g("kmom_exp")), _ptr(g("hbar")),
        _ptr(g("q8")), _ptr(g("k8")), _ptr(g("v8")), _ptr(g("exp8")), skim_fmt, *_fp4_ptrs(pooled),
        _ptr(idx), _ptr(cnt), cap, _ptr(idx2), _ptr(cnt2), cap2,
        _ptr(out), _ptr(lse), _stream(q)))
    return out, lse


def sparse_attn_residual(q, k, v, out, N: int, scale: float, phase: int = 0, ridge: float = 1e-3,
                         rank: int = 8, workspace=None) -> dict:
    """SparsePR probe-fitted residual correction of `out` (bf16, in place).

    Returns views into the workspace: "xp" / "od" (sparse / dense output at
    the probes, fp32 [B,H,Mp,d]), "W" [B,H,d,d] and "c" [B,H,d].
    """
    lib = _lib.load()
    _contig(q, k, v, out)
    B, H, Np, d = q.shape
    shape = _shape(q, N)
    nbytes = lib.sparse_attn_residual_workspace(ctypes.byref(shape))
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    _contig(workspace)
    _lib.check(lib.sparse_attn_residual(
        ctypes.byref(shape), _dtype(q), scale, _ptr(q), _ptr(k), _ptr(v), _ptr(out), phase, ridge, rank,
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(q)))
    nb = Np // BLK
    mp = BLK * ((nb + BLK - 1) // BLK)
    bh = B * H
    off = bh * 8 * (3 * d * d + 2 * d) * 8 + bh * 3 * d * d * 8
    f32 = workspace[off:].view(torch.float32)
    xp = f32[:bh * mp * d].view(B, H, mp, d)
    od = f32[bh * mp * d:2 * bh * mp * d].view(B, H, mp, d)
    wc = f32[2 * bh * mp * d:2 * bh * mp * d + bh * (d * d + d)].view(B, H, d * d + d)
    return {"xp": xp, "od": od, "W": wc[:, :, :d * d].view(B, H, d, d), "c": wc[:, :, d * d:],
            "workspace": workspace}
