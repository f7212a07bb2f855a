"""CPU checks of the C ABI: the library loads, exports every declared symbol,
and rejects bad arguments on the host before any HIP call."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_attn.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:sa_status|int32_t|size_t|const char\*)\s+(sparse_attn_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    from free_block_sparse_attn_amd import _lib
    return _lib.load()


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("sparse_attn_pool", "sparse_attn_route", "sparse_attn_fwd", "sparse_attn_residual",
              "sparse_attn_residual_workspace"):
        assert n in names


def test_missing_library_raises():
    """No fallback: with the library absent, the first call raises."""
    import subprocess
    import sys
    env = dict(os.environ, SPARSE_ATTN_LIB=os.path.join(ROOT, "_no_such_dir", "libsparse_attn.so"))
    code = ("import free_block_sparse_attn_amd as f\n"
            "try:\n    f.abi_version()\nexcept RuntimeError as e:\n    print('raised:', e)\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "raised:" in r.stdout and "missing" in r.stdout, r.stdout


def test_library_exports_every_declared_symbol(lib):
    from free_block_sparse_attn_amd import _lib
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in _lib.EXPORTED, name
    assert lib.sparse_attn_abi_version() == 9


def shape(B=1, H=2, N=100, N_pad=128, d=128):
    from free_block_sparse_attn_amd import _lib
    return ctypes.byref(_lib.Shape(B, H, N, N_pad, d))


P = ctypes.c_void_p(4096)        # aligned, never dereferenced: validation fails first
MIS = ctypes.c_void_p(4097)


def pool(lib, sh, dtype=1, **kw):
    a = dict(q=P, k=P, v=P, qbar=P, kbar=P, vbar=P, kcount=P, cent=None, v16=None, kmom=None, kmom_exp=None,
             hbar=None, hbar_ws=None, kcov=None, klam=None, q8=None, k8=None, v8=None, exp8=None, q4=None, k4=None,
             v4=None, qs4=None, ks4=None, vs4=None)
    a.update(kw)
    return lib.sparse_attn_pool(sh, dtype, a["q"], a["k"], a["v"], a["qbar"], a["kbar"], a["vbar"],
                                a["kcount"], a["cent"], a["v16"], a["kmom"], a["kmom_exp"], a["hbar"], a["hbar_ws"],
                                a["kcov"], a["klam"], a["q8"], a["k8"], a["v8"], a["exp8"], a["q4"], a["k4"], a["v4"],
                                a["qs4"], a["ks4"], a["vs4"], None)


def test_pool_rejects_bad_arguments(lib):
    assert pool(lib, None) == 1
    assert pool(lib, shape(N_pad=192)) == 1                  # N_pad != 64*ceil(N/64)
    assert pool(lib, shape(d=96)) == 1
    assert pool(lib, shape(B=-1)) == 1
    assert pool(lib, shape(), dtype=7) == 1
    assert pool(lib, shape(), q=None) == 1
    assert pool(lib, shape(), kbar=MIS) == 1
    assert b"kbar" in lib.sparse_attn_last_error()
    assert pool(lib, shape(), q8=P) == 1                     # fp8 copies: all four or none
    assert pool(lib, shape(), dtype=0, kmom=P, kmom_exp=P) == 2   # moments need bf16, d=128
    assert pool(lib, shape(d=64), kmom=P, kmom_exp=P) == 2
    assert pool(lib, shape(), kmom=P) == 1                   # moments come with their exponents
    assert b"kmom_exp" in lib.sparse_attn_last_error()
    assert pool(lib, shape(), kmom_exp=P) == 1
    assert pool(lib, shape(), dtype=0, v16=P) == 2           # the fp16 copy of V needs bf16, d=128
    assert pool(lib, shape(d=64), v16=P) == 2
    assert pool(lib, shape(), v16=MIS) == 1
    assert pool(lib, shape(), dtype=0, cent=P) == 2          # centroid planes need bf16, d=128
    assert pool(lib, shape(d=64), cent=P) == 2
    assert pool(lib, shape(), cent=MIS) == 1
    assert pool(lib, shape(), hbar=P) == 1                   # the mean moment needs its scratch
    assert pool(lib, shape(), hbar_ws=P) == 1
    assert pool(lib, shape(), dtype=0, hbar=P, hbar_ws=P) == 2
    assert pool(lib, shape(), kcov=P) == 1                   # M_j is taken against H_bar
    assert b"hbar" in lib.sparse_attn_last_error()
    assert pool(lib, shape(), dtype=0, kcov=P, hbar=P, hbar_ws=P) == 2
    assert pool(lib, shape(), q4=P, k4=P) == 1               # MXFP4 copies: all six or none
    assert b"q4" in lib.sparse_attn_last_error()
    assert pool(lib, shape(d=64), q4=P, k4=P, v4=P, qs4=P, ks4=P, vs4=P) == 2   # bf16, d = 128 only
    assert pool(lib, shape(B=0)) == 0                        # empty problem: nothing launched
    assert pool(lib, shape(N=0, N_pad=0)) == 0


def route(lib, sh, spec, idx=P, cnt=P, cap=4, idx2=None, cnt2=None, cap2=0, klam=None, kcount=None):
    return lib.sparse_attn_route(sh, ctypes.byref(spec), P, P, kcount, klam, idx, cnt, cap, idx2, cnt2, cap2, None)


def test_route_rejects_bad_arguments(lib):
    from free_block_sparse_attn_amd import _lib
    S = _lib.RouteSpec
    assert route(lib, shape(), S(0, 0)) == 1                  # topk 0
    assert route(lib, shape(), S(0, 3)) == 1                  # topk > nb = 2
    assert route(lib, shape(), S(0, 2), cap=1) == 1           # cap < topk
    assert route(lib, shape(), S(9, 1)) == 1                  # unknown mode
    assert route(lib, shape(), S(1, 0)) == 1                  # LVSA without frame ranges
    sp = S(1, 0, P, P, -1)
    assert route(lib, shape(), sp) == 1                       # negative window
    sp = S(1, 0, P, P, 2, 3)
    assert route(lib, shape(), sp) == 1                       # anchors > nb
    sp = S(2, 0, None, None, 0, 0, 0, 0, 2, 1, 1.0)
    assert route(lib, shape(), sp) == 1                       # triage without klam
    assert route(lib, shape(), sp, klam=P, kcount=P, cap=1, cap2=0, cnt2=P) == 1   # cap2 too small
    sp = S(2, 0, None, None, 0, 0, 0, 0, 2, 3, 1.0)
    assert route(lib, shape(), sp, klam=P, kcount=P, cnt2=P, idx2=P, cap2=2) == 1  # n_refine > n_keep
    sp = S(3, 1, None, None, 0, 0, 0, 0, 0, 0, 1.0)
    assert route(lib, shape(), sp) == 1                       # covariance top-k without ln M_j
    assert b"kterm" in lib.sparse_attn_last_error()
    assert route(lib, shape(), S(3, 0, None, None, 0, 0, 0, 0, 0, 0, 1.0), klam=P) == 1   # topk 0
    assert route(lib, shape(), S(3, 2, None, None, 0, 0, 0, 0, 0, 0, 1.0), klam=P, cap=1) == 1  # cap < topk
    assert route(lib, shape(), S(3, 1, None, None, 0, 0, 0, 0, 0, 0, float("inf")), klam=P) == 1
    sp = S(4, 1, None, None, 0, 0, 0, 0, 0, 0, 1.0, None, P)
    assert route(lib, shape(), sp, kcount=P) == 1              # error-aware routing without keys
    assert b"keys" in lib.sparse_attn_last_error()
    sp = S(4, 1, None, None, 0, 0, 0, 0, 0, 0, 1.0, P, None)
    assert route(lib, shape(), sp, kcount=P) == 1              # ... without its workspace
    sp = S(4, 1, None, None, 0, 0, 0, 0, 0, 0, 1.0, P, P)
    assert route(lib, shape(), sp) == 1                        # ... without kcount
    assert route(lib, shape(d=64), sp, kcount=P) == 2          # d == 128 only
    sp = S(4, 3, None, None, 0, 0, 0, 0, 0, 0, 1.0, P, P)
    assert route(lib, shape(), sp, kcount=P) == 1              # topk > nb
    big = shape(N=64 * 5000, N_pad=64 * 5000, H=1)
    assert route(lib, big, S(0, 4)) == 2                      # beyond the block limit


def fwd(lib, sh, dtype=1, comp=0, scale=1.0, **kw):
    a = dict(q=P, k=P, v=P, kbar=P, vbar=P, cent=P, v16=P, kcount=P, kmom=None, kmom_exp=None, hbar=None, q8=None,
             k8=None, v8=None, exp8=None, skim_fmt=0, q4=None, k4=None, v4=None, qs4=None, ks4=None, vs4=None,
             idx=P, cnt=P, cap=2, idx2=None, cnt2=None, cap2=0, out=P, lse=None)
    a.update(kw)
    return lib.sparse_attn_fwd(sh, dtype, comp, scale, a["q"], a["k"], a["v"], a["kbar"], a["vbar"],
                               a["cent"], a["v16"], a["kcount"], a["kmom"], a["kmom_exp"], a["hbar"], a["q8"],
                               a["k8"], a["v8"], a["exp8"],
                               a["skim_fmt"], a["q4"], a["k4"], a["v4"], a["qs4"], a["ks4"], a["vs4"],
                               a["idx"],
                               a["cnt"], a["cap"], a["idx2"], a["cnt2"], a["cap2"], a["out"], a["lse"], None)


def test_fwd_rejects_bad_arguments(lib):
    assert fwd(lib, shape(), comp=1) == 1                     # order 1 without kmom
    assert fwd(lib, shape(), comp=1, kmom=P) == 1             # ... or without its exponents
    assert b"kmom_exp" in lib.sparse_attn_last_error()
    assert fwd(lib, shape(), v16=None) == 1                   # the bf16 path reads the fp16 copy of V
    assert b"v16" in lib.sparse_attn_last_error()
    assert fwd(lib, shape(), comp=2) == 1                     # global order 1 without hbar
    assert fwd(lib, shape(), comp=3) == 1
    assert fwd(lib, shape(d=64), dtype=0, comp=2, hbar=P) == 2   # fp32 path has no first-order term
    assert fwd(lib, shape(), scale=float("inf")) == 1
    assert fwd(lib, shape(), out=None) == 1
    assert fwd(lib, shape(), cent=None) == 1                  # bf16 order 0 needs the centroid planes
    assert fwd(lib, shape(d=64), dtype=0, kbar=None) == 1     # fp32 order 0 needs the means
    assert fwd(lib, shape(), scale=0.0) == 1                  # scale must be > 0
    assert fwd(lib, shape(), scale=-1.0) == 1
    assert fwd(lib, shape(), cap=-1) == 1
    assert fwd(lib, shape(), comp=-1, cap=0, idx=None, cnt=None) == 1   # nothing to attend to
    assert fwd(lib, shape(d=64)) == 2                         # bf16 needs d = 128
    assert fwd(lib, shape(), dtype=0) == 2                    # fp32 needs d = 64
    assert fwd(lib, shape(d=64), dtype=0, comp=1, kmom=P, kmom_exp=P) == 2
    assert fwd(lib, shape(), skim_fmt=2) == 1                 # unknown skim format
    sk = dict(idx2=P, cnt2=P, cap2=2)
    assert fwd(lib, shape(), **sk) == 1                       # e4m3 skim without its copies
    assert fwd(lib, shape(), skim_fmt=1, q8=P, k8=P, v8=P, exp8=P, **sk) == 1   # MXFP4 skim needs q4 ...
    assert b"q4" in lib.sparse_attn_last_error()
    assert fwd(lib, shape(B=0)) == 0


def test_residual_rejects_bad_arguments(lib):
    from free_block_sparse_attn_amd import _lib
    sh = shape()
    need = lib.sparse_attn_residual_workspace(sh)
    assert need > 0
    def res(dtype=1, scale=1.0, phase=0, ridge=1e-3, rank=8, ws=P, nbytes=None, **kw):
        a = dict(q=P, k=P, v=P, out=P)
        a.update(kw)
        return lib.sparse_attn_residual(sh, dtype, scale, a["q"], a["k"], a["v"], a["out"], phase, ridge, rank,
                                        ws, need if nbytes is None else nbytes, None)
    assert res(dtype=0) == 2                                  # bf16 only
    assert res(rank=0) == 1 and res(rank=9) == 1
    assert res(ridge=-1.0) == 1 and res(ridge=float("nan")) == 1
    assert res(phase=-1) == 1
    assert res(scale=0.0) == 1
    assert res(nbytes=need - 1) == 1                          # workspace too small
    assert b"workspace" in lib.sparse_attn_last_error()
    assert res(out=None) == 1
    assert lib.sparse_attn_residual(shape(d=64), 1, 1.0, P, P, P, P, 0, 1e-3, 8, P, 1 << 30, None) == 2


def test_status_strings(lib):
    assert lib.sparse_attn_status_string(0) == b"ok"
    assert lib.sparse_attn_status_string(1) == b"invalid argument"
    assert lib.sparse_attn_status_string(2) == b"unsupported"
    assert lib.sparse_attn_status_string(3) == b"HIP error"


def test_lvsa_capacity_bounds_every_row():
    import numpy as np
    from free_block_sparse_attn_amd import sparse_attn_lvsa_capacity
    from oracle import routing
    from workloads import get_workload, tile_major_coords, block_frame_ranges
    wl = get_workload(4, small=True)
    lo, hi = block_frame_ranges(tile_major_coords(wl.T, wl.Y, wl.X))
    cap = sparse_attn_lvsa_capacity(lo, hi, wl.window, wl.anchors)
    for phase in range(wl.anchor_period):
        _, cnt = routing.route_lvsa(lo, hi, wl.window, wl.anchors, phase, 0)
        assert cnt.max() <= cap


@pytest.mark.parametrize("B,H,N_pad", [(1, 2, 128), (2, 3, 64 * 70), (1, 12, 32768)])
def test_residual_workspace_matches_the_documented_layout(lib, B, H, N_pad):
    """sparse_attn_residual_workspace() is the sum of the blocks the header
    lists (Mp = 64 ceil(nb / 64), K = min(8, nb) key chunks, d = 128)."""
    d, bh, nb = 128, B * H, N_pad // 64
    mp = 64 * ((nb + 63) // 64)
    kc = min(8, nb)
    f64 = bh * 8 * (3 * d * d + 2 * d) + bh * 3 * d * d          # Gram partial sums; X^T X, X^T R, R^T R
    f32 = (2 * bh * mp * d                                         # X and the dense output at the probes
           + bh * (d * d + d)                                      # W, c
           + kc * bh * mp * d + kc * bh * mp                       # per-chunk dense output and lse
           + bh * 2 * d * 8)                                       # Z and V_r
    b16 = bh * mp * d + bh * N_pad * d                             # gathered probe queries; fp16 copy of V
    assert lib.sparse_attn_residual_workspace(shape(B=B, H=H, N=N_pad, N_pad=N_pad)) == 8 * f64 + 4 * f32 + 2 * b16
