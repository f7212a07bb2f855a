"""ctypes binding of libsparse_attn.so (the C ABI in include/sparse_attn.h).

Argument marshalling only: every step of the hot path runs in the HIP
kernels behind the C ABI.  PyTorch provides device memory and the stream.
There is no fallback: a missing library raises.
"""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# SPARSE_ATTN_LIB may name another build of the same library (same ABI).
LIB_PATH = os.environ.get("SPARSE_ATTN_LIB", os.path.join(HERE, "libsparse_attn.so"))

SA_OK, SA_ERR_INVALID_ARG, SA_ERR_UNSUPPORTED, SA_ERR_HIP = 0, 1, 2, 3
SA_F32, SA_BF16 = 0, 1
SA_COMP_DROP, SA_COMP_ORDER0, SA_COMP_ORDER1_BLOCK, SA_COMP_ORDER1_GLOBAL = -1, 0, 1, 2
SA_ROUTE_TOPK, SA_ROUTE_LVSA, SA_ROUTE_TRIAGE, SA_ROUTE_TOPK_COV, SA_ROUTE_ERROR = 0, 1, 2, 3, 4
SA_SKIM_E4M3, SA_SKIM_MXFP4 = 0, 1

EXPORTED = (
    "sparse_attn_pool", "sparse_attn_route", "sparse_attn_fwd", "sparse_attn_lvsa_capacity",
    "sparse_attn_status_string", "sparse_attn_last_error", "sparse_attn_abi_version",
    "sparse_attn_residual", "sparse_attn_residual_workspace", "sparse_attn_pool_static",
)


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32),
                ("N_pad", ctypes.c_int32), ("d", ctypes.c_int32)]


class RouteSpec(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("frame_lo", ctypes.c_void_p), ("frame_hi", ctypes.c_void_p),
                ("window", ctypes.c_int32), ("anchors", ctypes.c_int32),
                ("anchor_phase", ctypes.c_int32), ("step", ctypes.c_int32),
                ("n_keep", ctypes.c_int32), ("n_refine", ctypes.c_int32),
                ("scale", ctypes.c_float), ("keys", ctypes.c_void_p), ("ekey", ctypes.c_void_p)]


class SparseAttnError(RuntimeError):
    def __init__(self, status, detail):
        super().__init__(f"sparse_attn status {status}: {detail}")
        self.status = status
        self.detail = detail


_lib = None


def load(path: str = LIB_PATH):
    """Load the library once and declare every exported signature."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                           "(python free_block_sparse_attn_amd/build.py)")
    lib = ctypes.CDLL(path)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    # shape, dtype, q, k, v, qbar, kbar, vbar, kcount, cent, v16, kmom, kmom_exp, hbar, hbar_ws, kcov,
    # klam, q8, k8, v8, exp8, q4, k4, v4, qs4, ks4, vs4, stream
    lib.sparse_attn_pool.argtypes = [ctypes.POINTER(Shape), i32] + [vp] * 26
    lib.sparse_attn_pool.restype = i32
    # as sparse_attn_pool without hbar_ws
    lib.sparse_attn_pool_static.argtypes = [ctypes.POINTER(Shape), i32] + [vp] * 25
    lib.sparse_attn_pool_static.restype = i32
    lib.sparse_attn_route.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(RouteSpec), vp, vp, vp, vp,
                                      vp, vp, i32, vp, vp, i32, vp]
    lib.sparse_attn_route.restype = i32
    # shape, dtype, comp, scale, q, k, v, kbar, vbar, cent, v16, kcount, kmom, kmom_exp, hbar, q8, k8,
    # v8, exp8, skim_fmt, q4, k4, v4, qs4, ks4, vs4, idx, cnt, cap, idx2, cnt2, cap2, out, lse, stream
    lib.sparse_attn_fwd.argtypes = [ctypes.POINTER(Shape), i32, i32, f32] + [vp] * 15 + [i32] + [vp] * 6 + \
                                   [vp, vp, i32, vp, vp, i32, vp, vp, vp]
    lib.sparse_attn_fwd.restype = i32
    lib.sparse_attn_lvsa_capacity.argtypes = [vp, vp, i32, i32, i32]
    lib.sparse_attn_lvsa_capacity.restype = i32
    lib.sparse_attn_status_string.argtypes = [i32]
    lib.sparse_attn_status_string.restype = ctypes.c_char_p
    lib.sparse_attn_last_error.argtypes = []
    lib.sparse_attn_last_error.restype = ctypes.c_char_p
    lib.sparse_attn_residual_workspace.argtypes = [ctypes.POINTER(Shape)]
    lib.sparse_attn_residual_workspace.restype = ctypes.c_size_t
    lib.sparse_attn_residual.argtypes = [ctypes.POINTER(Shape), i32, f32, vp, vp, vp, vp, i32, f32, i32, vp,
                                         ctypes.c_size_t, vp]
    lib.sparse_attn_residual.restype = i32
    lib.sparse_attn_abi_version.argtypes = []
    lib.sparse_attn_abi_version.restype = i32
    _lib = lib
    return lib


def check(status: int):
    if status != SA_OK:
        lib = load()
        raise SparseAttnError(status, f"{lib.sparse_attn_status_string(status).decode()}: "
                                      f"{lib.sparse_attn_last_error().decode()}")
