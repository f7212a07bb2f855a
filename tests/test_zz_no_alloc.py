"""The allocation-free pooling entry point, sparse_attn_pool_static, against
sparse_attn_pool with its caller-owned hbar_ws scratch: the same results bit
for bit, on two calls in a row (the second on a smaller problem, so it reads
only partial sums it wrote itself), and the size limit refused on the host."""

import ctypes

import numpy as np
import pytest
import torch

import gpu_cases as gc


def _compare(wl, **kw):
    import free_block_sparse_attn_amd as fbsa
    (q, k, v), dev, _ = gc.inputs(wl)
    print(f"\n[case] pool_static {wl.name} B={wl.B} H={wl.H} N={wl.N} nb={wl.nb} {kw}", flush=True)
    ref = fbsa.sparse_attn_pool(*dev, wl.N, **kw)
    got = fbsa.sparse_attn_pool_static(*dev, wl.N, **kw)
    torch.cuda.synchronize()
    assert "hbar_ws" in ref and "hbar_ws" not in got
    for n, t in got.items():
        assert torch.equal(t, ref[n]), n
    return got


@pytest.mark.gpu
def test_static_pool_matches_the_workspace_pool():
    from dataclasses import replace
    from workloads import configs as C
    big = replace(C.GLOBAL_COV_SMALL, T=9, Y=20, X=45, B=2, H=3)       # 8100 tokens, 127 blocks, 6 heads
    small = replace(C.GLOBAL_ORDER1_SMALL, B=1, H=1)                    # 1080 tokens, 17 blocks, 1 head
    g1 = _compare(big, global_moment=True, cov=True)
    g2 = _compare(small, global_moment=True)
    # the second call's H_bar is its own (not the first call's partial sums)
    assert g1["hbar"].shape != g2["hbar"].shape
    (q, k, v), _, _ = gc.inputs(small)
    from oracle import pooling
    ref = np.swapaxes(pooling.global_moment(k, v, small.N), -1, -2)
    err = np.abs(g2["hbar"].cpu().numpy().astype(np.float64) - ref)
    assert err.max() <= 1e-4 * np.abs(ref).max(), err.max()


@pytest.mark.gpu
def test_static_pool_refuses_more_heads_than_its_scratch_holds():
    from free_block_sparse_attn_amd import _lib
    lib = _lib.load()
    n = 64
    t = torch.zeros(1, 33, n, 128, dtype=torch.bfloat16, device="cuda")
    fq, fk, fv = (torch.zeros(1, 33, 1, 128, dtype=torch.float32, device="cuda") for _ in range(3))
    hb = torch.zeros(1, 33, 128, 128, dtype=torch.float32, device="cuda")
    kc = torch.zeros(1, dtype=torch.int32, device="cuda")
    p = lambda x: ctypes.c_void_p(x.data_ptr())
    sh = ctypes.byref(_lib.Shape(1, 33, n, n, 128))
    st = lib.sparse_attn_pool_static(sh, 1, p(t), p(t), p(t), p(fq), p(fk), p(fv), p(kc), None, None, None, None,
                                     p(hb), None, None, None, None, None, None, None, None, None, None, None, None,
                                     None)
    assert st == 2, st
    assert b"B*H <= 32" in lib.sparse_attn_last_error()
    # without H_bar there is no scratch and no limit: 33 heads pool normally
    st = lib.sparse_attn_pool_static(sh, 1, p(t), p(t), p(t), p(fq), p(fk), p(fv), p(kc), None, None, None, None,
                                     None, None, None, None, None, None, None, None, None, None, None, None, None,
                                     None)
    torch.cuda.synchronize()
    assert st == 0, lib.sparse_attn_last_error()
