"""asp_sparse_decode_static, the attention entry point that allocates nothing
(GPU required): through the C ABI it must give, bit for bit, what
asp_sparse_decode gives with a workspace, on two calls in a row (the second on
a smaller problem, over the scratch the first call left behind), and match the
oracle within 1e-2; a shape whose partials exceed the built-in scratch is
refused before anything is enqueued."""
import numpy as np
import pytest
import torch

import oracle
import query_aware_sparse_amd as A
from query_aware_sparse_amd import workload as wk
from asp_testutil import dims_for, kv_np, np_, require_gpu

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(B, Hkv, G, D, T_cap, C, kv, n_sels, seed, recent=0, lens=None):
    Hq = Hkv * G
    q = wk.randn((B, Hq, D), seed=seed)
    k = (wk.randn((B, Hkv, T_cap, D), seed=seed, sub=1) * 2).to(torch.bfloat16 if kv == "bf16" else torch.float32)
    v = wk.randn((B, Hkv, T_cap, D), seed=seed, sub=2).to(k.dtype)
    r = np.random.default_rng(seed)
    idx = np.full((B, Hkv, C), -1, np.int32)
    n_sel = np.zeros((B, Hkv), np.int32)
    for b in range(B):
        for g in range(Hkv):
            n = n_sels[(b * Hkv + g) % len(n_sels)]
            idx[b, g, :n] = np.sort(r.choice(T_cap, n, replace=False))
            n_sel[b, g] = n
    dims = dims_for(A, B, Hq, Hkv, D, T_cap, kv)
    cfg = A.Cfg(8, C, 1e-2, recent)
    g = dict(q=q.to(DEV), k=k.to(DEV), v=v.to(DEV), idx=torch.from_numpy(idx).to(DEV),
             n_sel=torch.from_numpy(n_sel).to(DEV),
             lens=None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV))
    return dims, cfg, (q, k, v, idx, n_sel), g


def _run_pair(dims, cfg, g):
    ws = torch.empty(A.asp_workspace_size(dims, cfg, A.OP_DECODE), dtype=torch.uint8, device=DEV)
    B, Hq, D = dims.batch, dims.n_q_heads, dims.head_dim
    ref = torch.full((B, Hq, D), 7.0, dtype=torch.float32, device=DEV)
    got = torch.full((B, Hq, D), -7.0, dtype=torch.float32, device=DEV)
    A.asp_sparse_decode(dims, cfg, g["q"], g["k"], g["v"], g["lens"], g["idx"], g["n_sel"], ref, ws)
    A.asp_sparse_decode_static(dims, cfg, g["q"], g["k"], g["v"], g["lens"], g["idx"], g["n_sel"], got)
    torch.cuda.synchronize()
    return np_(ref), np_(got)


def test_static_scratch_matches_the_workspace_entry_point_twice():
    require_gpu()
    # 1: bf16, 64 units, four splits per unit (partials in the scratch);
    # 2: smaller, fp32 K/V (the VALU path, more splits), the newest tokens on
    cases = [
        dict(B=8, Hkv=8, G=4, D=128, T_cap=4096, C=2048, kv="bf16", n_sels=[2048, 1500, 513, 0], seed=11),
        dict(B=2, Hkv=2, G=2, D=64, T_cap=1000, C=300, kv="f32", n_sels=[300, 17, 1], seed=12, recent=50,
             lens=[1000, 40]),
    ]
    for i, c in enumerate(cases):
        dims, cfg, host, g = _case(**c)
        assert A.asp_workspace_size(dims, cfg, A.OP_DECODE) <= A.STATIC_SCRATCH_BYTES
        ref, got = _run_pair(dims, cfg, g)
        np.testing.assert_array_equal(got, ref, err_msg="call %d" % i)
        q, k, v, idx, n_sel = host
        if c.get("recent"):
            orc = oracle.attend_with_recent(q.numpy(), kv_np(k), kv_np(v), idx, n_sel,
                                            np.array(c["lens"], np.int32), c["recent"])
        else:
            orc = oracle.attend(q.numpy(), kv_np(k), kv_np(v), idx, n_sel)
        err = np.abs(got.astype(np.float64) - orc).max()
        assert err <= 1e-2, (i, err)


def test_static_scratch_refuses_shapes_beyond_it():
    require_gpu()
    # 65528 units of 8 heads at head_dim 128: partials of ~272 MB
    dims = A.Dims(8191, 64, 8, 128, 4096, A.KV_BF16)
    cfg = A.Cfg(8, 2048, 1e-2, 0)
    assert A.asp_workspace_size(dims, cfg, A.OP_DECODE) > A.STATIC_SCRATCH_BYTES
    fake = torch.empty(16, dtype=torch.float32, device=DEV)
    lib = A.load()
    import ctypes
    p = ctypes.c_void_p(fake.data_ptr())
    st = lib.asp_sparse_decode_static(ctypes.byref(dims), ctypes.byref(cfg), p, p, p, None, p, p, p, None)
    assert st == 6, st  # ASP_ERR_SCRATCH, nothing enqueued
