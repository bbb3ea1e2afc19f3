"""Seeded random shapes through every stage against the oracle (GPU required).

Each case draws a shape the fixed-shape tests do not pin down: batch 1-5,
1-3 KV heads, group 1/2/4/8, head_dim 64/128, bf16 or fp32 K/V, a t_cap that
is rarely a multiple of the 512-key score block, C anywhere in [1, t_cap],
window 4-32, ragged lengths that include 0 and t_cap, sometimes the newest-token
window.  Per case:
  * ring push and predictor against the oracle (push bit-exact, prediction
    within 1e-4 of max|q| per head);
  * scores within the bound their arithmetic guarantees: per key, 2^-15 of
    the largest sum over the group's heads of |q_d k_d| (q carried as two bf16
    terms, fp32 accumulation); the fixed-shape tests use the tighter
    1e-5 * max|score| per unit, which a unit with one or a few keys whose
    score cancels need not meet;
  * the top-C selection bit-exact against the oracle on the GPU's own fp32
    scores, and the candidate route (with a random threshold hint) equal to it
    bit for bit;
  * the attention over that selection within 1e-2 (observed ~1e-6).
"""
import os

import numpy as np
import pytest
import torch

import oracle
import query_aware_sparse_amd as A
from query_aware_sparse_amd import workload as wk
from asp_testutil import assert_pred_close, dims_for, kv_np, np_, require_gpu

pytestmark = pytest.mark.gpu
DEV = "cuda"
N_CASES = int(os.environ.get("ASP_RANDOM_SHAPES", "64"))  # more cases: set the variable


def draw(seed: int) -> dict:
    r = np.random.default_rng(1000 + seed)
    B = int(r.integers(1, 6))
    Hkv = int(r.integers(1, 4))
    G = int(r.choice([1, 2, 4, 8]))
    D = int(r.choice([64, 128]))
    kv = str(r.choice(["bf16", "f32"]))
    T_cap = int(r.choice([r.integers(1, 600), r.integers(600, 6000), 512 * int(r.integers(1, 9))]))
    C = int(r.choice([1, r.integers(1, T_cap + 1), T_cap, min(T_cap, 2048)]))
    W = int(r.choice([4, 8, 12, 16, 32]))
    lens = r.integers(0, T_cap + 1, size=B)
    if B > 1:
        lens[0] = T_cap
        lens[-1] = int(r.choice([0, 1, T_cap, lens[-1]]))
    recent = int(r.choice([0, 0, r.integers(1, T_cap + 1)]))
    pushes = int(r.integers(1, W + 4))  # the ring may or may not be full
    return dict(B=B, Hkv=Hkv, G=G, D=D, kv=kv, T_cap=T_cap, C=C, W=W, lens=lens.astype(np.int32), recent=recent,
                pushes=pushes, seed=seed)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_shape_end_to_end(seed):
    require_gpu()
    p = draw(seed)
    B, Hkv, G, D, kv, T_cap, C, W = (p[x] for x in ("B", "Hkv", "G", "D", "kv", "T_cap", "C", "W"))
    Hq = G * Hkv
    lens_np = p["lens"]
    dims = dims_for(A, B, Hq, Hkv, D, T_cap, kv)
    cfg = A.Cfg(W, C, 1e-2, p["recent"])
    kdt = torch.bfloat16 if kv == "bf16" else torch.float32
    k = (wk.randn((B, Hkv, T_cap, D), seed=seed, sub=1) * 2).to(kdt)
    v = wk.randn((B, Hkv, T_cap, D), seed=seed, sub=2).to(kdt)
    lens = torch.from_numpy(lens_np).to(DEV)
    kd, vd = k.to(DEV), v.to(DEV)

    # ring push and predictor
    q_hist = torch.zeros((B, Hq, W, D), device=DEV)
    newest = torch.full((B,), W - 1, dtype=torch.int32, device=DEV)
    length = torch.zeros((B,), dtype=torch.int32, device=DEV)
    h_np, n_np, l_np = np_(q_hist).astype(np.float32), np_(newest), np_(length)
    for t in range(p["pushes"]):
        q_t = (wk.randn((B, Hq, D), seed=seed, sub=10 + t) * 0.5).float()
        A.asp_push_query(dims, cfg, q_t.to(DEV), q_hist, newest, length)
        h_np, n_np, l_np = oracle.push(q_t.numpy(), h_np, n_np, l_np)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(np_(q_hist), h_np)
    np.testing.assert_array_equal(np_(newest), n_np)
    np.testing.assert_array_equal(np_(length), l_np)
    q_pred = torch.empty((B, Hq, D), device=DEV)
    A.asp_predict_query(dims, cfg, q_hist, newest, length, q_pred)
    assert_pred_close(np_(q_pred), oracle.predict(h_np, n_np, l_np, 1e-2))

    # scores, exact selection on them, and the candidate route
    scores = torch.empty((B, Hkv, T_cap), device=DEV)
    A.asp_score_keys(dims, q_pred, kd, lens, scores)
    got = np_(scores).astype(np.float64)
    ref = oracle.score(np_(q_pred), kv_np(k), lens_np)
    qa = np.abs(np_(q_pred).astype(np.float64))
    ka = np.abs(k.float().numpy().astype(np.float64))
    for b in range(B):
        T = int(lens_np[b])
        for g in range(Hkv):
            # the arithmetic's bound per key: q is carried as two bf16 terms
            # (residual <= 2^-18 |q|) and 2D exact products accumulate in
            # fp32 (<= 2D 2^-24 of their magnitude), together <= 2^-15 of
            # max over the group's heads of sum_d |q_d k_d|
            mag = (ka[b, g, :T] @ qa[b, g * G:(g + 1) * G].T).max(axis=1) if T else np.zeros(0)
            err = np.abs(got[b, g, :T] - ref[b, g, :T])
            assert (err <= 2.0 ** -15 * mag + 1e-30).all(), (b, g, err.max(), mag[err.argmax()] if T else 0)
    idx = torch.full((B, Hkv, C), -9, dtype=torch.int32, device=DEV)
    n_sel = torch.full((B, Hkv), -9, dtype=torch.int32, device=DEV)
    A.asp_select_topc(dims, cfg, scores, lens, idx, n_sel)
    ri, rn = oracle.select(np_(scores), lens_np, C)
    np.testing.assert_array_equal(np_(n_sel), rn)
    np.testing.assert_array_equal(np_(idx), ri)

    ws = torch.empty(A.asp_workspace_size(dims, cfg, A.OP_CANDIDATES), dtype=torch.uint8, device=DEV)
    ws.zero_()
    r = np.random.default_rng(seed)
    hints = torch.from_numpy(r.integers(0, 2**32, size=B * Hkv, dtype=np.uint64).astype(np.uint32).view(np.int32))
    ws[: 4 * B * Hkv].copy_(hints.view(torch.uint8))  # the threshold hints lead the workspace
    idx2 = torch.full_like(idx, -9)
    n2 = torch.full_like(n_sel, -9)
    A.asp_score_candidates(dims, cfg, q_pred, kd, lens, ws)
    A.asp_select_candidates(dims, cfg, q_pred, kd, lens, idx2, n2, ws)
    np.testing.assert_array_equal(np_(n2), rn)
    np.testing.assert_array_equal(np_(idx2), ri)

    # attention over that selection (and the newest tokens when asked)
    q = wk.randn((B, Hq, D), seed=seed, sub=3)
    out = torch.full((B, Hq, D), 99.0, device=DEV)
    wsd = torch.empty(A.asp_workspace_size(dims, cfg, A.OP_DECODE), dtype=torch.uint8, device=DEV)
    A.asp_sparse_decode(dims, cfg, q.to(DEV), kd, vd, lens, idx, n_sel, out, wsd)
    if p["recent"]:
        ref_o = oracle.attend_with_recent(q.numpy(), kv_np(k), kv_np(v), ri, rn, lens_np, p["recent"])
    else:
        ref_o = oracle.attend(q.numpy(), kv_np(k), kv_np(v), ri, rn)
    err = np.abs(np_(out).astype(np.float64) - ref_o).max()
    assert err <= 1e-2, (p, err)
