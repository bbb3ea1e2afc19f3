"""The largest shapes the header admits, through every stage (GPU required).

* The longest token stride, t_cap = 2^22 (4,194,304 keys), one unit of four
  query heads at head_dim 64 with bf16 K/V and the sequence full:
  - scores within the bound their arithmetic guarantees (q carried as two bf16
    terms, fp32 accumulation: 2^-15 of the largest sum over the group's heads of
    |q_d k_d|) against the oracle's fp64 scores of every key;
  - the score-row route and the candidate route bit-exact against the oracle's
    selection on the GPU's own scores, at C = 65536 (the largest list the
    head_dim-64 bf16 attention takes) and at C = 1.  The candidate route runs
    first with every key kept (all 4M keys: far more than a select workgroup
    stages, so the unit is rescored and selected from memory), then with the
    threshold hint that call left;
  - the attention over the C = 65536 selection within 1e-2 (observed ~1e-6):
    256 splits of one unit and their merge, the most the merge takes;
  - asp_step (bootstrap and two pipelined steps, one stream and two streams)
    bit-identical to the same schedule built from the entry points.
* The attention at its largest token list for each row width, with one unit
  (every split on one unit) and with four (the newest-token window on):
  bf16 head_dim 128 and fp32 head_dim 64 (C + R = 32768), fp32 head_dim 128
  (16384).
"""
import numpy as np
import pytest
import torch

import oracle
import query_aware_sparse_amd as A
from query_aware_sparse_amd import workload as wk
from asp_testutil import dims_for, kv_np, np_, require_gpu
from test_gpu_step import Problem, _manual_run, _step_run

pytestmark = pytest.mark.gpu
DEV = "cuda"
T_MAX = 1 << 22
C_MAX_D64_BF16 = 65536


@pytest.fixture(scope="module")
def longest():
    """One unit (B=1, 4 query heads / 1 KV head, head_dim 64, bf16) with a
    full sequence of 2^22 keys, and its predicted-query stand-in."""
    require_gpu()
    B, Hq, Hkv, D = 1, 4, 1, 64
    g = torch.Generator(device=DEV).manual_seed(2024)
    k = (torch.randn((B, Hkv, T_MAX, D), generator=g, device=DEV) * 2).to(torch.bfloat16)
    v = torch.randn((B, Hkv, T_MAX, D), generator=g, device=DEV).to(torch.bfloat16)
    q = torch.randn((B, Hq, D), generator=g, device=DEV) * 0.5
    lens = torch.tensor([T_MAX], dtype=torch.int32, device=DEV)
    torch.cuda.synchronize()
    print("t_cap %d: K and V %.0f MiB each" % (T_MAX, k.numel() * 2 / 2**20), flush=True)
    return dict(B=B, Hq=Hq, Hkv=Hkv, D=D, k=k, v=v, q=q, lens=lens, k_np=kv_np(k))


def _scores(s):
    dims = dims_for(A, s["B"], s["Hq"], s["Hkv"], s["D"], T_MAX, "bf16")
    scores = torch.empty((s["B"], s["Hkv"], T_MAX), device=DEV)
    A.asp_score_keys(dims, s["q"], s["k"], s["lens"], scores)
    torch.cuda.synchronize()
    return dims, scores


def test_longest_stride_scores_within_their_arithmetic_bound(longest):
    s = longest
    _, scores = _scores(s)
    got = np_(scores).astype(np.float64)[0, 0]
    q = np_(s["q"])
    ref = oracle.score(q, s["k_np"], np.array([T_MAX], np.int32))[0, 0]
    ka = np.abs(s["k"][0, 0].float().cpu().numpy().astype(np.float64))
    mag = (ka @ np.abs(q[0].astype(np.float64)).T).max(axis=1)
    err = np.abs(got - ref)
    assert (err <= 2.0 ** -15 * mag + 1e-30).all(), (err.max(), mag[err.argmax()])


@pytest.mark.parametrize("C", [C_MAX_D64_BF16, 1])
def test_longest_stride_selection_both_routes_bit_exact(longest, C):
    s = longest
    dims, scores = _scores(s)
    cfg = A.Cfg(16, C, 1e-2)
    ri, rn = oracle.select(np_(scores), np.array([T_MAX], np.int32), C)
    idx = torch.full((1, 1, C), -9, dtype=torch.int32, device=DEV)
    n_sel = torch.full((1, 1), -9, dtype=torch.int32, device=DEV)
    A.asp_select_topc(dims, cfg, scores, s["lens"], idx, n_sel)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(np_(n_sel), rn)
    np.testing.assert_array_equal(np_(idx), ri)

    ws = torch.zeros(A.asp_workspace_size(dims, cfg, A.OP_CANDIDATES), dtype=torch.uint8, device=DEV)  # hint 0
    for call in ("every key kept", "the hint the first call left"):
        idx2 = torch.full_like(idx, -9)
        n2 = torch.full_like(n_sel, -9)
        A.asp_score_candidates(dims, cfg, s["q"], s["k"], s["lens"], ws)
        A.asp_select_candidates(dims, cfg, s["q"], s["k"], s["lens"], idx2, n2, ws)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(np_(n2), rn, err_msg=call)
        np.testing.assert_array_equal(np_(idx2), ri, err_msg=call)


def test_longest_stride_attention_over_the_largest_selection(longest):
    s = longest
    dims, scores = _scores(s)
    C = C_MAX_D64_BF16
    cfg = A.Cfg(16, C, 1e-2)
    assert A.asp_workspace_size(dims, A.Cfg(16, C + 1, 1e-2), A.OP_DECODE) == 0  # the longest list taken
    idx = torch.empty((1, 1, C), dtype=torch.int32, device=DEV)
    n_sel = torch.empty((1, 1), dtype=torch.int32, device=DEV)
    A.asp_select_topc(dims, cfg, scores, s["lens"], idx, n_sel)
    q_t = torch.randn((1, s["Hq"], s["D"]), generator=torch.Generator(device=DEV).manual_seed(7), device=DEV)
    out = torch.full((1, s["Hq"], s["D"]), 99.0, device=DEV)
    ws = torch.empty(A.asp_workspace_size(dims, cfg, A.OP_DECODE), dtype=torch.uint8, device=DEV)
    A.asp_sparse_decode(dims, cfg, q_t, s["k"], s["v"], s["lens"], idx, n_sel, out, ws)
    torch.cuda.synchronize()
    assert int(np_(n_sel)[0, 0]) == C
    ref = oracle.attend(np_(q_t), s["k_np"], kv_np(s["v"]), np_(idx), np_(n_sel))
    err = np.abs(np_(out).astype(np.float64) - ref).max()
    assert err <= 1e-2, err
    print("attention over %d tokens: max err %.2e" % (C, err), flush=True)


def test_longest_stride_step_modes_bit_identical(longest):
    s = longest
    wl = wk.TINY.replace(name="longest-stride", batch=1, n_q_heads=s["Hq"], n_kv_heads=1, head_dim=s["D"],
                         t_cap=T_MAX, kv_dtype="bf16", window=16, top_c=C_MAX_D64_BF16, history_steps=18,
                         heavy_count=8, recent=0, seed=91)
    n = 3
    runs = {}
    for mode in ("manual", "one_stream", "two_streams"):
        p = Problem(wl, n_steps=n, kv=(s["k"], s["v"]), lens=[T_MAX])
        p.fill_history()
        torch.cuda.synchronize()
        runs[mode] = _manual_run(p, n) if mode == "manual" else _step_run(p, mode, n)
        del p
    for mode in ("one_stream", "two_streams"):
        for st in range(n):
            for a, b in zip(runs["manual"][st], runs[mode][st]):
                np.testing.assert_array_equal(a, b, err_msg="%s step %d" % (mode, st))


def _largest_list_case(kv, D, C, R, B, Hkv, T_cap, lens, seed):
    G = 4
    Hq = G * Hkv
    # the list is the longest the library takes: one more token is refused
    d = dims_for(A, B, Hq, Hkv, D, T_cap, kv)
    assert A.asp_workspace_size(d, A.Cfg(8, C, 1e-2, R), A.OP_DECODE) > 0
    assert A.asp_workspace_size(d, A.Cfg(8, C + 1, 1e-2, R), A.OP_DECODE) == 0
    g = torch.Generator(device="cpu").manual_seed(seed)
    kdt = torch.bfloat16 if kv == "bf16" else torch.float32
    k = (torch.randn((B, Hkv, T_cap, D), generator=g) * 2).to(kdt)
    v = torch.randn((B, Hkv, T_cap, D), generator=g).to(kdt)
    q = torch.randn((B, Hq, D), generator=g)
    r = np.random.default_rng(seed)
    idx = np.full((B, Hkv, C), -1, np.int32)
    n_sel = np.zeros((B, Hkv), np.int32)
    for b in range(B):
        for h in range(Hkv):
            n = C if (b + h) % 2 == 0 else C - 1 - 37 * (b + h)  # full lists and lists ending inside a split
            n = min(n, lens[b])
            idx[b, h, :n] = np.sort(r.choice(lens[b], n, replace=False))
            n_sel[b, h] = n
    dims = dims_for(A, B, Hq, Hkv, D, T_cap, kv)
    cfg = A.Cfg(8, C, 1e-2, R)
    ws = torch.empty(A.asp_workspace_size(dims, cfg, A.OP_DECODE), dtype=torch.uint8, device=DEV)
    out = torch.full((B, Hq, D), 99.0, device=DEV)
    glens = torch.tensor(lens, dtype=torch.int32, device=DEV)
    A.asp_sparse_decode(dims, cfg, q.to(DEV), k.to(DEV), v.to(DEV), glens, torch.from_numpy(idx).to(DEV),
                        torch.from_numpy(n_sel).to(DEV), out, ws)
    torch.cuda.synchronize()
    if R:
        ref = oracle.attend_with_recent(q.numpy(), kv_np(k), kv_np(v), idx, n_sel, np.array(lens, np.int32), R)
    else:
        ref = oracle.attend(q.numpy(), kv_np(k), kv_np(v), idx, n_sel)
    err = np.abs(np_(out).astype(np.float64) - ref).max()
    assert err <= 1e-2, err
    assert err < 1e-4, err
    return err


@pytest.mark.parametrize("kv,D,C", [("bf16", 128, 32768), ("f32", 64, 32768), ("f32", 128, 16384)])
def test_attention_at_its_largest_list_one_unit(kv, D, C):
    require_gpu()
    _largest_list_case(kv, D, C, 0, 1, 1, C + 5000, [C + 5000], seed=C + D)


@pytest.mark.parametrize("kv,D,C", [("bf16", 128, 32768), ("f32", 64, 32768), ("f32", 128, 16384)])
def test_attention_at_its_largest_list_with_the_newest_tokens(kv, D, C):
    require_gpu()
    R = 768
    T_cap = C + 4000
    # the last sequence is shorter than the list: its newest tokens and a short selection
    _largest_list_case(kv, D, C - R, R, 2, 2, T_cap, [T_cap, C // 2], seed=C + D + 1)
