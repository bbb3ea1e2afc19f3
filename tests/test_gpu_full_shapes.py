"""Full-size parity at the remaining workload shapes (GPU required).

One decoder layer of each workload at its real size: the Qwen3-8B stack layer
(B=32, T=16384), the Qwen3-32B layer (B=16, 64q/8kv: GQA group 8, T=32768) and
the ragged long-CoT batch (B=64, lengths in [8192, 131072], several (W, C)
points).  Every unit is computed on the GPU; the oracle checks the sampled
sequences stage by stage (ring bit-exact, predictor, scores, selection, and
attention), and the bench's launch configuration (asp_step with two streams)
must reproduce the entry points bit for bit on every unit.
"""
import numpy as np
import pytest
import torch

import query_aware_sparse_amd as A
from query_aware_sparse_amd import workload as wk
from asp_testutil import np_, require_gpu
from test_gpu_step import DEV, Problem, _staged_check

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _ring(p):
    return p.q_hist.clone(), p.newest.clone(), p.length.clone()


def _set_ring(p, r):
    p.q_hist.copy_(r[0])
    p.newest.copy_(r[1])
    p.length.copy_(r[2])


def _snap(p, idx, n_sel):
    return [np_(x).copy() for x in (p.out, idx, n_sel, p.q_hist, p.newest, p.length)]


def _full_shape_check(p: Problem, units):
    wl, d, c = p.wl, p.dims, p.cfg
    B, Hkv, C = wl.batch, wl.n_kv_heads, wl.top_c
    t = wl.history_steps
    q0, q1 = p.queries[t], p.queries[t + 1]
    ring0 = _ring(p)
    # Entry points, checked against the oracle on the sampled sequences.
    _staged_check(p, q0, units=units)
    ref0 = _snap(p, p.idx, p.n_sel)
    ring1 = _ring(p)
    idx0, n0 = p.idx.clone(), p.n_sel.clone()
    # The next step through the entry points (reference for the pipelined step).
    A.asp_sparse_decode(d, c, q1.to(DEV), p.k, p.v, p.seq_lens, idx0, n0, p.out, p.ws_dec)
    A.asp_push_query(d, c, q1.to(DEV), p.q_hist, p.newest, p.length)
    A.asp_predict_query(d, c, p.q_hist, p.newest, p.length, p.q_pred)
    A.asp_score_keys(d, p.q_pred, p.k, p.seq_lens, p.scores)
    A.asp_select_topc(d, c, p.scores, p.seq_lens, p.idx, p.n_sel)
    torch.cuda.synchronize()
    ref1 = _snap(p, p.idx, p.n_sel)

    # asp_step: bootstrap, then one pipelined step on two streams.
    _set_ring(p, ring0)
    ws = torch.empty(A.asp_workspace_size(d, c, A.OP_STEP), dtype=torch.uint8, device=DEV)
    idx = [torch.full((B, Hkv, C), -7, dtype=torch.int32, device=DEV) for _ in range(2)]
    nsel = [torch.zeros((B, Hkv), dtype=torch.int32, device=DEV) for _ in range(2)]
    ev = [A.HipEvent(), A.HipEvent()]
    ctx = A.AspContext()
    attn, sel = torch.cuda.Stream(), torch.cuda.Stream()
    attn.wait_stream(torch.cuda.current_stream())
    q0d, q1d = q0.to(DEV), q1.to(DEV)  # held until the streams are done with them
    attn.wait_stream(torch.cuda.current_stream())
    A.asp_step(d, c, q0d, p.q_hist, p.newest, p.length, p.k, p.v, p.seq_lens, None, None, idx[0], nsel[0],
               p.out, ws, attn_stream=attn, idx_next_ready=ev[0])
    torch.cuda.synchronize()
    got0 = _snap(p, idx[0], nsel[0])
    assert np.array_equal(np_(p.q_hist), np_(ring1[0]))
    A.asp_step(d, c, q1d, p.q_hist, p.newest, p.length, p.k, p.v, p.seq_lens, idx[0], nsel[0], idx[1],
               nsel[1], p.out, ws, attn_stream=attn, sel_stream=sel, ctx=ctx, idx_cur_ready=ev[0],
               idx_next_ready=ev[1])
    torch.cuda.synchronize()
    got1 = _snap(p, idx[1], nsel[1])
    names = ("out", "idx", "n_sel", "q_hist", "newest", "len")
    for s, (ref, got) in enumerate(((ref0, got0), (ref1, got1))):
        for name, a, b in zip(names, ref, got):
            np.testing.assert_array_equal(a, b, err_msg="step %d %s" % (s, name))


def test_qwen3_8b_stack_layer_full_size():
    wl = wk.Q8B_STACK
    p = Problem(wl, kv_device=DEV, layer=5, n_steps=3)
    p.fill_history()
    _full_shape_check(p, units=[0, 17, 31])


def test_qwen3_32b_layer_full_size():
    wl = wk.Q32B
    p = Problem(wl, kv_device=DEV, layer=9, n_steps=3)
    p.fill_history()
    _full_shape_check(p, units=[0, 7, 15])


@pytest.fixture(scope="module")
def ragged_kv():
    """K/V of the full ragged long-CoT batch (2 x 16 GiB), shared by the (W, C) points."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wl = wk.RAGGED
    lens = wk.make_seq_lens(wl)
    k, v = wk.make_kv(wl, lens, layer=0, device=DEV)
    yield k, v
    del k, v
    torch.cuda.empty_cache()


@pytest.mark.parametrize("W,C", [(16, 2048), (32, 4096), (8, 512), (16, 1024)])
def test_ragged_long_cot_full_size(ragged_kv, W, C):
    wl = wk.RAGGED.replace(window=W, top_c=C, history_steps=W + 4)
    p = Problem(wl, n_steps=3, kv=ragged_kv)
    p.fill_history()
    lens = np_(p.seq_lens)
    # the shortest, the longest and one mid-length sequence
    order = np.argsort(lens)
    _full_shape_check(p, units=sorted({int(order[0]), int(order[len(order) // 2]), int(order[-1])}))


def test_ragged_long_cot_page_baseline_full_size(ragged_kv):
    # The page-level baseline on the full ragged batch (8192 page rows per
    # unit, pages of 16, C = 2048): summaries bit-exact and the selection by
    # the gap rule on the shortest, a mid-length and the longest sequence.
    import oracle
    from asp_testutil import kv_np
    from test_gpu_page import _check_selection, _check_summaries
    k, _ = ragged_kv
    wl = wk.RAGGED
    B, Hq, Hkv, D, T, P, C = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.t_cap, 16, wl.top_c
    lens_t = wk.make_seq_lens(wl, device=DEV)
    q = wk.make_queries(wl, 1, device=DEV)[0].contiguous()
    dims = A.Dims(B, Hq, Hkv, D, T, A.KV_BF16)
    cfg = A.Cfg(wl.window, C, wl.lam)
    NP = A.page_count(T, P)
    kmin = torch.empty((B, Hkv, NP, D), dtype=torch.bfloat16, device=DEV)
    kmax = torch.empty_like(kmin)
    A.asp_page_summary(dims, P, k, lens_t, kmin, kmax)
    idx = torch.empty((B, Hkv, C), dtype=torch.int32, device=DEV)
    n_sel = torch.empty((B, Hkv), dtype=torch.int32, device=DEV)
    A.asp_page_select(dims, cfg, P, q, kmin, kmax, lens_t, idx, n_sel)
    torch.cuda.synchronize()
    lens = np_(lens_t)
    order = np.argsort(lens)
    bs = sorted({int(order[0]), int(order[len(order) // 2]), int(order[-1])})
    sl = [int(lens[b]) for b in bs]
    o_min, o_max = oracle.page_summary(kv_np(k[bs]), sl, P)
    n_pages = oracle.page_counts(sl, T, P)
    _check_summaries(kmin[bs], kmax[bs], o_min, o_max, n_pages)
    s_orc = oracle.page_scores(np_(q[bs]), o_min, o_max, n_pages)
    _check_selection(np_(idx[bs]), np_(n_sel[bs]), s_orc, n_pages, sl, P, C)
    del kmin, kmax
