"""The entry points recorded into a HIP graph (GPU required).

One decode step built from the individual entry points (push, predict, score
with its histogram, select, sparse attention over the previous selection) is
captured on one stream into a graph.  The graph is replayed several times,
with eager work (a new query copied into the captured input buffer) and a
synchronisation between replays; after every replay the attention output,
the selection and the query ring must equal, bit for bit, the same entry
points run eagerly on a second copy of the state.  The same holds for
asp_step in its one-stream pipelined mode (two steps captured, with their
selection events) and in its two-stream mode (two layers in rotation, two
steps each, one context joined back before the capture ends).  A two-stream
step whose selection stream is capturing into another graph is refused with
ASP_ERR_UNSUPPORTED and enqueues nothing.
"""
import numpy as np
import pytest
import torch

import query_aware_sparse_amd as A
from query_aware_sparse_amd import workload as wk
from asp_testutil import np_, require_gpu
from test_gpu_step import DEV, Problem, SMALL_STEP_CASES, STEP_LENS

pytestmark = pytest.mark.gpu


class _State:
    def __init__(self, p: Problem):
        wl = p.wl
        B, Hkv, Hq, D, C = wl.batch, wl.n_kv_heads, wl.n_q_heads, wl.head_dim, wl.top_c
        self.q_hist, self.newest, self.length = p.q_hist.clone(), p.newest.clone(), p.length.clone()
        self.q_pred = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
        self.scores = torch.empty((B, Hkv, wl.t_cap), dtype=torch.float32, device=DEV)
        self.hist = torch.empty((B, Hkv, A.HIST_BINS), dtype=torch.int32, device=DEV)
        self.idx = [torch.full((B, Hkv, C), -1, dtype=torch.int32, device=DEV) for _ in range(2)]
        self.n_sel = [torch.zeros((B, Hkv), dtype=torch.int32, device=DEV) for _ in range(2)]
        self.out = torch.zeros((B, Hq, D), dtype=torch.float32, device=DEV)
        self.ws_sel = torch.empty(A.asp_workspace_size(p.dims, p.cfg, A.OP_SELECT), dtype=torch.uint8, device=DEV)
        self.ws_dec = torch.empty(A.asp_workspace_size(p.dims, p.cfg, A.OP_DECODE), dtype=torch.uint8, device=DEV)

    def step(self, p: Problem, q, cur: int):
        """Attention over selection `cur`, then the next selection into 1 - cur."""
        d, c = p.dims, p.cfg
        A.asp_sparse_decode(d, c, q, p.k, p.v, p.seq_lens, self.idx[cur], self.n_sel[cur], self.out, self.ws_dec)
        A.asp_push_query(d, c, q, self.q_hist, self.newest, self.length)
        A.asp_predict_query(d, c, self.q_hist, self.newest, self.length, self.q_pred)
        A.asp_score_keys(d, self.q_pred, p.k, p.seq_lens, self.scores, hist=self.hist)
        A.asp_select_topc(d, c, self.scores, p.seq_lens, self.idx[1 - cur], self.n_sel[1 - cur], ws=self.ws_sel,
                          hist=self.hist)

    def snapshot(self, nxt: int):
        return [np_(x).copy() for x in (self.out, self.idx[nxt], self.n_sel[nxt], self.q_hist, self.newest,
                                        self.length)]


@pytest.mark.parametrize("wl_name", ["g4-recent", "g8-d64-w64"])
def test_captured_entry_point_step_replays_match_eager(wl_name):
    require_gpu()
    wl = SMALL_STEP_CASES[wl_name]
    n_rep = 4
    p = Problem(wl, kv_device=DEV, n_steps=n_rep + 2, lens=STEP_LENS.get(wl_name))
    p.fill_history()
    torch.cuda.synchronize()
    graph_state, eager_state = _State(p), _State(p)
    warm = _State(p)  # one eager step on throwaway state before the capture
    warm.step(p, p.queries[wl.history_steps].to(DEV), 0)
    torch.cuda.synchronize()
    del warm
    q_buf = torch.empty((wl.batch, wl.n_q_heads, wl.head_dim), dtype=torch.float32, device=DEV)
    t0 = wl.history_steps

    # Two captured steps (selection 0 -> 1 -> 0), so that the graph leaves the
    # buffers in the parity it started from and can be replayed as is.
    q_buf2 = torch.empty_like(q_buf)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        graph_state.step(p, q_buf, 0)
        graph_state.step(p, q_buf2, 1)
    torch.cuda.synchronize()
    # Capturing ran nothing: the graph state is still the initial one.
    for rep in range(n_rep):
        qa, qb = p.queries[t0 + rep].to(DEV), p.queries[t0 + rep + 1].to(DEV)
        q_buf.copy_(qa)
        q_buf2.copy_(qb)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager_state.step(p, qa, 0)
        eager_state.step(p, qb, 1)
        torch.cuda.synchronize()
        for name, a, b in zip(("out", "idx", "n_sel", "q_hist", "newest", "len"), graph_state.snapshot(0),
                              eager_state.snapshot(0)):
            np.testing.assert_array_equal(a, b, err_msg="replay %d %s" % (rep, name))


def test_captured_page_step_replays_match_eager():
    # The page-level baseline's step (page selection with the current query,
    # then attention over the chosen pages' tokens) in a graph.
    require_gpu()
    B, Hq, Hkv, D, T, P, C = 3, 16, 4, 128, 5000, 16, 1024
    wl = wk.Q8B_LAYER.replace(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, t_cap=T, seed=21)
    lens = torch.tensor([5000, 3001, 100], dtype=torch.int32)
    k, v = wk.make_kv(wl, lens, device=DEV)
    lens = lens.to(DEV)
    qs = wk.make_queries(wl, 6, device=DEV)
    dims = A.Dims(B, Hq, Hkv, D, T, A.KV_BF16)
    cfg = A.Cfg(16, C, 1e-2)
    NP = A.page_count(T, P)
    kmin = torch.empty((B, Hkv, NP, D), dtype=torch.bfloat16, device=DEV)
    kmax = torch.empty_like(kmin)
    A.asp_page_summary(dims, P, k, lens, kmin, kmax)

    def buffers():
        return dict(idx=torch.full((B, Hkv, C), -5, dtype=torch.int32, device=DEV),
                    n=torch.zeros((B, Hkv), dtype=torch.int32, device=DEV),
                    out=torch.zeros((B, Hq, D), device=DEV),
                    ws=torch.empty(A.asp_page_select_workspace_size(dims, cfg, P), dtype=torch.uint8, device=DEV),
                    wsd=torch.empty(A.asp_workspace_size(dims, cfg, A.OP_DECODE), dtype=torch.uint8, device=DEV))

    def step(bf, q, stream=None):
        A.asp_page_select(dims, cfg, P, q, kmin, kmax, lens, bf["idx"], bf["n"], bf["ws"], stream=stream)
        A.asp_sparse_decode(dims, cfg, q, k, v, lens, bf["idx"], bf["n"], bf["out"], bf["wsd"], stream=stream)

    gb, eb = buffers(), buffers()
    q_buf = qs[0].clone()
    step(buffers(), q_buf)  # one eager call before the capture
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        step(gb, q_buf, stream=side)
    torch.cuda.synchronize()
    for rep in range(1, 6):
        q_buf.copy_(qs[rep])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        step(eb, qs[rep])
        torch.cuda.synchronize()
        for name in ("idx", "n", "out"):
            np.testing.assert_array_equal(np_(gb[name]), np_(eb[name]), err_msg="replay %d %s" % (rep, name))


def _step_state(p: Problem):
    wl = p.wl
    B, Hkv, Hq, D, C = wl.batch, wl.n_kv_heads, wl.n_q_heads, wl.head_dim, wl.top_c
    st = dict(q_hist=p.q_hist.clone(), newest=p.newest.clone(), length=p.length.clone(),
              idx=[torch.full((B, Hkv, C), -1, dtype=torch.int32, device=DEV) for _ in range(2)],
              n_sel=[torch.zeros((B, Hkv), dtype=torch.int32, device=DEV) for _ in range(2)],
              out=torch.zeros((B, Hq, D), dtype=torch.float32, device=DEV),
              ws=torch.empty(A.asp_workspace_size(p.dims, p.cfg, A.OP_STEP), dtype=torch.uint8, device=DEV),
              ev=[A.HipEvent(), A.HipEvent()])
    return st


def _asp_step(p: Problem, st, q, cur, stream, bootstrap=False):
    nxt = 1 - cur
    A.asp_step(p.dims, p.cfg, q, st["q_hist"], st["newest"], st["length"], p.k, p.v, p.seq_lens,
               None if bootstrap else st["idx"][cur], None if bootstrap else st["n_sel"][cur], st["idx"][nxt],
               st["n_sel"][nxt], st["out"], st["ws"], attn_stream=stream, idx_next_ready=st["ev"][nxt])


@pytest.mark.parametrize("wl_name", ["g4-recent", "g8-d64-w64"])
def test_captured_one_stream_asp_step_replays_match_eager(wl_name):
    # Two one-stream pipelined asp_step calls (selection 1 -> 0 -> 1), with the
    # events they record, captured once and replayed with new queries; every
    # replay equals the same calls made eagerly on a second copy of the state.
    require_gpu()
    wl = SMALL_STEP_CASES[wl_name]
    n_rep = 4
    p = Problem(wl, kv_device=DEV, n_steps=2 * n_rep + 2, lens=STEP_LENS.get(wl_name))
    p.fill_history()
    torch.cuda.synchronize()
    t0 = wl.history_steps
    gs, es = _step_state(p), _step_state(p)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    q0 = p.queries[t0].to(DEV)
    for st in (gs, es):  # the bootstrap step, eager on both copies: selection 1
        _asp_step(p, st, q0, 0, side, bootstrap=True)
    torch.cuda.synchronize()
    qa_buf = torch.empty((wl.batch, wl.n_q_heads, wl.head_dim), dtype=torch.float32, device=DEV)
    qb_buf = torch.empty_like(qa_buf)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        _asp_step(p, gs, qa_buf, 1, side)   # attends selection 1, selects 0
        _asp_step(p, gs, qb_buf, 0, side)   # attends selection 0, selects 1
    torch.cuda.synchronize()
    for rep in range(n_rep):
        qa, qb = p.queries[t0 + 1 + 2 * rep].to(DEV), p.queries[t0 + 2 + 2 * rep].to(DEV)
        qa_buf.copy_(qa)
        qb_buf.copy_(qb)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _asp_step(p, es, qa, 1, side)
        _asp_step(p, es, qb, 0, side)
        torch.cuda.synchronize()
        for name in ("out", "q_hist", "newest", "length"):
            np.testing.assert_array_equal(np_(gs[name]), np_(es[name]), err_msg="replay %d %s" % (rep, name))
        for i in (0, 1):
            np.testing.assert_array_equal(np_(gs["idx"][i]), np_(es["idx"][i]), err_msg="replay %d idx" % rep)
            np.testing.assert_array_equal(np_(gs["n_sel"][i]), np_(es["n_sel"][i]), err_msg="replay %d n" % rep)


@pytest.mark.parametrize("ctx_flags", [A.CTX_SCORE_ALL_CUS, 0], ids=["all-cus", "masked"])
@pytest.mark.parametrize("wl_name", ["g4-recent", "g8-d64-w64"])
def test_captured_two_stream_steps_replay_match_eager(wl_name, ctx_flags):
    # Two layers, each bootstrapped eagerly; then two pipelined two-stream
    # steps of each layer (layers in rotation, one shared context) captured
    # with attn as the origin: the first steps order themselves after the
    # selection they read by the graph's replay order (no idx_cur_ready), the
    # second ones wait for the events the first recorded in the capture; the
    # context's stream and sel join attn before the capture ends.  Every
    # replay, with new queries, equals the same steps made eagerly on copies.
    require_gpu()
    wl = SMALL_STEP_CASES[wl_name]
    L, n_rep = 2, 3
    probs = [Problem(wl, kv_device=DEV, layer=l, n_steps=2 * n_rep + 2, lens=STEP_LENS.get(wl_name))
             for l in range(L)]
    for p in probs:
        p.fill_history()
    torch.cuda.synchronize()
    t0 = wl.history_steps
    gs = [_step_state(p) for p in probs]
    es = [_step_state(p) for p in probs]
    attn, sel = torch.cuda.Stream(), torch.cuda.Stream()
    attn.wait_stream(torch.cuda.current_stream())
    for l, p in enumerate(probs):  # bootstrap steps (selection 1), eager on both copies
        q0 = p.queries[t0].to(DEV)
        for st in (gs[l], es[l]):
            _asp_step(p, st, q0, 0, attn, bootstrap=True)
    torch.cuda.synchronize()
    shape = (wl.batch, wl.n_q_heads, wl.head_dim)
    q_buf = [[torch.empty(shape, device=DEV) for _ in range(2)] for _ in range(L)]
    ctx_g, ctx_e = A.AspContext(flags=ctx_flags), A.AspContext(flags=ctx_flags)

    def two_stream_step(p, st, q, cur, ctx, wait):
        nxt = 1 - cur
        A.asp_step(p.dims, p.cfg, q, st["q_hist"], st["newest"], st["length"], p.k, p.v, p.seq_lens,
                   st["idx"][cur], st["n_sel"][cur], st["idx"][nxt], st["n_sel"][nxt], st["out"], st["ws"],
                   attn_stream=attn, sel_stream=sel, ctx=ctx, idx_cur_ready=st["ev"][cur] if wait else None,
                   idx_next_ready=st["ev"][nxt])

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=attn):
        for j, cur in enumerate((1, 0)):  # selection 1 -> 0, then 0 -> 1
            for l, p in enumerate(probs):
                two_stream_step(p, gs[l], q_buf[l][j], cur, ctx_g, wait=j > 0)
        ctx_g.join(attn)
        attn.wait_stream(sel)
    torch.cuda.synchronize()
    for rep in range(n_rep):
        qs = [[p.queries[t0 + 1 + 2 * rep + j].to(DEV) for j in range(2)] for p in probs]
        for l in range(L):
            for j in range(2):
                q_buf[l][j].copy_(qs[l][j])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        attn.wait_stream(torch.cuda.current_stream())
        for j, cur in enumerate((1, 0)):
            for l, p in enumerate(probs):
                two_stream_step(p, es[l], qs[l][j], cur, ctx_e, wait=True)
        attn.wait_stream(sel)
        torch.cuda.synchronize()
        for l in range(L):
            for name in ("out", "q_hist", "newest", "length"):
                np.testing.assert_array_equal(np_(gs[l][name]), np_(es[l][name]),
                                              err_msg="replay %d layer %d %s" % (rep, l, name))
            for i in (0, 1):
                np.testing.assert_array_equal(np_(gs[l]["idx"][i]), np_(es[l]["idx"][i]),
                                              err_msg="replay %d layer %d idx" % (rep, l))
                np.testing.assert_array_equal(np_(gs[l]["n_sel"][i]), np_(es[l]["n_sel"][i]),
                                              err_msg="replay %d layer %d n_sel" % (rep, l))
    ctx_g.close()
    ctx_e.close()


@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")  # the refused step enqueues nothing
def test_two_stream_step_refuses_a_selection_stream_in_another_capture():
    # sel_stream capturing while attn_stream is not: refused before anything is enqueued
    require_gpu()
    wl = SMALL_STEP_CASES["g4-recent"]
    p = Problem(wl, kv_device=DEV, n_steps=3, lens=STEP_LENS.get("g4-recent"))
    p.fill_history()
    st = _step_state(p)
    attn, sel = torch.cuda.Stream(), torch.cuda.Stream()
    attn.wait_stream(torch.cuda.current_stream())
    q = p.queries[wl.history_steps].to(DEV)
    _asp_step(p, st, q, 0, attn, bootstrap=True)
    torch.cuda.synchronize()
    ctx = A.AspContext()
    before = np_(st["idx"][0]).copy()
    g = torch.cuda.CUDAGraph()
    with pytest.raises(A.AspError) as e:
        with torch.cuda.graph(g, stream=sel):
            A.asp_step(p.dims, p.cfg, q, st["q_hist"], st["newest"], st["length"], p.k, p.v, p.seq_lens,
                       st["idx"][1], st["n_sel"][1], st["idx"][0], st["n_sel"][0], st["out"], st["ws"],
                       attn_stream=attn, sel_stream=sel, ctx=ctx, idx_cur_ready=st["ev"][1],
                       idx_next_ready=st["ev"][0])
    assert e.value.status == 2  # ASP_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    np.testing.assert_array_equal(np_(st["idx"][0]), before)  # nothing ran
    ctx.close()
