"""The entry points recorded into a HIP graph (GPU required).

One decode step built from the individual entry points (push, predict, score
with its histogram, select, sparse attention over the previous selection) is
captured on one stream into a graph.  The graph is replayed several times,
with eager work (a new query copied into the captured input buffer) and a
synchronisation between replays; after every replay the attention output,
the selection and the query ring must equal, bit for bit, the same entry
points run eagerly on a second copy of the state.  (asp_step itself refuses
stream capture.)
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
