"""End-to-end parity of the decode step (GPU required).

* Staged parity of the whole path against the oracle over a multi-step walk of
  the tiny workload and at the full Qwen3-8B-layer shape: ring bit-exact,
  predictor within 1e-4, scores within 1e-5 * max|score| of oracle scores
  computed from the GPU's prediction, selection bit-exact on the GPU's fp32
  scores and within the 1e-5 * max|score| boundary gap of the oracle's own fp64
  selection, attention within 1e-2 on the GPU's selection.
* asp_step (bootstrap, pipelined on one stream, pipelined on two streams with
  a context, also with the context destroyed and a new one made mid-run, and
  with a context whose score stream may use every CU) is bit-identical to the
  same schedule built from the individual entry points.
"""
import numpy as np
import pytest
import torch

import oracle
import query_aware_sparse_amd as A
from query_aware_sparse_amd import workload as wk
from asp_testutil import assert_pred_close, assert_selection_within_gap, kv_np, np_, require_gpu

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


class Problem:
    """Device-resident inputs and state of one layer of a workload."""

    def __init__(self, wl: wk.Workload, kv_device="cpu", layer=0, n_steps=8, kv=None, lens=None):
        self.wl = wl
        self.dims = A.Dims(wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.t_cap,
                           A.KV_BF16 if wl.kv_dtype == "bf16" else A.KV_F32)
        self.cfg = A.Cfg(wl.window, wl.top_c, wl.lam, wl.recent)
        # lens: context lengths that replace the workload's (K/V stay as generated)
        self.seq_lens = (wk.make_seq_lens(wl) if lens is None else torch.tensor(lens, dtype=torch.int32)).to(DEV)
        if kv is None:  # else K/V already generated for this workload's batch and lengths
            kv = wk.make_kv(wl, wk.make_seq_lens(wl), layer=layer, device=kv_device)
        self.k, self.v = kv[0].to(DEV), kv[1].to(DEV)
        self.queries = wk.make_queries(wl, wl.history_steps + n_steps, layer=layer)
        self.q_hist, self.newest, self.length = [x.to(DEV) for x in wk.empty_history(wl)]
        B, Hq, Hkv, D, C = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.top_c
        self.q_pred = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
        self.scores = torch.empty((B, Hkv, wl.t_cap), dtype=torch.float32, device=DEV)
        self.idx = torch.empty((B, Hkv, C), dtype=torch.int32, device=DEV)
        self.n_sel = torch.empty((B, Hkv), dtype=torch.int32, device=DEV)
        self.out = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
        self.ws_dec = torch.empty(A.asp_workspace_size(self.dims, self.cfg, A.OP_DECODE), dtype=torch.uint8,
                                  device=DEV)

    def fill_history(self):
        for t in range(self.wl.history_steps):
            A.asp_push_query(self.dims, self.cfg, self.queries[t].to(DEV), self.q_hist, self.newest, self.length)


def _staged_check(p: Problem, q_t: torch.Tensor, units=None):
    """Run push..attend through the entry points for actual query q_t and check
    every stage against the oracle (optionally on a subset of sequences)."""
    d, c = p.dims, p.cfg
    hist_before = (np_(p.q_hist), np_(p.newest), np_(p.length))
    A.asp_push_query(d, c, q_t.to(DEV), p.q_hist, p.newest, p.length)
    A.asp_predict_query(d, c, p.q_hist, p.newest, p.length, p.q_pred)
    A.asp_score_keys(d, p.q_pred, p.k, p.seq_lens, p.scores)
    A.asp_select_topc(d, c, p.scores, p.seq_lens, p.idx, p.n_sel)
    A.asp_sparse_decode(d, c, q_t.to(DEV), p.k, p.v, p.seq_lens, p.idx, p.n_sel, p.out, p.ws_dec)
    torch.cuda.synchronize()
    bs = list(range(p.wl.batch)) if units is None else units
    oh, on, ol = oracle.push(q_t.numpy(), *hist_before)
    np.testing.assert_array_equal(np_(p.q_hist), oh)
    np.testing.assert_array_equal(np_(p.newest), on)
    np.testing.assert_array_equal(np_(p.length), ol)
    q_pred = np_(p.q_pred)
    q_orc = oracle.predict(oh, on, ol, c.lam)
    assert_pred_close(q_pred[bs], q_orc[bs])
    lens = np_(p.seq_lens)[bs]
    k_s = kv_np(p.k[bs])
    v_s = kv_np(p.v[bs])
    s_orc = oracle.score(q_pred[bs], k_s, lens)
    with np.errstate(invalid="ignore"):  # rows past each length are unwritten: any bits
        s_gpu = np_(p.scores)[bs].astype(np.float64)
    for i, b in enumerate(bs):
        T = int(lens[i])
        for g in range(p.wl.n_kv_heads):
            err = np.abs(s_gpu[i, g, :T] - s_orc[i, g, :T]).max()
            assert err <= 1e-5 * np.abs(s_orc[i, g, :T]).max(), (b, g, err)
    idx_g, n_g = np_(p.idx)[bs], np_(p.n_sel)[bs]
    ri, rn = oracle.select(s_gpu, lens, c.top_c)   # bit-exact on the GPU's own fp32 scores
    np.testing.assert_array_equal(idx_g, ri)
    np.testing.assert_array_equal(n_g, rn)
    assert_selection_within_gap(idx_g, n_g, s_orc, lens, c.top_c)
    o_orc = oracle.attend(q_t.numpy()[bs], k_s, v_s, idx_g, n_g)
    err = np.abs(np_(p.out)[bs].astype(np.float64) - o_orc).max()
    assert err <= 1e-2, err
    # Not gated: overlap with the fully independent oracle path (its own prediction).
    s_ind = oracle.score(q_orc[bs].astype(np.float32), k_s, lens)
    ii, _ = oracle.select(s_ind, lens, c.top_c)
    inter = np.mean([len(set(a[a >= 0]) & set(b_[b_ >= 0])) / max(1, (a >= 0).sum())
                     for a, b_ in zip(idx_g.reshape(-1, c.top_c), ii.reshape(-1, c.top_c))])
    print("independent-path selection overlap %.6f, attention max err %.2e" % (inter, err), flush=True)


def test_tiny_workload_staged_walk():
    wl = wk.TINY
    p = Problem(wl, n_steps=6)
    # Walk the whole 64-query history, checking every step from the first push.
    for t in range(wl.history_steps + 6):
        _staged_check(p, p.queries[t])


@pytest.mark.parametrize("W", [8, 16, 32])
@pytest.mark.parametrize("C", [512, 2048])
def test_ragged_small_staged(W, C):
    wl = wk.RAGGED.replace(batch=3, t_cap=9000, seq_len_range=(1, 9000), window=W, top_c=C, history_steps=W + 2)
    p = Problem(wl, n_steps=2)
    p.seq_lens = torch.tensor([9000, 511, 4097], dtype=torch.int32, device=DEV)
    p.fill_history()
    _staged_check(p, p.queries[wl.history_steps])


def test_qwen3_8b_layer_full_shape_staged():
    # Full Qwen3-8B-layer shape (B=8, 32q/8kv, D=128, T=32768, C=2048, W=16); the
    # oracle checks every unit of one step after the ring is full.
    wl = wk.Q8B_LAYER
    p = Problem(wl, kv_device=DEV, n_steps=2)
    p.fill_history()
    _staged_check(p, p.queries[wl.history_steps])


def _step_run(p: Problem, mode: str, n_steps: int, release_after=None, hints=None, ctx_flags=0):
    """Run n_steps decode steps with asp_step in `mode`; return per-step outputs.
    release_after: step after which the context is destroyed and a new one
    made for the next two-stream step.  hints: {step: value} written over the
    workspace's per-unit threshold hints after that step.  ctx_flags: flags of
    the contexts made."""
    wl, d, c = p.wl, p.dims, p.cfg
    B, Hkv, C = wl.batch, wl.n_kv_heads, wl.top_c
    ws = torch.empty(A.asp_workspace_size(d, c, A.OP_STEP), dtype=torch.uint8, device=DEV)
    idx = [torch.full((B, Hkv, C), -5, dtype=torch.int32, device=DEV) for _ in range(2)]
    nsel = [torch.zeros((B, Hkv), dtype=torch.int32, device=DEV) for _ in range(2)]
    ev = [A.HipEvent(), A.HipEvent()]
    ctx = A.AspContext(flags=ctx_flags) if mode == "two_streams" else None
    attn = torch.cuda.Stream()
    sel = torch.cuda.Stream() if mode == "two_streams" else None
    results = []
    for s in range(n_steps):
        t = wl.history_steps + s
        q = p.queries[t].to(DEV)
        cur, nxt = s % 2, (s + 1) % 2
        attn.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(attn):
            if s == 0:
                A.asp_step(d, c, q, p.q_hist, p.newest, p.length, p.k, p.v, p.seq_lens, None, None, idx[nxt],
                           nsel[nxt], p.out, ws, attn_stream=attn, idx_next_ready=ev[nxt])
            else:
                A.asp_step(d, c, q, p.q_hist, p.newest, p.length, p.k, p.v, p.seq_lens, idx[cur], nsel[cur],
                           idx[nxt], nsel[nxt], p.out, ws, attn_stream=attn, sel_stream=sel, ctx=ctx,
                           idx_cur_ready=ev[cur], idx_next_ready=ev[nxt])
        torch.cuda.synchronize()
        results.append((np_(p.out).copy(), np_(idx[nxt]).copy(), np_(nsel[nxt]).copy(), np_(p.q_hist).copy(),
                        np_(p.newest).copy(), np_(p.length).copy()))
        if s == release_after and ctx is not None:
            ctx.close()
            ctx = A.AspContext(flags=ctx_flags)
        if hints and s in hints:
            ws[:4 * B * Hkv].view(torch.int32).fill_(hints[s])
            torch.cuda.synchronize()
    return results


def _manual_run(p: Problem, n_steps: int):
    """The pipelined schedule built from the individual entry points."""
    wl, d, c = p.wl, p.dims, p.cfg
    results = []
    idx_prev = n_prev = None
    for s in range(n_steps):
        q = p.queries[wl.history_steps + s].to(DEV)
        if s > 0:
            A.asp_sparse_decode(d, c, q, p.k, p.v, p.seq_lens, idx_prev, n_prev, p.out, p.ws_dec)
        A.asp_push_query(d, c, q, p.q_hist, p.newest, p.length)
        A.asp_predict_query(d, c, p.q_hist, p.newest, p.length, p.q_pred)
        A.asp_score_keys(d, p.q_pred, p.k, p.seq_lens, p.scores)
        idx = torch.empty_like(p.idx)
        n_sel = torch.empty_like(p.n_sel)
        A.asp_select_topc(d, c, p.scores, p.seq_lens, idx, n_sel)
        if s == 0:
            A.asp_sparse_decode(d, c, q, p.k, p.v, p.seq_lens, idx, n_sel, p.out, p.ws_dec)
        torch.cuda.synchronize()
        results.append((np_(p.out).copy(), np_(idx).copy(), np_(n_sel).copy(), np_(p.q_hist).copy(),
                        np_(p.newest).copy(), np_(p.length).copy()))
        idx_prev, n_prev = idx, n_sel
    return results


SMALL_STEP_CASES = {
    # ragged bf16, GQA group 8, head_dim 64, the largest window
    "g8-d64-w64": wk.RAGGED.replace(name="g8-d64-w64", batch=3, n_q_heads=16, n_kv_heads=2, head_dim=64,
                                    t_cap=5000, seq_len_range=(100, 5000), window=64, top_c=300, history_steps=70),
    # fp32 KV, group 2, head_dim 128, window 32 (ring not yet full when the steps start)
    "g2-d128-w32-f32": wk.TINY.replace(name="g2-d128-w32-f32", batch=2, n_q_heads=4, n_kv_heads=2, head_dim=128,
                                       t_cap=3000, window=32, top_c=500, history_steps=20),
    # window 4, group 1
    "g1-d128-w4": wk.TINY.replace(name="g1-d128-w4", batch=2, n_q_heads=2, n_kv_heads=2, head_dim=128,
                                  t_cap=1000, kv_dtype="bf16", window=4, top_c=1000, history_steps=6),
    # an empty sequence, one shorter than a split, one ending inside a split, one full
    "g4-short-empty": wk.TINY.replace(name="g4-short-empty", batch=4, n_q_heads=8, n_kv_heads=2, head_dim=128,
                                      t_cap=2000, kv_dtype="bf16", window=8, top_c=700, history_steps=10),
    # the newest 200 tokens attended beside the selection (which overlaps them)
    "g4-recent": wk.TINY.replace(name="g4-recent", batch=4, n_q_heads=8, n_kv_heads=2, head_dim=128,
                                 t_cap=2000, kv_dtype="bf16", window=8, top_c=300, history_steps=10, recent=200),
}
STEP_LENS_RECENT = [2000, 150, 0, 1234]
STEP_LENS = {"g4-short-empty": [0, 37, 650, 2000], "g4-recent": STEP_LENS_RECENT}


@pytest.mark.parametrize("wl_name", ["tiny", "qwen3-8b-layer"] + list(SMALL_STEP_CASES))
def test_step_modes_bit_identical_to_entry_points(wl_name):
    wl = wk.CONFIGS.get(wl_name) or SMALL_STEP_CASES[wl_name]
    n = 5
    runs = {}
    modes = ("one_stream", "two_streams", "two_streams_release", "two_streams_all_cus", "two_streams_hints",
             "one_stream_hints")
    for mode in ("manual",) + modes:
        p = Problem(wl, kv_device=DEV if wl.batch > 1 else "cpu", n_steps=n, lens=STEP_LENS.get(wl_name))
        p.fill_history()
        torch.cuda.synchronize()
        if mode == "manual":
            runs[mode] = _manual_run(p, n)
        elif mode == "two_streams_release":  # the context destroyed mid-run and a new one made
            runs[mode] = _step_run(p, "two_streams", n, release_after=2)
        elif mode == "two_streams_all_cus":  # a score stream without a CU mask
            runs[mode] = _step_run(p, "two_streams", n, ctx_flags=A.CTX_SCORE_ALL_CUS)
        elif mode.endswith("_hints"):  # hints that keep nothing (every unit rescored), then every key
            runs[mode] = _step_run(p, mode[:-len("_hints")], n, hints={0: -1, 1: 0, 3: -1})
        else:
            runs[mode] = _step_run(p, mode, n)
    for mode in modes:
        for s in range(n):
            for a, b in zip(runs["manual"][s], runs[mode][s]):
                np.testing.assert_array_equal(a, b, err_msg="%s step %d" % (mode, s))


@pytest.mark.parametrize("wl_name,L,n", [("g8-d64-w64", 3, 4), ("g1-d128-w4", 3, 4), ("g4-recent", 3, 4),
                                         ("qwen3-8b-layer", 4, 3)])
def test_two_stream_layer_rotation_matches_entry_points(wl_name, L, n):
    """The bench's schedule: L layers in rotation on two streams, one workspace,
    idx pair and event pair per layer and one shared context; every step
    of every layer equals the entry-point schedule of that layer (at the bench
    shape too: four 1 GiB layers)."""
    base = wk.CONFIGS.get(wl_name) or SMALL_STEP_CASES[wl_name]
    probs = [Problem(base, kv_device=DEV, layer=l, n_steps=n) for l in range(L)]
    for p in probs:
        p.fill_history()
    torch.cuda.synchronize()
    rings = [(p.q_hist.clone(), p.newest.clone(), p.length.clone()) for p in probs]
    manual = [_manual_run(p, n) for p in probs]
    for p, r in zip(probs, rings):
        p.q_hist.copy_(r[0]); p.newest.copy_(r[1]); p.length.copy_(r[2])
    torch.cuda.synchronize()
    B, Hkv, C = base.batch, base.n_kv_heads, base.top_c
    d, c = probs[0].dims, probs[0].cfg
    ws = [torch.empty(A.asp_workspace_size(d, c, A.OP_STEP), dtype=torch.uint8, device=DEV) for _ in range(L)]
    idx = [[torch.full((B, Hkv, C), -5, dtype=torch.int32, device=DEV) for _ in range(2)] for _ in range(L)]
    nsel = [[torch.zeros((B, Hkv), dtype=torch.int32, device=DEV) for _ in range(2)] for _ in range(L)]
    ev = [[A.HipEvent(), A.HipEvent()] for _ in range(L)]
    outs = [torch.empty_like(p.out) for p in probs]
    ctx = A.AspContext()
    attn, sel = torch.cuda.Stream(), torch.cuda.Stream()
    attn.wait_stream(torch.cuda.current_stream())
    got = [[] for _ in range(L)]
    # every step's query stays allocated until the end: the streams read it
    # long after the host has moved on (a freed block could be refilled by the
    # next upload on the default stream while a step still reads it)
    alive = []
    for s in range(n):
        for l, p in enumerate(probs):  # one step of every layer, in layer order, nothing synchronised
            q = p.queries[base.history_steps + s].to(DEV)
            alive.append(q)
            cur, nxt = s % 2, (s + 1) % 2
            attn.wait_stream(torch.cuda.current_stream())
            if s == 0:
                A.asp_step(d, c, q, p.q_hist, p.newest, p.length, p.k, p.v, p.seq_lens, None, None, idx[l][nxt],
                           nsel[l][nxt], outs[l], ws[l], attn_stream=attn, idx_next_ready=ev[l][nxt])
            else:
                A.asp_step(d, c, q, p.q_hist, p.newest, p.length, p.k, p.v, p.seq_lens, idx[l][cur], nsel[l][cur],
                           idx[l][nxt], nsel[l][nxt], outs[l], ws[l], attn_stream=attn, sel_stream=sel,
                           ctx=ctx, idx_cur_ready=ev[l][cur], idx_next_ready=ev[l][nxt])
            # snapshots in each writer's stream order: the attention output on the
            # attention stream, the selection and the ring where the step completes
            # them (the selection stream once pipelined)
            with torch.cuda.stream(attn if s == 0 else sel):
                sel_snap = (idx[l][nxt].clone(), nsel[l][nxt].clone(), p.q_hist.clone(), p.newest.clone(),
                            p.length.clone())
            with torch.cuda.stream(attn):
                got[l].append((outs[l].clone(),) + sel_snap)
    torch.cuda.synchronize()
    for l in range(L):
        for s in range(n):
            for i, (a, b) in enumerate(zip(manual[l][s], got[l][s])):
                np.testing.assert_array_equal(a, np_(b), err_msg="layer %d step %d field %d" % (l, s, i))
