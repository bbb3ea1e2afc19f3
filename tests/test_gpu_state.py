"""Determinism and saved state (GPU required).

* Every entry point run twice on the same inputs, with its outputs and its
  workspace filled with different bytes before each run, gives the same
  outputs bit for bit (the workspaces need no initialisation; the candidate
  route's threshold hints, an input, are the same in both runs).
* Checkpoint and resume: the library keeps no state between calls, so a
  decode loop is resumed from what the caller saves.  A layer decoded for
  six two-stream steps gives, bit for bit, the outputs of one decoded for
  three, whose ring (q_hist, hist_newest, hist_len) and current selection
  (idx, n_sel) are copied to the host, then into new buffers with a new
  workspace, new streams, events and context, and decoded for three more.
  The threshold hints at the head of the workspace only steer the candidate
  route's cost: the resumed run matches with the hints restored and with a
  zeroed workspace (every key kept on the first resumed step).
"""
import numpy as np
import pytest
import torch

import query_aware_sparse_amd as A
from query_aware_sparse_amd import workload as wk
from asp_testutil import np_, require_gpu
from test_gpu_step import Problem

pytestmark = pytest.mark.gpu
DEV = "cuda"

WL = wk.TINY.replace(name="state", batch=3, n_q_heads=8, n_kv_heads=2, head_dim=128, t_cap=3000, kv_dtype="bf16",
                     window=16, top_c=400, history_steps=20, heavy_count=8, seed=12)
LENS = [3000, 1234, 0]


def _garbage(t: torch.Tensor, seed: int) -> None:
    g = torch.Generator(device=DEV).manual_seed(seed)
    t.view(torch.uint8).view(-1).copy_(torch.randint(0, 256, (t.numel() * t.element_size(),), generator=g,
                                                     device=DEV, dtype=torch.int32).to(torch.uint8))


def test_every_entry_point_is_deterministic():
    require_gpu()
    p = Problem(WL, kv_device=DEV, n_steps=2, lens=LENS)
    p.fill_history()
    d, c = p.dims, p.cfg
    B, Hq, Hkv, D, T, C = WL.batch, WL.n_q_heads, WL.n_kv_heads, WL.head_dim, WL.t_cap, WL.top_c
    q = p.queries[WL.history_steps].to(DEV)
    P = 16
    NP = A.page_count(T, P)
    hints = torch.zeros(A.asp_workspace_size(d, c, A.OP_CANDIDATES), dtype=torch.uint8, device=DEV)
    _garbage(hints[: 4 * B * Hkv], 99)  # the same hints in both runs
    hints = hints[: 4 * B * Hkv].clone()

    def run(seed):
        outs = {}
        q_hist, newest, length = p.q_hist.clone(), p.newest.clone(), p.length.clone()
        A.asp_push_query(d, c, q, q_hist, newest, length)
        q_pred = torch.empty((B, Hq, D), device=DEV)
        _garbage(q_pred, seed)
        A.asp_predict_query(d, c, q_hist, newest, length, q_pred)
        scores = torch.empty((B, Hkv, T), device=DEV)
        hist = torch.empty((B, Hkv, 2048), dtype=torch.int32, device=DEV)
        _garbage(scores, seed + 1)
        _garbage(hist, seed + 2)
        A.asp_score_keys(d, q_pred, p.k, p.seq_lens, scores, hist=hist)
        idx = torch.empty((B, Hkv, C), dtype=torch.int32, device=DEV)
        n_sel = torch.empty((B, Hkv), dtype=torch.int32, device=DEV)
        ws = torch.empty(A.asp_workspace_size(d, c, A.OP_SELECT), dtype=torch.uint8, device=DEV)
        for t_, s_ in ((idx, 3), (n_sel, 4), (ws, 5)):
            _garbage(t_, seed + s_)
        A.asp_select_topc(d, c, scores, p.seq_lens, idx, n_sel, ws=ws, hist=hist)
        cws = torch.empty(A.asp_workspace_size(d, c, A.OP_CANDIDATES), dtype=torch.uint8, device=DEV)
        _garbage(cws, seed + 6)
        cws[: 4 * B * Hkv].copy_(hints)
        idx2, n2 = torch.empty_like(idx), torch.empty_like(n_sel)
        _garbage(idx2, seed + 7)
        A.asp_score_candidates(d, c, q_pred, p.k, p.seq_lens, cws)
        A.asp_select_candidates(d, c, q_pred, p.k, p.seq_lens, idx2, n2, cws)
        out = torch.empty((B, Hq, D), device=DEV)
        dws = torch.empty(A.asp_workspace_size(d, c, A.OP_DECODE), dtype=torch.uint8, device=DEV)
        _garbage(out, seed + 8)
        _garbage(dws, seed + 9)
        A.asp_sparse_decode(d, c, q, p.k, p.v, p.seq_lens, idx, n_sel, out, dws)
        out_s = torch.empty_like(out)
        _garbage(out_s, seed + 10)
        A.asp_sparse_decode_static(d, c, q, p.k, p.v, p.seq_lens, idx, n_sel, out_s)
        ovl = torch.empty((B, Hkv), dtype=torch.int32, device=DEV)
        A.asp_selection_overlap(d, c, idx, n_sel, idx2, n2, ovl)
        kmin = torch.empty((B, Hkv, NP, D), dtype=p.k.dtype, device=DEV)
        kmax = torch.empty_like(kmin)
        _garbage(kmin, seed + 11)
        A.asp_page_summary(d, P, p.k, p.seq_lens, kmin, kmax)
        pidx, pn = torch.empty_like(idx), torch.empty_like(n_sel)
        pws = torch.empty(A.asp_page_select_workspace_size(d, c, P), dtype=torch.uint8, device=DEV)
        _garbage(pws, seed + 12)
        A.asp_page_select(d, c, P, q, kmin, kmax, p.seq_lens, pidx, pn, pws)
        torch.cuda.synchronize()
        for name, t_ in (("ring", q_hist), ("newest", newest), ("length", length), ("q_pred", q_pred),
                         ("scores", scores), ("hist", hist), ("idx", idx), ("n_sel", n_sel), ("idx_cand", idx2),
                         ("n_cand", n2), ("hints_next", cws[: 4 * B * Hkv]), ("out", out), ("out_static", out_s),
                         ("overlap", ovl), ("kmin", kmin), ("kmax", kmax), ("page_idx", pidx), ("page_n", pn)):
            outs[name] = np_(t_.view(torch.int16) if t_.dtype == torch.bfloat16 else t_).copy()  # bits
        # rows past a sequence's tokens (scores) or pages (summaries) are not written
        outs["scores"] = np.concatenate([outs["scores"][b, :, :n].ravel() for b, n in enumerate(LENS)])
        for name in ("kmin", "kmax"):
            outs[name] = np.concatenate([outs[name][b, :, :(n + P - 1) // P].ravel() for b, n in enumerate(LENS)])
        return outs

    a, b = run(1000), run(2000)
    for name in a:
        np.testing.assert_array_equal(a[name], b[name], err_msg=name)


def _steps(p, s0, s1, state, ws):
    """Two-stream steps s0 .. s1-1 of the layer from `state` (its ring and the
    selection step s0 attends over, as device tensors); new streams, events
    and context.  Returns each step's (out, idx_next, n_sel_next) on the host
    and the state after the last step."""
    d, c = p.dims, p.cfg
    q_hist, newest, length, idx_cur, n_cur = state
    idx = [idx_cur, torch.empty_like(idx_cur)]
    nsel = [n_cur, torch.empty_like(n_cur)]
    ev = [A.HipEvent(), A.HipEvent()]
    ctx = A.AspContext()
    attn, sel = torch.cuda.Stream(), torch.cuda.Stream()
    out = torch.empty((WL.batch, WL.n_q_heads, WL.head_dim), device=DEV)
    attn.wait_stream(torch.cuda.current_stream())
    res = []
    for i, s in enumerate(range(s0, s1)):
        cur, nxt = i % 2, (i + 1) % 2
        q = p.queries[WL.history_steps + s].to(DEV)
        attn.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(attn):
            A.asp_step(d, c, q, q_hist, newest, length, p.k, p.v, p.seq_lens, idx[cur], nsel[cur], idx[nxt],
                       nsel[nxt], out, ws, attn_stream=attn, sel_stream=sel, ctx=ctx, idx_cur_ready=ev[cur],
                       idx_next_ready=ev[nxt])
        torch.cuda.synchronize()
        res.append((np_(out).copy(), np_(idx[nxt]).copy(), np_(nsel[nxt]).copy()))
    last = (s1 - s0) % 2
    ctx.close()
    return res, (q_hist, newest, length, idx[last], nsel[last])


def _bootstrap(p, ws):
    d, c = p.dims, p.cfg
    idx = torch.empty((WL.batch, WL.n_kv_heads, WL.top_c), dtype=torch.int32, device=DEV)
    n_sel = torch.empty((WL.batch, WL.n_kv_heads), dtype=torch.int32, device=DEV)
    out = torch.empty((WL.batch, WL.n_q_heads, WL.head_dim), device=DEV)
    A.asp_step(d, c, p.queries[WL.history_steps].to(DEV), p.q_hist, p.newest, p.length, p.k, p.v, p.seq_lens,
               None, None, idx, n_sel, out, ws)
    torch.cuda.synchronize()
    return (p.q_hist, p.newest, p.length, idx, n_sel)


@pytest.mark.parametrize("hints", ["restored", "zeroed"])
def test_decode_resumes_from_saved_state(hints):
    require_gpu()
    kv = wk.make_kv(WL, torch.tensor(LENS, dtype=torch.int32), device=DEV)
    ws_bytes = A.asp_workspace_size(A.Dims(WL.batch, WL.n_q_heads, WL.n_kv_heads, WL.head_dim, WL.t_cap,
                                           A.KV_BF16), A.Cfg(WL.window, WL.top_c, WL.lam), A.OP_STEP)
    n_hint = 4 * WL.batch * WL.n_kv_heads

    # straight through: the bootstrap step, then steps 1 .. 6
    p = Problem(WL, n_steps=8, kv=kv, lens=LENS)
    p.fill_history()
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=DEV)
    straight, _ = _steps(p, 1, 7, _bootstrap(p, ws), ws)

    # steps 1 .. 3, the caller's state saved to the host and everything dropped
    p = Problem(WL, n_steps=8, kv=kv, lens=LENS)
    p.fill_history()
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=DEV)
    first, state = _steps(p, 1, 4, _bootstrap(p, ws), ws)
    saved = [t.cpu().clone() for t in state] + [ws[:n_hint].cpu().clone()]
    del state, ws
    torch.cuda.synchronize()

    # resumed in new buffers (the old ones are still held, so the addresses differ)
    q_hist, newest, length, idx, n_sel = [t.to(DEV).clone() for t in saved[:5]]
    p.q_hist = None  # the Problem's own ring is not used again
    ws2 = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    _garbage(ws2, 5)
    if hints == "restored":
        ws2[:n_hint].copy_(saved[5].to(DEV))
    else:
        ws2.zero_()
    torch.cuda.synchronize()
    resumed, _ = _steps(p, 4, 7, (q_hist, newest, length, idx, n_sel), ws2)

    for s, (a, b) in enumerate(zip(straight, first + resumed)):
        for x, y, name in zip(a, b, ("out", "idx_next", "n_sel_next")):
            np.testing.assert_array_equal(x, y, err_msg="step %d %s" % (s + 1, name))
