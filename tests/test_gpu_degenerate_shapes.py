"""Degenerate shapes (GPU required).

* Batch 0: every entry point validates its arguments and returns ASP_OK
  without touching the caller's arrays (asp.h: "batch >= 0 (0 is a no-op)");
  asp_check_device_args still clears its status word, and the two-stream step
  still orders its streams.  Every array pointer points into one zero-filled
  device buffer, which must read zero afterwards; the status word starts at a
  nonzero sentinel.
* The smallest non-empty shape: one query head per KV head, a token stride of
  one (t_cap = 1, C = 1), the shortest window (W = 4), one sequence holding
  its single token and one empty, through a bootstrap and four pipelined
  steps in every mode.  Closed forms pin the outputs: the full sequence
  selects token 0 and its attention over that one token returns V[0] exactly
  (a softmax over one logit is 1); the empty one selects nothing (index -1,
  count 0) and returns 0.  The modes agree bit for bit with the entry-point
  schedule.
"""
import ctypes

import numpy as np
import pytest
import torch

import query_aware_sparse_amd as A
from query_aware_sparse_amd import workload as wk
from asp_testutil import require_gpu
from test_gpu_step import Problem, _manual_run, _step_run

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("kv", [A.KV_BF16, A.KV_F32])
def test_every_entry_point_with_an_empty_batch_is_a_no_op(kv):
    require_gpu()
    lib = A.load()
    dims = A.Dims(0, 8, 2, 128, 1000, kv)
    cfg = A.Cfg(8, 100, 1e-2, 16)
    buf = torch.zeros(1 << 20, dtype=torch.int32, device=DEV)
    status = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    p = ctypes.c_void_p(buf.data_ptr())
    d, c = ctypes.byref(dims), ctypes.byref(cfg)
    ws = {op: A.asp_workspace_size(dims, cfg, op) for op in (A.OP_SELECT, A.OP_DECODE, A.OP_STEP, A.OP_CANDIDATES)}
    assert max(ws.values()) <= buf.numel() * 4
    attn, sel = torch.cuda.Stream(), torch.cuda.Stream()
    ha, hs = ctypes.c_void_p(attn.cuda_stream), ctypes.c_void_p(sel.cuda_stream)
    ctx = A.AspContext()
    ev_cur, ev_next = A.HipEvent(), A.HipEvent()
    st = ws[A.OP_STEP]
    calls = {
        "asp_push_query": lambda: lib.asp_push_query(d, c, p, p, p, p, None),
        "asp_predict_query": lambda: lib.asp_predict_query(d, c, p, p, p, p, None),
        "asp_score_keys": lambda: lib.asp_score_keys(d, p, p, p, p, None, None),
        "asp_score_keys with a histogram": lambda: lib.asp_score_keys(d, p, p, p, p, p, None),
        "asp_select_topc": lambda: lib.asp_select_topc(d, c, p, None, p, p, p, p, ws[A.OP_SELECT], None),
        "asp_select_topc with a histogram": lambda: lib.asp_select_topc(d, c, p, p, p, p, p, p, ws[A.OP_SELECT], None),
        "asp_score_candidates": lambda: lib.asp_score_candidates(d, c, p, p, p, p, ws[A.OP_CANDIDATES], None),
        "asp_select_candidates": lambda: lib.asp_select_candidates(d, c, p, p, p, p, p, p, ws[A.OP_CANDIDATES], None),
        "asp_selection_overlap": lambda: lib.asp_selection_overlap(d, c, p, p, p, p, p, None),
        "asp_sparse_decode": lambda: lib.asp_sparse_decode(d, c, p, p, p, p, p, p, p, p, ws[A.OP_DECODE], None),
        "asp_sparse_decode_static": lambda: lib.asp_sparse_decode_static(d, c, p, p, p, p, p, p, p, None),
        "asp_step bootstrap": lambda: lib.asp_step(None, d, c, p, p, p, p, p, p, p, None, None, p, p, p, p, st, ha,
                                                   None, None, ev_next.handle),
        "asp_step one stream": lambda: lib.asp_step(None, d, c, p, p, p, p, p, p, p, p, p, p, p, p, p, st, ha, ha,
                                                    ev_cur.handle, ev_next.handle),
        "asp_step two streams": lambda: lib.asp_step(ctx.handle, d, c, p, p, p, p, p, p, p, p, p, p, p, p, p, st, ha,
                                                     hs, ev_cur.handle, ev_next.handle),
        "asp_context_join": lambda: lib.asp_context_join(ctx.handle, ha),
        "asp_check_device_args": lambda: lib.asp_check_device_args(d, c, p, p, p, p, p,
                                                                   ctypes.c_void_p(status.data_ptr()), None),
    }
    for name, call in calls.items():
        assert call() == 0, name
    torch.cuda.synchronize()
    assert int(status.item()) == 0  # cleared: no violation in an empty batch
    assert int(torch.count_nonzero(buf).item()) == 0
    ctx.close()


@pytest.mark.parametrize("kv", ["bf16", "f32"])
def test_smallest_shape_through_every_step_mode(kv):
    require_gpu()
    wl = wk.TINY.replace(name="smallest", batch=2, n_q_heads=1, n_kv_heads=1, head_dim=64, t_cap=1, kv_dtype=kv,
                         window=4, top_c=1, history_steps=0, heavy_count=1, recent=0, seed=3)
    n = 5
    runs = {}
    for mode in ("manual", "one_stream", "two_streams"):
        p = Problem(wl, n_steps=n, lens=[1, 0])
        runs[mode] = _manual_run(p, n) if mode == "manual" else _step_run(p, mode, n)
    v0 = p.v[0, 0, 0].float().cpu().numpy()
    for mode in ("manual", "one_stream", "two_streams"):
        for st in range(n):
            out, idx, n_sel = runs[mode][st][:3]
            np.testing.assert_array_equal(idx.reshape(2), [0, -1], err_msg="%s step %d" % (mode, st))
            np.testing.assert_array_equal(n_sel.reshape(2), [1, 0], err_msg="%s step %d" % (mode, st))
            np.testing.assert_array_equal(out[0, 0], v0, err_msg="%s step %d" % (mode, st))
            np.testing.assert_array_equal(out[1, 0], np.zeros(64, np.float32), err_msg="%s step %d" % (mode, st))
            if mode != "manual":
                for a, b in zip(runs["manual"][st], runs[mode][st]):
                    np.testing.assert_array_equal(a, b, err_msg="%s step %d" % (mode, st))
