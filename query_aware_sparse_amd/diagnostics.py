"""Prediction-quality diagnostics on synthetic inputs.

Reproduction card, "What reproduces (and what does not)", claim C5: temporal
locality of the top-k selection inside a recent 16-query window, and the share
of the true next-step top-k selection that the ridge one-step-ahead prediction
recovers.  The card gives the figures (on real queries of Qwen3-8B/32B-class
models), not their definitions; the readings taken here:

* the selection S(q) of a query q is the exact top-C of the GQA-group-max scores
  max_h q_h . k_i, the rule the decode step applies to the predicted query;
* temporal overlap at lag k: |S(q_t) & S(q_{t-k})| / |S(q_t)|; the window
  figure is its mean over k = 1..window and over the steps that have a full
  window behind them;
* prediction recall: |S(q^_{t+1}) & S(q_{t+1})| / |S(q_{t+1})|, where q^_{t+1}
  is the prediction made at step t from the ring of recent queries; beside it,
  the "last query" baseline |S(q_t) & S(q_{t+1})| / |S(q_{t+1})|;
* page-level recall: the same share for the page-level baseline (Quest's
  selection, asp_page_select: the top C / P pages by their min/max bound, with
  the current query q_{t+1}), whose C tokens come in whole pages.

Every score pass, selection, prediction and overlap count runs in the library's
kernels (asp_score_keys, asp_select_topc, asp_push_query, asp_predict_query,
asp_selection_overlap, asp_page_summary, asp_page_select); this module only orders the calls and turns counts into
ratios.  The synthetic queries are AR(1) sequences, so the numbers measure the
predictor on that process, not on a model's queries.

    python -m query_aware_sparse_amd.diagnostics --workload qwen3-8b-layer --steps 48
"""
from __future__ import annotations

import argparse
import json
from typing import Dict, List, Tuple

import torch

from . import (Cfg, Dims, KV_BF16, KV_F32, OP_SELECT, asp_page_select, asp_page_select_workspace_size,
               asp_page_summary, asp_predict_query, asp_push_query, asp_score_keys, asp_select_topc,
               asp_selection_overlap, asp_workspace_size, page_count)
from . import workload as wk


class Selector:
    """Selections of arbitrary queries over one layer's keys (device resident)."""

    def __init__(self, wl: wk.Workload, seq_lens: torch.Tensor, k: torch.Tensor, device: str, page_size: int = 0):
        self.wl = wl
        self.dims = Dims(wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.t_cap,
                         KV_BF16 if wl.kv_dtype == "bf16" else KV_F32)
        self.cfg = Cfg(wl.window, wl.top_c, wl.lam)
        self.seq_lens, self.k = seq_lens, k
        B, Hkv, C = wl.batch, wl.n_kv_heads, wl.top_c
        self.scores = torch.empty((B, Hkv, wl.t_cap), dtype=torch.float32, device=device)
        self.ws = torch.empty(asp_workspace_size(self.dims, self.cfg, OP_SELECT), dtype=torch.uint8, device=device)
        self.device = device
        self.page_size = page_size
        if page_size > 0:  # page summaries of these keys, for the page-level baseline
            shape = (B, Hkv, page_count(wl.t_cap, page_size), wl.head_dim)
            self.kmin = torch.empty(shape, dtype=k.dtype, device=device)
            self.kmax = torch.empty(shape, dtype=k.dtype, device=device)
            asp_page_summary(self.dims, page_size, k, seq_lens, self.kmin, self.kmax)
            self.ws_page = torch.empty(asp_page_select_workspace_size(self.dims, self.cfg, page_size),
                                       dtype=torch.uint8, device=device)

    def page_select(self, q: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
        wl = self.wl
        idx = torch.empty((wl.batch, wl.n_kv_heads, wl.top_c), dtype=torch.int32, device=self.device)
        n_sel = torch.empty((wl.batch, wl.n_kv_heads), dtype=torch.int32, device=self.device)
        asp_page_select(self.dims, self.cfg, self.page_size, q, self.kmin, self.kmax, self.seq_lens, idx, n_sel,
                        ws=self.ws_page)
        return idx, n_sel

    def select(self, q: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
        wl = self.wl
        idx = torch.empty((wl.batch, wl.n_kv_heads, wl.top_c), dtype=torch.int32, device=self.device)
        n_sel = torch.empty((wl.batch, wl.n_kv_heads), dtype=torch.int32, device=self.device)
        asp_score_keys(self.dims, q, self.k, self.seq_lens, self.scores)
        asp_select_topc(self.dims, self.cfg, self.scores, self.seq_lens, idx, n_sel, ws=self.ws)
        return idx, n_sel

    def overlap(self, a, b) -> torch.Tensor:
        out = torch.empty((self.wl.batch, self.wl.n_kv_heads), dtype=torch.int32, device=self.device)
        asp_selection_overlap(self.dims, self.cfg, a[0], a[1], b[0], b[1], out)
        return out


def collect(wl: wk.Workload, steps: int, window: int = 16, layer: int = 0, device: str = "cuda",
            page_size: int = 16) -> Dict:
    """Selections and overlap counts of one synthetic layer.

    Returns device tensors: ``true[t]`` = S(q_t) for every query t in
    0 .. H+steps (H = wl.history_steps), ``pred[t]`` = S(q^_t) for t in
    H+1 .. H+steps, and the counts ``lag[(t, k)]`` = |S(q_t) & S(q_{t-k})|,
    ``rec_pred[t]``, ``rec_last[t]`` and, with page_size > 0 dividing C,
    ``rec_page[t]`` (overlaps with S(q_t); ``page[t]`` is the page-level
    selection with q_t)."""
    H = wl.history_steps
    lens = wk.make_seq_lens(wl, device=device)
    k, _ = wk.make_kv(wl, lens, layer=layer, device=device)
    qs = wk.make_queries(wl, H + steps + 1, layer=layer, device=device)
    if page_size <= 0 or wl.top_c % page_size != 0:
        page_size = 0
    sel = Selector(wl, lens, k, device, page_size)
    true = [sel.select(qs[t]) for t in range(H + steps + 1)]
    q_hist, newest, length = [x.to(device) for x in wk.empty_history(wl)]
    for t in range(H):
        asp_push_query(sel.dims, sel.cfg, qs[t], q_hist, newest, length)
    q_pred = torch.empty_like(qs[0])
    pred: Dict[int, Tuple[torch.Tensor, torch.Tensor]] = {}
    rec_pred, rec_last, rec_page = {}, {}, {}
    page: Dict[int, Tuple[torch.Tensor, torch.Tensor]] = {}
    for t in range(H, H + steps):
        asp_push_query(sel.dims, sel.cfg, qs[t], q_hist, newest, length)
        asp_predict_query(sel.dims, sel.cfg, q_hist, newest, length, q_pred)   # q^_{t+1}
        pred[t + 1] = sel.select(q_pred)
        rec_pred[t + 1] = sel.overlap(pred[t + 1], true[t + 1])
        rec_last[t + 1] = sel.overlap(true[t], true[t + 1])
        if page_size:
            page[t + 1] = sel.page_select(qs[t + 1])
            rec_page[t + 1] = sel.overlap(page[t + 1], true[t + 1])
    lag = {}
    for t in range(H, H + steps + 1):
        for kk in range(1, window + 1):
            if t - kk >= 0:
                lag[(t, kk)] = sel.overlap(true[t], true[t - kk])
    return {"true": true, "pred": pred, "lag": lag, "rec_pred": rec_pred, "rec_last": rec_last,
            "page": page, "rec_page": rec_page, "page_size": page_size, "H": H, "steps": steps, "window": window}


def summarize(wl: wk.Workload, res: Dict) -> Dict:
    """Ratios from the counts of ``collect`` (means over units and steps)."""
    H, steps, window = res["H"], res["steps"], res["window"]

    def ratio(count: torch.Tensor, base: torch.Tensor) -> float:
        c, n = count.double(), base.double()
        ok = n > 0
        return float((c[ok] / n[ok]).mean()) if bool(ok.any()) else float("nan")

    by_lag: List[float] = []
    for kk in range(1, window + 1):
        vals = [ratio(res["lag"][(t, kk)], res["true"][t][1]) for t in range(H, H + steps + 1)
                if (t, kk) in res["lag"]]
        by_lag.append(sum(vals) / len(vals))
    full = [t for t in range(H, H + steps + 1) if t - window >= 0]
    win = [sum(ratio(res["lag"][(t, kk)], res["true"][t][1]) for kk in range(1, window + 1)) / window for t in full]
    rp = [ratio(res["rec_pred"][t], res["true"][t][1]) for t in sorted(res["rec_pred"])]
    rl = [ratio(res["rec_last"][t], res["true"][t][1]) for t in sorted(res["rec_last"])]
    rg = [ratio(res["rec_page"][t], res["true"][t][1]) for t in sorted(res.get("rec_page", {}))]
    return {
        "workload": wl.name, "steps": steps, "window": window, "top_c": wl.top_c, "ring_window": wl.window,
        "temporal_overlap_window_mean": sum(win) / len(win) if win else float("nan"),
        "temporal_overlap_by_lag": by_lag,
        "recall_predicted": sum(rp) / len(rp), "recall_last_query": sum(rl) / len(rl),
        "recall_page_current_query": sum(rg) / len(rg) if rg else None, "page_size": res.get("page_size", 0),
        "recall_predicted_by_step": rp,
    }


def main() -> int:
    ap = argparse.ArgumentParser(description="Prediction-quality diagnostics on synthetic inputs (one GPU).")
    ap.add_argument("--workload", default="qwen3-8b-layer", choices=sorted(wk.CONFIGS))
    ap.add_argument("--steps", type=int, default=48)
    ap.add_argument("--window", type=int, default=16)
    ap.add_argument("--page-size", type=int, default=16, help="page size of the page-level baseline (0 = skip)")
    args = ap.parse_args()
    wl = wk.CONFIGS[args.workload]
    res = collect(wl, args.steps, args.window, page_size=args.page_size)
    torch.cuda.synchronize()
    print(json.dumps(summarize(wl, res)))
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
