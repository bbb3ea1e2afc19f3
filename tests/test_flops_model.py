"""The analytic decode cost model against the figures the pages print.

* The FLOPs reduction at the Qwen3-8B shape, 32k context, C = 2k, is the
  reproduction card's 54.5% (claim C2), to the printed digit.
* The page-scan gap of page-level selection spans the card's 1-4% over page
  sizes 64 .. 16.
* Properties: no saving when C >= T; the saving grows with the context; the
  hot-path byte count equals the benchmark's own step-byte count.
"""
import json
import os

import pytest

import bench
from query_aware_sparse_amd import flops_model as fm
from query_aware_sparse_amd import workload as wk

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "decode_flops_reduction.json")


def test_reduction_matches_the_printed_figure():
    g = json.load(open(GOLDEN))
    r = fm.reduction(fm.ARCHS[g["model"]], g["context"], g["top_c"])
    assert round(100 * r, 1) == g["flops_reduction_percent"]


def test_page_scan_gap_spans_the_printed_range():
    g = json.load(open(GOLDEN))
    a = fm.ARCHS[g["model"]]
    lo, hi = g["page_scan_gap_percent_range"]
    gaps = {p: 100 * fm.page_scan_gap(a, g["context"], g["top_c"], p) for p in (16, 32, 64)}
    assert gaps[64] == pytest.approx(lo, abs=0.05)
    assert gaps[16] == pytest.approx(hi, abs=0.05)
    assert lo <= gaps[32] <= hi


@pytest.mark.parametrize("model", sorted(fm.ARCHS))
def test_no_saving_without_sparsity_and_monotone_in_context(model):
    a = fm.ARCHS[model]
    assert fm.reduction(a, 2048, 2048) == 0.0
    assert fm.reduction(a, 1000, 2048) == 0.0
    rs = [fm.reduction(a, T, 2048) for T in (4096, 8192, 32768, 131072)]
    assert all(x < y for x, y in zip(rs, rs[1:]))
    f = fm.decode_flops(a, 32768, 2048)
    assert f["full"] > f["sparse"] > 0


@pytest.mark.parametrize("wl", [wk.Q8B_LAYER, wk.Q8B_STACK, wk.Q32B, wk.RAGGED])
def test_hot_path_bytes_match_the_benchmark_count(wl):
    a = fm.ARCHS["qwen3-32b" if wl.group == 8 else "qwen3-8b"]
    assert (a.n_q_heads, a.n_kv_heads, a.head_dim) == (wl.n_q_heads, wl.n_kv_heads, wl.head_dim)
    lens = [int(x) for x in wk.make_seq_lens(wl).tolist()]
    B = wl.batch
    assert fm.hot_path_bytes(a, lens, wl.top_c) == bench.step_bytes(wl, lens)["score_select_attend"]
    kb = fm.kv_bytes(a, B, wl.t_cap, wl.top_c)
    assert kb["selection_scan"] * 2 == kb["full_attention"]
