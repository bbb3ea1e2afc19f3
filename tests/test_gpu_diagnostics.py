"""Selection overlap and the prediction-quality diagnostics (GPU required).

* asp_selection_overlap against the oracle's set intersection, bit-exact, on
  ascending selections of random, identical, disjoint, empty and partial lists,
  up to the largest selection (32768 entries).
* The diagnostics' counts (temporal-overlap lags, predicted and last-query
  recall) against the oracle on the GPU's own selections, and the summary
  ratios recomputed from those counts.
"""
import numpy as np
import pytest
import torch

import oracle
import query_aware_sparse_amd as A
from query_aware_sparse_amd import diagnostics as dg
from query_aware_sparse_amd import workload as wk
from asp_testutil import np_, require_gpu

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _sorted_selection(rng, T, n, C):
    row = np.full(C, -1, np.int32)
    row[:n] = np.sort(rng.choice(T, size=n, replace=False))
    return row


@pytest.mark.parametrize("B,Hkv,T_cap,C", [(3, 4, 5000, 700), (2, 2, 40000, 32768), (1, 1, 64, 64)])
def test_selection_overlap_matches_oracle(B, Hkv, T_cap, C):
    rng = np.random.default_rng(B * 1000 + C)
    d = A.Dims(B, 4 * Hkv, Hkv, 128, T_cap, A.KV_BF16)
    c = A.Cfg(16, C, 1e-2)
    ia = np.full((B, Hkv, C), -1, np.int32)
    ib = np.full((B, Hkv, C), -1, np.int32)
    na = np.zeros((B, Hkv), np.int32)
    nb = np.zeros((B, Hkv), np.int32)
    for u, (b, g) in enumerate(np.ndindex(B, Hkv)):
        kind = u % 5
        n1 = C if kind != 3 else 0
        n2 = [C, C, rng.integers(0, C + 1), C, C // 3][kind]
        ia[b, g] = _sorted_selection(rng, T_cap, n1, C)
        if kind == 0:
            ib[b, g] = ia[b, g]                                    # identical
        elif kind == 1 and 2 * C <= T_cap:                         # disjoint
            rest = np.setdiff1d(np.arange(T_cap), ia[b, g][:n1])
            ib[b, g, :n2] = np.sort(rng.choice(rest, size=n2, replace=False))
        else:
            ib[b, g] = _sorted_selection(rng, T_cap, int(n2), C)
        na[b, g], nb[b, g] = n1, n2
        if kind == 4:
            na[b, g] = C + 5                                       # clamped to C
    out = torch.empty((B, Hkv), dtype=torch.int32, device=DEV)
    A.asp_selection_overlap(d, c, torch.from_numpy(ia).to(DEV), torch.from_numpy(na).to(DEV),
                            torch.from_numpy(ib).to(DEV), torch.from_numpy(nb).to(DEV), out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(np_(out), oracle.overlap(ia, na, ib, nb, T_cap))


def test_selection_overlap_rejects_selections_beyond_lds():
    # head_dim 64 bf16 lets top_c reach 65536; the overlap stages 32768 at most
    d = A.Dims(1, 4, 1, 64, 50000, A.KV_BF16)
    c = A.Cfg(16, 40000, 1e-2)
    t = torch.zeros((1, 1, 40000), dtype=torch.int32, device=DEV)
    n = torch.zeros((1, 1), dtype=torch.int32, device=DEV)
    with pytest.raises(A.AspError, match="ASP_ERR_UNSUPPORTED"):
        A.asp_selection_overlap(d, c, t, n, t, n, torch.empty_like(n))


def test_diagnostics_counts_match_oracle():
    wl = wk.RAGGED.replace(name="diag-small", batch=2, n_q_heads=8, n_kv_heads=2, head_dim=64, t_cap=3000,
                           seq_len_range=(1000, 3000), window=8, top_c=256, history_steps=10)
    res = dg.collect(wl, steps=6, window=4)
    torch.cuda.synchronize()
    T_cap = wl.t_cap
    host = lambda s: (np_(s[0]), np_(s[1]))  # noqa: E731
    for (t, k), cnt in res["lag"].items():
        a, b = host(res["true"][t]), host(res["true"][t - k])
        np.testing.assert_array_equal(np_(cnt), oracle.overlap(a[0], a[1], b[0], b[1], T_cap))
    for t, cnt in res["rec_pred"].items():
        a, b = host(res["pred"][t]), host(res["true"][t])
        np.testing.assert_array_equal(np_(cnt), oracle.overlap(a[0], a[1], b[0], b[1], T_cap))
    for t, cnt in res["rec_last"].items():
        a, b = host(res["true"][t - 1]), host(res["true"][t])
        np.testing.assert_array_equal(np_(cnt), oracle.overlap(a[0], a[1], b[0], b[1], T_cap))
    assert res["page_size"] == 16 and sorted(res["rec_page"]) == sorted(res["rec_pred"])
    for t, cnt in res["rec_page"].items():
        a, b = host(res["page"][t]), host(res["true"][t])
        np.testing.assert_array_equal(np_(cnt), oracle.overlap(a[0], a[1], b[0], b[1], T_cap))
    s = dg.summarize(wl, res)
    assert 0.0 <= s["recall_page_current_query"] <= 1.0
    rp = [np.mean(np_(res["rec_pred"][t]) / np_(res["true"][t][1])) for t in sorted(res["rec_pred"])]
    assert s["recall_predicted"] == pytest.approx(np.mean(rp), rel=1e-12)
    assert 0.0 <= s["recall_last_query"] <= 1.0 and 0.0 <= s["temporal_overlap_window_mean"] <= 1.0
    assert len(s["temporal_overlap_by_lag"]) == 4
