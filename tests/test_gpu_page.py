"""Parity of the page-level (Quest) selection against the CPU oracle (GPU required).

The baseline the pages compare AsyncSpade with selects whole pages with the
current query (research-map summary, "Problem" and the baselines of
"Experimental setup"); the page
score is Quest's published min/max bound.  Checks, on the bytes the GPU used:
  * page summaries: bit-exact (they are copies of key elements);
  * page scores: bit-exact on small-integer inputs, else within 1e-5 of the
    page's absolute bound sum_d max(|q_d min_d|, |q_d max_d|) (fp32 sums of D
    terms against fp64);
  * page selection: every page in the symmetric difference with the oracle's
    top-K lies within 1e-5 * max|score| of the oracle's K-th score, and the
    token list is exactly the tokens of the GPU's pages, ascending;
  * the page step's attention (page selection, then asp_sparse_decode with the
    same query): max-abs 1e-2 against the oracle on the same tokens.
Sizes span several blocks and ragged page tails; the last case is the
Qwen3-8B layer shape (32k tokens, pages of 16, C = 2048) on sampled units.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import query_aware_sparse_amd as A
from query_aware_sparse_amd import workload as wk
from asp_testutil import assert_selection_within_gap, dims_for, kv_np, np_, require_gpu

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()
    print("\n[case]", flush=True)


def _inputs(B, Hq, Hkv, D, T_cap, kv, lens, seed, heavy=0.01, integers=False):
    lens_t = torch.tensor(lens, dtype=torch.int32)
    if integers:  # values in {-3..3}: every product and sum is exact in fp32
        k = (wk.randn((B, Hkv, T_cap, D), seed=seed) * 2).round().clamp(-3, 3)
        q = (wk.randn((B, Hq, D), seed=seed, sub=1) * 2).round().clamp(-3, 3)
        k = k.to(torch.bfloat16 if kv == "bf16" else torch.float32)
    else:
        wl = wk.Q8B_LAYER.replace(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, t_cap=T_cap, kv_dtype=kv,
                                  heavy_frac=heavy, seed=seed)
        k, _ = wk.make_kv(wl, lens_t)
        q = wk.randn((B, Hq, D), seed=seed, sub=1)
    return k.to(DEV), q.to(DEV), lens_t.to(DEV)


def _summaries(dims, P, k, lens):
    NP = A.page_count(dims.t_cap, P)
    shape = (dims.batch, dims.n_kv_heads, NP, dims.head_dim)
    kmin = torch.zeros(shape, dtype=k.dtype, device=DEV)
    kmax = torch.zeros(shape, dtype=k.dtype, device=DEV)
    A.asp_page_summary(dims, P, k, lens, kmin, kmax)
    return kmin, kmax


def _as_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()


def _check_summaries(kmin, kmax, o_min, o_max, n_pages):
    g_min, g_max = _as_f64(kmin), _as_f64(kmax)
    for b, n in enumerate(n_pages):
        np.testing.assert_array_equal(g_min[b, :, :n], o_min[b, :, :n])
        np.testing.assert_array_equal(g_max[b, :, :n], o_max[b, :, :n])


def _abs_bound(q, kmin, kmax, G):
    """sum_d max(|q_d min_d|, |q_d max_d|), maxed over the group: the scale of
    a page score's rounding error."""
    B, Hkv, NP, D = kmin.shape
    qa = np.abs(q.astype(np.float64)).reshape(B, Hkv, G, D)
    m = np.maximum(np.abs(np.nan_to_num(kmin)), np.abs(np.nan_to_num(kmax)))  # [B][Hkv][NP][D]
    return np.einsum("bghd,bgpd->bghp", qa, m).max(axis=2)


def _pages_of(idx, n, P):
    return sorted(set((idx[:n] // P).tolist()))


def _check_selection(idx_g, n_g, s_orc, n_pages, lens, P, C):
    """GPU token lists against the oracle's page scores (from the same inputs)."""
    K = C // P
    pidx_o, pn_o = oracle.select(s_orc, n_pages, K)
    B, Hkv, _ = s_orc.shape
    for b in range(B):
        for g in range(Hkv):
            pages = _pages_of(idx_g[b, g], int(n_g[b, g]), P)
            ke = min(K, int(n_pages[b]))
            assert len(pages) == ke, (b, g, len(pages), ke)
            want = sorted(pidx_o[b, g, :ke].tolist())
            if pages != want:
                row = s_orc[b, g, : n_pages[b]]
                thr = np.sort(row)[::-1][ke - 1]
                tol = 1e-5 * np.abs(row).max()
                for p in set(pages) ^ set(want):
                    assert abs(row[p] - thr) <= tol, (b, g, p, row[p], thr, tol)
            # the token list is exactly the tokens of the GPU's pages, ascending
            toks, _ = oracle.page_tokens(np.array(pages + [-1] * (K - ke), np.int32).reshape(1, 1, K),
                                         np.array([[ke]], np.int32), [lens[b]], P, C, s_orc.shape[2] * P)
            np.testing.assert_array_equal(idx_g[b, g], toks[0, 0])
            assert n_g[b, g] == int((toks[0, 0] >= 0).sum())


CASES = [
    # B, Hq, Hkv, D, T_cap, kv, lens, P, C
    (3, 8, 2, 128, 3000, "bf16", [3000, 1234, 17], 16, 512),
    (2, 16, 2, 128, 2500, "bf16", [2500, 2491], 7, 700),
    (2, 8, 1, 64, 4096, "bf16", [4096, 4000], 64, 1024),
    (3, 4, 2, 128, 1500, "f32", [1500, 777, 1], 16, 256),
    (2, 4, 4, 64, 1030, "f32", [1030, 1029], 1, 96),
    (2, 16, 2, 128, 2048, "bf16", [2048, 0], 32, 32),
    # more pages than one workgroup holds: the row-selection route
    (2, 4, 2, 64, 17000, "bf16", [17000, 16500], 1, 256),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%d_G%d_D%d_T%d_%s_P%d_C%d" % (
    c[0], c[1] // c[2], c[3], c[4], c[5], c[7], c[8]))
def test_page_summary_scores_and_selection(case):
    B, Hq, Hkv, D, T_cap, kv, lens, P, C = case
    G = Hq // Hkv
    print("[case] page", case, flush=True)
    k, q, lens_t = _inputs(B, Hq, Hkv, D, T_cap, kv, lens, seed=sum(lens) + P)
    dims = dims_for(A, B, Hq, Hkv, D, T_cap, kv)
    cfg = A.Cfg(16, C, 1e-2)
    NP = A.page_count(T_cap, P)
    kmin, kmax = _summaries(dims, P, k, lens_t)
    scores = torch.full((B, Hkv, NP), float("nan"), device=DEV)
    A.asp_page_scores(dims, P, q, kmin, kmax, lens_t, scores)
    idx = torch.full((B, Hkv, C), -7, dtype=torch.int32, device=DEV)
    n_sel = torch.full((B, Hkv), -7, dtype=torch.int32, device=DEV)
    A.asp_page_select(dims, cfg, P, q, kmin, kmax, lens_t, idx, n_sel)
    torch.cuda.synchronize()

    o_min, o_max = oracle.page_summary(kv_np(k), lens, P)
    n_pages = oracle.page_counts(lens, T_cap, P)
    _check_summaries(kmin, kmax, o_min, o_max, n_pages)
    s_orc = oracle.page_scores(np_(q), o_min, o_max, n_pages)
    s_gpu = np_(scores).astype(np.float64)
    bound = _abs_bound(np_(q), o_min, o_max, G)
    for b in range(B):
        n = n_pages[b]
        err = np.abs(s_gpu[b, :, :n] - s_orc[b, :, :n])
        assert (err <= 1e-5 * bound[b, :, :n] + 1e-30).all(), err.max()
    _check_selection(np_(idx), np_(n_sel), s_orc, n_pages, lens, P, C)


@pytest.mark.parametrize("kv", ["bf16", "f32"])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_integer_inputs_are_bit_exact(kv, G):
    B, Hkv, D, T_cap, P, C = 2, 2, 128, 1600, 16, 320
    Hq = Hkv * G
    lens = [1600, 1001]
    k, q, lens_t = _inputs(B, Hq, Hkv, D, T_cap, kv, lens, seed=G, integers=True)
    dims = dims_for(A, B, Hq, Hkv, D, T_cap, kv)
    cfg = A.Cfg(16, C, 1e-2)
    kmin, kmax = _summaries(dims, P, k, lens_t)
    scores = torch.zeros((B, Hkv, A.page_count(T_cap, P)), device=DEV)
    A.asp_page_scores(dims, P, q, kmin, kmax, lens_t, scores)
    idx = torch.empty((B, Hkv, C), dtype=torch.int32, device=DEV)
    n_sel = torch.empty((B, Hkv), dtype=torch.int32, device=DEV)
    A.asp_page_select(dims, cfg, P, q, kmin, kmax, lens_t, idx, n_sel)
    torch.cuda.synchronize()
    o_min, o_max = oracle.page_summary(kv_np(k), lens, P)
    idx_o, n_o, _, _ = oracle.page_select(np_(q), o_min, o_max, lens, P, C)
    n_pages = oracle.page_counts(lens, T_cap, P)
    s_orc = oracle.page_scores(np_(q), o_min, o_max, n_pages)
    for b in range(B):
        np.testing.assert_array_equal(np_(scores)[b, :, : n_pages[b]], s_orc[b, :, : n_pages[b]])
    np.testing.assert_array_equal(np_(idx), idx_o)
    np.testing.assert_array_equal(np_(n_sel), n_o)


def test_one_token_pages_match_the_token_selection():
    # P = 1: each page is one key and its bound is that key's score.
    B, Hq, Hkv, D, T_cap, C = 2, 8, 2, 128, 3000, 300
    lens = [3000, 2222]
    k, q, lens_t = _inputs(B, Hq, Hkv, D, T_cap, "bf16", lens, seed=5)
    dims = dims_for(A, B, Hq, Hkv, D, T_cap, "bf16")
    cfg = A.Cfg(16, C, 1e-2)
    kmin, kmax = _summaries(dims, 1, k, lens_t)
    idx = torch.empty((B, Hkv, C), dtype=torch.int32, device=DEV)
    n_sel = torch.empty((B, Hkv), dtype=torch.int32, device=DEV)
    A.asp_page_select(dims, cfg, 1, q, kmin, kmax, lens_t, idx, n_sel)
    scores = torch.empty((B, Hkv, T_cap), device=DEV)
    A.asp_score_keys(dims, q, k, lens_t, scores)
    idx_t = torch.empty_like(idx)
    n_t = torch.empty_like(n_sel)
    A.asp_select_topc(dims, cfg, scores, lens_t, idx_t, n_t)
    torch.cuda.synchronize()
    for b, T in enumerate(lens):  # one-token pages summarise to the keys themselves
        assert torch.equal(kmin[b, :, :T], k[b, :, :T]) and torch.equal(kmax[b, :, :T], k[b, :, :T])
    # Both routes sum D products in fp32, in different orders: compare each
    # with the oracle's token-level top-C on the fp64 scores.
    s_orc = oracle.score(np_(q), kv_np(k), lens)
    assert_selection_within_gap(np_(idx), np_(n_sel), s_orc, lens, C)
    assert_selection_within_gap(np_(idx_t), np_(n_t), s_orc, lens, C)


@pytest.mark.parametrize("P", [16, 7])
def test_partial_last_page_chosen(P):
    # The last page of each sequence holds a few tokens whose keys stand out,
    # so it is chosen; it must be listed last and only with its valid tokens.
    B, Hq, Hkv, D, T_cap = 2, 8, 2, 128, 1000
    lens = [995, 990]
    C = 10 * P
    k, q, lens_t = _inputs(B, Hq, Hkv, D, T_cap, "bf16", lens, seed=11 + P)
    q = q.abs()
    for b, T in enumerate(lens):
        last = (T - 1) // P * P
        k[b, :, last:T] = 4.0
    dims = dims_for(A, B, Hq, Hkv, D, T_cap, "bf16")
    cfg = A.Cfg(16, C, 1e-2)
    kmin, kmax = _summaries(dims, P, k, lens_t)
    idx = torch.empty((B, Hkv, C), dtype=torch.int32, device=DEV)
    n_sel = torch.empty((B, Hkv), dtype=torch.int32, device=DEV)
    A.asp_page_select(dims, cfg, P, q, kmin, kmax, lens_t, idx, n_sel)
    torch.cuda.synchronize()
    o_min, o_max = oracle.page_summary(kv_np(k), lens, P)
    n_pages = oracle.page_counts(lens, T_cap, P)
    s_orc = oracle.page_scores(np_(q), o_min, o_max, n_pages)
    _check_selection(np_(idx), np_(n_sel), s_orc, n_pages, lens, P, C)
    for b, T in enumerate(lens):
        part = T - (T - 1) // P * P
        for g in range(Hkv):
            n = int(np_(n_sel)[b, g])
            assert n == C - P + part
            np.testing.assert_array_equal(np_(idx)[b, g, n - part:n], np.arange(T - part, T))


def test_page_step_attention_matches_the_oracle():
    # The baseline's decode step: page selection with the current query, then
    # attention with that query over the selected tokens.
    B, Hq, Hkv, D, T_cap, P, C = 3, 16, 4, 128, 4100, 16, 1024
    lens = [4100, 3333, 40]
    k, q, lens_t = _inputs(B, Hq, Hkv, D, T_cap, "bf16", lens, seed=8)
    wl = wk.Q8B_LAYER.replace(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, t_cap=T_cap, seed=9)
    _, v = wk.make_kv(wl, lens_t.cpu())
    v = v.to(DEV)
    dims = dims_for(A, B, Hq, Hkv, D, T_cap, "bf16")
    cfg = A.Cfg(16, C, 1e-2)
    kmin, kmax = _summaries(dims, P, k, lens_t)
    idx = torch.empty((B, Hkv, C), dtype=torch.int32, device=DEV)
    n_sel = torch.empty((B, Hkv), dtype=torch.int32, device=DEV)
    out = torch.empty((B, Hq, D), device=DEV)
    ws = torch.empty(A.asp_workspace_size(dims, cfg, A.OP_DECODE), dtype=torch.uint8, device=DEV)
    A.asp_page_select(dims, cfg, P, q, kmin, kmax, lens_t, idx, n_sel)
    A.asp_sparse_decode(dims, cfg, q, k, v, lens_t, idx, n_sel, out, ws)
    torch.cuda.synchronize()
    o = oracle.attend(np_(q), kv_np(k), kv_np(v), np_(idx), np_(n_sel))
    assert np.abs(np_(out) - o).max() <= 1e-2
    # sequence 2 has 3 pages, fewer than the budget: every token, i.e. dense attention
    assert (np_(n_sel)[2] == 40).all()
    np.testing.assert_array_equal(np_(idx)[2, :, :40], np.tile(np.arange(40), (Hkv, 1)))


def test_empty_batch_enqueues_nothing():
    dims = A.Dims(0, 8, 2, 128, 1000, A.KV_BF16)
    cfg = A.Cfg(16, 160, 1e-2)
    e = torch.empty((0, 2, 1000, 128), dtype=torch.bfloat16, device=DEV)
    s = torch.empty((0, 2, A.page_count(1000, 16), 128), dtype=torch.bfloat16, device=DEV)
    lens = torch.empty((0,), dtype=torch.int32, device=DEV)
    q = torch.empty((0, 8, 128), device=DEV)
    # zero-size tensors have no storage: hand the C ABI placeholder addresses
    ph = torch.empty(64, dtype=torch.uint8, device=DEV)
    lib = A.load()
    p = ctypes.c_void_p(ph.data_ptr())
    assert lib.asp_page_summary(ctypes.byref(dims), 16, p, p, p, p, None) == 0
    assert lib.asp_page_scores(ctypes.byref(dims), 16, p, p, p, p, p, None) == 0
    assert lib.asp_page_select(ctypes.byref(dims), ctypes.byref(cfg), 16, p, p, p, p, p, p, p,
                               A.asp_page_select_workspace_size(dims, cfg, 16) + 256, None) == 0
    torch.cuda.synchronize()
    del e, s, lens, q


def test_qwen3_8b_layer_shape_sampled_units():
    # The bench layer: 8 x 8 units of 32768 bf16 keys, pages of 16, C = 2048.
    wl = wk.Q8B_LAYER
    B, Hq, Hkv, D, T, P, C = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.t_cap, 16, wl.top_c
    lens_t = wk.make_seq_lens(wl)
    k, _ = wk.make_kv(wl, lens_t, device=DEV)
    q = wk.make_queries(wl, 1, device=DEV)[0].contiguous()
    lens_t = lens_t.to(DEV)
    dims = dims_for(A, B, Hq, Hkv, D, T, "bf16")
    cfg = A.Cfg(wl.window, C, wl.lam)
    kmin, kmax = _summaries(dims, P, k, lens_t)
    idx = torch.empty((B, Hkv, C), dtype=torch.int32, device=DEV)
    n_sel = torch.empty((B, Hkv), dtype=torch.int32, device=DEV)
    A.asp_page_select(dims, cfg, P, q, kmin, kmax, lens_t, idx, n_sel)
    torch.cuda.synchronize()
    bs = [0, 5, 7]  # sampled sequences, all their KV heads
    lens = [T] * len(bs)
    k_s = kv_np(k[bs])
    o_min, o_max = oracle.page_summary(k_s, lens, P)
    n_pages = oracle.page_counts(lens, T, P)
    _check_summaries(kmin[bs], kmax[bs], o_min, o_max, n_pages)
    s_orc = oracle.page_scores(np_(q[bs]), o_min, o_max, n_pages)
    _check_selection(np_(idx[bs]), np_(n_sel[bs]), s_orc, n_pages, lens, P, C)
    assert (np_(n_sel) == C).all()
