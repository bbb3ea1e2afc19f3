"""Per-kernel parity of the HIP library against the CPU oracle (GPU required).

Each test hands the oracle the exact bytes the GPU consumed and compares
element by element:
  * ring push: bit-exact;
  * predictor: max-abs error within 1e-4 of max|q_pred| per (sequence, head);
  * scores: bit-exact on small-integer inputs, else within 1e-5 * max|score|;
    the optional coarse histograms count the GPU's own scores exactly;
  * selection: bit-exact index sets on identical fp32 scores;
  * attention: max-abs error 1e-2 on the same index set (fp32 accumulation of
    bf16 inputs; observed errors are ~1e-6), also with the newest-token window.
Sizes span several workgroup tiles and a ragged tail.
"""
import numpy as np
import pytest
import torch

import oracle
import query_aware_sparse_amd as A
from query_aware_sparse_amd import workload as wk
from asp_testutil import assert_pred_close, dims_for, kv_np, np_, require_gpu

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()
    print("\n[case]", flush=True)


def _history(B, Hq, W, D, n_push, seed, start_newest=None):
    """Push n_push AR(1)-like queries through both the GPU ring and the oracle ring."""
    cfgW = A.Cfg(W, 1, 1e-2)
    dims = A.Dims(B, Hq, Hq, D, 1, A.KV_F32)
    q_hist = torch.zeros((B, Hq, W, D), dtype=torch.float32)
    newest = torch.full((B,), W - 1, dtype=torch.int32) if start_newest is None else start_newest.clone()
    length = torch.zeros((B,), dtype=torch.int32)
    seq = wk.randn((max(n_push, 1), B, Hq, D), seed=seed) * 0.7
    gh, gn, gl = q_hist.to(DEV), newest.to(DEV), length.to(DEV)
    oh, on, ol = q_hist.numpy(), newest.numpy(), length.numpy()
    for t in range(n_push):
        q = seq[t].to(DEV)
        A.asp_push_query(dims, cfgW, q, gh, gn, gl)
        oh, on, ol = oracle.push(seq[t].numpy(), oh, on, ol)
    torch.cuda.synchronize()
    return gh, gn, gl, oh, on, ol


def test_push_ring_is_bit_exact():
    B, Hq, W, D = 3, 8, 8, 128
    gh, gn, gl, oh, on, ol = _history(B, Hq, W, D, 19, seed=1)
    np.testing.assert_array_equal(np_(gh), oh)
    np.testing.assert_array_equal(np_(gn), on)
    np.testing.assert_array_equal(np_(gl), ol)


@pytest.mark.parametrize("W", [4, 8, 16, 32, 64])
@pytest.mark.parametrize("D", [64, 128])
def test_predict_matches_oracle(W, D):
    B, Hq = 2, 4
    for n_push in sorted({0, 1, 2, 3, W // 4, W // 2, W - 1, W, W + 3}):
        gh, gn, gl, oh, on, ol = _history(B, Hq, W, D, n_push, seed=100 + n_push)
        lam = 1e-2
        dims = A.Dims(B, Hq, Hq, D, 1, A.KV_F32)
        cfg = A.Cfg(W, 1, lam)
        q_pred = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
        A.asp_predict_query(dims, cfg, gh, gn, gl, q_pred)
        torch.cuda.synchronize()
        ref = oracle.predict(oh, on, ol, lam)
        assert_pred_close(np_(q_pred), ref)


def test_predict_tiny_workload_walk():
    # The tiny workload: 64 AR(1) queries through an 8-slot ring, checked at every step.
    wl = wk.TINY
    qs = wk.make_queries(wl, wl.history_steps)
    dims = A.Dims(wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.t_cap, A.KV_F32)
    cfg = A.Cfg(wl.window, wl.top_c, wl.lam)
    gh, gn, gl = [x.to(DEV) for x in wk.empty_history(wl)]
    oh, on, ol = [x.numpy() for x in wk.empty_history(wl)]
    q_pred = torch.empty((wl.batch, wl.n_q_heads, wl.head_dim), dtype=torch.float32, device=DEV)
    for t in range(wl.history_steps):
        A.asp_push_query(dims, cfg, qs[t].to(DEV), gh, gn, gl)
        A.asp_predict_query(dims, cfg, gh, gn, gl, q_pred)
        oh, on, ol = oracle.push(qs[t].numpy(), oh, on, ol)
        assert_pred_close(np_(q_pred), oracle.predict(oh, on, ol, wl.lam))


def _score_inputs(B, Hq, Hkv, D, T_cap, kv, integer, seed):
    G = Hq // Hkv
    if integer:
        q = torch.randint(-3, 4, (B, Hq, D), generator=torch.Generator().manual_seed(seed)).float()
        k = torch.randint(-3, 4, (B, Hkv, T_cap, D), generator=torch.Generator().manual_seed(seed + 1)).float()
    else:
        q = wk.randn((B, Hq, D), seed=seed)
        k = wk.randn((B, Hkv, T_cap, D), seed=seed, sub=1)
    k = k.to(torch.bfloat16 if kv == "bf16" else torch.float32)
    return q, k


@pytest.mark.parametrize("kv", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_score_integer_inputs_bit_exact(kv, D, G):
    B, Hkv, T_cap = 3, 2, 4500          # 3 key blocks with a ragged tail
    Hq = G * Hkv
    q, k = _score_inputs(B, Hq, Hkv, D, T_cap, kv, True, seed=G * 10 + D)
    lens = torch.tensor([T_cap, 2049, 0], dtype=torch.int32)
    dims = dims_for(A, B, Hq, Hkv, D, T_cap, kv)
    scores = torch.full((B, Hkv, T_cap), -7.0, dtype=torch.float32, device=DEV)
    A.asp_score_keys(dims, q.to(DEV), k.to(DEV), lens.to(DEV), scores)
    got = np_(scores)
    ref = oracle.score(q.numpy(), kv_np(k), lens.numpy())
    for b in range(B):
        T = int(lens[b])
        np.testing.assert_array_equal(got[b, :, :T], ref[b, :, :T])
        assert (got[b, :, T:] == -7.0).all()   # past the length: untouched


@pytest.mark.parametrize("kv", ["bf16", "f32"])
@pytest.mark.parametrize("G", [4, 8])
def test_score_random_inputs_within_tolerance(kv, G):
    B, Hkv, D, T_cap = 2, 4, 128, 6001
    Hq = G * Hkv
    q, k = _score_inputs(B, Hq, Hkv, D, T_cap, kv, False, seed=7)
    lens = torch.tensor([T_cap, 5000], dtype=torch.int32)
    dims = dims_for(A, B, Hq, Hkv, D, T_cap, kv)
    scores = torch.empty((B, Hkv, T_cap), dtype=torch.float32, device=DEV)
    A.asp_score_keys(dims, q.to(DEV), k.to(DEV), lens.to(DEV), scores)
    got = np_(scores).astype(np.float64)
    ref = oracle.score(q.numpy(), kv_np(k), lens.numpy())
    for b in range(B):
        T = int(lens[b])
        for g in range(Hkv):
            err = np.abs(got[b, g, :T] - ref[b, g, :T]).max()
            assert err <= 1e-5 * np.abs(ref[b, g, :T]).max(), (b, g, err)


def _coarse_bins(scores: np.ndarray) -> np.ndarray:
    """Top 11 bits of the order key of fp32 scores: NaN ranks as -inf, -0 as +0,
    negative values reversed below the positive ones (the selection's ranking)."""
    u = scores.astype(np.float32).view(np.uint32).copy()
    u[np.isnan(scores)] = np.uint32(0xFF800000)
    u[u == np.uint32(0x80000000)] = np.uint32(0)
    key = np.where(u >> 31, ~u, u | np.uint32(0x80000000)).astype(np.uint32)
    return (key >> 21).astype(np.int64)


@pytest.mark.parametrize("kv,G", [("bf16", 4), ("bf16", 8), ("f32", 2)])
def test_score_histogram_counts_the_gpu_scores(kv, G):
    B, Hkv, D, T_cap = 3, 2, 128, 5003
    Hq = G * Hkv
    q, k = _score_inputs(B, Hq, Hkv, D, T_cap, kv, False, seed=11 + G)
    lens = torch.tensor([T_cap, 1777, 0], dtype=torch.int32)
    dims = dims_for(A, B, Hq, Hkv, D, T_cap, kv)
    s_plain = torch.empty((B, Hkv, T_cap), dtype=torch.float32, device=DEV)
    s_hist = torch.empty_like(s_plain)
    hist = torch.full((B, Hkv, A.HIST_BINS), 12345, dtype=torch.int32, device=DEV)  # overwritten
    A.asp_score_keys(dims, q.to(DEV), k.to(DEV), lens.to(DEV), s_plain)
    A.asp_score_keys(dims, q.to(DEV), k.to(DEV), lens.to(DEV), s_hist, hist=hist)
    got, h = np_(s_hist), np_(hist)
    for b in range(B):
        T = int(lens[b])
        np.testing.assert_array_equal(got[b, :, :T], np_(s_plain)[b, :, :T])  # same arithmetic
        for g in range(Hkv):
            ref = np.bincount(_coarse_bins(got[b, g, :T]), minlength=A.HIST_BINS)
            np.testing.assert_array_equal(h[b, g], ref)


def test_select_with_the_score_histogram():
    B, Hkv, G, D, T_cap, C = 3, 2, 4, 128, 33000, 2048
    q, k = _score_inputs(B, G * Hkv, Hkv, D, T_cap, "bf16", False, seed=21)
    lens = torch.tensor([T_cap, 20001, 1500], dtype=torch.int32, device=DEV)
    dims = dims_for(A, B, G * Hkv, Hkv, D, T_cap, "bf16")
    cfg = A.Cfg(16, C, 1e-2)
    scores = torch.empty((B, Hkv, T_cap), dtype=torch.float32, device=DEV)
    hist = torch.empty((B, Hkv, A.HIST_BINS), dtype=torch.int32, device=DEV)
    A.asp_score_keys(dims, q.to(DEV), k.to(DEV), lens, scores, hist=hist)
    out = []
    for h in (hist, None):
        idx = torch.full((B, Hkv, C), -9, dtype=torch.int32, device=DEV)
        n_sel = torch.full((B, Hkv), -9, dtype=torch.int32, device=DEV)
        A.asp_select_topc(dims, cfg, scores, lens, idx, n_sel, hist=h)
        out.append((np_(idx), np_(n_sel)))
    ri, rn = oracle.select(np_(scores), np_(lens), C)
    for idx, n_sel in out:
        np.testing.assert_array_equal(n_sel, rn)
        np.testing.assert_array_equal(idx, ri)


def _select_case(B, Hkv, T_cap, lens, C, seed, kind):
    r = np.random.default_rng(seed)
    if kind == "normal":
        s = r.standard_normal((B, Hkv, T_cap)).astype(np.float32) * 10
    elif kind == "ties":
        s = r.choice(np.array([-1.5, -0.0, 0.0, 0.25, 2.0, 7.0, np.nan, np.inf, -np.inf], np.float32),
                     size=(B, Hkv, T_cap))
    elif kind == "quantized":   # many exact ties deep in the mantissa
        s = (np.round(r.standard_normal((B, Hkv, T_cap)) * 64) / 64).astype(np.float32)
    else:
        raise ValueError(kind)
    dims = A.Dims(B, Hkv, Hkv, 64, T_cap, A.KV_F32)
    cfg = A.Cfg(8, C, 1e-2)
    gs = torch.from_numpy(s).to(DEV)
    gl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    idx = torch.full((B, Hkv, C), -9, dtype=torch.int32, device=DEV)
    n_sel = torch.full((B, Hkv), -9, dtype=torch.int32, device=DEV)
    A.asp_select_topc(dims, cfg, gs, gl, idx, n_sel)
    ridx, rn = oracle.select(s, np.array(lens, np.int32), C)
    np.testing.assert_array_equal(np_(n_sel), rn)
    np.testing.assert_array_equal(np_(idx), ridx)


@pytest.mark.parametrize("kind", ["normal", "ties", "quantized"])
def test_select_bit_exact_small_rows(kind):
    lens = [1000, 999, 64, 63, 1, 0, 700, 1000]
    _select_case(len(lens), 2, 1000, lens, 64, seed=3, kind=kind)


@pytest.mark.parametrize("kind", ["normal", "quantized", "ties"])
def test_select_bit_exact_32k_rows(kind):
    lens = [32768, 32767, 20000, 2048, 2047]
    _select_case(len(lens), 2, 32768, lens, 2048, seed=5, kind=kind)


@pytest.mark.parametrize("T_cap", [4097, 4098, 4099, 4100])
def test_select_bit_exact_any_row_stride(T_cap):
    # Row strides that are not a multiple of 4 floats: only some rows are
    # 16-byte aligned, and the last row ends at the end of the buffer.
    lens = [T_cap, T_cap - 1, 3001, T_cap]
    _select_case(len(lens), 3, T_cap, lens, 700, seed=T_cap, kind="quantized")


@pytest.mark.parametrize("kind", ["normal", "quantized"])
def test_select_bit_exact_rows_longer_than_lds(kind):
    lens = [131072, 70001, 32769, 8192]
    _select_case(len(lens), 1, 131072, lens, 4096, seed=9, kind=kind)


def test_select_all_equal_and_c_equals_t():
    B, T_cap = 2, 5000
    s = np.full((B, 1, T_cap), 3.0, np.float32)
    dims = A.Dims(B, 1, 1, 64, T_cap, A.KV_F32)
    for C in (1, 777, T_cap):
        cfg = A.Cfg(8, C, 1e-2)
        idx = torch.empty((B, 1, C), dtype=torch.int32, device=DEV)
        n_sel = torch.empty((B, 1), dtype=torch.int32, device=DEV)
        lens = torch.tensor([T_cap, 10], dtype=torch.int32, device=DEV)
        A.asp_select_topc(dims, cfg, torch.from_numpy(s).to(DEV), lens, idx, n_sel)
        ri, rn = oracle.select(s, np.array([T_cap, 10], np.int32), C)
        np.testing.assert_array_equal(np_(idx), ri)
        np.testing.assert_array_equal(np_(n_sel), rn)


def _attend_case(B, Hkv, G, D, T_cap, C, kv, n_sels, seed, sorted_idx=True, recent=0, lens=None):
    Hq = Hkv * G
    q = wk.randn((B, Hq, D), seed=seed)
    k = (wk.randn((B, Hkv, T_cap, D), seed=seed, sub=1) * 2).to(torch.bfloat16 if kv == "bf16" else torch.float32)
    v = wk.randn((B, Hkv, T_cap, D), seed=seed, sub=2).to(k.dtype)
    r = np.random.default_rng(seed)
    idx = np.full((B, Hkv, C), -1, np.int32)
    n_sel = np.zeros((B, Hkv), np.int32)
    for b in range(B):
        for g in range(Hkv):
            n = n_sels[(b * Hkv + g) % len(n_sels)]
            sel = r.choice(T_cap, n, replace=False)
            idx[b, g, :n] = np.sort(sel) if sorted_idx else sel
            n_sel[b, g] = n
    dims = dims_for(A, B, Hq, Hkv, D, T_cap, kv)
    cfg = A.Cfg(8, C, 1e-2, recent)
    ws = torch.empty(A.asp_workspace_size(dims, cfg, A.OP_DECODE), dtype=torch.uint8, device=DEV)
    out = torch.full((B, Hq, D), 99.0, dtype=torch.float32, device=DEV)
    glens = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    A.asp_sparse_decode(dims, cfg, q.to(DEV), k.to(DEV), v.to(DEV), glens, torch.from_numpy(idx).to(DEV),
                        torch.from_numpy(n_sel).to(DEV), out, ws)
    if recent:
        ref = oracle.attend_with_recent(q.numpy(), kv_np(k), kv_np(v), idx, n_sel, np.array(lens, np.int32), recent)
    else:
        ref = oracle.attend(q.numpy(), kv_np(k), kv_np(v), idx, n_sel)
    err = np.abs(np_(out).astype(np.float64) - ref).max()
    assert err <= 1e-2, err
    return err


@pytest.mark.parametrize("kv", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_attend_matches_oracle(kv, D, G):
    err = _attend_case(2, 2, G, D, 3000, 700, kv, [700, 513, 1, 0], seed=G + D)
    assert err < 1e-4


@pytest.mark.parametrize("kv,G,D", [("bf16", 4, 128), ("f32", 2, 64), ("bf16", 8, 64)])
@pytest.mark.parametrize("recent", [1, 100, 700])
def test_attend_with_the_newest_tokens(kv, G, D, recent):
    # Selections drawn over the whole cache overlap the recent window; lengths
    # include an empty sequence and ones shorter than the window.
    lens = [3000, 1000, 60, 0]
    err = _attend_case(4, 2, G, D, 3000, 300, kv, [300, 0, 17, 1], seed=recent + G, recent=recent, lens=lens)
    assert err < 1e-4


def test_attend_dense_case_and_unsorted_indices():
    # C = T: every token selected (dense decode attention); order of idx irrelevant.
    _attend_case(1, 2, 4, 128, 1024, 1024, "bf16", [1024], seed=31)
    _attend_case(1, 2, 4, 128, 1024, 1024, "bf16", [1024], seed=31, sorted_idx=False)


@pytest.mark.parametrize("G,D", [(4, 128), (8, 128), (2, 64)])
def test_attend_many_units_one_split(G, D):
    # 256 units: the bf16 attention runs one block per unit, which writes the
    # normalised output itself (no partials, no merge launch); lists of every
    # length from empty to full, and a list that ends inside a chunk.
    err = _attend_case(32, 8, G, D, 2048, 512, "bf16", [512, 0, 1, 31, 33, 300, 511], seed=7 + G + D)
    assert err < 1e-4


def test_attend_split_boundaries():
    # 64 units at C = 2048 (four splits of 512 positions) with lists that end
    # exactly on and just past a split and a chunk boundary.
    err = _attend_case(8, 8, 4, 128, 4096, 2048, "bf16", [2048, 512, 513, 1536, 1537, 32, 33, 0], seed=5)
    assert err < 1e-4


@pytest.mark.parametrize("kv", ["bf16", "f32"])
def test_nonfinite_keys_leave_finite_rows_exact_and_selection_well_formed(kv):
    # Keys must be finite (asp.h).  Rows holding +-inf or NaN elements get
    # unspecified scores, but every finite row still scores exactly (integer
    # inputs), and both selection routes still give C_eff distinct ascending
    # in-range indices; the candidate route equals the score-row route on the
    # GPU's own scores.
    B, Hkv, G, D, T_cap, C = 2, 2, 4, 128, 3000, 700
    Hq = G * Hkv
    q, k = _score_inputs(B, Hq, Hkv, D, T_cap, kv, True, seed=33)
    bad = {(0, 0, 5): np.inf, (0, 1, 17): -np.inf, (1, 0, 2999): np.nan, (1, 1, 0): np.inf, (0, 0, 2048): np.nan}
    kf = k.float()
    for (b, g, i), val in bad.items():
        kf[b, g, i, (i * 7) % D] = val
    k = kf.to(k.dtype)
    lens = torch.tensor([T_cap, T_cap], dtype=torch.int32)
    dims = dims_for(A, B, Hq, Hkv, D, T_cap, kv)
    cfg = A.Cfg(8, C, 1e-2)
    gq, gk, gl = q.to(DEV), k.to(DEV), lens.to(DEV)
    scores = torch.empty((B, Hkv, T_cap), dtype=torch.float32, device=DEV)
    A.asp_score_keys(dims, gq, gk, gl, scores)
    got = np_(scores)
    ref = oracle.score(q.numpy(), kv_np(k), lens.numpy())
    finite = np.isfinite(k.float().numpy()).all(axis=3)
    np.testing.assert_array_equal(got[finite], ref[finite])
    idx_rows = torch.empty((B, Hkv, C), dtype=torch.int32, device=DEV)
    n_rows = torch.empty((B, Hkv), dtype=torch.int32, device=DEV)
    A.asp_select_topc(dims, cfg, scores, gl, idx_rows, n_rows)
    ws = torch.zeros(A.asp_workspace_size(dims, cfg, A.OP_CANDIDATES), dtype=torch.uint8, device=DEV)
    idx_c = torch.empty_like(idx_rows)
    n_c = torch.empty_like(n_rows)
    A.asp_score_candidates(dims, cfg, gq, gk, gl, ws)
    A.asp_select_candidates(dims, cfg, gq, gk, gl, idx_c, n_c, ws)
    torch.cuda.synchronize()
    ri, rn = oracle.select(got, lens.numpy(), C)  # bit-exact on the GPU's own scores, non-finite ones included
    for i_, n_ in ((np_(idx_rows), np_(n_rows)), (np_(idx_c), np_(n_c))):
        np.testing.assert_array_equal(i_, ri)
        np.testing.assert_array_equal(n_, rn)
        for b in range(B):
            for g in range(Hkv):
                sel = i_[b, g, :C]
                assert n_[b, g] == C and (np.diff(sel) > 0).all() and sel[0] >= 0 and sel[-1] < T_cap
