"""Pins for the oracle's page-level selection, the baseline the pages compare
against (research-map summary, "Problem" and the baselines of "Experimental
setup"; arXiv abstract: Quest's page-level selection with the current query).  The page score is the
criticality estimate Quest publishes (Tang et al., ICML 2024, method section):
each page keeps the element-wise min and max of its keys, and a query scores
the page by the largest value its dot product can take over that box.

The pins: min/max by numpy over page slices, the box maximum by enumerating
every corner, the upper-bound property against the oracle's token scores, the
one-token-page case that must reproduce the token-level selection exactly, and
a small example worked by hand.
"""
import itertools

import numpy as np
import pytest
import torch


def bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_values(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("kv", ["f32", "bf16"])
@pytest.mark.parametrize("P", [1, 4, 16])
def test_summary_is_min_max_of_each_page(orc, kv, P):
    r = np.random.default_rng(P)
    B, Hkv, T_cap, D = 3, 2, 70, 64
    k = r.standard_normal((B, Hkv, T_cap, D)).astype(np.float32)
    lens = np.array([70, 37, 0], np.int32)
    kin = k if kv == "f32" else bf16_bits(k)
    kval = k.astype(np.float64) if kv == "f32" else bf16_values(kin)
    kmin, kmax = orc.page_summary(kin, lens, P)
    NP = (T_cap + P - 1) // P
    assert kmin.shape == (B, Hkv, NP, D)
    for b in range(B):
        for p in range(NP):
            lo, hi = p * P, min(p * P + P, int(lens[b]))
            if lo >= hi:
                assert np.isnan(kmin[b, :, p]).all() and np.isnan(kmax[b, :, p]).all()
                continue
            np.testing.assert_array_equal(kmin[b, :, p], kval[b, :, lo:hi].min(axis=1))
            np.testing.assert_array_equal(kmax[b, :, p], kval[b, :, lo:hi].max(axis=1))


def test_worked_example(orc):
    # q = (1, -2).  Page 0 holds (0, 1) and (2, -1): min (0, -1), max (2, 1),
    # bound max(0, 2) + max(2, -2) = 4, attained by the key (2, -1).
    # Page 1 holds (1, 1) and (-1, 0): min (-1, 0), max (1, 1),
    # bound max(-1, 1) + max(0, -2) = 1, above both keys' -1 and -1.
    k = np.array([[[[0, 1], [2, -1], [1, 1], [-1, 0]]]], np.float32)
    q = np.array([[[1, -2]]], np.float32)
    kmin, kmax = orc.page_summary(k, np.array([4], np.int32), 2)
    np.testing.assert_array_equal(kmin[0, 0], [[0, -1], [-1, 0]])
    np.testing.assert_array_equal(kmax[0, 0], [[2, 1], [1, 1]])
    s = orc.page_scores(q, kmin, kmax, np.array([2], np.int32))
    np.testing.assert_array_equal(s[0, 0], [4.0, 1.0])
    idx, n, pidx, pn = orc.page_select(q, kmin, kmax, np.array([4], np.int32), 2, 2)
    assert pn[0, 0] == 1 and pidx[0, 0, 0] == 0
    np.testing.assert_array_equal(idx[0, 0], [0, 1])
    assert n[0, 0] == 2


@pytest.mark.parametrize("G", [1, 2, 4])
def test_score_is_the_box_maximum_over_every_corner(orc, G):
    r = np.random.default_rng(10 + G)
    B, Hkv, NP, D = 2, 2, 5, 6
    Hq = Hkv * G
    a = r.standard_normal((B, Hkv, NP, D))
    c = r.standard_normal((B, Hkv, NP, D))
    kmin, kmax = np.minimum(a, c), np.maximum(a, c)
    q = r.standard_normal((B, Hq, D)).astype(np.float32)
    n_pages = np.array([5, 3], np.int32)
    s = orc.page_scores(q, kmin, kmax, n_pages)
    corners = np.array(list(itertools.product([0, 1], repeat=D)), bool)  # 64 corners
    for b in range(B):
        for g in range(Hkv):
            for p in range(NP):
                if p >= n_pages[b]:
                    assert np.isnan(s[b, g, p])
                    continue
                pts = np.where(corners, kmax[b, g, p], kmin[b, g, p])  # [64][D]
                qs = q[b, g * G:(g + 1) * G].astype(np.float64)  # [G][D]
                best = (qs @ pts.T).max()
                assert s[b, g, p] == pytest.approx(best, rel=1e-13, abs=1e-13)


@pytest.mark.parametrize("P", [2, 8, 16])
def test_page_score_bounds_every_token_score(orc, P):
    r = np.random.default_rng(20 + P)
    B, Hq, Hkv, T_cap, D = 2, 8, 2, 96, 64
    k = bf16_bits(r.standard_normal((B, Hkv, T_cap, D)).astype(np.float32) * 2)
    q = r.standard_normal((B, Hq, D)).astype(np.float32)
    lens = np.array([96, 45], np.int32)
    kmin, kmax = orc.page_summary(k, lens, P)
    ps = orc.page_scores(q, kmin, kmax, orc.page_counts(lens, T_cap, P))
    ts = orc.score(q, k, lens)
    for b in range(B):
        T = int(lens[b])
        page_of = np.arange(T) // P
        assert (ts[b, :, :T] <= ps[b][:, page_of] + 1e-9).all()
        # A page's bound is never below its best token.
        for p in range((T + P - 1) // P):
            assert (ps[b, :, p] >= ts[b, :, p * P:min(p * P + P, T)].max(axis=1) - 1e-9).all()


@pytest.mark.parametrize("kv", ["f32", "bf16"])
def test_one_token_pages_reproduce_the_token_selection(orc, kv):
    # With P = 1 each page's box is a single key, the bound is that key's
    # score, and the page selection is the token-level top-C.
    r = np.random.default_rng(3)
    B, Hq, Hkv, T_cap, D, C = 3, 8, 2, 300, 64, 40
    k = r.standard_normal((B, Hkv, T_cap, D)).astype(np.float32)
    kin = k if kv == "f32" else bf16_bits(k)
    q = r.standard_normal((B, Hq, D)).astype(np.float32)
    lens = np.array([300, 129, 17], np.int32)
    kmin, kmax = orc.page_summary(kin, lens, 1)
    ps = orc.page_scores(q, kmin, kmax, lens)
    ts = orc.score(q, kin, lens)
    np.testing.assert_array_equal(ps, ts)  # NaN past each length on both
    idx, n, _, _ = orc.page_select(q, kmin, kmax, lens, 1, C)
    idx_t, n_t = orc.select(ts, lens, C)
    np.testing.assert_array_equal(idx, idx_t)
    np.testing.assert_array_equal(n, n_t)


def test_selected_pages_rank_above_the_rest_and_expand_to_their_tokens(orc):
    r = np.random.default_rng(4)
    B, Hq, Hkv, T_cap, D, P, C = 3, 4, 2, 200, 64, 8, 48  # 6 pages of 8
    k = bf16_bits(r.standard_normal((B, Hkv, T_cap, D)).astype(np.float32))
    q = r.standard_normal((B, Hq, D)).astype(np.float32)
    lens = np.array([200, 101, 20], np.int32)  # 25, 13 (last holds 5) and 3 pages
    kmin, kmax = orc.page_summary(k, lens, P)
    n_pages = orc.page_counts(lens, T_cap, P)
    np.testing.assert_array_equal(n_pages, [25, 13, 3])
    ps = orc.page_scores(q, kmin, kmax, n_pages)
    idx, n, pidx, pn = orc.page_select(q, kmin, kmax, lens, P, C)
    for b in range(B):
        for g in range(Hkv):
            K = min(C // P, int(n_pages[b]))
            assert pn[b, g] == K
            chosen = pidx[b, g, :K]
            assert (np.diff(chosen) > 0).all()
            rest = np.setdiff1d(np.arange(n_pages[b]), chosen)
            if len(rest):
                assert ps[b, g, chosen].min() >= ps[b, g, rest].max()
            toks = np.concatenate([np.arange(p * P, min(p * P + P, int(lens[b]))) for p in chosen])
            assert n[b, g] == len(toks)
            np.testing.assert_array_equal(idx[b, g, :len(toks)], toks)
            assert (idx[b, g, len(toks):] == -1).all()
    # Sequence 2 has fewer pages than the budget: every token is selected.
    np.testing.assert_array_equal(idx[2, 0, :20], np.arange(20))


def test_equal_page_scores_take_the_lowest_pages(orc):
    # q = 0 scores every page 0; ties go to the lower page index.
    B, Hq, Hkv, T_cap, D, P, C = 1, 2, 1, 64, 64, 4, 12
    k = np.random.default_rng(5).standard_normal((B, Hkv, T_cap, D)).astype(np.float32)
    q = np.zeros((B, Hq, D), np.float32)
    lens = np.array([64], np.int32)
    kmin, kmax = orc.page_summary(k, lens, P)
    idx, n, pidx, pn = orc.page_select(q, kmin, kmax, lens, P, C)
    np.testing.assert_array_equal(pidx[0, 0, :3], [0, 1, 2])
    np.testing.assert_array_equal(idx[0, 0], np.arange(12))
