"""Pins for the oracle's key scoring and top-C selection (runs on the CPU).

Scoring: token-level scoring of every cached key against the predicted query
(AsyncSpade research-map summary, "Approach"; arXiv abstract).  Selection:
the C best tokens per (sequence, KV head) (reproduction card, "Key finding";
summary, "Key results").  The pins are exact integer arithmetic for the score
and a rank-counting brute force for the selection, which never sorts.
"""
import itertools

import numpy as np
import pytest
import torch


def bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("kv", ["f32", "bf16"])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_score_is_exact_on_small_integers(orc, kv, G):
    # Values in {-3..3} are exact in bf16 and fp32; the exact score is an
    # integer max over the group of integer dot products.
    r = np.random.default_rng(G)
    B, Hkv, T, D = 2, 2, 37, 64
    Hq = Hkv * G
    q = r.integers(-3, 4, (B, Hq, D)).astype(np.float32)
    k = r.integers(-3, 4, (B, Hkv, T, D)).astype(np.float32)
    lens = np.array([T, 29], np.int32)
    kin = k if kv == "f32" else bf16_bits(k)
    s = orc.score(q, kin, lens)
    qi = q.astype(np.int64).reshape(B, Hkv, G, D)
    ki = k.astype(np.int64)
    exact = np.einsum("bgtd,bghd->bght", ki, qi).max(axis=2)  # [B][Hkv][T]
    for b in range(B):
        np.testing.assert_array_equal(s[b, :, : lens[b]], exact[b, :, : lens[b]])
        assert np.isnan(s[b, :, lens[b]:]).all()


def test_score_decodes_bf16_bit_patterns(orc):
    # bf16 0x3F80 = 1, 0xC040 = -3, 0x3F81 = 1 + 2^-7, 0x0001 = 2^-133 (subnormal).
    D = 64
    q = np.zeros((1, 1, D), np.float32)
    q[0, 0, :4] = [1.0, 2.0, 4.0, 2.0 ** 100]
    k = np.zeros((1, 1, 1, D), np.uint16)
    k[0, 0, 0, :4] = [0x3F80, 0xC040, 0x3F81, 0x0001]
    s = orc.score(q, k, np.array([1], np.int32))
    assert s[0, 0, 0] == 1.0 - 6.0 + 4.0 * (1 + 2.0 ** -7) + 2.0 ** -33


def test_score_uses_group_max_not_sum(orc):
    # Two heads share a KV head; each key is aligned with exactly one head.
    D = 64
    q = np.zeros((1, 2, D), np.float32)
    q[0, 0, 0] = 1.0
    q[0, 1, 1] = 1.0
    k = np.zeros((1, 1, 3, D), np.float32)
    k[0, 0, 0, 0] = 5.0   # head 0 sees 5, head 1 sees 0
    k[0, 0, 1, 1] = 7.0   # head 1 sees 7
    k[0, 0, 2, :2] = -2.0  # both heads see -2
    s = orc.score(q, k, np.array([3], np.int32))
    np.testing.assert_array_equal(s[0, 0], [5.0, 7.0, -2.0])


def test_empty_sequence_scores_nothing(orc):
    q = np.ones((2, 1, 64), np.float32)
    k = np.ones((2, 1, 8, 64), np.float32)
    s = orc.score(q, k, np.array([0, 8], np.int32))
    assert np.isnan(s[0]).all() and (s[1] == 64.0).all()


# ---------------------------------------------------------------- selection


def brute_select(vals, T, C):
    """Rank counting: token i is kept iff fewer than C_eff tokens beat it, where
    j beats i when v_j > v_i, or v_j == v_i and j < i (NaN counts as -inf)."""
    v = [(-np.inf if np.isnan(x) else float(x)) for x in vals[:T]]
    c_eff = min(C, T)
    keep = []
    for i in range(T):
        beats = sum(1 for j in range(T) if v[j] > v[i] or (v[j] == v[i] and j < i))
        if beats < c_eff:
            keep.append(i)
    return keep


SPECIAL = [-1.0, 0.0, -0.0, 1.0, np.nan, np.inf, -np.inf]


@pytest.mark.parametrize("C", [1, 2, 3, 4, 5])
def test_select_exhaustive_special_values(orc, C):
    # Every array of length 4 over {-1, 0, -0, 1, NaN, +inf, -inf}, each also
    # truncated to lengths 0..4 through the per-sequence length.
    T_cap = 4
    rows = np.array(list(itertools.product(SPECIAL, repeat=T_cap)), np.float64)
    n = len(rows)
    lens = np.arange(n, dtype=np.int32) % (T_cap + 1)
    idx, n_sel = orc.select(rows.reshape(n, 1, T_cap), lens, C)
    for r in range(n):
        keep = brute_select(rows[r], int(lens[r]), C)
        assert n_sel[r, 0] == len(keep)
        assert list(idx[r, 0, : len(keep)]) == keep
        assert (idx[r, 0, len(keep):] == -1).all()


def test_select_random_ties_against_brute_force(orc):
    r = np.random.default_rng(41)
    for trial in range(200):
        T = int(r.integers(1, 40))
        C = int(r.integers(1, 45))
        pool = r.choice([-2.5, -1.0, 0.0, -0.0, 0.5, 3.0, np.nan], size=int(r.integers(1, 7)), replace=False)
        vals = r.choice(pool, size=T)
        idx, n_sel = orc.select(vals.reshape(1, 1, T), np.array([T], np.int32), C)
        keep = brute_select(vals, T, C)
        assert list(idx[0, 0, : n_sel[0, 0]]) == keep, (trial, vals, C)


def test_select_large_row_invariants(orc):
    # T = 4096 normal scores with forced ties around the threshold.
    r = np.random.default_rng(43)
    T, C = 4096, 300
    vals = np.round(r.standard_normal(T), 1)       # many exact ties
    idx, n_sel = orc.select(vals.reshape(1, 1, T), np.array([T], np.int32), C)
    sel = idx[0, 0, : n_sel[0, 0]]
    assert n_sel[0, 0] == C and (np.diff(sel) > 0).all()
    # vectorised rank counting
    vi = vals[:, None]
    vj = vals[None, :]
    j_lt_i = np.arange(T)[None, :] < np.arange(T)[:, None]
    beats = ((vj > vi) | ((vj == vi) & j_lt_i)).sum(axis=1)
    np.testing.assert_array_equal(sel, np.nonzero(beats < C)[0])
    thr = vals[sel].min()
    unsel = np.setdiff1d(np.arange(T), sel)
    assert vals[unsel].max() <= thr
    tied = np.nonzero(vals == thr)[0]              # ties taken in index order
    taken = np.intersect1d(tied, sel)
    np.testing.assert_array_equal(taken, tied[: len(taken)])


def test_select_special_cases(orc):
    T_cap, C = 50, 8
    eq = np.full((1, 1, T_cap), 0.25)
    idx, n_sel = orc.select(eq, np.array([T_cap], np.int32), C)
    np.testing.assert_array_equal(idx[0, 0], np.arange(C))
    short = np.random.default_rng(0).standard_normal((1, 1, T_cap))
    idx, n_sel = orc.select(short, np.array([5], np.int32), C)   # T < C: all of them
    np.testing.assert_array_equal(idx[0, 0], [0, 1, 2, 3, 4, -1, -1, -1])
    assert n_sel[0, 0] == 5
    idx, n_sel = orc.select(short, np.array([0], np.int32), C)   # empty
    assert n_sel[0, 0] == 0 and (idx == -1).all()
