"""Pins for the oracle's next-query predictor (runs on the CPU).

The pages give the predictor's ingredients (a short window of recent queries,
ridge regression, softmax-normalised weights, multi-window average pooling:
AsyncSpade research-map summary, "Approach"; arXiv abstract) but print no
equations and no worked example.  These tests therefore pin the oracle's
reading with facts that follow from the mathematics rather than from the
oracle's own code: a second least-squares route, closed forms, limits,
symmetries and hand-worked fixtures under tests/golden/.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def ar1_lags(n, D, seed, a=0.9, sigma=0.3):
    """n AR(1) queries returned newest-first (row j = q_{t-j})."""
    r = np.random.default_rng(seed)
    q = np.empty((n, D))
    q[0] = r.standard_normal(D) * sigma / math.sqrt(1 - a * a)
    for s in range(1, n):
        q[s] = a * q[s - 1] + sigma * r.standard_normal(D)
    return q[::-1].copy()


def test_window_of_two_returns_newest_query(orc):
    # One lag (p = 1): beta = <q_t, q_{t-1}> / (|q_{t-1}|^2 + lambda), softmax of
    # one value is 1, so the one-step-ahead prediction is q_t itself.
    lags = np.random.default_rng(1).standard_normal((2, 24))
    lam = 0.37
    q, wins, betas, alphas = orc.predict_one(lags, W=4, lam=lam)
    assert wins == [2]
    expect = lags[0] @ lags[1] / (lags[1] @ lags[1] + lam)
    assert betas[0][0] == pytest.approx(expect, rel=1e-14)
    assert alphas[0][0] == 1.0
    np.testing.assert_array_equal(q, lags[0])


@pytest.mark.parametrize("lam", [0.3, 1e-2])
@pytest.mark.parametrize("seed", [0, 1])
def test_ridge_coefficients_match_augmented_least_squares(orc, lam, seed):
    # Ridge regression is ordinary least squares on the system augmented with
    # sqrt(lambda) I; numpy's SVD-based lstsq is an independent route.
    W, D = 16, 64
    lags = ar1_lags(W, D, seed)
    _, wins, betas, _ = orc.predict_one(lags, W=W, lam=lam)
    assert wins == [16, 8, 4]
    for w, beta in zip(wins, betas):
        p = w - 1
        X = lags[1:p + 1].T                       # D x p: lag j in column j-1
        A = np.vstack([X, math.sqrt(lam) * np.eye(p)])
        y = np.concatenate([lags[0], np.zeros(p)])
        ref = np.linalg.lstsq(A, y, rcond=None)[0]
        np.testing.assert_allclose(beta, ref, rtol=1e-7, atol=1e-9 * np.abs(ref).max())


def test_huge_lambda_reduces_to_average_pooling(orc):
    # lambda -> infinity drives beta -> 0, the softmax becomes uniform, and each
    # window predicts the plain mean of q_t .. q_{t-w+2}; pooling averages those.
    W, D = 16, 32
    lags = ar1_lags(W, D, 7)
    q, wins, _, alphas = orc.predict_one(lags, W=W, lam=1e30)
    assert wins == [16, 8, 4]
    for w, a in zip(wins, alphas):
        np.testing.assert_allclose(a, np.full(w - 1, 1.0 / (w - 1)), rtol=1e-12)
    expect = np.mean([lags[: w - 1].mean(axis=0) for w in wins], axis=0)
    np.testing.assert_allclose(q, expect, rtol=1e-12, atol=1e-15)


def test_constant_history_predicts_the_constant(orc):
    c = np.random.default_rng(3).standard_normal(48)
    lags = np.tile(c, (8, 1))
    q, wins, betas, _ = orc.predict_one(lags, W=8, lam=0.05)
    assert wins == [8, 4, 2]
    for beta in betas:  # symmetric system: all lag coefficients equal
        np.testing.assert_allclose(beta, np.full_like(beta, beta[0]), rtol=1e-12)
    np.testing.assert_allclose(q, c, rtol=1e-12)


def test_orthogonal_history_closed_form(orc):
    # Lags j >= 1 along distinct coordinate axes with signed lengths c_j make the
    # Gram matrix diagonal: beta_j = c_j q_t[axis_j] / (c_j^2 + lambda).  Negative
    # beta_j must still get positive softmax weight exp(beta_j) / sum exp(beta).
    W, D, lam = 8, 16, 0.25
    r = np.random.default_rng(5)
    axes = r.permutation(D)[: W - 1]
    cj = np.array([1.5, -0.7, 2.0, -1.1, 0.4, 3.0, -2.2])
    lags = np.zeros((W, D))
    lags[0] = r.standard_normal(D)
    for j in range(1, W):
        lags[j, axes[j - 1]] = cj[j - 1]
    q, wins, betas, alphas = orc.predict_one(lags, W=W, lam=lam)
    assert wins == [8, 4, 2]
    beta_cf = cj * lags[0][axes] / (cj ** 2 + lam)
    assert (beta_cf < 0).any()
    expect_q = np.zeros(D)
    for w, beta, alpha in zip(wins, betas, alphas):
        p = w - 1
        np.testing.assert_allclose(beta, beta_cf[:p], rtol=1e-13)
        e = np.exp(beta_cf[:p])
        np.testing.assert_allclose(alpha, e / e.sum(), rtol=1e-13)
        expect_q += (e / e.sum()) @ lags[:p] / len(wins)
    np.testing.assert_allclose(q, expect_q, rtol=1e-12, atol=1e-15)


def test_rotation_and_permutation_equivariance(orc):
    # The Gram matrix is invariant under an orthogonal map of the coordinates,
    # so the prediction must rotate with the history.
    W, D = 16, 32
    lags = ar1_lags(W, D, 11)
    q, _, _, _ = orc.predict_one(lags, W=W, lam=1e-2)
    R, _ = np.linalg.qr(np.random.default_rng(12).standard_normal((D, D)))
    qr, _, _, _ = orc.predict_one(lags @ R.T, W=W, lam=1e-2)
    np.testing.assert_allclose(qr, R @ q, rtol=1e-8, atol=1e-10)
    perm = np.random.default_rng(13).permutation(D)
    qp, _, _, _ = orc.predict_one(lags[:, perm], W=W, lam=1e-2)
    np.testing.assert_allclose(qp, q[perm], rtol=1e-10, atol=1e-13)


def test_scale_covariance_pins_where_lambda_enters(orc):
    # Scaling every query by s and lambda by s^2 leaves beta unchanged, so the
    # prediction scales by s.  A lambda scaled by D, or added to r, breaks this.
    W, D, s = 8, 40, 3.5
    lags = ar1_lags(W, D, 17)
    q, _, b1, _ = orc.predict_one(lags, W=W, lam=0.2)
    qs, _, b2, _ = orc.predict_one(s * lags, W=W, lam=0.2 * s * s)
    for x, y in zip(b1, b2):
        np.testing.assert_allclose(x, y, rtol=1e-10)
    np.testing.assert_allclose(qs, s * q, rtol=1e-10)


def test_prediction_lies_in_convex_hull_of_recent_queries(orc):
    W, D = 32, 64
    lags = ar1_lags(W, D, 19)
    q, wins, _, alphas = orc.predict_one(lags, W=W, lam=1e-2)
    assert wins == [32, 16, 8]
    for a in alphas:
        assert (a >= 0).all() and abs(a.sum() - 1.0) < 1e-13
    lo = lags[: W - 1].min(axis=0)
    hi = lags[: W - 1].max(axis=0)
    assert (q >= lo - 1e-12).all() and (q <= hi + 1e-12).all()


@pytest.mark.parametrize("W,cases", [
    (16, {0: None, 1: [], 3: [], 4: [4], 7: [4], 8: [8, 4], 15: [8, 4], 16: [16, 8, 4]}),
    (8, {1: [], 2: [2], 3: [2], 4: [4, 2], 8: [8, 4, 2]}),
    (4, {2: [2], 4: [4, 2]}),
])
def test_window_set_follows_history_length(orc, W, cases):
    D = 8
    for n, expect in cases.items():
        lags = ar1_lags(max(n, 1), D, 23)[:n]
        q, wins, _, _ = orc.predict_one(lags, W=W, lam=1e-2)
        if expect is None:          # no history at all: zero prediction
            assert wins == [] and not q.any()
        else:
            assert wins == expect
            if not expect:          # one query held: predict it unchanged
                np.testing.assert_array_equal(q, lags[0])


def test_ring_push_and_read_match_linear_history(orc):
    # Push 21 queries through an 8-slot ring (wrapping twice) and check the
    # ring by plain indexing, then that predicting from the ring equals
    # predicting from the same queries listed newest-first.
    B, Hq, W, D = 2, 3, 8, 16
    r = np.random.default_rng(29)
    seq = r.standard_normal((21, B, Hq, D)).astype(np.float32)
    ring = np.zeros((B, Hq, W, D), np.float32)
    newest = np.array([W - 1, 2], np.int32)   # arbitrary starting slots
    length = np.zeros(B, np.int32)
    start = newest.copy()
    for t in range(21):
        ring, newest, length = orc.push(seq[t], ring, newest, length)
        assert (length == min(t + 1, W)).all()
        np.testing.assert_array_equal(newest, (start + t + 1) % W)
    for b in range(B):
        for j in range(W):
            np.testing.assert_array_equal(ring[b, :, (newest[b] - j) % W], seq[20 - j, b])
    got = orc.predict(ring, newest, length, lam=1e-2)
    for b in range(B):
        for h in range(Hq):
            lags = seq[20:20 - W:-1, b, h].astype(np.float64)
            q, _, _, _ = orc.predict_one(lags, W=W, lam=1e-2)
            np.testing.assert_array_equal(got[b, h], q)


def _solve_fraction(A, y):
    """Exact rational Gaussian elimination (an independent solver)."""
    n = len(y)
    M = [[Fraction(v) for v in row] + [Fraction(yv)] for row, yv in zip(A, y)]
    for c in range(n):
        piv = next(r for r in range(c, n) if M[r][c] != 0)
        M[c], M[piv] = M[piv], M[c]
        for r in range(n):
            if r != c and M[r][c] != 0:
                f = M[r][c] / M[c][c]
                M[r] = [a - f * b for a, b in zip(M[r], M[c])]
    return [M[i][n] / M[i][i] for i in range(n)]


@pytest.mark.parametrize("name", ["predictor_handworked_1.json", "predictor_handworked_2.json"])
def test_hand_worked_predictor_examples(orc, name):
    with open(os.path.join(GOLDEN, name)) as f:
        fx = json.load(f)
    lags = np.array(fx["lags_newest_first"], dtype=np.float64)
    lam = Fraction(fx["lambda"])
    q, wins, betas, alphas = orc.predict_one(lags, W=fx["W"], lam=float(lam))
    assert wins == fx["windows"]
    qexp = np.zeros(lags.shape[1])
    for w, beta in zip(wins, betas):
        hand = [Fraction(s) for s in fx["beta"][str(w)]]
        # the hand-worked values are themselves re-derived exactly here
        p = w - 1
        G = [[sum(Fraction(a) * Fraction(b) for a, b in zip(fx["lags_newest_first"][j], fx["lags_newest_first"][k]))
              + (lam if j == k else 0) for k in range(1, p + 1)] for j in range(1, p + 1)]
        rr = [sum(Fraction(a) * Fraction(b) for a, b in zip(fx["lags_newest_first"][j], fx["lags_newest_first"][0]))
              for j in range(1, p + 1)]
        assert _solve_fraction(G, rr) == hand
        np.testing.assert_allclose(beta, [float(x) for x in hand], rtol=1e-14, atol=1e-15)
        e = np.array([math.exp(float(x)) for x in hand])
        qexp += (e / e.sum()) @ lags[:p] / len(wins)
    np.testing.assert_allclose(q, qexp, rtol=1e-13)
