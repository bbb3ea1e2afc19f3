"""Pins of the selection-overlap oracle: hand-worked cases and an independent
pairwise count (no marker array, no sets) on random small selections."""
import numpy as np

import oracle


def _pairwise(a, na, b, nb, T):
    """Count values of B[:nb] in [0, T) equal to some value of A[:na], each value once."""
    seen = []
    for j in range(max(0, min(nb, len(b)))):
        x = int(b[j])
        if x < 0 or x >= T or x in seen:
            continue
        for i in range(max(0, min(na, len(a)))):
            if int(a[i]) == x:
                seen.append(x)
                break
    return len(seen)


def test_hand_worked():
    idx_a = np.array([[[1, 4, 7, 9, -1, -1]]], np.int32)
    idx_b = np.array([[[0, 4, 9, 10, 11, -1]]], np.int32)
    # {1,4,7,9} and {0,4,9,10,11}: {4, 9}
    assert oracle.overlap(idx_a, np.array([[4]]), idx_b, np.array([[5]]), 12)[0, 0] == 2
    # only the first 2 entries of B count: {0, 4}
    assert oracle.overlap(idx_a, np.array([[4]]), idx_b, np.array([[2]]), 12)[0, 0] == 1
    # a selection against itself, against an empty one, and index 11 beyond T=11
    assert oracle.overlap(idx_b, np.array([[5]]), idx_b, np.array([[5]]), 12)[0, 0] == 5
    assert oracle.overlap(idx_b, np.array([[5]]), idx_b, np.array([[5]]), 11)[0, 0] == 4
    assert oracle.overlap(idx_a, np.array([[0]]), idx_b, np.array([[5]]), 12)[0, 0] == 0
    # n_sel beyond C is clamped to C; negative to 0
    assert oracle.overlap(idx_a, np.array([[99]]), idx_a, np.array([[99]]), 12)[0, 0] == 4
    assert oracle.overlap(idx_a, np.array([[-3]]), idx_a, np.array([[4]]), 12)[0, 0] == 0


def test_against_pairwise_count():
    rng = np.random.default_rng(3)
    U, C, T = 7, 40, 90
    a = np.full((U, C), -1, np.int32)
    b = np.full((U, C), -1, np.int32)
    na = rng.integers(0, C + 1, U).astype(np.int32)
    nb = rng.integers(0, C + 1, U).astype(np.int32)
    for u in range(U):
        a[u, :na[u]] = np.sort(rng.choice(T + 5, na[u], replace=False)) - 2   # a few out of range
        b[u, :nb[u]] = rng.integers(-1, T + 1, nb[u])                          # any order, repeats
    got = oracle.overlap(a, na, b, nb, T)
    want = [_pairwise(a[u], na[u], b[u], nb[u], T) for u in range(U)]
    np.testing.assert_array_equal(got, want)
