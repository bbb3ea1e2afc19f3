"""asp_check_device_args (GPU required): the check of the arguments that live in
device memory reports nothing for the states the library's own producers leave
(a pushed ring; selections from the token route, the candidate route, the step
and the page route), and exactly the conditions that planted values violate.

The expected bits come from `expected_bits`, which states the header's
conditions for this call in plain Python over host copies; the check launch
only reads its inputs, so planted out-of-range values are safe to pass.
"""
import numpy as np
import pytest
import torch

import query_aware_sparse_amd as A
from asp_testutil import np_, require_gpu

pytestmark = pytest.mark.gpu
DEV = "cuda"

B, HQ, HKV, D, TCAP, C, W = 3, 8, 2, 64, 1000, 128, 8
LENS = [1000, 300, 50]  # the last one shorter than C


def expected_bits(seq_lens, hist_newest, hist_len, idx, n_sel, t_cap=TCAP, c=C, w=W, hkv=HKV):
    bits = 0
    for b, t in enumerate(seq_lens):
        if t < 0 or t > t_cap:
            bits |= A.CHECK_SEQ_LEN
        if hist_len is not None:
            n = hist_len[b]
            if n < 0 or n > w:
                bits |= A.CHECK_HIST_LEN
            elif n > 0 and not 0 <= hist_newest[b] < w:
                bits |= A.CHECK_HIST_NEWEST
    if idx is not None:
        rows = idx.reshape(-1, c)
        for u, row in enumerate(rows):
            t = min(max(int(seq_lens[u // hkv]), 0), t_cap)
            n_raw = int(n_sel.reshape(-1)[u])
            if n_raw < 0 or n_raw > min(c, t):
                bits |= A.CHECK_N_SEL
            n = min(max(n_raw, 0), c)
            for j in range(c):
                x = int(row[j])
                if j < n:
                    if x < 0 or x >= t or (j + 1 < n and int(row[j + 1]) <= x):
                        bits |= A.CHECK_IDX
                elif x != -1:
                    bits |= A.CHECK_IDX_PAD
    return bits


def run_check(dims, cfg, seq_lens, hist_newest=None, hist_len=None, idx=None, n_sel=None):
    status = torch.full((1,), -7, dtype=torch.int32, device=DEV)  # the call clears it first
    A.asp_check_device_args(dims, cfg, seq_lens, status, hist_newest=hist_newest, hist_len=hist_len, idx=idx,
                            n_sel=n_sel)
    torch.cuda.synchronize()
    return int(status.item())


@pytest.fixture(scope="module")
def state():
    require_gpu()
    g = torch.Generator(device="cpu").manual_seed(5)
    dims = A.Dims(B, HQ, HKV, D, TCAP, A.KV_F32)
    cfg = A.Cfg(W, C, 1e-2)
    lens = torch.tensor(LENS, dtype=torch.int32, device=DEV)
    k = torch.randn((B, HKV, TCAP, D), generator=g).to(DEV)
    v = torch.randn((B, HKV, TCAP, D), generator=g).to(DEV)
    q_hist = torch.zeros((B, HQ, W, D), device=DEV)
    newest = torch.zeros((B,), dtype=torch.int32, device=DEV)
    length = torch.zeros((B,), dtype=torch.int32, device=DEV)
    for _ in range(W + 3):  # the ring wraps around
        A.asp_push_query(dims, cfg, torch.randn((B, HQ, D), generator=g).to(DEV), q_hist, newest, length)
    q = torch.randn((B, HQ, D), generator=g).to(DEV)
    scores = torch.empty((B, HKV, TCAP), device=DEV)
    A.asp_score_keys(dims, q, k, lens, scores)
    idx = torch.empty((B, HKV, C), dtype=torch.int32, device=DEV)
    n_sel = torch.empty((B, HKV), dtype=torch.int32, device=DEV)
    A.asp_select_topc(dims, cfg, scores, lens, idx, n_sel,
                      ws=torch.empty(A.asp_workspace_size(dims, cfg, A.OP_SELECT), dtype=torch.uint8, device=DEV))
    torch.cuda.synchronize()
    return dict(dims=dims, cfg=cfg, lens=lens, k=k, v=v, q=q, q_hist=q_hist, newest=newest, length=length, idx=idx,
                n_sel=n_sel)


def test_states_left_by_the_producers_pass(state):
    s = state
    d, c = s["dims"], s["cfg"]
    assert run_check(d, c, s["lens"]) == 0
    assert run_check(d, c, s["lens"], s["newest"], s["length"], s["idx"], s["n_sel"]) == 0
    # the candidate route's selection
    ws = torch.empty(A.asp_workspace_size(d, c, A.OP_CANDIDATES), dtype=torch.uint8, device=DEV)
    ws.zero_()  # hints 0: every key kept
    idx2, n2 = torch.empty_like(s["idx"]), torch.empty_like(s["n_sel"])
    A.asp_score_candidates(d, c, s["q"], s["k"], s["lens"], ws)
    A.asp_select_candidates(d, c, s["q"], s["k"], s["lens"], idx2, n2, ws)
    assert run_check(d, c, s["lens"], idx=idx2, n_sel=n2) == 0
    # a bootstrap step's selection and ring
    q_hist, newest, length = s["q_hist"].clone(), s["newest"].clone(), s["length"].clone()
    idx3, n3 = torch.empty_like(s["idx"]), torch.empty_like(s["n_sel"])
    out = torch.empty((B, HQ, D), device=DEV)
    wst = torch.empty(A.asp_workspace_size(d, c, A.OP_STEP), dtype=torch.uint8, device=DEV)
    A.asp_step(d, c, s["q"], q_hist, newest, length, s["k"], s["v"], s["lens"], None, None, idx3, n3, out, wst)
    assert run_check(d, c, s["lens"], newest, length, idx3, n3) == 0
    # an empty ring (any newest slot) and an all-empty batch
    assert run_check(d, c, s["lens"], torch.full_like(newest, 99), torch.zeros_like(length)) == 0
    zero = torch.zeros_like(s["lens"])
    assert run_check(d, c, zero, idx=torch.full_like(idx3, -1), n_sel=torch.zeros_like(n3)) == 0


def test_page_selection_passes(state):
    s = state
    d, c, P = s["dims"], s["cfg"], 16
    NP = A.page_count(TCAP, P)
    kmin = torch.empty((B, HKV, NP, D), device=DEV)
    kmax = torch.empty_like(kmin)
    A.asp_page_summary(d, P, s["k"], s["lens"], kmin, kmax)
    idx, n = torch.empty_like(s["idx"]), torch.empty_like(s["n_sel"])
    ws = torch.empty(A.asp_page_select_workspace_size(d, c, P), dtype=torch.uint8, device=DEV)
    A.asp_page_select(d, c, P, s["q"], kmin, kmax, s["lens"], idx, n, ws)
    torch.cuda.synchronize()
    want = expected_bits(np_(s["lens"]), None, None, np_(idx), np_(n))
    assert want == 0
    assert run_check(d, c, s["lens"], idx=idx, n_sel=n) == 0


def _plant(state, what):
    lens, newest, length = np_(state["lens"]).copy(), np_(state["newest"]).copy(), np_(state["length"]).copy()
    idx, n_sel = np_(state["idx"]).copy(), np_(state["n_sel"]).copy()
    what(lens, newest, length, idx, n_sel)
    return lens, newest, length, idx, n_sel


def _swap(L, N, H, I, S):
    I[0, 1, 5], I[0, 1, 6] = I[0, 1, 6], I[0, 1, 5]


def _empty_ring_any_slot(L, N, H, I, S):
    H[1] = 0
    N[1] = 1234


def _set(arr_pos, at, value):
    def f(*arrays):
        arrays[arr_pos][at] = value(arrays) if callable(value) else value
    return f


# name: (plant, the single bit it violates, or None when it also breaks what follows from it)
PLANTS = {
    "length past t_cap": (_set(0, 1, TCAP + 1), A.CHECK_SEQ_LEN),
    "ring longer than the window": (_set(2, 0, W + 1), A.CHECK_HIST_LEN),
    "negative ring length": (_set(2, 2, -1), A.CHECK_HIST_LEN),
    "newest slot outside the window": (_set(1, 1, W), A.CHECK_HIST_NEWEST),
    "negative newest slot": (_set(1, 0, -3), A.CHECK_HIST_NEWEST),
    "empty ring, any newest slot": (_empty_ring_any_slot, 0),
    "two entries swapped": (_swap, A.CHECK_IDX),
    "a repeated entry": (_set(3, (1, 0, 7), lambda a: a[3][1, 0, 6]), A.CHECK_IDX),
    "an entry at the length": (_set(3, (2, 1, LENS[2] - 1), LENS[2]), A.CHECK_IDX),
    "a padding entry not -1": (_set(3, (2, 0, C - 1), 3), A.CHECK_IDX_PAD),
    "count below zero": (_set(4, (0, 0), -1), None),  # the row's entries become padding
    "count above C_eff": (_set(4, (2, 1), LENS[2] + 1), None),  # a -1 entry falls inside the count
}


@pytest.mark.parametrize("name", sorted(PLANTS))
def test_planted_violations_are_reported(state, name):
    fn, single = PLANTS[name]
    lens, newest, length, idx, n_sel = _plant(state, fn)
    want = expected_bits(lens, newest, length, idx, n_sel)
    if single is not None:
        assert want == single  # the reference agrees with the plant's intent
    else:
        assert want & A.CHECK_N_SEL
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    got = run_check(state["dims"], state["cfg"], t(lens), t(newest), t(length), t(idx), t(n_sel))
    assert got == want, (name, got, want)


def test_random_corruptions_match_the_reference(state):
    rng = np.random.default_rng(11)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    seen = 0
    for _ in range(40):
        lens, newest, length, idx, n_sel = _plant(state, lambda *a: None)
        for _ in range(rng.integers(1, 4)):
            which = rng.integers(0, 5)
            if which == 0:
                lens[rng.integers(0, B)] = rng.choice([-2, -1, 0, 1, 50, 300, TCAP, TCAP + 1, 5000])
            elif which == 1:
                length[rng.integers(0, B)] = rng.integers(-1, W + 2)
            elif which == 2:
                newest[rng.integers(0, B)] = rng.integers(-2, W + 2)
            elif which == 3:
                n_sel[rng.integers(0, B), rng.integers(0, HKV)] = rng.integers(-1, C + 2)
            else:
                idx[rng.integers(0, B), rng.integers(0, HKV), rng.integers(0, C)] = rng.integers(-2, TCAP + 2)
        want = expected_bits(lens, newest, length, idx, n_sel)
        got = run_check(state["dims"], state["cfg"], t(lens), t(newest), t(length), t(idx), t(n_sel))
        assert got == want
        seen |= want
    assert seen == 63  # every condition was hit at least once
