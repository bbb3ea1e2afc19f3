"""The candidate route of the selection (GPU required).

asp_score_candidates keeps, per unit, the keys at or above a threshold hint
held in the workspace; asp_select_candidates picks the exact top C_eff among
them, rescoring with every key kept a unit whose candidates fall short.  The
index sets must equal, bit for bit, the oracle's selection on the GPU's own
fp32 scores (asp_score_keys, whose values the score tests check against the
oracle), for every hint: all keys kept (hint 0), none kept (every unit
rescored), random hints, and the hints a previous selection left (the steady
state of a decode loop).  Inputs include exact ties (small-integer keys and
queries), +-inf and NaN scores, empty rows, rows of at most C tokens, and rows
whose candidates do not fit the select's LDS stage.
"""
import numpy as np
import pytest
import torch

import oracle
import query_aware_sparse_amd as A
from query_aware_sparse_amd import workload as wk
from asp_testutil import dims_for, np_, require_gpu

pytestmark = pytest.mark.gpu

DEV = "cuda"
FINE_SHIFT = 10  # the hints are lower edges of bins of the top 22 bits of the order key


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()
    print("\n[case]", flush=True)


def order_keys(s: np.ndarray) -> np.ndarray:
    """The monotone float -> uint32 map the selection ranks by (NaN as -inf, -0 as +0)."""
    s = np.where(np.isnan(s), np.float32(-np.inf), s).astype(np.float32)
    s = np.where(s == 0, np.float32(0.0), s)
    u = s.view(np.uint32)
    return np.where(u >> 31, ~u, u | np.uint32(0x80000000)).astype(np.uint32)


def _inputs(B, Hq, Hkv, D, T_cap, kv, kind, seed):
    g = torch.Generator().manual_seed(seed)
    if kind == "integer":   # exact scores, many ties
        q = torch.randint(-3, 4, (B, Hq, D), generator=g).float()
        k = torch.randint(-3, 4, (B, Hkv, T_cap, D), generator=g).float()
    else:
        q = wk.randn((B, Hq, D), seed=seed)
        k = wk.randn((B, Hkv, T_cap, D), seed=seed, sub=1)
        if kind == "special":   # +-inf / NaN scores from infinite rows, +-0 scores from zero rows
            r = np.random.default_rng(seed)
            for b in range(B):
                for h in range(Hkv):
                    rows = r.choice(T_cap, size=min(T_cap, 24), replace=False)
                    k[b, h, rows[:8]] = float("inf")
                    k[b, h, rows[8:12]] = -float("inf")
                    k[b, h, rows[12:]] = 0.0
    return q, k.to(torch.bfloat16 if kv == "bf16" else torch.float32)


class Case:
    def __init__(self, B, Hq, Hkv, D, T_cap, lens, C, kv, kind, seed):
        self.dims = dims_for(A, B, Hq, Hkv, D, T_cap, kv)
        self.cfg = A.Cfg(8, C, 1e-2)
        self.B, self.Hkv, self.C, self.T_cap = B, Hkv, C, T_cap
        q, k = _inputs(B, Hq, Hkv, D, T_cap, kv, kind, seed)
        self.q, self.k = q.to(DEV), k.to(DEV)
        self.lens_np = np.array(lens, np.int32)
        self.lens = torch.tensor(lens, dtype=torch.int32, device=DEV)
        self.ws = torch.zeros(A.asp_workspace_size(self.dims, self.cfg, A.OP_CANDIDATES), dtype=torch.uint8,
                              device=DEV)
        self.hints = self.ws[:4 * B * Hkv].view(torch.int32)

    def gpu_scores(self, q):
        s = torch.empty((self.B, self.Hkv, self.T_cap), dtype=torch.float32, device=DEV)
        A.asp_score_keys(self.dims, q, self.k, self.lens, s)
        torch.cuda.synchronize()
        return np_(s)

    def run(self, q):
        idx = torch.full((self.B, self.Hkv, self.C), -9, dtype=torch.int32, device=DEV)
        n_sel = torch.full((self.B, self.Hkv), -9, dtype=torch.int32, device=DEV)
        A.asp_score_candidates(self.dims, self.cfg, q, self.k, self.lens, self.ws)
        A.asp_select_candidates(self.dims, self.cfg, q, self.k, self.lens, idx, n_sel, self.ws)
        torch.cuda.synchronize()
        return np_(idx), np_(n_sel)

    def check(self, q, label):
        s = self.gpu_scores(q)
        ri, rn = oracle.select(s, self.lens_np, self.C)
        idx, n_sel = self.run(q)
        np.testing.assert_array_equal(n_sel, rn, err_msg=label)
        np.testing.assert_array_equal(idx, ri, err_msg=label)
        # the new hints: bin edges that keep at least C_eff keys of these scores
        hints = np_(self.hints).view(np.uint32).reshape(self.B, self.Hkv)
        assert ((hints & np.uint32((1 << FINE_SHIFT) - 1)) == 0).all(), label
        keys = order_keys(s)
        for b in range(self.B):
            T = int(self.lens_np[b])
            c_eff = min(self.C, T)
            for g in range(self.Hkv):
                kept = int((keys[b, g, :T] >= hints[b, g]).sum())
                assert kept >= c_eff, (label, b, g, kept, c_eff)
        return hints


def _walk(case: Case, seed):
    """Selections under every kind of hint, then a few steps of a drifting query."""
    case.hints.fill_(0)                      # every key kept
    case.check(case.q, "hint 0")
    case.hints.fill_(-1)                     # nothing kept: every short unit rescored
    case.check(case.q, "hint max")
    r = np.random.default_rng(seed)
    case.hints.copy_(torch.from_numpy(r.integers(0, 2**32, size=case.B * case.Hkv, dtype=np.uint64)
                                      .astype(np.uint32).view(np.int32)).to(DEV))
    case.check(case.q, "random hints")
    case.check(case.q, "hints of the same scores")
    q = case.q
    for t in range(3):                       # AR(1)-like drift, the hints of the previous step
        q = (0.9 * q + 0.3 * wk.randn(tuple(q.shape), seed=seed + 100 + t).to(DEV)).contiguous()
        case.check(q, "drift step %d" % t)
    # a sudden change of scale: the hints of the previous scores keep too few
    # keys (every unit rescored), then far too many
    case.check((q * 0.01).contiguous(), "scale 1/100")
    case.check(q, "scale back")
    case.check(q, "same scores again")


@pytest.mark.parametrize("kind", ["normal", "integer", "special"])
def test_candidates_bf16_g4_ragged_rows(kind):
    # a full row, one ending inside a score block, one of at most C tokens, an empty one
    lens = [9000, 4097, 700, 0]
    _walk(Case(4, 8, 2, 128, 9000, lens, 1000, "bf16", kind, seed=11), seed=11)


@pytest.mark.parametrize("kind", ["normal", "integer"])
def test_candidates_bf16_g8_d64(kind):
    lens = [5000, 1, 2048]
    _walk(Case(3, 16, 2, 64, 5000, lens, 2048, "bf16", kind, seed=12), seed=12)


@pytest.mark.parametrize("kind", ["normal", "integer", "special"])
def test_candidates_f32_g2_and_g1(kind):
    _walk(Case(2, 4, 2, 128, 3000, [3000, 2999], 300, "f32", kind, seed=13), seed=13)
    _walk(Case(3, 2, 2, 64, 1000, [1000, 64, 65], 64, "f32", kind, seed=14), seed=14)


def test_candidates_rows_longer_than_the_lds_stage():
    # 131072-key rows with C = 4096: a rescoring keeps every key (more than
    # the select stages in LDS), the steady state keeps about 2 C of them.
    lens = [131072, 70001]
    _walk(Case(2, 4, 1, 128, 131072, lens, 4096, "bf16", "normal", seed=15), seed=15)


def test_candidates_qwen3_8b_layer_shape():
    # B=8, 32q/8kv, D=128, T=32768, C=2048 on the workload's own K and queries
    wl = wk.Q8B_LAYER
    case = Case(wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.t_cap, [wl.t_cap] * wl.batch, wl.top_c,
                "bf16", "normal", seed=16)
    case.k = wk.make_kv(wl, wk.make_seq_lens(wl), layer=0, device=DEV)[0]
    case.lens = wk.make_seq_lens(wl).to(DEV)
    case.lens_np = np_(case.lens)
    qs = wk.make_queries(wl, 4, layer=0)
    case.hints.fill_(0)
    for t in range(4):
        case.check(qs[t].to(DEV), "query %d" % t)


def test_candidates_hints_at_exact_ranks():
    # Hints placed on the order key of a chosen rank of each row, so that the
    # kept set holds exactly C_eff - 1 (every unit rescored), C_eff, C_eff + 1
    # or 2 C_eff - 1 keys: the boundaries of the kept-count rules.
    lens = [4096, 3000, 700, 1]
    case = Case(4, 16, 4, 128, 4096, lens, 512, "bf16", "normal", seed=17)
    s = case.gpu_scores(case.q)
    keys = order_keys(s)
    for extra in (-1, 0, 1, 511, 2000):
        h = np.zeros((case.B, case.Hkv), np.uint32)
        for b in range(case.B):
            T = int(case.lens_np[b])
            r = min(case.C, T) + extra
            for g in range(case.Hkv):
                if T and 0 < r <= T:
                    h[b, g] = np.sort(keys[b, g, :T])[::-1][r - 1]
        case.hints.copy_(torch.from_numpy(h.view(np.int32).reshape(-1)).to(DEV))
        case.check(case.q, "rank C_eff%+d" % extra)


def test_candidates_any_workspace_contents():
    # Whatever the workspace holds before the first call (hints, flags, region
    # counts and slots left by other work), the selection is the oracle's.
    lens = [4096, 3000, 700, 1]
    case = Case(4, 16, 4, 128, 4096, lens, 512, "bf16", "normal", seed=18)
    g = torch.Generator(device=DEV).manual_seed(18)
    for fill in range(4):
        case.ws.copy_(torch.randint(0, 256, tuple(case.ws.shape), generator=g, device=DEV, dtype=torch.int32)
                      .to(torch.uint8))
        case.check(case.q, "random workspace %d" % fill)


def test_candidates_empty_batch_is_a_no_op():
    # batch 0: validated, nothing enqueued, nothing dereferenced (placeholder pointers)
    import ctypes
    lib = A.load()
    dims = A.Dims(0, 8, 2, 128, 1000, A.KV_BF16)
    cfg = A.Cfg(8, 100, 1e-2)
    p = ctypes.c_void_p(256)
    nbytes = A.asp_workspace_size(dims, cfg, A.OP_CANDIDATES)
    assert lib.asp_score_candidates(ctypes.byref(dims), ctypes.byref(cfg), p, p, p, p, nbytes, None) == 0
    assert lib.asp_select_candidates(ctypes.byref(dims), ctypes.byref(cfg), p, p, p, p, p, p, nbytes, None) == 0
    torch.cuda.synchronize()


@pytest.mark.parametrize("C", [1, 2, 998, 999])
@pytest.mark.parametrize("kind", ["normal", "integer"])
def test_candidates_extreme_budgets(C, kind):
    # C = 1 and C = T - 1 on rows of 1000 keys, beside rows of 999 and 2 keys
    # (C_eff = T there for the larger budgets), with every kind of hint
    lens = [1000, 999, 2]
    _walk(Case(3, 8, 2, 128, 1000, lens, C, "bf16", kind, seed=20 + C), seed=20 + C)
