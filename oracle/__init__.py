"""CPU oracle for the AsyncSpade sparse decode step (fp64, plain, slow).

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  It shares no
code with the HIP library in ``query_aware_sparse_amd`` and never calls it.

The arithmetic lives in ``asp_oracle.c`` (compiled with gcc, no fast-math);
this module only builds it, marshals numpy arrays through ctypes, shapes the
results, lists the tokens of the optional newest-token window
(``attend_with_recent``) before handing them to the C attention, and lists the
tokens of selected pages (``page_tokens``).  Each wrapper names the definition
it follows; the C file states the readings adopted where the pages are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "asp_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libasp_oracle.so")

KV_BF16 = 0
KV_F32 = 1

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, IEEE semantics kept)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int
    Dbl = ctypes.c_double
    lib.oracle_num_threads.restype = I
    lib.oracle_predict_one.argtypes = [I, I, I, Dbl, P, P, P, P, P, P]
    lib.oracle_predict_one.restype = I
    lib.oracle_predict.argtypes = [I, I, I, I, P, P, P, Dbl, P]
    lib.oracle_predict.restype = I
    lib.oracle_push.argtypes = [I, I, I, I, P, P, P, P]
    lib.oracle_push.restype = None
    lib.oracle_score.argtypes = [I, I, I, I, I, I, P, P, P, P]
    lib.oracle_score.restype = None
    lib.oracle_select.argtypes = [I, I, I, I, P, P, P, P]
    lib.oracle_select.restype = None
    lib.oracle_attend.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P]
    lib.oracle_attend.restype = I
    lib.oracle_overlap.argtypes = [I, I, I, P, P, P, P, P]
    lib.oracle_overlap.restype = None
    lib.oracle_page_summary.argtypes = [I, I, I, I, I, I, P, P, P, P]
    lib.oracle_page_summary.restype = None
    lib.oracle_page_score.argtypes = [I, I, I, I, I, P, P, P, P, P]
    lib.oracle_page_score.restype = None
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype) -> np.ndarray:
    # Rows past a sequence's length may hold any bits (the GPU path leaves them
    # unwritten, and the oracle never reads them): widening a signalling NaN
    # there is not worth a warning.
    with np.errstate(invalid="ignore"):
        return np.ascontiguousarray(a, dtype=dtype)


def _kv(a: np.ndarray):
    """K/V arrays: float32 values, or uint16 raw bfloat16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, KV_F32
    if a.dtype == np.uint16 or a.dtype == np.int16:
        return a.view(np.uint16), KV_BF16
    raise TypeError("K/V must be float32 or uint16 (bfloat16 bits), got %s" % a.dtype)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def predict_one(lags, W: int, lam: float):
    """Predictor for one head.  ``lags[j]`` is q_{t-j} (row 0 newest).

    Returns (q_pred[D], windows list, beta[nw][p], alpha[nw][p]) in fp64.
    """
    lags = _c(lags, np.float64)
    n, D = lags.shape
    q = np.zeros(D, np.float64)
    win = np.zeros(3, np.int32)
    nw = np.zeros(1, np.int32)
    beta = np.zeros((3, W), np.float64)
    alpha = np.zeros((3, W), np.float64)
    rc = _load().oracle_predict_one(n, D, W, float(lam), _ptr(lags) if n else None, _ptr(q),
                                    _ptr(win), _ptr(nw), _ptr(beta), _ptr(alpha))
    if rc != 0:
        raise ArithmeticError("oracle_predict_one: singular ridge system")
    k = int(nw[0])
    windows = [int(w) for w in win[:k]]
    betas = [beta[i, : windows[i] - 1].copy() for i in range(k)]
    alphas = [alpha[i, : windows[i] - 1].copy() for i in range(k)]
    return q, windows, betas, alphas


def predict(q_hist, newest, length, lam: float):
    """q_hist[B][Hq][W][D] fp32 ring, newest[B], len[B] -> q_pred[B][Hq][D] fp64."""
    q_hist = _c(q_hist, np.float32)
    B, Hq, W, D = q_hist.shape
    newest = _c(newest, np.int32)
    length = _c(length, np.int32)
    out = np.zeros((B, Hq, D), np.float64)
    rc = _load().oracle_predict(B, Hq, W, D, _ptr(q_hist), _ptr(newest), _ptr(length), float(lam), _ptr(out))
    if rc != 0:
        raise ArithmeticError("oracle_predict: singular ridge system")
    return out


def push(q_cur, q_hist, newest, length):
    """Returns (q_hist, newest, len) after pushing q_cur[B][Hq][D]; inputs untouched."""
    q_hist = np.array(q_hist, dtype=np.float32, copy=True, order="C")
    newest = np.array(newest, dtype=np.int32, copy=True)
    length = np.array(length, dtype=np.int32, copy=True)
    q_cur = _c(q_cur, np.float32)
    B, Hq, W, D = q_hist.shape
    _load().oracle_push(B, Hq, W, D, _ptr(q_cur), _ptr(q_hist), _ptr(newest), _ptr(length))
    return q_hist, newest, length


def score(q_pred, k, seq_lens):
    """q_pred[B][Hq][D] fp32, K[B][Hkv][T_cap][D] -> scores[B][Hkv][T_cap] fp64 (NaN past seq_len)."""
    q_pred = _c(q_pred, np.float32)
    k, kvd = _kv(k)
    B, Hkv, T_cap, D = k.shape
    Hq = q_pred.shape[1]
    seq_lens = _c(seq_lens, np.int32)
    out = np.empty((B, Hkv, T_cap), np.float64)
    _load().oracle_score(B, Hq, Hkv, D, T_cap, kvd, _ptr(q_pred), _ptr(k), _ptr(seq_lens), _ptr(out))
    return out


def select(scores, seq_lens, C: int):
    """scores[B][Hkv][T_cap] (any float dtype, widened to fp64) -> (idx[B][Hkv][C], n_sel[B][Hkv])."""
    scores = _c(scores, np.float64)
    B, Hkv, T_cap = scores.shape
    seq_lens = _c(seq_lens, np.int32)
    idx = np.empty((B, Hkv, C), np.int32)
    n_sel = np.empty((B, Hkv), np.int32)
    _load().oracle_select(B, Hkv, T_cap, int(C), _ptr(scores), _ptr(seq_lens), _ptr(idx), _ptr(n_sel))
    return idx, n_sel


def attend(q, k, v, idx, n_sel):
    """q[B][Hq][D] fp32, K/V[B][Hkv][T_cap][D], idx[B][Hkv][C], n_sel[B][Hkv] -> out[B][Hq][D] fp64."""
    q = _c(q, np.float32)
    k, kvd = _kv(k)
    v, kvd2 = _kv(v)
    if kvd != kvd2:
        raise TypeError("K and V must share a dtype")
    B, Hkv, T_cap, D = k.shape
    Hq = q.shape[1]
    idx = _c(idx, np.int32)
    C = idx.shape[2]
    n_sel = _c(n_sel, np.int32)
    out = np.empty((B, Hq, D), np.float64)
    rc = _load().oracle_attend(B, Hq, Hkv, D, T_cap, kvd, C, _ptr(q), _ptr(k), _ptr(v), _ptr(idx),
                               _ptr(n_sel), _ptr(out))
    if rc != 0:
        raise IndexError("oracle_attend: selected index outside [0, T_cap)")
    return out


def attend_with_recent(q, k, v, idx, n_sel, seq_lens, recent: int):
    """Attention over each unit's selection and its sequence's newest `recent`
    tokens: the entries idx[j], j < n, with 0 <= idx[j] < T_cap and outside
    [T - r, T) (as listed), followed by every token of [T - r, T) once;
    n = n_sel clamped to [0, C], T = seq_len clamped to [0, T_cap],
    r = min(recent, T).  The pages do not treat tokens newer than the
    selection; this is the library's optional newest-token window, written as
    the list of attended tokens followed by attend()."""
    B, Hkv, T_cap = np.shape(k)[:3]
    idx = np.asarray(idx, np.int32)
    n_sel = np.asarray(n_sel, np.int32)
    lens = np.asarray(seq_lens, np.int32)
    C = idx.shape[2]
    width = C + max(int(recent), 0)
    u_idx = np.full((B, Hkv, max(width, 1)), -1, np.int32)
    u_n = np.zeros((B, Hkv), np.int32)
    for b in range(B):
        T = min(max(int(lens[b]), 0), T_cap)
        r = min(max(int(recent), 0), T)
        for g in range(Hkv):
            n = min(max(int(n_sel[b, g]), 0), C)
            sel = [int(x) for x in idx[b, g, :n] if 0 <= x < T_cap and not (T - r <= x < T)]
            tokens = sel + list(range(T - r, T))
            u_idx[b, g, :len(tokens)] = tokens
            u_n[b, g] = len(tokens)
    return attend(q, k, v, u_idx, u_n)


def overlap(idx_a, n_a, idx_b, n_b, T_cap: int):
    """Per unit, the number of distinct indices in [0, T_cap) present in both
    selections (idx_*[..., C] int32, n_*[...] int32, leading dims = units) --
    the set intersection behind the temporal-locality and prediction-recall
    measurements of the reproduction card ("What reproduces")."""
    idx_a, idx_b = _c(idx_a, np.int32), _c(idx_b, np.int32)
    n_a, n_b = _c(n_a, np.int32), _c(n_b, np.int32)
    C = idx_a.shape[-1]
    units = int(np.prod(idx_a.shape[:-1]))
    out = np.empty(idx_a.shape[:-1], np.int32)
    _load().oracle_overlap(units, C, int(T_cap), _ptr(idx_a), _ptr(n_a), _ptr(idx_b), _ptr(n_b), _ptr(out))
    return out


def page_counts(seq_lens, T_cap: int, P: int) -> np.ndarray:
    """Pages holding at least one token: ceil(T_b / P), T_b clamped to [0, T_cap]."""
    T = np.clip(np.asarray(seq_lens, np.int64), 0, T_cap)
    return ((T + P - 1) // P).astype(np.int32)


def page_summary(k, seq_lens, P: int):
    """Quest page summaries (per page of P tokens, the element-wise min and max
    of its keys; asp_oracle.c states the source and the readings):
    K[B][Hkv][T_cap][D] -> (kmin, kmax) [B][Hkv][NP][D] fp64, NaN for pages
    with no token."""
    k, kvd = _kv(k)
    B, Hkv, T_cap, D = k.shape
    NP = (T_cap + P - 1) // P
    seq_lens = _c(seq_lens, np.int32)
    kmin = np.empty((B, Hkv, NP, D), np.float64)
    kmax = np.empty((B, Hkv, NP, D), np.float64)
    _load().oracle_page_summary(B, Hkv, D, T_cap, kvd, int(P), _ptr(k), _ptr(seq_lens), _ptr(kmin), _ptr(kmax))
    return kmin, kmax


def page_scores(q, kmin, kmax, n_pages):
    """Quest page scores: max over the KV head's query heads of
    sum_d max(q_d * min_d, q_d * max_d); q[B][Hq][D] fp32, kmin/kmax
    [B][Hkv][NP][D] (widened to fp64), n_pages[B] -> [B][Hkv][NP] fp64, NaN
    past each sequence's pages."""
    q = _c(q, np.float32)
    kmin = _c(kmin, np.float64)
    kmax = _c(kmax, np.float64)
    B, Hkv, NP, D = kmin.shape
    Hq = q.shape[1]
    n_pages = _c(n_pages, np.int32)
    out = np.empty((B, Hkv, NP), np.float64)
    _load().oracle_page_score(B, Hq, Hkv, D, NP, _ptr(q), _ptr(kmin), _ptr(kmax), _ptr(n_pages), _ptr(out))
    return out


def page_tokens(page_idx, n_pages_sel, seq_lens, P: int, C: int, T_cap: int):
    """Token list of a page selection: the tokens of the selected pages in
    ascending order, each page p contributing [p*P, min(p*P + P, T_b)); padded
    with -1 to C.  Returns (idx[B][Hkv][C], n_sel[B][Hkv])."""
    page_idx = np.asarray(page_idx, np.int32)
    n_pages_sel = np.asarray(n_pages_sel, np.int32)
    B, Hkv = n_pages_sel.shape
    T = np.clip(np.asarray(seq_lens, np.int64), 0, T_cap)
    idx = np.full((B, Hkv, C), -1, np.int32)
    n_sel = np.zeros((B, Hkv), np.int32)
    for b in range(B):
        for g in range(Hkv):
            toks = []
            for p in sorted(int(x) for x in page_idx[b, g, : n_pages_sel[b, g]]):
                toks.extend(range(p * P, min(p * P + P, int(T[b]))))
            idx[b, g, : len(toks)] = toks
            n_sel[b, g] = len(toks)
    return idx, n_sel


def page_select(q, kmin, kmax, seq_lens, P: int, C: int):
    """Quest selection with a budget of C tokens: the top C / P pages of each
    unit by page score (score descending, lower page first on ties), as the
    token list of page_tokens.  Returns (idx, n_sel, page_idx, n_pages_sel)."""
    B, Hkv, NP, D = np.shape(kmin)
    T_cap = NP * P
    n_pages = page_counts(seq_lens, T_cap, P)
    scores = page_scores(q, kmin, kmax, n_pages)
    page_idx, n_pages_sel = select(scores, n_pages, C // P)
    idx, n_sel = page_tokens(page_idx, n_pages_sel, seq_lens, P, C, T_cap)
    return idx, n_sel, page_idx, n_pages_sel
