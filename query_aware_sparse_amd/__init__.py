"""Python binding of libasp.so, the MI355X (gfx950) AsyncSpade sparse decode step.

Argument marshalling only: every function below checks tensor shapes, dtypes
and devices, then calls the C entry point of the same name (include/asp.h) on
raw device pointers and a HIP stream.  All arithmetic runs in the HIP kernels.
PyTorch supplies device memory and streams.  There is no fallback: if the HIP
library is not built, every call raises ``AspError``.
"""
from __future__ import annotations

import ctypes
import os
import weakref
from typing import Optional

import torch

__all__ = [
    "AspError", "Dims", "Cfg", "HipEvent", "library_path", "load",
    "OP_PUSH", "OP_PREDICT", "OP_SCORE", "OP_SELECT", "OP_DECODE", "OP_STEP", "OP_CANDIDATES",
    "KV_BF16", "KV_F32", "HIST_BINS",
    "asp_workspace_size", "asp_status_string", "asp_push_query", "asp_predict_query", "asp_score_keys",
    "asp_select_topc", "asp_score_candidates", "asp_select_candidates", "asp_sparse_decode", "asp_step",
    "asp_selection_overlap", "AspContext", "CTX_SCORE_ALL_CUS", "PreparedStep", "asp_sparse_decode_static",
    "STATIC_SCRATCH_BYTES", "asp_check_device_args", "CHECK_SEQ_LEN", "CHECK_HIST_LEN", "CHECK_HIST_NEWEST",
    "CHECK_N_SEL", "CHECK_IDX", "CHECK_IDX_PAD",
    "asp_page_summary_size", "asp_page_summary", "asp_page_scores", "asp_page_select_workspace_size",
    "asp_page_select", "page_count",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libasp.so")

OP_PUSH, OP_PREDICT, OP_SCORE, OP_SELECT, OP_DECODE, OP_STEP, OP_CANDIDATES = range(7)
KV_BF16, KV_F32 = 0, 1
HIST_BINS = 2048  # bins of the coarse score histograms (ASP_HIST_BINS)
CTX_SCORE_ALL_CUS = 1  # asp_context_create flag: the score stream may use every CU
STATIC_SCRATCH_BYTES = 8 << 20  # built-in scratch of asp_sparse_decode_static (ASP_STATIC_SCRATCH_BYTES)
# asp_check_device_args status bits (ASP_CHECK_*)
CHECK_SEQ_LEN, CHECK_HIST_LEN, CHECK_HIST_NEWEST, CHECK_N_SEL, CHECK_IDX, CHECK_IDX_PAD = 1, 2, 4, 8, 16, 32
_STATUS_NAMES = {0: "ASP_OK", 1: "ASP_ERR_INVALID_ARG", 2: "ASP_ERR_UNSUPPORTED", 3: "ASP_ERR_WORKSPACE",
                 4: "ASP_ERR_HIP", 5: "ASP_ERR_HOST_MEMORY", 6: "ASP_ERR_SCRATCH"}


class AspError(RuntimeError):
    def __init__(self, msg: str, status: Optional[int] = None):
        super().__init__(msg)
        self.status = status


class Dims(ctypes.Structure):
    """asp_dims: batch, n_q_heads, n_kv_heads, head_dim, t_cap, kv_dtype."""
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("t_cap", ctypes.c_int32), ("kv_dtype", ctypes.c_int32)]

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


class Cfg(ctypes.Structure):
    """asp_cfg: window (ring length W), top_c (C), lam (ridge lambda), recent
    (newest tokens attended beside the selection; 0 by default)."""
    _fields_ = [("window", ctypes.c_int32), ("top_c", ctypes.c_int32), ("lam", ctypes.c_double),
                ("recent", ctypes.c_int32)]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load libasp.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise AspError("libasp.so is not built (%s); run __graft_entry__.build()" % _LIB_PATH)
    lib = ctypes.CDLL(_LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    D, C = ctypes.POINTER(Dims), ctypes.POINTER(Cfg)
    lib.asp_workspace_size.argtypes = [D, C, ctypes.c_int]
    lib.asp_workspace_size.restype = SZ
    lib.asp_status_string.argtypes = [ctypes.c_int]
    lib.asp_status_string.restype = ctypes.c_char_p
    lib.asp_push_query.argtypes = [D, C, P, P, P, P, P]
    lib.asp_predict_query.argtypes = [D, C, P, P, P, P, P]
    lib.asp_score_keys.argtypes = [D, P, P, P, P, P, P]
    lib.asp_select_topc.argtypes = [D, C, P, P, P, P, P, P, SZ, P]
    lib.asp_score_candidates.argtypes = [D, C, P, P, P, P, SZ, P]
    lib.asp_select_candidates.argtypes = [D, C, P, P, P, P, P, P, SZ, P]
    lib.asp_sparse_decode.argtypes = [D, C, P, P, P, P, P, P, P, P, SZ, P]
    lib.asp_sparse_decode_static.argtypes = [D, C, P, P, P, P, P, P, P, P]
    lib.asp_step.argtypes = [P, D, C, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P, P, P, P]
    lib.asp_selection_overlap.argtypes = [D, C, P, P, P, P, P, P]
    lib.asp_check_device_args.argtypes = [D, C, P, P, P, P, P, P, P]
    lib.asp_context_create.argtypes = [ctypes.c_int32, ctypes.c_uint32, ctypes.POINTER(ctypes.c_void_p)]
    lib.asp_context_destroy.argtypes = [P]
    lib.asp_context_join.argtypes = [P, P]
    I32 = ctypes.c_int32
    lib.asp_page_summary_size.argtypes = [D, I32]
    lib.asp_page_summary_size.restype = SZ
    lib.asp_page_summary.argtypes = [D, I32, P, P, P, P, P]
    lib.asp_page_scores.argtypes = [D, I32, P, P, P, P, P, P]
    lib.asp_page_select_workspace_size.argtypes = [D, C, I32]
    lib.asp_page_select_workspace_size.restype = SZ
    lib.asp_page_select.argtypes = [D, C, I32, P, P, P, P, P, P, P, SZ, P]
    for name in ("asp_push_query", "asp_predict_query", "asp_score_keys", "asp_select_topc",
                 "asp_score_candidates", "asp_select_candidates", "asp_sparse_decode", "asp_step",
                 "asp_selection_overlap", "asp_context_create", "asp_context_destroy", "asp_sparse_decode_static",
                 "asp_context_join", "asp_check_device_args"):
        getattr(lib, name).restype = I32
    _lib = lib
    return lib


# ----------------------------------------------------------------------------- helpers

def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t: torch.Tensor, name: str, shape, dtype):
    if not isinstance(t, torch.Tensor):
        raise AspError("%s must be a torch.Tensor" % name)
    if not t.is_cuda:
        raise AspError("%s must be a device tensor" % name)
    if t.dtype != dtype:
        raise AspError("%s must have dtype %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise AspError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise AspError("%s must be contiguous" % name)


def _kv_dtype(d: Dims) -> torch.dtype:
    return torch.bfloat16 if d.kv_dtype == KV_BF16 else torch.float32


def _raise(name: str, status: int):
    if status != 0:
        text = load().asp_status_string(status).decode()
        raise AspError("%s: %s (%s)" % (name, _STATUS_NAMES.get(status, status), text), status)


def _ws(ws: Optional[torch.Tensor]):
    if ws is None:
        return None, 0
    if not ws.is_cuda or not ws.is_contiguous():
        raise AspError("workspace must be a contiguous device tensor")
    return ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size()


class HipEvent:
    """A HIP event for asp_step's ordering of two streams on one device.

    Created with timing disabled and without the system-scope fence: the event
    only orders work between streams of the same GPU (each kernel already
    publishes its writes device-wide when it ends), so the cache writeback a
    system-scope release would add to every record is not needed.
    """

    _hip = None

    def __init__(self):
        if HipEvent._hip is None:
            hip = ctypes.CDLL("libamdhip64.so")
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventCreateWithFlags.restype = ctypes.c_int
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            hip.hipEventDestroy.restype = ctypes.c_int
            HipEvent._hip = hip
        h = ctypes.c_void_p()
        # hipEventDisableTiming | hipEventDisableSystemFence
        rc = HipEvent._hip.hipEventCreateWithFlags(ctypes.byref(h), 0x2 | 0x20000000)
        if rc != 0:
            raise AspError("hipEventCreateWithFlags failed (%d)" % rc)
        self.handle = h

    def __del__(self):
        hip = getattr(HipEvent, "_hip", None)
        if getattr(self, "handle", None) and hip is not None:
            hip.hipEventDestroy(self.handle)
            self.handle = None


def _ev(e: Optional[HipEvent]):
    return None if e is None else e.handle


# ----------------------------------------------------------------------------- entry points

def asp_workspace_size(dims: Dims, cfg: Cfg, op: int) -> int:
    return int(load().asp_workspace_size(ctypes.byref(dims), ctypes.byref(cfg), int(op)))


def asp_status_string(status: int) -> str:
    return load().asp_status_string(int(status)).decode()


def asp_push_query(dims: Dims, cfg: Cfg, q_cur, q_hist, hist_newest, hist_len, stream=None) -> None:
    B, Hq, W, D = dims.batch, dims.n_q_heads, cfg.window, dims.head_dim
    _check(q_cur, "q_cur", (B, Hq, D), torch.float32)
    _check(q_hist, "q_hist", (B, Hq, W, D), torch.float32)
    _check(hist_newest, "hist_newest", (B,), torch.int32)
    _check(hist_len, "hist_len", (B,), torch.int32)
    _raise("asp_push_query", load().asp_push_query(ctypes.byref(dims), ctypes.byref(cfg), _ptr(q_cur), _ptr(q_hist),
                                                   _ptr(hist_newest), _ptr(hist_len), _stream_handle(stream)))


def asp_predict_query(dims: Dims, cfg: Cfg, q_hist, hist_newest, hist_len, q_pred, stream=None) -> None:
    B, Hq, W, D = dims.batch, dims.n_q_heads, cfg.window, dims.head_dim
    _check(q_hist, "q_hist", (B, Hq, W, D), torch.float32)
    _check(hist_newest, "hist_newest", (B,), torch.int32)
    _check(hist_len, "hist_len", (B,), torch.int32)
    _check(q_pred, "q_pred", (B, Hq, D), torch.float32)
    _raise("asp_predict_query", load().asp_predict_query(ctypes.byref(dims), ctypes.byref(cfg), _ptr(q_hist),
                                                         _ptr(hist_newest), _ptr(hist_len), _ptr(q_pred),
                                                         _stream_handle(stream)))


def asp_score_keys(dims: Dims, q_pred, k, seq_lens, scores, hist=None, stream=None) -> None:
    """hist: None, or an int32 [B][Hkv][HIST_BINS] tensor that receives the
    coarse histograms (a uint32 count per bin, stored in int32)."""
    B, Hq, Hkv, D, T = dims.batch, dims.n_q_heads, dims.n_kv_heads, dims.head_dim, dims.t_cap
    _check(q_pred, "q_pred", (B, Hq, D), torch.float32)
    _check(k, "k", (B, Hkv, T, D), _kv_dtype(dims))
    _check(seq_lens, "seq_lens", (B,), torch.int32)
    _check(scores, "scores", (B, Hkv, T), torch.float32)
    if hist is not None:
        _check(hist, "hist", (B, Hkv, HIST_BINS), torch.int32)
    _raise("asp_score_keys", load().asp_score_keys(ctypes.byref(dims), _ptr(q_pred), _ptr(k), _ptr(seq_lens),
                                                   _ptr(scores), _ptr(hist), _stream_handle(stream)))


def asp_select_topc(dims: Dims, cfg: Cfg, scores, seq_lens, idx, n_sel, ws=None, stream=None, hist=None) -> None:
    """hist: None, or the histograms asp_score_keys wrote for these scores."""
    B, Hkv, T, C = dims.batch, dims.n_kv_heads, dims.t_cap, cfg.top_c
    _check(scores, "scores", (B, Hkv, T), torch.float32)
    _check(seq_lens, "seq_lens", (B,), torch.int32)
    _check(idx, "idx", (B, Hkv, C), torch.int32)
    _check(n_sel, "n_sel", (B, Hkv), torch.int32)
    if hist is not None:
        _check(hist, "hist", (B, Hkv, HIST_BINS), torch.int32)
    if ws is None:  # scratch of the selection launches, sized by the library
        ws = torch.empty(asp_workspace_size(dims, cfg, OP_SELECT), dtype=torch.uint8, device=scores.device)
    wp, wb = _ws(ws)
    _raise("asp_select_topc", load().asp_select_topc(ctypes.byref(dims), ctypes.byref(cfg), _ptr(scores),
                                                     _ptr(hist), _ptr(seq_lens), _ptr(idx), _ptr(n_sel), wp, wb,
                                                     _stream_handle(stream)))


def _check_candidates(dims: Dims, cfg: Cfg, q_pred, k, seq_lens, ws):
    B, Hq, Hkv, D, T = dims.batch, dims.n_q_heads, dims.n_kv_heads, dims.head_dim, dims.t_cap
    _check(q_pred, "q_pred", (B, Hq, D), torch.float32)
    _check(k, "k", (B, Hkv, T, D), _kv_dtype(dims))
    _check(seq_lens, "seq_lens", (B,), torch.int32)
    if ws is None:
        raise AspError("the candidate workspace carries the threshold hints between calls: pass one "
                       "(asp_workspace_size(dims, cfg, OP_CANDIDATES) bytes)")
    return _ws(ws)


def asp_score_candidates(dims: Dims, cfg: Cfg, q_pred, k, seq_lens, ws, stream=None) -> None:
    """Score pass that keeps, per unit, the keys at or above the hint held in ws."""
    wp, wb = _check_candidates(dims, cfg, q_pred, k, seq_lens, ws)
    _raise("asp_score_candidates", load().asp_score_candidates(ctypes.byref(dims), ctypes.byref(cfg), _ptr(q_pred),
                                                               _ptr(k), _ptr(seq_lens), wp, wb,
                                                               _stream_handle(stream)))


def asp_select_candidates(dims: Dims, cfg: Cfg, q_pred, k, seq_lens, idx, n_sel, ws, stream=None) -> None:
    """Exact top-C from the candidates of the last asp_score_candidates call on ws."""
    B, Hkv, C = dims.batch, dims.n_kv_heads, cfg.top_c
    wp, wb = _check_candidates(dims, cfg, q_pred, k, seq_lens, ws)
    _check(idx, "idx", (B, Hkv, C), torch.int32)
    _check(n_sel, "n_sel", (B, Hkv), torch.int32)
    _raise("asp_select_candidates", load().asp_select_candidates(ctypes.byref(dims), ctypes.byref(cfg), _ptr(q_pred),
                                                                 _ptr(k), _ptr(seq_lens), _ptr(idx), _ptr(n_sel), wp,
                                                                 wb, _stream_handle(stream)))


def asp_selection_overlap(dims: Dims, cfg: Cfg, idx_a, n_sel_a, idx_b, n_sel_b, overlap, stream=None) -> None:
    B, Hkv, C = dims.batch, dims.n_kv_heads, cfg.top_c
    for name, t in (("idx_a", idx_a), ("idx_b", idx_b)):
        _check(t, name, (B, Hkv, C), torch.int32)
    for name, t in (("n_sel_a", n_sel_a), ("n_sel_b", n_sel_b), ("overlap", overlap)):
        _check(t, name, (B, Hkv), torch.int32)
    _raise("asp_selection_overlap", load().asp_selection_overlap(ctypes.byref(dims), ctypes.byref(cfg), _ptr(idx_a),
                                                                 _ptr(n_sel_a), _ptr(idx_b), _ptr(n_sel_b),
                                                                 _ptr(overlap), _stream_handle(stream)))


def asp_check_device_args(dims: Dims, cfg: Cfg, seq_lens, status, hist_newest=None, hist_len=None, idx=None,
                          n_sel=None, stream=None) -> None:
    """status: a one-element int32 tensor on the device; after the stream has run the
    call it holds the OR of the CHECK_* bits of the violated conditions (0: none)."""
    B, Hkv, C = dims.batch, dims.n_kv_heads, cfg.top_c
    _check(seq_lens, "seq_lens", (B,), torch.int32)
    _check(status, "status", (1,), torch.int32)
    if hist_newest is not None or hist_len is not None:
        _check(hist_newest, "hist_newest", (B,), torch.int32)
        _check(hist_len, "hist_len", (B,), torch.int32)
    if idx is not None or n_sel is not None:
        _check(idx, "idx", (B, Hkv, C), torch.int32)
        _check(n_sel, "n_sel", (B, Hkv), torch.int32)
    _raise("asp_check_device_args", load().asp_check_device_args(ctypes.byref(dims), ctypes.byref(cfg),
                                                                 _ptr(seq_lens), _ptr(hist_newest), _ptr(hist_len),
                                                                 _ptr(idx), _ptr(n_sel), _ptr(status),
                                                                 _stream_handle(stream)))


def asp_sparse_decode(dims: Dims, cfg: Cfg, q, k, v, seq_lens, idx, n_sel, out, ws, stream=None) -> None:
    """seq_lens may be None when cfg.recent is 0."""
    B, Hq, Hkv, D, T, C = dims.batch, dims.n_q_heads, dims.n_kv_heads, dims.head_dim, dims.t_cap, cfg.top_c
    _check(q, "q", (B, Hq, D), torch.float32)
    _check(k, "k", (B, Hkv, T, D), _kv_dtype(dims))
    _check(v, "v", (B, Hkv, T, D), _kv_dtype(dims))
    if seq_lens is not None:
        _check(seq_lens, "seq_lens", (B,), torch.int32)
    _check(idx, "idx", (B, Hkv, C), torch.int32)
    _check(n_sel, "n_sel", (B, Hkv), torch.int32)
    _check(out, "out", (B, Hq, D), torch.float32)
    wp, wb = _ws(ws)
    _raise("asp_sparse_decode", load().asp_sparse_decode(ctypes.byref(dims), ctypes.byref(cfg), _ptr(q), _ptr(k),
                                                         _ptr(v), _ptr(seq_lens), _ptr(idx), _ptr(n_sel), _ptr(out),
                                                         wp, wb,
                                                         _stream_handle(stream)))


def asp_sparse_decode_static(dims: Dims, cfg: Cfg, q, k, v, seq_lens, idx, n_sel, out, stream=None) -> None:
    """asp_sparse_decode with the library's built-in scratch instead of a
    workspace: it allocates nothing.  Calls whose work overlaps on one GPU race
    (they share that GPU's scratch).  seq_lens may be None when cfg.recent is 0."""
    B, Hq, Hkv, D, T, C = dims.batch, dims.n_q_heads, dims.n_kv_heads, dims.head_dim, dims.t_cap, cfg.top_c
    _check(q, "q", (B, Hq, D), torch.float32)
    _check(k, "k", (B, Hkv, T, D), _kv_dtype(dims))
    _check(v, "v", (B, Hkv, T, D), _kv_dtype(dims))
    if seq_lens is not None:
        _check(seq_lens, "seq_lens", (B,), torch.int32)
    _check(idx, "idx", (B, Hkv, C), torch.int32)
    _check(n_sel, "n_sel", (B, Hkv), torch.int32)
    _check(out, "out", (B, Hq, D), torch.float32)
    _raise("asp_sparse_decode_static", load().asp_sparse_decode_static(
        ctypes.byref(dims), ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(seq_lens), _ptr(idx), _ptr(n_sel),
        _ptr(out), _stream_handle(stream)))


class AspContext:
    """asp_context: the stream and events of two-stream asp_step calls, owned
    by this object (asp_context_create / asp_context_destroy).

    device: the CUDA/HIP device index (default: the current device).  flags: 0
    (the score stream leaves the last 32-CU group to the step's latency-bound
    launches) or CTX_SCORE_ALL_CUS.  One context serves one asp_step call at a
    time; use one per host thread.  close() (or the end of the process)
    releases it.
    """

    def __init__(self, device: Optional[int] = None, flags: int = 0):
        lib = load()
        dev = torch.cuda.current_device() if device is None else int(device)
        h = ctypes.c_void_p()
        _raise("asp_context_create", lib.asp_context_create(dev, int(flags), ctypes.byref(h)))
        self.handle = h
        self.device = dev
        # released before the HIP runtime is torn down at interpreter exit
        self._finalizer = weakref.finalize(self, lib.asp_context_destroy, h)

    def close(self) -> None:
        """Wait for the context's stream and release it (idempotent)."""
        if self._finalizer.alive:
            status = self._finalizer()
            _raise("asp_context_destroy", status)

    def join(self, stream) -> None:
        """asp_context_join: `stream` waits for every score pass enqueued on the
        context so far (under graph capture, the join a capture with two-stream
        steps needs before it ends)."""
        _raise("asp_context_join", load().asp_context_join(self.handle, _stream_handle(stream)))


def _step_args(ctx, dims, cfg, q_cur, q_hist, hist_newest, hist_len, k, v, seq_lens, idx_cur, n_sel_cur, idx_next,
               n_sel_next, out, ws, attn_stream, sel_stream, idx_cur_ready, idx_next_ready):
    B, Hq, Hkv, D, T = dims.batch, dims.n_q_heads, dims.n_kv_heads, dims.head_dim, dims.t_cap
    W, C = cfg.window, cfg.top_c
    _check(q_cur, "q_cur", (B, Hq, D), torch.float32)
    _check(q_hist, "q_hist", (B, Hq, W, D), torch.float32)
    _check(hist_newest, "hist_newest", (B,), torch.int32)
    _check(hist_len, "hist_len", (B,), torch.int32)
    _check(k, "k", (B, Hkv, T, D), _kv_dtype(dims))
    _check(v, "v", (B, Hkv, T, D), _kv_dtype(dims))
    _check(seq_lens, "seq_lens", (B,), torch.int32)
    if idx_cur is not None:
        _check(idx_cur, "idx_cur", (B, Hkv, C), torch.int32)
        _check(n_sel_cur, "n_sel_cur", (B, Hkv), torch.int32)
    _check(idx_next, "idx_next", (B, Hkv, C), torch.int32)
    _check(n_sel_next, "n_sel_next", (B, Hkv), torch.int32)
    _check(out, "out", (B, Hq, D), torch.float32)
    if ctx is not None and not isinstance(ctx, AspContext):
        raise AspError("ctx must be an AspContext or None")
    wp, wb = _ws(ws)
    attn = _stream_handle(attn_stream)
    sel = None if sel_stream is None else _stream_handle(sel_stream)
    return (None if ctx is None else ctx.handle, ctypes.byref(dims), ctypes.byref(cfg), _ptr(q_cur), _ptr(q_hist),
            _ptr(hist_newest), _ptr(hist_len), _ptr(k), _ptr(v), _ptr(seq_lens), _ptr(idx_cur), _ptr(n_sel_cur),
            _ptr(idx_next), _ptr(n_sel_next), _ptr(out), wp, wb, attn, sel, _ev(idx_cur_ready), _ev(idx_next_ready))


def asp_step(dims: Dims, cfg: Cfg, q_cur, q_hist, hist_newest, hist_len, k, v, seq_lens, idx_cur, n_sel_cur,
             idx_next, n_sel_next, out, ws, attn_stream=None, sel_stream=None, ctx: Optional[AspContext] = None,
             idx_cur_ready: Optional[HipEvent] = None, idx_next_ready: Optional[HipEvent] = None) -> None:
    """One decode step of one layer (include/asp.h).  Two distinct streams need
    ctx (an AspContext on the current device) and idx_cur_ready."""
    args = _step_args(ctx, dims, cfg, q_cur, q_hist, hist_newest, hist_len, k, v, seq_lens, idx_cur, n_sel_cur,
                      idx_next, n_sel_next, out, ws, attn_stream, sel_stream, idx_cur_ready, idx_next_ready)
    _raise("asp_step", load().asp_step(*args))


class PreparedStep:
    """asp_step with its arguments checked and marshalled once, for a decode
    loop that calls the same step (same tensors, streams and events) again and
    again: calling the object makes the C call with the stored arguments.

    The tensors, streams, events and context are referenced until the object is
    dropped.  Their contents may change between calls (a new query written
    into q_cur, for instance); their storage must not.
    """

    def __init__(self, dims: Dims, cfg: Cfg, q_cur, q_hist, hist_newest, hist_len, k, v, seq_lens, idx_cur,
                 n_sel_cur, idx_next, n_sel_next, out, ws, attn_stream=None, sel_stream=None,
                 ctx: Optional[AspContext] = None, idx_cur_ready: Optional[HipEvent] = None,
                 idx_next_ready: Optional[HipEvent] = None):
        self._keep = (dims, cfg, q_cur, q_hist, hist_newest, hist_len, k, v, seq_lens, idx_cur, n_sel_cur,
                      idx_next, n_sel_next, out, ws, attn_stream, sel_stream, ctx, idx_cur_ready, idx_next_ready)
        self._args = _step_args(ctx, dims, cfg, q_cur, q_hist, hist_newest, hist_len, k, v, seq_lens, idx_cur,
                                n_sel_cur, idx_next, n_sel_next, out, ws, attn_stream, sel_stream, idx_cur_ready,
                                idx_next_ready)
        self._fn = load().asp_step

    def __call__(self) -> None:
        status = self._fn(*self._args)
        if status != 0:
            _raise("asp_step", status)


def page_count(t_cap: int, page_size: int) -> int:
    """Page rows per unit of the page summaries and page scores: ceil(t_cap / page_size)."""
    return (int(t_cap) + int(page_size) - 1) // int(page_size)


def asp_page_summary_size(dims: Dims, page_size: int) -> int:
    return int(load().asp_page_summary_size(ctypes.byref(dims), int(page_size)))


def _check_summaries(dims: Dims, page_size: int, kmin, kmax):
    B, Hkv, D = dims.batch, dims.n_kv_heads, dims.head_dim
    shape = (B, Hkv, page_count(dims.t_cap, page_size), D)
    _check(kmin, "kmin", shape, _kv_dtype(dims))
    _check(kmax, "kmax", shape, _kv_dtype(dims))


def asp_page_summary(dims: Dims, page_size: int, k, seq_lens, kmin, kmax, stream=None) -> None:
    """Per page of page_size tokens, the element-wise min and max of its keys."""
    B, Hkv, D, T = dims.batch, dims.n_kv_heads, dims.head_dim, dims.t_cap
    _check(k, "k", (B, Hkv, T, D), _kv_dtype(dims))
    _check(seq_lens, "seq_lens", (B,), torch.int32)
    _check_summaries(dims, page_size, kmin, kmax)
    _raise("asp_page_summary", load().asp_page_summary(ctypes.byref(dims), int(page_size), _ptr(k), _ptr(seq_lens),
                                                       _ptr(kmin), _ptr(kmax), _stream_handle(stream)))


def asp_page_scores(dims: Dims, page_size: int, q, kmin, kmax, seq_lens, scores, stream=None) -> None:
    """Page scores [B][Hkv][NP] fp32 from the page summaries and the query q."""
    B, Hq, Hkv, D = dims.batch, dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    _check(q, "q", (B, Hq, D), torch.float32)
    _check_summaries(dims, page_size, kmin, kmax)
    _check(seq_lens, "seq_lens", (B,), torch.int32)
    _check(scores, "scores", (B, Hkv, page_count(dims.t_cap, page_size)), torch.float32)
    _raise("asp_page_scores", load().asp_page_scores(ctypes.byref(dims), int(page_size), _ptr(q), _ptr(kmin),
                                                     _ptr(kmax), _ptr(seq_lens), _ptr(scores),
                                                     _stream_handle(stream)))


def asp_page_select_workspace_size(dims: Dims, cfg: Cfg, page_size: int) -> int:
    return int(load().asp_page_select_workspace_size(ctypes.byref(dims), ctypes.byref(cfg), int(page_size)))


def asp_page_select(dims: Dims, cfg: Cfg, page_size: int, q, kmin, kmax, seq_lens, idx, n_sel, ws=None,
                    stream=None) -> None:
    """The top top_c / page_size pages per unit, written as their tokens."""
    B, Hq, Hkv, D, C = dims.batch, dims.n_q_heads, dims.n_kv_heads, dims.head_dim, cfg.top_c
    _check(q, "q", (B, Hq, D), torch.float32)
    _check_summaries(dims, page_size, kmin, kmax)
    _check(seq_lens, "seq_lens", (B,), torch.int32)
    _check(idx, "idx", (B, Hkv, C), torch.int32)
    _check(n_sel, "n_sel", (B, Hkv), torch.int32)
    if ws is None:
        ws = torch.empty(max(asp_page_select_workspace_size(dims, cfg, page_size), 1), dtype=torch.uint8,
                         device=q.device)
    wp, wb = _ws(ws)
    _raise("asp_page_select", load().asp_page_select(ctypes.byref(dims), ctypes.byref(cfg), int(page_size), _ptr(q),
                                                     _ptr(kmin), _ptr(kmax), _ptr(seq_lens), _ptr(idx), _ptr(n_sel),
                                                     wp, wb, _stream_handle(stream)))
