"""The C ABI: libasp.so loads, exports every function include/asp.h declares, and
rejects invalid arguments on the host before touching the GPU (CPU only: no
compute call is made here)."""
import ctypes
import os
import re

import pytest

import query_aware_sparse_amd as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "asp.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(asp_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(A.library_path()):
        pytest.fail("libasp.so is not built; run __graft_entry__.build()")
    return A.load()


def test_header_declares_the_boundary():
    assert declared_functions() == sorted([
        "asp_workspace_size", "asp_status_string", "asp_push_query", "asp_predict_query", "asp_score_keys",
        "asp_select_topc", "asp_score_candidates", "asp_select_candidates", "asp_sparse_decode", "asp_step",
        "asp_selection_overlap", "asp_context_create", "asp_context_destroy", "asp_sparse_decode_static",
        "asp_check_device_args", "asp_context_join", "asp_page_summary_size",
        "asp_page_summary",
        "asp_page_scores", "asp_page_select_workspace_size", "asp_page_select"])


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(A.library_path())
    for name in declared_functions():
        assert hasattr(raw, name), name


def test_context_argument_checks(lib):
    # rejected on the host before any HIP call; destroying NULL is a no-op
    h = ctypes.c_void_p(1234)
    assert lib.asp_context_create(0, 0, None) == 1
    assert lib.asp_context_create(0, 2, ctypes.byref(h)) == 1  # unknown flag bit
    assert h.value is None  # *ctx is cleared on failure
    assert lib.asp_context_create(0, 0x80000000, ctypes.byref(h)) == 1
    assert lib.asp_context_destroy(None) == 0
    assert lib.asp_context_join(None, None) == 1


def test_status_strings(lib):
    for code in range(7):
        assert A.asp_status_string(code)
    assert A.asp_status_string(77) == "unknown status"


def _dims(**kw):
    base = dict(batch=8, n_q_heads=32, n_kv_heads=8, head_dim=128, t_cap=32768, kv_dtype=A.KV_BF16)
    base.update(kw)
    return A.Dims(**base)


def test_workspace_sizes(lib):
    d, c = _dims(), A.Cfg(16, 2048, 1e-2)
    assert A.asp_workspace_size(d, c, A.OP_PUSH) == 0
    assert A.asp_workspace_size(d, c, A.OP_SCORE) == 0
    sel = A.asp_workspace_size(d, c, A.OP_SELECT)
    # coarse histograms, per-region candidate lists, counts and bitmaps
    assert sel % 256 == 0 and sel >= 8 * 8 * (2048 * 4 + 32768 * 4 + 32768 // 8)
    dec = A.asp_workspace_size(d, c, A.OP_DECODE)
    step = A.asp_workspace_size(d, c, A.OP_STEP)
    assert dec > 0 and dec % 256 == 0
    cand = A.asp_workspace_size(d, c, A.OP_CANDIDATES)
    # hints and flags per unit, a count per 128-key region, an 8-byte slot per key
    assert cand % 256 == 0 and cand >= 8 * 8 * (4 + 4 + (32768 // 128) * 4 + 32768 * 8)
    # the step holds the candidate workspace, the predicted queries and the attention partials
    assert step >= cand + 8 * 32 * 128 * 4 + dec
    assert A.asp_workspace_size(_dims(head_dim=96), c, A.OP_STEP) == 0
    assert A.asp_workspace_size(_dims(head_dim=96), c, A.OP_CANDIDATES) == 0
    # a ragged t_cap rounds up to whole 512-key score blocks
    c7 = A.Cfg(16, 64, 1e-2)
    assert A.asp_workspace_size(_dims(t_cap=700), c7, A.OP_CANDIDATES) >= 8 * 8 * (1024 // 128) * (4 + 128 * 8)


BAD_DIMS = [
    (dict(batch=-1), 1), (dict(n_q_heads=0), 1), (dict(n_kv_heads=3), 1), (dict(n_q_heads=48, n_kv_heads=8), 2),
    (dict(n_q_heads=128, n_kv_heads=8), 2), (dict(head_dim=96), 2), (dict(head_dim=0), 1), (dict(t_cap=0), 1),
    (dict(t_cap=(1 << 22) + 1), 1), (dict(kv_dtype=5), 1),
]
BAD_CFG = [
    (A.Cfg(6, 64, 1e-2), 1), (A.Cfg(0, 64, 1e-2), 1), (A.Cfg(68, 64, 1e-2), 1), (A.Cfg(16, 0, 1e-2), 1),
    (A.Cfg(16, 40000, 1e-2), 1), (A.Cfg(16, 64, 0.0), 1), (A.Cfg(16, 64, -1.0), 1),
    (A.Cfg(16, 64, float("nan")), 1), (A.Cfg(16, 64, float("inf")), 1),
    (A.Cfg(16, 64, 1e-2, -1), 1), (A.Cfg(16, 64, 1e-2, 40000), 1),
    (A.Cfg(16, 32768, 1e-2, 128), 2),   # C + R past 256 attention splits (128 tokens each here)
]


def _call_score(lib, d):
    one = ctypes.c_void_p(16)   # never dereferenced: validation fails first
    return lib.asp_score_keys(ctypes.byref(d), one, one, one, one, None, None)


def _call_select(lib, d, c, ws=None, nbytes=0):
    one = ctypes.c_void_p(16)
    return lib.asp_select_topc(ctypes.byref(d), ctypes.byref(c), one, None, one, one, one, ws, nbytes, None)


def _call_decode(lib, d, c, ws=None, nbytes=0, null_out=False):
    one = ctypes.c_void_p(16)
    return lib.asp_sparse_decode(ctypes.byref(d), ctypes.byref(c), one, one, one, None, one, one,
                                 None if null_out else one, ws, nbytes, None)


@pytest.mark.parametrize("kw,code", BAD_DIMS)
def test_invalid_dims_rejected_before_any_launch(lib, kw, code):
    assert _call_score(lib, _dims(**kw)) == code
    assert _call_select(lib, _dims(**kw), A.Cfg(16, 64, 1e-2)) == code


@pytest.mark.parametrize("cfg,code", BAD_CFG)
def test_invalid_cfg_rejected_before_any_launch(lib, cfg, code):
    assert _call_select(lib, _dims(), cfg) == code
    assert _call_decode(lib, _dims(), cfg, ctypes.c_void_p(256), 1 << 30) == code


def test_null_pointers_and_short_workspace_rejected(lib):
    d, c = _dims(), A.Cfg(16, 2048, 1e-2)
    assert lib.asp_score_keys(ctypes.byref(d), None, ctypes.c_void_p(16), ctypes.c_void_p(16),
                              ctypes.c_void_p(16), None, None) == 1
    # a histogram that is not 16-byte aligned
    assert lib.asp_score_keys(ctypes.byref(d), ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(16),
                              ctypes.c_void_p(16), ctypes.c_void_p(20), None) == 1
    assert lib.asp_select_topc(ctypes.byref(d), ctypes.byref(c), ctypes.c_void_p(16), ctypes.c_void_p(20),
                               ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(256),
                               1 << 40, None) == 1
    assert _call_decode(lib, d, c, ctypes.c_void_p(256), 1 << 30, null_out=True) == 1
    # recent tokens need the sequence lengths
    assert _call_decode(lib, d, A.Cfg(16, 2048, 1e-2, 16), ctypes.c_void_p(256), 1 << 40) == 1
    need = A.asp_workspace_size(d, c, A.OP_DECODE)
    assert _call_decode(lib, d, c, None, 0) == 3
    need_sel = A.asp_workspace_size(d, c, A.OP_SELECT)
    assert _call_select(lib, d, c, None, 0) == 3
    assert _call_select(lib, d, c, ctypes.c_void_p(256), need_sel - 1) == 3
    assert _call_decode(lib, d, c, ctypes.c_void_p(256), need - 1) == 3
    assert lib.asp_score_keys(None, None, None, None, None, None, None) == 1
    # candidate route: missing, short or misaligned workspace; null outputs
    need_c = A.asp_workspace_size(d, c, A.OP_CANDIDATES)
    for ws, nb in ((None, 0), (ctypes.c_void_p(256), need_c - 1), (ctypes.c_void_p(264), need_c)):
        assert lib.asp_score_candidates(ctypes.byref(d), ctypes.byref(c), ctypes.c_void_p(16), ctypes.c_void_p(16),
                                        ctypes.c_void_p(16), ws, nb, None) == 3
        assert lib.asp_select_candidates(ctypes.byref(d), ctypes.byref(c), ctypes.c_void_p(16), ctypes.c_void_p(16),
                                         ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(16), ws, nb,
                                         None) == 3
    assert lib.asp_score_candidates(ctypes.byref(d), ctypes.byref(c), None, ctypes.c_void_p(16), ctypes.c_void_p(16),
                                    ctypes.c_void_p(256), need_c, None) == 1
    assert lib.asp_select_candidates(ctypes.byref(d), ctypes.byref(c), ctypes.c_void_p(16), ctypes.c_void_p(16),
                                     ctypes.c_void_p(16), None, ctypes.c_void_p(16), ctypes.c_void_p(256), need_c,
                                     None) == 1
    assert lib.asp_score_candidates(ctypes.byref(d), ctypes.byref(A.Cfg(6, 64, 1e-2)), ctypes.c_void_p(16),
                                    ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(256), need_c, None) == 1
    one = ctypes.c_void_p(16)
    # asp_step: idx_cur without n_sel_cur; missing workspace
    args = [None, ctypes.byref(d), ctypes.byref(c)] + [one] * 7  # ctx, dims, cfg, q_cur .. seq_lens
    #                   idx_cur n_sel_cur idx_nx nsel_nx out  ws    ws_bytes  attn  sel   events
    assert lib.asp_step(*args, one, None, one, one, one, one, 1 << 40, None, None, None, None) == 1
    assert lib.asp_step(*args, None, None, one, one, one, None, 0, None, None, None, None) == 3
    # two distinct streams need a context and an idx_cur_ready event
    assert lib.asp_step(*args, one, one, one, one, one, one, 1 << 40, ctypes.c_void_p(1), ctypes.c_void_p(2),
                        None, None) == 1
    assert lib.asp_step(*args, one, one, one, one, one, one, 1 << 40, ctypes.c_void_p(1), ctypes.c_void_p(2),
                        ctypes.c_void_p(3), None) == 1
    args[0] = ctypes.c_void_p(64)  # a context (never dereferenced before the event check)
    assert lib.asp_step(*args, one, one, one, one, one, one, 1 << 40, ctypes.c_void_p(1), ctypes.c_void_p(2),
                        None, None) == 1


# Array arguments per entry point after (dims[, cfg]): "16" must be 16-byte
# aligned, "4" 4-byte aligned, "o4" 4-byte aligned and may be NULL here (the
# sequence lengths of an attention without the newest-token window), "ws" is a
# workspace (16), "n" a byte count or other scalar, "-" an optional pointer
# left NULL.
ALIGNED_ARGS = {
    "asp_push_query": ("dc", ["16", "16", "4", "4"]),
    "asp_predict_query": ("dc", ["16", "4", "4", "4"]),
    "asp_score_keys": ("d", ["4", "16", "4", "4", "-"]),
    "asp_select_topc": ("dc", ["4", "-", "4", "4", "4", "ws", "n"]),
    "asp_score_candidates": ("dc", ["4", "16", "4", "ws", "n"]),
    "asp_select_candidates": ("dc", ["4", "16", "4", "4", "4", "ws", "n"]),
    "asp_selection_overlap": ("dc", ["4", "4", "4", "4", "4"]),
    "asp_sparse_decode": ("dc", ["4", "16", "16", "o4", "4", "4", "4", "ws", "n"]),
    "asp_sparse_decode_static": ("dc", ["4", "16", "16", "o4", "4", "4", "4"]),
    # pipelined on one stream: q_cur .. n_sel_next, out, ws, ws_bytes
    "asp_step": ("xdc", ["16", "16", "4", "4", "16", "16", "4", "4", "4", "4", "4", "4", "ws", "n"]),
}


@pytest.mark.parametrize("name", sorted(ALIGNED_ARGS))
@pytest.mark.parametrize("fault", ["misaligned", "null"])
def test_every_bad_array_pointer_is_rejected_before_any_launch(lib, name, fault):
    # One argument at a time moved off its alignment (by 2 bytes for 4-byte
    # arrays, by 4 for 16-byte ones), or one required pointer NULL:
    # ASP_ERR_INVALID_ARG, or ASP_ERR_WORKSPACE for a workspace, before
    # anything reaches HIP (no GPU is needed here).
    d, c = _dims(), A.Cfg(16, 2048, 1e-2)
    lead, kinds = ALIGNED_ARGS[name]
    fn = getattr(lib, name)
    for i, kind in enumerate(kinds):
        if kind in ("n", "-") or (fault == "null" and kind == "o4"):
            continue
        args = []
        for j, kj in enumerate(kinds):
            if kj == "n":
                args.append(1 << 40)
            elif kj == "-":
                args.append(None)
            elif j == i:
                args.append(None if fault == "null" else ctypes.c_void_p(4096 + (2 if kj in ("4", "o4") else 4)))
            else:
                args.append(ctypes.c_void_p(4096))
        head = {"x": None, "d": ctypes.byref(d), "c": ctypes.byref(c)}
        tail = [None] * (4 if name == "asp_step" else 1)  # streams (and the step's events)
        got = fn(*([head[ch] for ch in lead] + args + tail))
        assert got == (3 if kind == "ws" else 1), (name, fault, i, kind, got)


def test_device_argument_check_rejects_bad_host_arguments(lib):
    # rejected on the host before any HIP call
    d, c = _dims(), A.Cfg(16, 2048, 1e-2)
    one, odd = ctypes.c_void_p(16), ctypes.c_void_p(18)
    chk = lib.asp_check_device_args
    assert chk(ctypes.byref(d), ctypes.byref(c), None, None, None, None, None, one, None) == 1  # no seq_lens
    assert chk(ctypes.byref(d), ctypes.byref(c), one, None, None, None, None, None, None) == 1  # no status
    assert chk(ctypes.byref(d), ctypes.byref(c), one, one, None, None, None, one, None) == 1  # half a ring
    assert chk(ctypes.byref(d), ctypes.byref(c), one, None, None, None, one, one, None) == 1  # half a selection
    assert chk(ctypes.byref(d), ctypes.byref(c), one, None, None, None, None, odd, None) == 1  # misaligned status
    assert chk(ctypes.byref(d), ctypes.byref(A.Cfg(6, 64, 1e-2)), one, None, None, None, None, one, None) == 1
    assert chk(None, ctypes.byref(c), one, None, None, None, None, one, None) == 1
    assert (A.CHECK_SEQ_LEN, A.CHECK_HIST_LEN, A.CHECK_HIST_NEWEST, A.CHECK_N_SEL, A.CHECK_IDX,
            A.CHECK_IDX_PAD) == (1, 2, 4, 8, 16, 32)
    text = open(HEADER).read()
    for name, bit in (("SEQ_LEN", 1), ("HIST_LEN", 2), ("HIST_NEWEST", 4), ("N_SEL", 8), ("IDX", 16),
                      ("IDX_PAD", 32)):
        assert re.search(r"#define ASP_CHECK_%s 0x%02xu" % (name, bit), text), name


def test_page_sizes_and_argument_checks(lib):
    d, c = _dims(), A.Cfg(16, 2048, 1e-2)
    # summaries: B * Hkv * ceil(t_cap / P) * D * 2 bytes (bf16) each
    assert A.asp_page_summary_size(d, 16) == 8 * 8 * 2048 * 128 * 2
    assert A.asp_page_summary_size(_dims(t_cap=33, kv_dtype=A.KV_F32), 16) == 8 * 8 * 3 * 128 * 4
    assert A.asp_page_summary_size(d, 0) == 0
    assert A.asp_page_summary_size(d, 32769) == 0
    assert A.asp_page_summary_size(_dims(head_dim=96), 16) == 0
    ws = A.asp_page_select_workspace_size(d, c, 16)
    assert ws >= 64 * 2048 * 4 + 64 * 128 * 4  # page scores and selected pages
    assert ws % 256 == 0
    assert A.asp_page_select_workspace_size(d, c, 24) == 0  # 2048 is not a multiple of 24
    assert A.asp_page_select_workspace_size(d, A.Cfg(6, 2048, 1e-2), 16) == 0
    one, P = ctypes.c_void_p(16), 16
    dr, cr = ctypes.byref(d), ctypes.byref(c)
    assert lib.asp_page_summary(dr, 0, one, one, one, one, None) == 1
    assert lib.asp_page_summary(dr, P, None, one, one, one, None) == 1
    assert lib.asp_page_summary(dr, P, one, one, ctypes.c_void_p(20), one, None) == 1  # kmin misaligned
    assert lib.asp_page_summary(ctypes.byref(_dims(head_dim=96)), P, one, one, one, one, None) == 2
    assert lib.asp_page_scores(dr, P, one, one, one, one, None, None) == 1
    assert lib.asp_page_scores(dr, P, one, one, ctypes.c_void_p(24), one, one, None) == 1
    assert lib.asp_page_select(dr, cr, 24, one, one, one, one, one, one, one, 1 << 40, None) == 1
    assert lib.asp_page_select(dr, cr, P, one, one, one, one, None, one, one, 1 << 40, None) == 1
    assert lib.asp_page_select(dr, cr, P, one, one, one, one, one, one, None, 1 << 40, None) == 3
    assert lib.asp_page_select(dr, cr, P, one, one, one, one, one, one, one, ws - 1, None) == 3
    assert lib.asp_page_select(dr, cr, P, one, one, one, one, one, one, ctypes.c_void_p(8), ws, None) == 3


def test_missing_library_fails_loudly(tmp_path):
    # No fallback: without libasp.so every entry point raises instead of
    # computing anything elsewhere.  Run in a child process so that this
    # process's loaded library is untouched.
    import subprocess
    import sys
    code = (
        "import query_aware_sparse_amd as A\n"
        "A._LIB_PATH = %r\n"
        "try:\n"
        "    A.asp_workspace_size(A.Dims(1, 2, 1, 64, 64, 0), A.Cfg(8, 8, 1e-2), A.OP_SELECT)\n"
        "except A.AspError as e:\n"
        "    print('raised:', e)\n"
        "else:\n"
        "    print('no error')\n" % str(tmp_path / "libasp.so"))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert "raised: libasp.so is not built" in r.stdout, r.stdout + r.stderr
