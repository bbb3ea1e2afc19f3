"""Benchmark of the AsyncSpade sparse decode step on one MI355X.

One step = one pass of the whole path for one decoder layer of the
Qwen3-8B-shaped workload (batch 8, 32 query / 8 KV heads, head_dim 128,
32768-token bf16 KV cache, C = 2048, W = 16): push the actual query, predict
the next query, score every key, select the top-C, and attend over the
selection made by the previous step.  Selection runs on a second HIP stream
concurrently with attention (the pipelined schedule); --mode one_stream runs
the same schedule serially.  Four independent KV caches (layers) are used in
rotation so that no step reads KV that the previous step left in the 256 MB
last-level cache; every step uses a fresh AR(1) query.

--workload measures one layer of another workload shape (the Qwen3-8B stack
layer, the Qwen3-32B layer or the ragged long-CoT batch; --top-c and --window
override C and W); the roofline's measured traffic is then null, since the
committed counter summary is of the Qwen3-8B layer.

The timed loop is run twice over the same layers: issued from Python through
the binding's prepared steps (one ctypes call per step; this gives `value`),
then issued from C++ through the C ABI (bench_driver.cpp; "loops.cpp"), so
that the host's issue cost can be told from the GPU's time.

Beside the step, the page-level (Quest) baseline is timed on the same layers
("page_baseline"): page scoring with the current query, top C / P pages and
attention over their tokens, all on one stream (--page-size, 0 skips it).  So
is dense decode attention over every cached token ("dense_baseline"): the
attention entry point given each unit's whole token list (--no-dense-baseline
skips it; null when the cache is longer than the attention's longest list).

Prints one JSON line on stdout.  Everything else goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


METRIC = "sparse decode steps/s + achieved HBM GB/s (score+select+attend), 32k ctx C=2048"
HBM_PEAK_GBPS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def step_bytes(wl, seq_lens) -> dict:
    """Algorithmic HBM bytes of one step (what the method must move).

    Per unit (sequence b, KV head g): the K scan T_b*D*2, the gathered K and V
    rows 2*C_eff*D*2, the index write and read 8*C_eff, and the predicted query
    read, actual query read and output write 3*G*D*4.  The full step adds the
    query history read G*W*D*4 and the predicted query write G*D*4 per unit.
    With a newest-token window of r tokens, its K and V rows 2*r*D*2 are added
    (counted apart from the selection, which may overlap them).  The transient
    score rows are excluded.
    """
    D, G, C, W, Hkv = wl.head_dim, wl.group, wl.top_c, wl.window, wl.n_kv_heads
    core = 0
    for T in seq_lens:
        ce, r = min(C, T), min(wl.recent, T)
        core += Hkv * (T * D * 2 + 2 * (ce + r) * D * 2 + 8 * ce + 3 * G * D * 4)
    full = core + wl.batch * Hkv * (G * W * D * 4 + G * D * 4)
    return {"score_select_attend": core, "full_step": full}


def score_kernel_bytes(wl, seq_lens) -> int:
    """Algorithmic bytes of one score launch of the step (the candidate
    route): the K rows read and the predicted queries read.  The candidates it
    writes (about 2*C_eff (key, index) pairs per unit) are the implementation's
    own traffic, as the score rows are not part of the method's bytes."""
    D, Hkv, G = wl.head_dim, wl.n_kv_heads, wl.group
    return sum(Hkv * (T * D * 2 + G * D * 4) for T in seq_lens)


SCORE_SOURCES = [os.path.join(ROOT, "query_aware_sparse_amd", "csrc", f)
                 for f in ("score.hip", "score_block.h", "asp_internal.h")]


def sources_hash(paths) -> str:
    """First 16 hex digits of the SHA-256 of the files' bytes, concatenated in order."""
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_sources):
    """HBM traffic of the score kernel from the committed rocprofv3 counter
    summary, or None when the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "score_candidates_qwen3-8b-layer_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256_16") != sources_hash(kernel_sources):
        return None
    return rec.get("bytes_per_launch")


STEP_SOURCES = [os.path.join(ROOT, "query_aware_sparse_amd", "csrc", f)
                for f in ("api.hip", "predict.hip", "score.hip", "score_block.h", "select.hip", "attend.hip",
                          "attend_mfma.h", "attend_block.h", "asp_internal.h")]


def in_step_score_launch_us():
    """Average duration of the step's score launch inside the overlapped steps
    of the default command, from the committed rocprofv3 kernel trace summary,
    or None when the step's sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "sparse_decode_step_qwen3-8b-layer_in_step.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256_16") != sources_hash(STEP_SOURCES):
        return None
    return rec.get("score_candidates_avg_us")


# Keys per oracle sample: about the Qwen3-8B layer (64 units x 32768 keys); at
# least two units per thread of a 16-core host, so that the sample keeps every
# thread busy as the whole layer does.
CPU_SAMPLE_KEYS = 64 * 32768
CPU_SAMPLE_MIN_UNITS = 32


def cpu_baseline(wl, layer, q_t) -> dict:
    """The oracle (fp64, plain) timed on the host cores for one full step of one
    layer (all units), on inputs copied back from the device.  A layer with
    many more keys than the Qwen3-8B layer (the ragged long-CoT batch) is
    timed on its first sequences (at least CPU_SAMPLE_MIN_UNITS units, more
    while the sample stays within CPU_SAMPLE_KEYS keys), and the step time is
    scaled by the keys the whole layer scans."""
    import numpy as np
    import torch
    import oracle

    lens_all = layer["seq_lens"].cpu().numpy()
    per_seq = wl.n_kv_heads * np.maximum(lens_all, 0).astype(np.int64)
    nb, acc = 0, 0
    min_seqs = -(-CPU_SAMPLE_MIN_UNITS // wl.n_kv_heads)
    while nb < wl.batch and (nb < min_seqs or acc + per_seq[nb] <= CPU_SAMPLE_KEYS):
        acc += per_seq[nb]
        nb += 1
    scale = float(per_seq.sum()) / float(per_seq[:nb].sum()) if nb < wl.batch else 1.0
    k, v = layer["k"][:nb], layer["v"][:nb]
    kn = k.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    vn = v.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    lens = lens_all[:nb].copy()
    hist = layer["q_hist"][:nb].cpu().numpy()
    newest = layer["newest"][:nb].cpu().numpy()
    length = layer["length"][:nb].cpu().numpy()
    q = q_t[:nb].cpu().numpy()
    idx_prev = layer["idx"][layer["cur"]][:nb].cpu().numpy()
    n_prev = layer["nsel"][layer["cur"]][:nb].cpu().numpy()

    def one_step():
        o = oracle.attend(q, kn, vn, idx_prev, n_prev)
        h, n, l = oracle.push(q, hist, newest, length)
        qp = oracle.predict(h, n, l, wl.lam).astype(np.float32)
        s = oracle.score(qp, kn, lens)
        oracle.select(s, lens, wl.top_c)
        return o

    one_step()  # warm-up
    reps, t0 = 0, time.perf_counter()
    while True:
        one_step()
        reps += 1
        el = time.perf_counter() - t0
        if (reps >= 3 and el >= 10.0) or el > 30.0:  # a bounded sample of ~10 s of CPU work
            break
    per_step = el / reps * scale
    if nb == wl.batch:
        what = "full step of one layer (all %d units)" % (wl.batch * wl.n_kv_heads)
    else:
        what = ("step of the first %d of %d sequences (%d of %d units, %d of %d keys), scaled by the keys "
                "(x%.2f)" % (nb, wl.batch, nb * wl.n_kv_heads, wl.batch * wl.n_kv_heads, int(per_seq[:nb].sum()),
                             int(per_seq.sum()), scale))
    return {"value": 1.0 / per_step, "unit": "steps/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "%s, %d timed repetitions (%.1f s) after 1 warm-up, %.3f s per full step"
                      % (what, reps, el, per_step),
            "host": host_cpu()}


def host_cpu() -> dict:
    """The host the oracle ran on: its CPU model and the processors the OS reports."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(),
            "usable": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None}


_DRIVER = None


def driver():
    """bench_driver.so (the C++ timing loop and the stream hold), built by
    __graft_entry__.build() beside this file."""
    global _DRIVER
    if _DRIVER is None:
        import ctypes
        _DRIVER = ctypes.CDLL(os.path.join(ROOT, "bench_driver.so"))
        _DRIVER.bench_hold.argtypes = [ctypes.c_void_p, ctypes.c_double]
        _DRIVER.bench_hold.restype = ctypes.c_int
    return _DRIVER


def hold(stream, us: float) -> None:
    """Holds `stream` for about `us` microseconds with a single-wave wait kernel."""
    if driver().bench_hold(stream.cuda_stream, float(us)) != 0:
        raise RuntimeError("bench_hold failed")


def raw_call(A, name, *args):
    """The C entry point `name` with its arguments marshalled once: tensors as
    device pointers, Dims/Cfg by reference, streams as handles, ints as they
    are.  Calling the result costs one ctypes call; the timing loops use it for
    arguments the binding has already accepted in their warm-up calls."""
    import ctypes
    import torch
    conv = []
    for a in args:
        if isinstance(a, torch.Tensor):
            conv.append(ctypes.c_void_p(a.data_ptr()))
        elif isinstance(a, (A.Dims, A.Cfg)):
            conv.append(ctypes.byref(a))
        elif isinstance(a, torch.cuda.Stream):
            conv.append(ctypes.c_void_p(a.cuda_stream))
        else:
            conv.append(a)
    fn = getattr(A.load(), name)

    def call():
        status = fn(*conv)
        if status != 0:
            raise RuntimeError("%s failed: %d" % (name, status))
    return call


def page_baseline(A, dims, cfg, wl, layers, P, time_entry, out, ws_dec, attn, n) -> dict:
    """The page-level (Quest) baseline on the same layers: its per-page min/max
    summaries are built once per KV cache; each of its decode steps scores the
    pages with the current query, keeps the top C / P pages and attends over
    their tokens, all on the decode critical path (one stream)."""
    import torch
    B, Hq, Hkv, D, C = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.top_c
    NP = A.page_count(wl.t_cap, P)
    dev = layers[0]["k"].device
    summ = []
    for lay in layers:
        kmin = torch.empty((B, Hkv, NP, D), dtype=lay["k"].dtype, device=dev)
        kmax = torch.empty_like(kmin)
        A.asp_page_summary(dims, P, lay["k"], lay["seq_lens"], kmin, kmax, stream=attn)
        summ.append((kmin, kmax))
    L = len(layers)
    ws = torch.empty(A.asp_page_select_workspace_size(dims, cfg, P), dtype=torch.uint8, device=dev)
    pscores = torch.empty((B, Hkv, NP), dtype=torch.float32, device=dev)
    idx = torch.empty((B, Hkv, C), dtype=torch.int32, device=dev)
    nsel = torch.empty((B, Hkv), dtype=torch.int32, device=dev)

    def q_of(i):
        lay = layers[i % L]
        return lay["qs"][lay["t"]]

    def page_step(i):
        lay, (kmin, kmax) = layers[i % L], summ[i % L]
        A.asp_page_select(dims, cfg, P, q_of(i), kmin, kmax, lay["seq_lens"], idx, nsel, ws, stream=attn)
        A.asp_sparse_decode(dims, cfg, q_of(i), lay["k"], lay["v"], lay["seq_lens"], idx, nsel, out, ws_dec,
                            stream=attn)

    def rc(name, *a):
        return raw_call(A, name, *a)

    def page_step_raw(i):
        lay, (kmin, kmax) = layers[i % L], summ[i % L]
        sel_call = rc("asp_page_select", dims, cfg, P, q_of(i), kmin, kmax, lay["seq_lens"], idx, nsel, ws, ws.numel(),
                      attn)
        dec_call = rc("asp_sparse_decode", dims, cfg, q_of(i), lay["k"], lay["v"], lay["seq_lens"], idx, nsel, out,
                      ws_dec, ws_dec.numel(), attn)

        def call():
            sel_call()
            dec_call()
        return call

    t = {
        "summary_us": time_entry(lambda i: A.asp_page_summary(dims, P, layers[i % L]["k"], layers[i % L]["seq_lens"],
                                                              summ[i % L][0], summ[i % L][1], stream=attn), 20),
        "page_scores_us": time_entry(
            lambda i: A.asp_page_scores(dims, P, q_of(i), summ[i % L][0], summ[i % L][1], layers[i % L]["seq_lens"],
                                        pscores, stream=attn), n,
            lambda i: rc("asp_page_scores", dims, P, q_of(i), summ[i][0], summ[i][1], layers[i]["seq_lens"], pscores,
                         attn)),
        "page_select_us": time_entry(
            lambda i: A.asp_page_select(dims, cfg, P, q_of(i), summ[i % L][0], summ[i % L][1],
                                        layers[i % L]["seq_lens"], idx, nsel, ws, stream=attn), n,
            lambda i: rc("asp_page_select", dims, cfg, P, q_of(i), summ[i][0], summ[i][1], layers[i]["seq_lens"], idx,
                         nsel, ws, ws.numel(), attn)),
        "step_us": time_entry(page_step, n, page_step_raw),
    }
    lens = [int(x) for x in layers[0]["seq_lens"].tolist()]
    esize = 2 if wl.kv_dtype == "bf16" else 4
    scan = sum(Hkv * ((T + P - 1) // P) * D * esize * 2 for T in lens)  # kmin + kmax rows read
    res = {k_: round(v_, 2) for k_, v_ in t.items()}
    res.update({"page_size": P, "pages_kept": C // P, "summary_bytes_read_per_step": scan,
                "page_scores_GBps": round(scan / (t["page_scores_us"] * 1e-6) / 1e9, 1),
                "steps_per_s": round(1e6 / t["step_us"], 1)})
    return res


def dense_baseline(A, dims, wl, layers, time_entry, out, attn, n):
    """Dense decode attention on the same layers: asp_sparse_decode with each
    unit's whole token list 0 .. seq_len - 1, so every cached K and V row is
    read (the full attention the pages compare against).  None when the cache
    is longer than the longest list the attention takes."""
    import torch
    B, Hq, Hkv, D, T = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.t_cap
    cfg_d = A.Cfg(wl.window, T, wl.lam, 0)
    need = A.asp_workspace_size(dims, cfg_d, A.OP_DECODE)
    if need == 0:
        return None
    dev = layers[0]["k"].device
    L = len(layers)
    idx = torch.arange(T, dtype=torch.int32, device=dev).expand(B, Hkv, T).contiguous()
    nsel = [lay["seq_lens"].view(B, 1).expand(B, Hkv).contiguous() for lay in layers]  # the whole list
    ws = torch.empty(need, dtype=torch.uint8, device=dev)

    def q_of(i):
        lay = layers[i % L]
        return lay["qs"][lay["t"]]

    us = time_entry(
        lambda i: A.asp_sparse_decode(dims, cfg_d, q_of(i), layers[i % L]["k"], layers[i % L]["v"],
                                      layers[i % L]["seq_lens"], idx, nsel[i % L], out, ws, stream=attn), n,
        lambda i: raw_call(A, "asp_sparse_decode", dims, cfg_d, q_of(i), layers[i]["k"], layers[i]["v"],
                           layers[i]["seq_lens"], idx, nsel[i], out, ws, ws.numel(), attn))
    esize = 2 if wl.kv_dtype == "bf16" else 4
    G = Hq // Hkv
    lens = [int(x) for x in layers[0]["seq_lens"].tolist()]
    nbytes = sum(Hkv * (2 * t * D * esize + 4 * t + 2 * G * D * 4) for t in lens)  # K, V, indices, q, out
    return {"attend_us": round(us, 2), "bytes_per_layer": nbytes, "GBps": round(nbytes / (us * 1e-6) / 1e9, 1)}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--mode", choices=["two_streams", "one_stream"], default="two_streams")
    ap.add_argument("--kv-buffers", type=int, default=4)
    ap.add_argument("--workload", default="qwen3-8b-layer",
                    choices=["qwen3-8b-layer", "qwen3-8b-stack", "qwen3-32b", "ragged-long-cot"],
                    help="one decoder layer of this workload (the headline metric is qwen3-8b-layer)")
    ap.add_argument("--top-c", type=int, default=None, help="override the workload's selection budget C")
    ap.add_argument("--window", type=int, default=None, help="override the workload's ridge window W")
    ap.add_argument("--recent", type=int, default=0, help="newest tokens attended beside the selection")
    ap.add_argument("--kernel-launches", type=int, default=200)
    ap.add_argument("--page-size", type=int, default=16,
                    help="page size of the page-level (Quest) baseline timed beside the step (0 = skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense-baseline", dest="dense_baseline", action="store_false",
                    help="skip the dense decode attention over every cached token")
    ap.add_argument("--hold-us", type=float, default=0.0,
                    help="hold the attention stream this long before each timed loop (a bounded wait kernel), so "
                         "that the host queues the timed steps first and the GPU sets their pace; for kernel traces, "
                         "whose tracer slows the host.  ms_per_step then comes from the GPU events alone")
    ap.add_argument("--no-cpp-driver", dest="cpp_driver", action="store_false",
                    help="skip the second timing of the same loop issued from C++ (bench_driver.so)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (rocprofv3 counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the sparse decode step here runs on a single device "
              "(--gpus %d was requested)" % args.gpus, file=sys.stderr)
        return 2

    import torch
    import query_aware_sparse_amd as A
    from query_aware_sparse_amd import workload as wk

    A.load()
    dev = "cuda"
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.randn(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copied %d MiB x5" % args.copy_calibration_mib)
        return 0

    wl = wk.CONFIGS[args.workload]
    if args.top_c is not None:
        wl = wl.replace(top_c=args.top_c)
    if args.window is not None:
        wl = wl.replace(window=args.window, history_steps=max(wl.history_steps, args.window + 4))
    if args.recent:
        wl = wl.replace(recent=args.recent)
    headline = wl == wk.Q8B_LAYER  # the counter summary in profiles/ is of this workload
    dims = A.Dims(wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.t_cap, A.KV_BF16)
    cfg = A.Cfg(wl.window, wl.top_c, wl.lam, wl.recent)
    B, Hq, Hkv, D, C = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.top_c
    L = args.kv_buffers
    drivers = ["python"] + (["cpp"] if args.cpp_driver else [])
    # each timing loop takes warmup + steps steps over the L layers in turn
    n_layer_steps = len(drivers) * ((args.warmup + args.steps) // L + 2)
    attn = torch.cuda.Stream()
    sel = torch.cuda.Stream() if args.mode == "two_streams" else None
    # one step workspace per layer, as a decode loop over layers keeps them
    ws_step = [torch.empty(A.asp_workspace_size(dims, cfg, A.OP_STEP), dtype=torch.uint8, device=dev)
               for _ in range(L)]
    ws_dec = torch.empty(A.asp_workspace_size(dims, cfg, A.OP_DECODE), dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    ctx = A.AspContext() if sel is not None else None

    t0 = time.perf_counter()
    layers = []
    for l in range(L):
        lens = wk.make_seq_lens(wl, device=dev)
        k, v = wk.make_kv(wl, lens, layer=l, device=dev)
        qs = wk.make_queries(wl, wl.history_steps + n_layer_steps + 1, layer=l, device=dev)
        q_hist, newest, length = [x.to(dev) for x in wk.empty_history(wl)]
        lay = dict(k=k, v=v, seq_lens=lens, qs=qs, q_hist=q_hist, newest=newest, length=length,
                   idx=[torch.empty((B, Hkv, C), dtype=torch.int32, device=dev) for _ in range(2)],
                   nsel=[torch.empty((B, Hkv), dtype=torch.int32, device=dev) for _ in range(2)],
                   ev=[A.HipEvent(), A.HipEvent()], ws=ws_step[l], cur=0, t=wl.history_steps)
        for t in range(wl.history_steps - 1):
            A.asp_push_query(dims, cfg, qs[t], q_hist, newest, length)
        # bootstrap step: selection made from the ring, attended at once
        A.asp_step(dims, cfg, qs[wl.history_steps - 1], q_hist, newest, length, k, v, lens, None, None,
                   lay["idx"][0], lay["nsel"][0], out, ws_step[l], idx_next_ready=lay["ev"][0])
        layers.append(lay)
    torch.cuda.synchronize()
    log("setup: %d KV caches of %.2f GiB (K+V) in %.1f s" % (L, 2 * k.numel() * 2 / 2**30, time.perf_counter() - t0))

    def prepare(lay, n):
        """The layer's next n steps (each with its own query and selection
        buffer order), checked and marshalled ahead: a step is then one
        ctypes call."""
        steps = []
        for j in range(n):
            cur, t = (lay["cur"] + j) % 2, lay["t"] + j
            steps.append(A.PreparedStep(dims, cfg, lay["qs"][t], lay["q_hist"], lay["newest"], lay["length"],
                                        lay["k"], lay["v"], lay["seq_lens"], lay["idx"][cur], lay["nsel"][cur],
                                        lay["idx"][1 - cur], lay["nsel"][1 - cur], out, lay["ws"], attn_stream=attn,
                                        sel_stream=sel, ctx=ctx, idx_cur_ready=lay["ev"][cur],
                                        idx_next_ready=lay["ev"][1 - cur]))
        return steps

    def time_python_loop():
        per_layer = (args.warmup + args.steps + L - 1) // L
        plan = [prepare(lay, per_layer) for lay in layers]
        order = [plan[i % L][i // L] for i in range(args.warmup + args.steps)]
        for i in range(args.warmup):
            order[i]()
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if args.hold_us > 0:
            hold(attn, args.hold_us)
        w0 = time.perf_counter()
        ev0.record(attn)
        for i in range(args.warmup, args.warmup + args.steps):
            order[i]()
        issued = time.perf_counter() - w0
        if sel is not None:
            attn.wait_stream(sel)
        ev1.record(attn)
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        if args.hold_us > 0:
            hold(attn, 1.0)  # a marker in kernel traces: the timed steps end here
        for i in range(args.warmup + args.steps):  # the layers' state moves on
            lay = layers[i % L]
            lay["cur"], lay["t"] = 1 - lay["cur"], lay["t"] + 1
        return ev0.elapsed_time(ev1), wall * 1e3, issued * 1e3

    def time_cpp_loop():
        import ctypes
        drv = driver()
        P = ctypes.c_void_p

        class Layer(ctypes.Structure):
            _fields_ = [("qs", P), ("q_hist", P), ("newest", P), ("len", P), ("k", P), ("v", P),
                        ("seq_lens", P), ("idx", P * 2), ("nsel", P * 2), ("ev", P * 2), ("out", P), ("ws", P),
                        ("ws_bytes", ctypes.c_size_t), ("cur", ctypes.c_int32), ("t", ctypes.c_int32)]

        arr = (Layer * L)()
        for i, lay in enumerate(layers):
            arr[i] = Layer(lay["qs"].data_ptr(), lay["q_hist"].data_ptr(), lay["newest"].data_ptr(),
                           lay["length"].data_ptr(), lay["k"].data_ptr(), lay["v"].data_ptr(),
                           lay["seq_lens"].data_ptr(), (P * 2)(*[x.data_ptr() for x in lay["idx"]]),
                           (P * 2)(*[x.data_ptr() for x in lay["nsel"]]),
                           (P * 2)(*[e.handle.value for e in lay["ev"]]), out.data_ptr(), lay["ws"].data_ptr(),
                           lay["ws"].numel(), lay["cur"], lay["t"])
        times = (ctypes.c_double * 3)()
        drv.bench_rotation.argtypes = [P, P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P, ctypes.c_double,
                                       P]
        drv.bench_rotation.restype = ctypes.c_int
        rc = drv.bench_rotation(None if ctx is None else ctx.handle, ctypes.byref(dims), ctypes.byref(cfg), arr, L,
                                args.warmup, args.steps, attn.cuda_stream, None if sel is None else sel.cuda_stream,
                                args.hold_us, times)
        if rc != 0:
            raise RuntimeError("bench_rotation failed: %d" % rc)
        for i, lay in enumerate(layers):
            lay["cur"], lay["t"] = arr[i].cur, arr[i].t
        return times[0], times[1], times[2]

    attn.wait_stream(torch.cuda.current_stream())
    loops = {}
    for name in drivers:
        gpu_ms, wall_ms, issue_ms = (time_python_loop if name == "python" else time_cpp_loop)()
        # with a hold before the loop the wall time includes it: the events alone time the steps
        per = (gpu_ms if args.hold_us > 0 else max(gpu_ms, wall_ms)) / args.steps
        loops[name] = {"ms_per_step": round(per, 5), "steps_per_s": round(1e3 / per, 2),
                       "events_ms_per_step": round(gpu_ms / args.steps, 5),
                       "wall_ms_per_step": round(wall_ms / args.steps, 5),
                       "host_issue_ms_per_step": round(issue_ms / args.steps, 5),
                       "host_issue_frac": round(issue_ms / max(gpu_ms, wall_ms), 3)}
        log("%s loop, timed %d steps: %.4f ms/step (events %.4f, wall %.4f, host issue %.4f)"
            % (name, args.steps, per, gpu_ms / args.steps, wall_ms / args.steps, issue_ms / args.steps))
    ms_per_step = loops["python"]["ms_per_step"]
    steps_per_s = 1e3 / ms_per_step
    lens_list = [int(x) for x in layers[0]["seq_lens"].tolist()]
    nbytes = step_bytes(wl, lens_list)

    # Per-kernel timing: each entry point launched alone, back to back on one
    # stream, over the rotating KV caches, bracketed by events on that stream.
    # The warm-up calls go through the binding (which checks the arguments);
    # the timed calls are the same C calls with their arguments marshalled
    # once, so that the host issues them faster than the GPU runs them.
    def time_entry(fn, n, raw=None):
        for i in range(5):
            fn(i)
        calls = [raw(i) for i in range(L)] if raw is not None else None
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(attn)
        for i in range(n):
            if calls is not None:
                calls[i % L]()
            else:
                fn(i)
        e1.record(attn)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n  # us per launch

    # Each layer's predicted query from its ring as the steps left it, so that
    # the candidate launches see the hints of that layer's steady state.
    q_pred = [torch.empty((B, Hq, D), dtype=torch.float32, device=dev) for _ in range(L)]
    scores = torch.empty((B, Hkv, wl.t_cap), dtype=torch.float32, device=dev)
    idx_t = torch.empty((B, Hkv, C), dtype=torch.int32, device=dev)
    nsel_t = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    ws_sel = torch.empty(A.asp_workspace_size(dims, cfg, A.OP_SELECT), dtype=torch.uint8, device=dev)
    for l, lay in enumerate(layers):
        A.asp_predict_query(dims, cfg, lay["q_hist"], lay["newest"], lay["length"], q_pred[l], stream=attn)
    n = args.kernel_launches

    def lay_(i):
        return layers[i % L]

    def rc(name, *a):
        return raw_call(A, name, *a)

    kern = {
        "predict_us": time_entry(
            lambda i: A.asp_predict_query(dims, cfg, lay_(i)["q_hist"], lay_(i)["newest"], lay_(i)["length"],
                                          q_pred[i % L], stream=attn), n,
            lambda i: rc("asp_predict_query", dims, cfg, lay_(i)["q_hist"], lay_(i)["newest"], lay_(i)["length"],
                         q_pred[i], attn)),
        # the step's score launch: keys at or above the layer's hints kept as candidates
        "score_us": time_entry(
            lambda i: A.asp_score_candidates(dims, cfg, q_pred[i % L], lay_(i)["k"], lay_(i)["seq_lens"],
                                             ws_step[i % L], stream=attn), n,
            lambda i: rc("asp_score_candidates", dims, cfg, q_pred[i], lay_(i)["k"], lay_(i)["seq_lens"], ws_step[i],
                         ws_step[i].numel(), attn)),
        "select_us": time_entry(
            lambda i: A.asp_select_candidates(dims, cfg, q_pred[i % L], lay_(i)["k"], lay_(i)["seq_lens"], idx_t,
                                              nsel_t, ws_step[i % L], stream=attn), n,
            lambda i: rc("asp_select_candidates", dims, cfg, q_pred[i], lay_(i)["k"], lay_(i)["seq_lens"], idx_t,
                         nsel_t, ws_step[i], ws_step[i].numel(), attn)),
        # the score-row route of the standalone entry points, for comparison
        "score_keys_us": time_entry(
            lambda i: A.asp_score_keys(dims, q_pred[i % L], lay_(i)["k"], lay_(i)["seq_lens"], scores, stream=attn),
            n, lambda i: rc("asp_score_keys", dims, q_pred[i], lay_(i)["k"], lay_(i)["seq_lens"], scores, None, attn)),
        "select_topc_us": time_entry(
            lambda i: A.asp_select_topc(dims, cfg, scores, layers[0]["seq_lens"], idx_t, nsel_t, ws_sel,
                                        stream=attn), n,
            lambda i: rc("asp_select_topc", dims, cfg, scores, None, layers[0]["seq_lens"], idx_t, nsel_t, ws_sel,
                         ws_sel.numel(), attn)),
        "attend_us": time_entry(
            lambda i: A.asp_sparse_decode(dims, cfg, lay_(i)["qs"][0], lay_(i)["k"], lay_(i)["v"],
                                          lay_(i)["seq_lens"], lay_(i)["idx"][0], lay_(i)["nsel"][0], out, ws_dec,
                                          stream=attn), n,
            lambda i: rc("asp_sparse_decode", dims, cfg, lay_(i)["qs"][0], lay_(i)["k"], lay_(i)["v"],
                         lay_(i)["seq_lens"], lay_(i)["idx"][0], lay_(i)["nsel"][0], out, ws_dec, ws_dec.numel(),
                         attn)),
    }
    sk_bytes = score_kernel_bytes(wl, lens_list)
    achieved = sk_bytes / (kern["score_us"] * 1e-6) / 1e9
    traffic = measured_traffic(SCORE_SOURCES) if headline else None
    in_step = in_step_score_launch_us() if headline and args.mode == "two_streams" else None
    roofline = {"kernel": "score_candidates", "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "algorithmic_bytes_per_launch": sk_bytes, "avg_launch_us": round(kern["score_us"], 2),
                # the same launch inside the overlapped steps, where the attention shares HBM with it
                # (kernel trace of the default command, committed in profiles/; null when stale)
                "in_step_avg_launch_us": in_step,
                "in_step_frac": (round(sk_bytes / (in_step * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4) if in_step else None)}
    log("per-kernel us: %s" % json.dumps({k_: round(v_, 2) for k_, v_ in kern.items()}))

    page = None
    if args.page_size > 0 and C % args.page_size == 0:
        page = page_baseline(A, dims, cfg, wl, layers, args.page_size, time_entry, out, ws_dec, attn, n)
        log("page baseline: %s" % json.dumps(page))

    dense = None
    if args.dense_baseline:
        dense = dense_baseline(A, dims, wl, layers, time_entry, out, attn, n)
        if dense is not None:
            # the overlapped step (scan, selection and sparse attention) against dense attention alone
            dense["step_over_dense"] = round(ms_per_step * 1e3 / dense["attend_us"], 3)
            dense["sparse_attention_over_dense"] = round(kern["attend_us"] / dense["attend_us"], 3)
        log("dense baseline: %s" % json.dumps(dense))

    cpu = None
    if not args.no_cpu_baseline:
        lay = layers[0]
        torch.cuda.synchronize()
        cpu = cpu_baseline(wl, lay, lay["qs"][lay["t"]])
        log("cpu baseline: %s" % json.dumps(cpu))

    rec = {
        "metric": METRIC, "value": round(steps_per_s, 2), "unit": "steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "arithmetic": "bf16 K/V; score: bf16 MFMA on hi+lo bf16 terms of the fp32 predicted query, fp32 "
                      "accumulate; attention: fp32 softmax and accumulation; predictor: fp64 Gram and solve",
        "config": {"workload": wl.name, "batch": B, "n_q_heads": Hq, "n_kv_heads": Hkv, "head_dim": D,
                   "context": wl.t_cap, "top_c": C, "window": wl.window, "recent": wl.recent, "kv_dtype": "bf16",
                   "kv_buffers": L, "mode": args.mode,
                   **({"context_range": list(wl.seq_len_range)} if wl.seq_len_range else {})},
        "achieved_GBps": round(nbytes["score_select_attend"] * steps_per_s / 1e9, 1),
        "achieved_GBps_full_step": round(nbytes["full_step"] * steps_per_s / 1e9, 1),
        "bytes_per_step": nbytes,
        # the same timed loop issued by the Python binding (value) and from C++ (bench_driver.cpp)
        "loops": loops,
        "hw_queues": os.environ.get("GPU_MAX_HW_QUEUES", "HIP default"),
        "hold_us": args.hold_us,
        "kernels_us": {k_: round(v_, 2) for k_, v_ in kern.items()},
        "roofline": roofline,
        "page_baseline": page,
        "dense_baseline": dense,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
