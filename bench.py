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

Beside the step, the page-level (Quest) baseline is timed on the same layers
("page_baseline"): page scoring with the current query, top C / P pages and
attention over their tokens, all on one stream (--page-size, 0 skips it).

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


def cpu_baseline(wl, layer, q_t) -> dict:
    """The oracle (fp64, plain) timed on the host cores for one full step of one
    layer (all units), on inputs copied back from the device."""
    import numpy as np
    import torch
    import oracle

    k, v = layer["k"], layer["v"]
    kn = k.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    vn = v.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    lens = layer["seq_lens"].cpu().numpy()
    hist = layer["q_hist"].cpu().numpy()
    newest = layer["newest"].cpu().numpy()
    length = layer["length"].cpu().numpy()
    q = q_t.cpu().numpy()
    idx_prev = layer["idx"][layer["cur"]].cpu().numpy()
    n_prev = layer["nsel"][layer["cur"]].cpu().numpy()

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
    per_step = el / reps
    return {"value": 1.0 / per_step, "unit": "steps/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "full step of one layer (all %d units), %d timed repetitions (%.1f s) after 1 warm-up, "
                      "%.3f s each" % (wl.batch * wl.n_kv_heads, reps, el, per_step),
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

    t = {
        "summary_us": time_entry(lambda i: A.asp_page_summary(dims, P, layers[i % L]["k"], layers[i % L]["seq_lens"],
                                                              summ[i % L][0], summ[i % L][1], stream=attn), 20),
        "page_scores_us": time_entry(lambda i: A.asp_page_scores(dims, P, q_of(i), summ[i % L][0], summ[i % L][1],
                                                                 layers[i % L]["seq_lens"], pscores, stream=attn), n),
        "page_select_us": time_entry(lambda i: A.asp_page_select(dims, cfg, P, q_of(i), summ[i % L][0],
                                                                 summ[i % L][1], layers[i % L]["seq_lens"], idx, nsel,
                                                                 ws, stream=attn), n),
        "step_us": time_entry(page_step, n),
    }
    lens = [int(x) for x in layers[0]["seq_lens"].tolist()]
    esize = 2 if wl.kv_dtype == "bf16" else 4
    scan = sum(Hkv * ((T + P - 1) // P) * D * esize * 2 for T in lens)  # kmin + kmax rows read
    res = {k_: round(v_, 2) for k_, v_ in t.items()}
    res.update({"page_size": P, "pages_kept": C // P, "summary_bytes_read_per_step": scan,
                "page_scores_GBps": round(scan / (t["page_scores_us"] * 1e-6) / 1e9, 1),
                "steps_per_s": round(1e6 / t["step_us"], 1)})
    return res


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
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (rocprofv3 counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the sparse decode step here runs on a single device "
              "(--gpus %d was requested)" % args.gpus, file=sys.stderr)
        return 2

    # The pipelined step keeps four streams busy at once (attention, predictor,
    # score pass, selection) beside the default stream; each needs a hardware
    # queue of its own, or streams that share one run in submission order.
    # HIP reads this at its first call (its default is 4 queues per process).
    os.environ["GPU_MAX_HW_QUEUES"] = str(max(8, int(os.environ.get("GPU_MAX_HW_QUEUES", "4"))))
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
    n_layer_steps = (args.warmup + args.steps) // L + 2
    attn = torch.cuda.Stream()
    sel = torch.cuda.Stream() if args.mode == "two_streams" else None
    # one step workspace per layer, as a decode loop over layers keeps them
    ws_step = [torch.empty(A.asp_workspace_size(dims, cfg, A.OP_STEP), dtype=torch.uint8, device=dev)
               for _ in range(L)]
    ws_dec = torch.empty(A.asp_workspace_size(dims, cfg, A.OP_DECODE), dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    q_ready = A.HipEvent()

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
                   ev=[A.HipEvent(), A.HipEvent()], cur=0, t=wl.history_steps)
        for t in range(wl.history_steps - 1):
            A.asp_push_query(dims, cfg, qs[t], q_hist, newest, length)
        # bootstrap step: selection made from the ring, attended at once
        A.asp_step(dims, cfg, qs[wl.history_steps - 1], q_hist, newest, length, k, v, lens, None, None,
                   lay["idx"][0], lay["nsel"][0], out, ws_step[l], idx_next_ready=lay["ev"][0])
        layers.append(lay)
    torch.cuda.synchronize()
    log("setup: %d KV caches of %.2f GiB (K+V) in %.1f s" % (L, 2 * k.numel() * 2 / 2**30, time.perf_counter() - t0))

    def one_step(i):
        lay = layers[i % L]
        cur = lay["cur"]
        nxt = 1 - cur
        q = lay["qs"][lay["t"]]
        A.asp_step(dims, cfg, q, lay["q_hist"], lay["newest"], lay["length"], lay["k"], lay["v"], lay["seq_lens"],
                   lay["idx"][cur], lay["nsel"][cur], lay["idx"][nxt], lay["nsel"][nxt], out, ws_step[i % L],
                   attn_stream=attn, sel_stream=sel, q_ready=q_ready, idx_cur_ready=lay["ev"][cur],
                   idx_next_ready=lay["ev"][nxt])
        lay["cur"] = nxt
        lay["t"] += 1

    attn.wait_stream(torch.cuda.current_stream())
    for i in range(args.warmup):
        one_step(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    ev0.record(attn)
    for i in range(args.warmup, args.warmup + args.steps):
        one_step(i)
    issued = time.perf_counter() - w0
    if sel is not None:
        attn.wait_stream(sel)
    ev1.record(attn)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    gpu_ms = ev0.elapsed_time(ev1)
    ms_per_step = max(gpu_ms, wall * 1e3) / args.steps
    steps_per_s = 1e3 / ms_per_step
    lens_list = [int(x) for x in layers[0]["seq_lens"].tolist()]
    nbytes = step_bytes(wl, lens_list)
    log("timed %d steps: %.4f ms/step (events %.4f, wall %.4f, host issue %.4f)"
        % (args.steps, ms_per_step, gpu_ms / args.steps, wall * 1e3 / args.steps, issued * 1e3 / args.steps))

    # Per-kernel timing: each entry point launched alone, back to back on one
    # stream, over the rotating KV caches, bracketed by events on that stream.
    def time_entry(fn, n):
        for i in range(5):
            fn(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(attn)
        for i in range(n):
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
    for l, lay in enumerate(layers):
        A.asp_predict_query(dims, cfg, lay["q_hist"], lay["newest"], lay["length"], q_pred[l], stream=attn)
    n = args.kernel_launches

    def lay_(i):
        return layers[i % L]

    kern = {
        "predict_us": time_entry(lambda i: A.asp_predict_query(dims, cfg, lay_(i)["q_hist"], lay_(i)["newest"],
                                                               lay_(i)["length"], q_pred[i % L], stream=attn), n),
        # the step's score launch: keys at or above the layer's hints kept as candidates
        "score_us": time_entry(lambda i: A.asp_score_candidates(dims, cfg, q_pred[i % L], lay_(i)["k"],
                                                                lay_(i)["seq_lens"], ws_step[i % L], stream=attn), n),
        "select_us": time_entry(lambda i: A.asp_select_candidates(dims, cfg, q_pred[i % L], lay_(i)["k"],
                                                                  lay_(i)["seq_lens"], idx_t, nsel_t, ws_step[i % L],
                                                                  stream=attn), n),
        # the score-row route of the standalone entry points, for comparison
        "score_keys_us": time_entry(lambda i: A.asp_score_keys(dims, q_pred[i % L], lay_(i)["k"],
                                                               lay_(i)["seq_lens"], scores, stream=attn), n),
        "select_topc_us": time_entry(lambda i: A.asp_select_topc(dims, cfg, scores, layers[0]["seq_lens"], idx_t,
                                                                 nsel_t, stream=attn), n),
        "attend_us": time_entry(lambda i: A.asp_sparse_decode(dims, cfg, layers[i % L]["qs"][0], layers[i % L]["k"],
                                                              layers[i % L]["v"], layers[i % L]["seq_lens"],
                                                              layers[i % L]["idx"][0],
                                                              layers[i % L]["nsel"][0], out, ws_dec, stream=attn), n),
    }
    sk_bytes = score_kernel_bytes(wl, lens_list)
    achieved = sk_bytes / (kern["score_us"] * 1e-6) / 1e9
    traffic = measured_traffic(SCORE_SOURCES) if headline else None
    roofline = {"kernel": "score_candidates", "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "algorithmic_bytes_per_launch": sk_bytes, "avg_launch_us": round(kern["score_us"], 2)}
    log("per-kernel us: %s" % json.dumps({k_: round(v_, 2) for k_, v_ in kern.items()}))

    page = None
    if args.page_size > 0 and C % args.page_size == 0:
        page = page_baseline(A, dims, cfg, wl, layers, args.page_size, time_entry, out, ws_dec, attn, n)
        log("page baseline: %s" % json.dumps(page))

    cpu = None
    if not args.no_cpu_baseline:
        lay = layers[0]
        torch.cuda.synchronize()
        cpu = cpu_baseline(wl, lay, lay["qs"][lay["t"]])
        log("cpu baseline: %s" % json.dumps(cpu))

    rec = {
        "metric": METRIC, "value": round(steps_per_s, 2), "unit": "steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "n_q_heads": Hq, "n_kv_heads": Hkv, "head_dim": D,
                   "context": wl.t_cap, "top_c": C, "window": wl.window, "recent": wl.recent, "kv_dtype": "bf16",
                   "kv_buffers": L, "mode": args.mode,
                   **({"context_range": list(wl.seq_len_range)} if wl.seq_len_range else {})},
        "achieved_GBps": round(nbytes["score_select_attend"] * steps_per_s / 1e9, 1),
        "achieved_GBps_full_step": round(nbytes["full_step"] * steps_per_s / 1e9, 1),
        "bytes_per_step": nbytes,
        "kernels_us": {k_: round(v_, 2) for k_, v_ in kern.items()},
        "roofline": roofline,
        "page_baseline": page,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
