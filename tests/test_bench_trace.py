"""bench_trace.py's summary of a kernel trace (CPU only): on a synthetic trace
whose timings are known, the timed steps are the launches between the end of
the first hold and the start of bench.py's marker (the second hold), the
launches after the marker are the standalone ones, and the score queue's
period, gap and predictor lead are the ones laid out."""
import csv
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench_trace  # noqa: E402

SCORE = "void asp::score_mfma_kernel<128, 4, false, 1>(float const*, ...)"
PRED = "void asp::predict_kernel<15, 128>(float*, ...)"
ATT = "void asp::attend_mfma_kernel<128, 4, false>(float const*, ...)"
HOLD = "hold_kernel(long long)"
ATTN_Q, SCORE_Q = 1, 2


def _write(tmp_path, rows):
    d = tmp_path / "trace"
    d.mkdir()
    with open(d / "t_kernel_trace.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Queue_Id"])
        w.writeheader()
        for name, t0, t1, q in rows:
            w.writerow({"Kernel_Name": name, "Start_Timestamp": t0, "End_Timestamp": t1, "Queue_Id": q})
    return str(d)


def _synthetic(n_steps, marker):
    """A hold of 1 ms, then n_steps steps of period 100 us (ns timestamps): a
    10 us predictor at the period's start on the attention queue, a 20 us
    attention after it, and an 85 us score launch starting 40 us after the
    predictor ends on the score queue; then (after the marker, if any) five
    standalone launches of each kernel, 1 us apart, within 1 ms of the last
    score launch."""
    us = 1000
    rows = [(HOLD, 0, 1000 * us, ATTN_Q)]
    t = 1000 * us
    for s in range(n_steps):
        p0 = t + s * 100 * us
        rows.append((PRED, p0, p0 + 10 * us, ATTN_Q))
        rows.append((ATT, p0 + 10 * us, p0 + 30 * us, ATTN_Q))
        rows.append((SCORE, p0 + 50 * us, p0 + 135 * us, SCORE_Q))
    t_end = t + n_steps * 100 * us + 40 * us
    if marker:
        rows.append((HOLD, t_end, t_end + 1 * us, ATTN_Q))
    t = t_end + 2 * us
    for name, dur in ((PRED, 8), (SCORE, 80), (ATT, 15)):
        for _ in range(5):
            rows.append((name, t, t + dur * us, ATTN_Q))
            t += (dur + 1) * us
    return rows


def test_marker_splits_timed_steps_from_standalone_launches(tmp_path):
    d = _write(tmp_path, _synthetic(20, marker=True))
    out = str(tmp_path / "s.json")
    bench_trace.trace(d, out)
    r = json.load(open(out))
    pred, att, score = "asp::predict_kernel<15, 128>", "asp::attend_mfma_kernel<128, 4, false>", \
        "asp::score_mfma_kernel<128, 4, false, 1>"
    assert r["in_step"][pred]["calls"] == 20 and r["in_step"][pred]["avg_us"] == 10.0
    assert r["in_step"][att]["calls"] == 20 and r["in_step"][att]["avg_us"] == 20.0
    assert r["in_step"][score]["calls"] == 20 and r["in_step"][score]["avg_us"] == 85.0
    assert r["standalone"][pred]["calls"] == 5 and r["standalone"][pred]["avg_us"] == 8.0
    assert r["standalone"][score]["calls"] == 5 and r["standalone"][score]["avg_us"] == 80.0
    q = r["score_queue"]
    assert q["step_score_launches"] == 20
    assert q["period_median_us"] == 100.0 and q["gap_median_us"] == 15.0
    assert q["pred_end_to_score_start_median_us"] == 40.0 and q["pred_ended_after_previous_score"] == 0.0


def test_without_a_marker_the_standalone_launches_leak_into_the_steps(tmp_path):
    # The fallback window (1 ms past the last step score launch) takes in the
    # standalone launches that start inside it: the reason for the marker.
    d = _write(tmp_path, _synthetic(20, marker=False))
    out = str(tmp_path / "s.json")
    bench_trace.trace(d, out)
    r = json.load(open(out))
    assert r["in_step"]["asp::predict_kernel<15, 128>"]["calls"] == 25
