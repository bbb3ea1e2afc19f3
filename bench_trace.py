"""Summaries of rocprofv3 output for profiles/ (small JSON; the raw CSVs stay
on the machine that took them).

  python3 bench_trace.py trace DIR OUT.json
      DIR holds a --kernel-trace [--stats] run of bench.py with --hold-us.
      Per kernel: the launches of the timed steps (from the end of the
      first bench_hold kernel to the start of the short one bench.py launches
      after the timed steps; for traces without it, to 1 ms after the last
      step score launch, which runs on a queue other than the held attention
      stream) and those of the per-entry-point timing loops after them (calls, average, median, min,
      max in us); on the score launches' queue, the median period and the
      median gap between consecutive step score launches, the median time
      from the end of each score launch's own predictor launch to its start
      and the share of score launches whose predictor ended after the
      previous score launch; on the attention queue, the median chain of a step (predictor
      start to the end of the step's last launch there) and the median idle
      time before each predictor launch.
  python3 bench_trace.py pmc DIR COUNTER OUT.json
      DIR holds a --pmc COUNTER run: per kernel, the dispatches and the
      median counter value per dispatch (KiB for FETCH_SIZE / WRITE_SIZE).
"""
import csv
import glob
import json
import os
import statistics as st
import sys
from collections import defaultdict


def _name(n: str) -> str:
    n = n.replace("void ", "")
    return n.split("(")[0] if "(" in n else n


def _stats(v):
    return {"calls": len(v), "avg_us": round(st.mean(v), 2), "median_us": round(st.median(v), 2),
            "min_us": round(min(v), 2), "max_us": round(max(v), 2)}


def trace(d: str, out: str) -> None:
    f = glob.glob(os.path.join(d, "*kernel_trace.csv"))[0]
    ks = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), _name(r["Kernel_Name"]), int(r["Queue_Id"]))
                for r in csv.DictReader(open(f)))
    res = {}
    holds = [k for k in ks if "hold_kernel" in k[2]]
    steps = [k for k in ks if "score_mfma_kernel<" in k[2] and k[2].endswith(", 1>")]
    if holds and steps:
        h_end, attn_q = holds[0][1], holds[0][3]
        # the timed steps end where bench.py's marker (a second, short hold)
        # starts; without one, 1 ms after the last step score launch
        marker = holds[1][0] if len(holds) > 1 else None
        sl = [k for k in steps if k[0] >= h_end and k[3] != attn_q and (marker is None or k[0] < marker)]
        hi = marker if marker is not None else (sl[-1][1] + 1_000_000 if sl else h_end)
        in_step, rest = defaultdict(list), defaultdict(list)
        for k in ks:
            if "hold_kernel" in k[2]:
                continue
            if h_end <= k[0] <= hi:
                in_step[k[2]].append((k[1] - k[0]) / 1000)
            elif k[0] > hi:
                rest[k[2]].append((k[1] - k[0]) / 1000)
        gaps = [(sl[i + 1][0] - sl[i][1]) / 1000 for i in range(len(sl) - 1)]
        periods = [(sl[i + 1][0] - sl[i][0]) / 1000 for i in range(len(sl) - 1)]
        res["score_queue"] = {"step_score_launches": len(sl),
                              "period_median_us": round(st.median(periods), 2) if periods else None,
                              "gap_median_us": round(st.median(gaps), 2) if gaps else None}
        # What each step score launch waited for: its own predictor launch
        # (the i-th of the timed steps on the attention queue; score launch i
        # uses prediction i) or the previous score launch.
        preds = [k for k in ks if "predict_kernel" in k[2] and k[3] == attn_q and h_end <= k[0] <= hi]
        after_pred, pred_last = [], 0
        for i in range(1, min(len(sl), len(preds))):
            after_pred.append((sl[i][0] - preds[i][1]) / 1000)
            pred_last += preds[i][1] > sl[i - 1][1]
        aq = [k for k in ks if k[3] == attn_q and h_end <= k[0] <= hi and "hold_kernel" not in k[2]]
        idle, chain = [], []
        for j, k in enumerate(aq):
            if "predict_kernel" not in k[2]:
                continue
            if j > 0:
                idle.append((k[0] - aq[j - 1][1]) / 1000)
            nxt = next((m for m in range(j + 1, len(aq)) if "predict_kernel" in aq[m][2]), len(aq))
            chain.append((aq[nxt - 1][1] - k[0]) / 1000)
        if after_pred:
            res["score_queue"]["pred_end_to_score_start_median_us"] = round(st.median(after_pred), 2)
            res["score_queue"]["pred_ended_after_previous_score"] = round(pred_last / len(after_pred), 3)
        if chain:
            res["attn_queue"] = {"chain_median_us": round(st.median(chain), 2),
                                 "idle_before_predictor_median_us": round(st.median(idle), 2) if idle else None}
        res["in_step"] = {n: _stats(v) for n, v in in_step.items()}
        res["standalone"] = {n: _stats(v) for n, v in rest.items()}
    allk = defaultdict(list)
    for k in ks:
        allk[k[2]].append((k[1] - k[0]) / 1000)
    res["all"] = {n: _stats(v) for n, v in allk.items()}
    with open(out, "w") as fo:
        json.dump(res, fo, indent=1)


def pmc(d: str, counter: str, out: str) -> None:
    f = glob.glob(os.path.join(d, "*counter_collection.csv"))[0]
    vals = defaultdict(list)
    for r in csv.DictReader(open(f)):
        if r.get("Counter_Name") == counter:
            vals[_name(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    with open(out, "w") as fo:
        json.dump({"counter": counter,
                   "kernels": {n: {"dispatches": len(v), "median": st.median(v)} for n, v in vals.items()}}, fo,
                  indent=1)


if __name__ == "__main__":
    if sys.argv[1] == "trace":
        trace(sys.argv[2], sys.argv[3])
    elif sys.argv[1] == "pmc":
        pmc(sys.argv[2], sys.argv[3], sys.argv[4])
    else:
        sys.exit(__doc__)
