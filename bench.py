"""Benchmark of the HiLS attention hot path on one MI355X.

Headline: the 7B-class GQA prefill (B=1, H=32 query heads over 8 kv heads,
d=128, T=32768, S=64, K=16, bf16 storage, float32 accumulation), the largest
prefill workload that fits one GPU. One step is the whole forward: landmark
summaries, chunk scoring + top-K, intra-chunk attention + inter-chunk fusion,
with inputs resident in HBM.

Also measured, each with a roofline block for its kernels: the 345M-class
prefill (B=1, H=16, d=64, T=8192), 128K-context decode (256 steps of
hils_decode under a HIP graph, with incremental summaries), the training step
(B=2, T=16384: forward + backward), and variants (group-max selection, the
pages' main setting K=32 with a 512-key window, Q-Cal, a host-resident decode
cache, 16 query rows per decode call).

Kernel durations come from HIP events recorded on the stream the kernels run
on. The CPU oracle (one thread, -O3 -march=native, compiled on the machine that
runs it) is timed on bounded samples of each workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       python bench.py --pmc-run WORKLOAD            (a short run for rocprofv3 --pmc)
       python bench.py --traffic WORKLOAD FETCH_CSV WRITE_CSV   (counter CSVs -> record)
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import tempfile
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP32_VECTOR_PEAK_TFLOPS = 157.3

ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(ROOT, "profiles")
CSRC = "hierarchical_sparse_attention_amd/csrc/"
COPY_BYTES = 256 << 20  # calibration copy: 256 MiB read + 256 MiB written

# kernels behind each measured call, and the sources they are built from (a
# counter record is used only while those sources are unchanged)
CALL_KERNELS = {
    "summarize": (("k_summarize",), ("k_summarize.hip", "hils_internal.h")),
    "score_topk": (("k_ksplit", "k_score_mfma"),
                   ("k_score_mfma.hip", "k_score_topk.hip", "mfma_common.h", "hils_internal.h")),
    "attend_fuse": (("k_kv_prep", "k_attend_mfma"),
                    ("k_attend_mfma.hip", "k_attend_fuse.hip", "hils_internal.h")),
    "decode": (("k_score_split_mfma", "k_decode_merge_partial", "k_decode_combine"),
               ("k_score_mfma.hip", "k_score_topk.hip", "k_attend_fuse.hip", "decode_slot.h",
                "decode_merge.h", "mfma_common.h", "hils_internal.h")),
    "backward": (("k_bwd_rowd", "k_sel_count", "k_sel_scan", "k_sel_fill", "k_bwd_kv_mfma",
                  "k_dq_reduce"), ("k_backward_mfma.hip", "k_backward.hip", "hils_internal.h")),
}
PMC_WORKLOADS = ("prefill_7b_gqa", "prefill_345m", "decode_128k", "train_345m")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=256)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra-configs", action="store_true",
                    help="only the headline workload and the 128K decode")
    ap.add_argument("--pmc-run", choices=PMC_WORKLOADS,
                    help="run 3 steps of one workload and a calibration copy, for counters")
    ap.add_argument("--traffic", nargs=3, metavar=("WORKLOAD", "FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter CSVs into the workload's record")
    ap.add_argument("--counters", nargs=2, metavar=("WORKLOAD", "DIR"),
                    help="summarise the counter passes DIR/p1..p4 of a --pmc-run of WORKLOAD "
                         "(FETCH_SIZE, WRITE_SIZE, SQ and TCC counters) into profiles/")
    ap.add_argument("--trace", nargs=2, metavar=("WHAT", "STATS_CSV"),
                    help="summarise a rocprofv3 --kernel-trace --stats kernel_stats.csv into "
                         "profiles/kernel_trace_<WHAT>.txt (WHAT: bench_all_workloads for a "
                         "run of bench.py --no-cpu-baseline, bench_headline for one of "
                         "bench.py --no-cpu-baseline --no-extra-configs, or a --pmc-run "
                         "workload)")
    return ap.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- counter records
def sources_hash(call):
    h = hashlib.sha256()
    for rel in CALL_KERNELS[call][1]:
        with open(os.path.join(ROOT, CSRC, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_path(workload):
    return os.path.join(PROFILES, f"traffic_{workload}.json")


def write_traffic_record(workload, fetch_csv, write_csv):
    """HBM bytes per dispatch of every kernel from FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch), each scaled by what the same counter reads for an elementwise copy
    (neg) of COPY_BYTES."""
    import csv

    def per_kernel(path, counter):
        acc = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            key = (r["Kernel_Name"], r["Dispatch_Id"])
            acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
        out = {}
        for (name, _), v in acc.items():
            out.setdefault(name, []).append(v * 1024.0)
        return {k: sum(v) / len(v) for k, v in out.items()}

    fetch, write = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")

    def copy_reading(d):
        vals = [v for k, v in d.items() if "neg" in k]
        return vals[0] if vals else None

    f_scale, w_scale = COPY_BYTES / copy_reading(fetch), COPY_BYTES / copy_reading(write)
    rec = {"workload": workload, "copy_bytes": COPY_BYTES, "fetch_scale": f_scale,
           "write_scale": w_scale, "sources_hash": {c: sources_hash(c) for c in CALL_KERNELS},
           "kernels": {}}
    for name in sorted(set(fetch) | set(write)):
        if "neg" in name:
            continue
        short = (name.replace("void ", "").replace("hils::(anonymous namespace)::", "")
                 .split("(")[0].split("<")[0].split("::")[-1].strip())
        rec["kernels"][name] = {"short": short,
                                "fetch_bytes": fetch.get(name, 0.0) * f_scale,
                                "write_bytes": write.get(name, 0.0) * w_scale}
    os.makedirs(PROFILES, exist_ok=True)
    with open(traffic_path(workload), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


PMC_PASSES = ("FETCH_SIZE", "WRITE_SIZE",
              "SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA SQ_INSTS_VALU SQ_INSTS_VALU_TRANS_F32 "
              "SQ_BUSY_CYCLES SQ_WAVES GRBM_GUI_ACTIVE",
              "TCC_HIT_sum TCC_MISS_sum SQ_WAIT_INST_ANY SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT")


def write_counter_summary(workload, directory):
    """profiles/counters_<workload>.txt: per kernel of a --pmc-run, the average per
    dispatch of every counter of the four passes, the dispatch duration and derived
    figures; and the traffic record from passes 1 and 2."""
    import csv
    import glob

    def load(i):
        path = glob.glob(os.path.join(directory, f"p{i}", "*counter_collection.csv"))[0]
        return path, list(csv.DictReader(open(path)))

    per = {}   # kernel -> counter -> [values]
    dur = {}
    for i in range(1, 5):
        _, rows = load(i)
        acc = {}
        for r in rows:
            key = (r["Kernel_Name"], r["Dispatch_Id"])
            acc.setdefault(key, {"name": r["Kernel_Name"], "c": {}, "t": (int(r["Start_Timestamp"]), int(r["End_Timestamp"])), "vgpr": r["VGPR_Count"], "lds": r["LDS_Block_Size"]})
            acc[key]["c"][r["Counter_Name"]] = acc[key]["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        for v in acc.values():
            d = per.setdefault(v["name"], {})
            for cn, cv in v["c"].items():
                d.setdefault(cn, []).append(cv)
            if i == 3:
                dur.setdefault(v["name"], []).append((v["t"][1] - v["t"][0]) / 1e3)
            d.setdefault("_vgpr", [v["vgpr"]])
            d.setdefault("_lds", [v["lds"]])
    write_traffic_record(workload, load(1)[0], load(2)[0])
    rec = json.load(open(traffic_path(workload)))
    scale = {"FETCH_SIZE": rec["fetch_scale"], "WRITE_SIZE": rec["write_scale"]}
    lines = [f"rocprofv3 counters per kernel, {workload} (bench.py --pmc-run {workload}: the "
             f"workload's inputs, 3 steps, then a 256 MiB elementwise copy for calibration), MI355X",
             "commands, one pass each (cd /tmp && export TMPDIR=/tmp first):"]
    for i, c in enumerate(PMC_PASSES, 1):
        lines.append(f"  timeout -s KILL 240 rocprofv3 --pmc {c} --output-format csv -d <dir>/p{i} "
                     f"-o pmc -- python3 bench.py --pmc-run {workload}")
    lines.append(f"  python3 bench.py --counters {workload} <dir>   (writes this file and "
                 f"traffic_{workload}.json)")
    lines.append(f"FETCH_SIZE / WRITE_SIZE are scaled to bytes by the calibration copy "
                 f"(fetch x{rec['fetch_scale']:.3f}, write x{rec['write_scale']:.3f}); other "
                 "counters are raw sums over the GPU per dispatch, averaged over dispatches.")
    lines.append("GRBM_GUI_ACTIVE is summed over the 8 XCDs: cycles = GRBM_GUI_ACTIVE / 8, and "
                 "MHz = cycles / us (the clock the kernel ran at; for kernels of a few tens of us "
                 "the count also takes in time around the dispatch, so MHz and mfma_busy are only "
                 "meaningful for the long ones); mfma_busy = "
                 "SQ_VALU_MFMA_BUSY_CYCLES (summed over SIMDs) / (cycles x 256 CUs x 4 SIMDs); "
                 "l2_hit = TCC_HIT / (TCC_HIT + TCC_MISS); us = dispatch duration in pass 3.")
    lines.append("")
    hdr = (f"{'kernel':44s} {'calls':>5s} {'us':>9s} {'fetch MB':>9s} {'write MB':>9s} "
           f"{'MHz':>5s} {'mfma_busy':>9s} {'MFMA inst':>10s} {'VALU inst':>11s} {'TRANS':>10s} {'l2_hit':>7s} "
           f"{'LDS inst':>10s} {'LDS bkcf':>10s} {'vgpr':>5s}")
    lines.append(hdr)
    avg = lambda xs: sum(xs) / len(xs) if xs else float("nan")  # noqa: E731
    order = sorted(per, key=lambda k: -avg(dur.get(k, [0])) * len(dur.get(k, [0])))
    for name in order:
        if "neg" in name:
            continue
        d = per[name]
        short = (name.replace("void ", "").replace("hils::(anonymous namespace)::", "")
                 .replace("at::native::", "").split("(")[0])
        g = avg(d.get("GRBM_GUI_ACTIVE", [])) / 8  # one instance per XCD
        busy = avg(d.get("SQ_VALU_MFMA_BUSY_CYCLES", [])) / (g * 256 * 4) if g else float("nan")
        mhz = g / avg(dur.get(name, [])) if g and dur.get(name) else float("nan")
        hit, miss = avg(d.get("TCC_HIT_sum", [])), avg(d.get("TCC_MISS_sum", []))
        l2 = hit / (hit + miss) if hit + miss else float("nan")
        lines.append(
            f"{short[:44]:44s} {len(dur.get(name, [])):5d} {avg(dur.get(name, [])):9.2f} "
            f"{avg(d.get('FETCH_SIZE', [])) * 1024 * scale['FETCH_SIZE'] / 1e6:9.2f} "
            f"{avg(d.get('WRITE_SIZE', [])) * 1024 * scale['WRITE_SIZE'] / 1e6:9.2f} "
            f"{mhz:5.0f} {busy:9.3f} {avg(d.get('SQ_INSTS_MFMA', [])):10.3g} "
            f"{avg(d.get('SQ_INSTS_VALU', [])):11.4g} {avg(d.get('SQ_INSTS_VALU_TRANS_F32', [])):10.3g} "
            f"{l2:7.3f} {avg(d.get('SQ_INSTS_LDS', [])):10.3g} "
            f"{avg(d.get('SQ_LDS_BANK_CONFLICT', [])):10.3g} {d['_vgpr'][0]:>5s}")
    out = os.path.join(PROFILES, f"counters_{workload}.txt")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def write_trace_summary(what, stats_csv):
    """profiles/kernel_trace_<what>.txt: per kernel, calls and duration statistics
    from a rocprofv3 --kernel-trace --stats run."""
    import csv
    if what == "bench_all_workloads":
        desc = ("one bench.py run: every workload and variant of the bench (7B GQA prefill "
                "headline, 128K decode with K=16, K=32 + 512-key window, pinned host cache, 16 "
                "positions per call and 16 sequences together, 345M prefill, 7B with group-max "
                "selection, 345M main setting, training step plain / Q-Cal / main setting); per "
                "kernel over all calls of the run (the per-workload figures are in bench.py's "
                "JSON line)")
        cmd = "python3 bench.py --no-cpu-baseline"
    elif what == "bench_headline":
        desc = ("the bench's headline run: the 7B GQA prefill steps with per-head selection "
                "(warmup and timed steps), then the 128K decode with K=16, its graph replays "
                "and eager steps; k_attend_mfma<128, false> here is the headline's attention "
                "launch alone")
        cmd = "python3 bench.py --no-cpu-baseline --no-extra-configs"
    else:
        desc = (f"bench.py --pmc-run {what}: the workload's inputs, one forward call of each "
                "kernel, then 3 steps and a 256 MiB elementwise copy")
        cmd = f"python3 bench.py --pmc-run {what}"
    lines = [f"rocprofv3 kernel trace on MI355X (gfx950) of {desc}.",
             "command: cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats "
             f"--output-format csv -d <dir> -o t -- {cmd}",
             f"then: python3 bench.py --trace {what} <dir>/t_kernel_stats.csv",
             "median_us: the median dispatch (from t_kernel_trace.csv beside the stats), which "
             "leaves out the first, cold calls", "",
             f"{'kernel':60s} {'calls':>8s} {'avg_us':>10s} {'median_us':>10s} {'min_us':>10s} "
             f"{'max_us':>10s} {'total_ms':>10s}"]
    durs = {}
    trace_csv = stats_csv.replace("kernel_stats", "kernel_trace")
    if os.path.exists(trace_csv):
        for r in csv.DictReader(open(trace_csv)):
            durs.setdefault(r["Kernel_Name"], []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    for r in csv.DictReader(open(stats_csv)):
        n = r["Name"].replace("void ", "").replace("hils::(anonymous namespace)::", "")
        n = n.split("(")[0] if not n.startswith("__amd") else n
        med = float(np.median(durs[r["Name"]])) if r["Name"] in durs else float("nan")
        lines.append(f"{n[:60]:60s} {int(r['Calls']):8d} {float(r['AverageNs']) / 1e3:10.2f} "
                     f"{med:10.2f} {float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} "
                     f"{float(r['TotalDurationNs']) / 1e6:10.2f}")
    out = os.path.join(PROFILES, f"kernel_trace_{what}.txt")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def call_traffic(workload, call):
    """HBM bytes per call from the committed counter record, or None when there is
    none or the call's kernel sources changed since it was taken."""
    try:
        rec = json.load(open(traffic_path(workload)))
    except (OSError, ValueError):
        return None
    if rec.get("sources_hash", {}).get(call) != sources_hash(call):
        return None
    pats = CALL_KERNELS[call][0]
    tot = [v["fetch_bytes"] + v["write_bytes"] for v in rec["kernels"].values()
           if any(p in v["short"] for p in pats)]
    return sum(tot) if tot else None


# ---------------------------------------------------------------- algorithmic work
def lstart_of(i, S, window):
    return max(0, i - window + 1) if window > 0 else i - i % S


def prefill_counts(w, idx_host, window=0):
    """Per-step algorithmic work of each prefill kernel (bytes the method must move,
    flops it must do; never the dense work it avoids)."""
    B, T, H, Hkv, d, S, K = w.B, w.T, w.H, w.Hkv, w.d, w.S, w.K
    NC = T // S
    esz = 2  # bf16
    sel_pairs = int((idx_host >= 0).sum())                 # (row, selected chunk) pairs
    own_keys = B * H * sum(i - lstart_of(i, S, window) + 1 for i in range(T))
    key_visits = sel_pairs * S + own_keys
    cand = B * H * sum(lstart_of(i, S, window) // S for i in range(T))
    summ_bytes = B * T * Hkv * d * esz + B * NC * H * d * esz + B * NC * H * (d + 2) * 4
    attend_bytes = (2 * B * T * H * d * esz + 2 * B * T * Hkv * d * esz + B * T * H * K * 8
                    + B * T * H * 8)
    return dict(summarize_bytes=summ_bytes, score_flops=2 * d * cand,
                attend_flops=4 * d * key_visits, attend_bytes=attend_bytes,
                backward_flops=10 * d * key_visits, key_visits=key_visits, sel_pairs=sel_pairs,
                candidates=cand)


def decode_step_bytes(wd, K_sel, window, p):
    """Algorithmic HBM bytes of one decode step at position p: the candidates'
    summaries and entropies, the selected chunks' keys and values, the local
    branch's keys and values, the query, output and selection."""
    H, Hkv, d, S = wd.H, wd.Hkv, wd.d, wd.S
    n = lstart_of(p, S, window) // S
    nloc = p - lstart_of(p, S, window) + 1
    return (n * H * (d + 1) * 4 + H * min(K_sel, n) * S * d * 2 * 2 + H * nloc * d * 2 * 2
            + 2 * H * d * 2 + H * K_sel * 8)


def decode_call_unique_bytes(wd, K_sel, window, p, nb, idx):
    """Algorithmic HBM bytes of one decode call of nb consecutive positions p ..
    p + nb - 1 of one sequence (idx [nb, H, K] their selections): the summaries
    and entropies of the last position's candidates once, each selected (head,
    chunk) once however many positions picked it, the keys and values of the
    local branch up to the last position once per head, and the queries,
    outputs and selections of every position."""
    H, d, S = wd.H, wd.d, wd.S
    last = p + nb - 1
    n = lstart_of(last, S, window) // S
    sel = sum(len(np.unique(idx[:, h][idx[:, h] >= 0])) for h in range(H))
    loc = last - lstart_of(p, S, window) + 1
    return (n * H * (d + 1) * 4 + sel * S * d * 2 * 2 + H * loc * d * 2 * 2
            + nb * (2 * H * d * 2 + H * K_sel * 8))


def roofline(kernel, bound, work, ms, traffic=None, note=None):
    """Roofline block: achieved = algorithmic work per launch / launch duration."""
    if bound == "mfma":
        achieved, peak, unit = work / (ms * 1e-3) / 1e12, BF16_PEAK_TFLOPS, "TFLOP/s"
    elif bound == "hbm":
        achieved, peak, unit = work / (ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s"
    else:  # "alu": float32 vector arithmetic
        achieved, peak, unit = work / (ms * 1e-3) / 1e12, FP32_VECTOR_PEAK_TFLOPS, "TFLOP/s"
    b = {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit, "frac": achieved / peak,
         "traffic": traffic, "kernel": kernel, "ms_per_launch": ms, "work_per_launch": work}
    if note:
        b["note"] = note
    return b


# ---------------------------------------------------------------- timing helpers
def make_timers(torch, stream):
    def ev_ms(fn, reps):
        """Average duration of fn over reps calls, HIP events on the kernels' stream."""
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(reps):
            fn()
        ev[1].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / reps

    def wall_ms(fn, reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / reps

    return ev_ms, wall_ms


def prefill_setup(torch, hsa, synth, dev, wname, K=None, group=False, window=0, qcal=False):
    w = synth.workloads()[wname]
    w = dataclasses.replace(w, K=K or w.K)
    log(f"generating {wname} inputs")
    x = synth.make_inputs(w)
    keys = ("Q", "K", "V", "Ql") + (("dO",) if w.need_dO else ())
    t = {k: torch.from_numpy(x[k]).to(dev, torch.bfloat16) for k in keys}
    if qcal:
        t["Qs"] = torch.from_numpy(synth.scoring_query(w, x)).to(dev, torch.bfloat16)
    Qs = t.get("Qs")
    f = hsa.forward(t["Q"], t["K"], t["V"], t["Ql"], w.K, w.S, group=group, Qs=Qs, window=window)
    calls = {
        "summarize": lambda: hsa.summarize(t["K"], t["Ql"], w.S, ksum=f["ksum"], ent=f["ent"],
                                           lse_l=f["lse_l"]),
        "score_topk": lambda: hsa.score_topk(t["Q"] if Qs is None else Qs, f["ksum"], f["ent"],
                                             w.K, w.S, 0, w.T, Hkv=w.Hkv, idx=f["idx"],
                                             score=f["score"], group=group, window=window),
        "attend_fuse": lambda: hsa.attend_fuse(t["Q"], t["K"], t["V"], f["idx"], f["score"],
                                               w.S, O=f["O"], lse_own=f["lse_own"],
                                               lse_tot=f["lse_tot"], window=window),
    }
    if w.need_dO:
        calls["backward"] = lambda: hsa.backward(t["Q"], t["K"], t["V"], t["Ql"], f["ksum"],
                                                 f["ent"], f["lse_l"], f["idx"], f["score"],
                                                 f["lse_tot"], f["O"], t["dO"], w.S, Qs=Qs,
                                                 window=window)
    return w, x, t, f, calls


def time_in_step(torch, stream, calls, reps):
    """Average duration of each call with the calls run in step order (each one
    sees the caches the previous ones left), HIP events between the calls on the
    kernels' stream."""
    names = list(calls)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
           for _ in range(reps)]
    for r in range(reps):
        evs[r][0].record(stream)
        for i, k in enumerate(names):
            calls[k]()
            evs[r][i + 1].record(stream)
    torch.cuda.synchronize()
    return {k: sum(evs[r][i].elapsed_time(evs[r][i + 1]) for r in range(reps)) / reps
            for i, k in enumerate(names)}


def measure_prefill(torch, ev_ms, w, f, calls, reps, workload, window=0, stream=None):
    for fn in calls.values():
        fn()
    torch.cuda.synchronize()
    km = time_in_step(torch, stream, calls, reps)
    # calls of a few tens of microseconds: an event pair around one launch weighs
    # on them, so they are timed over 100 launches back to back
    for k, fn in calls.items():
        if km[k] < 0.1:
            km[k] = ev_ms(fn, 100)
    cnt = prefill_counts(w, f["idx"].cpu().numpy(), window)
    fwd_ms = km["summarize"] + km["score_topk"] + km["attend_fuse"]
    blocks = {
        "summarize": roofline("hils_summarize (k_summarize_mfma)", "hbm", cnt["summarize_bytes"],
                              km["summarize"], call_traffic(workload, "summarize")),
        "score_topk": roofline("hils_score_topk", "alu", cnt["score_flops"], km["score_topk"],
                               call_traffic(workload, "score_topk"),
                               note="float32-accurate products on bf16 MFMAs over a hi/lo split "
                                    "of the summary key, against the float32 vector peak"),
        "attend_fuse": roofline("hils_attend_fuse (k_kv_prep + k_attend_mfma)", "mfma",
                                cnt["attend_flops"], km["attend_fuse"],
                                call_traffic(workload, "attend_fuse")),
    }
    rec = {"kernels_ms": km, "forward_ms": fwd_ms, "roofline": blocks,
           "key_visits": cnt["key_visits"], "candidates": cnt["candidates"],
           "attend_algorithmic_bytes": cnt["attend_bytes"], "K": w.K}
    if "backward" in km:
        blocks["backward"] = roofline("hils_backward", "mfma", cnt["backward_flops"],
                                      km["backward"], call_traffic(workload, "backward"))
        rec["train_tokens_per_s"] = w.B * w.T / ((fwd_ms + km["backward"]) * 1e-3)
    else:
        rec["prefill_tokens_per_s"] = w.B * w.T / (fwd_ms * 1e-3)
    return rec


def measure_decode(torch, hsa, stream, td, wd, K_sel, window, Kc, Vc, nsteps, dev, nb=1,
                   traffic=None):
    """(record, idx of every step) for a sequence of decode steps: step s queries the
    nb positions p0 + nb s .. over a cache that ends with them; a chunk's summary is
    made when it completes. Timed eagerly and as one captured HIP graph. nb > 1
    stands in for nb sequences decoding together (each row its own position).
    traffic: the counter record's HBM bytes per step, for the configuration it
    was taken on."""
    p0, S = wd.q_pos0, wd.S
    NCd = wd.T // S
    nsteps = nsteps // nb
    Bq = Kc.shape[0]  # sequences decoding together, each with its own cache
    dk = torch.empty(Bq, NCd, wd.H, wd.d, device=dev)
    de = torch.empty(Bq, NCd, wd.H, device=dev)
    dl = torch.empty(Bq, NCd, wd.H, device=dev)
    hsa.summarize(Kc, td["Ql"], S, 0, p0 // S, Tkv=p0, ksum=dk, ent=de, lse_l=dl)
    didx = torch.empty(nsteps, Bq, nb, wd.H, K_sel, dtype=torch.int32, device=dev)
    dsc = torch.empty(nsteps, Bq, nb, wd.H, K_sel, device=dev)
    dO = torch.empty(Bq, nb, wd.H, wd.d, dtype=torch.bfloat16, device=dev)
    dlo = torch.empty(Bq, nb, wd.H, device=dev)
    dlt = torch.empty(Bq, nb, wd.H, device=dev)
    ws = hsa.decode_workspace(td["Q"][:, :nb], Kc, dk, K_sel, S, wd.T - nb, wd.T, window=window)
    qs = [td["Q"][:, nb * s:nb * s + nb].contiguous() for s in range(nsteps)]

    def dstep(s):
        p = p0 + nb * s
        if p % S == 0 and p > p0:  # chunk p/S - 1 just completed
            c = p // S - 1
            hsa.summarize(Kc, td["Ql"], S, c, c + 1, Tkv=p, ksum=dk, ent=de, lse_l=dl)
        hsa.decode(qs[s], Kc, Vc, dk, de, K_sel, S, p, p + nb, idx=didx[s], score=dsc[s], O=dO,
                   lse_own=dlo, lse_tot=dlt, ws=ws, window=window)

    for s in range(8):
        dstep(s)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for s in range(nsteps):
        dstep(s)
    ev[1].record(stream)
    torch.cuda.synchronize()
    eager = ev[0].elapsed_time(ev[1]) * 1e3 / nsteps
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            for s in range(nsteps):
                dstep(s)
    stream.wait_stream(cap)
    graph.replay()
    torch.cuda.synchronize()
    reps = 3
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(reps):
        graph.replay()
    ev[1].record(stream)
    torch.cuda.synchronize()
    us = ev[0].elapsed_time(ev[1]) * 1e3 / (nsteps * reps)
    if nb == 1:  # every sequence moves its own bytes
        mean_bytes = Bq * float(np.mean([decode_step_bytes(wd, K_sel, window, p0 + s)
                                         for s in range(nsteps)]))
    else:  # nb positions of one sequence share its summaries and chunks
        mean_bytes = float(np.mean([decode_call_unique_bytes(wd, K_sel, window, p0 + nb * s, nb,
                                                             didx[s, 0].cpu().numpy())
                                    for s in range(nsteps)]))
    rec = {"us_per_token": us / (nb * Bq), "us_per_step": us,
           "us_per_token_eager": eager / (nb * Bq), "steps": nsteps,
           "rows_per_step": Bq * nb * wd.H, "bytes_per_step": mean_bytes,
           "roofline": roofline("hils_decode (split scoring; list merge and slot attention; slot "
                                "fusion: three launches; a k_summarize every 64 positions)",
                                "hbm", mean_bytes, us * 1e-3, traffic),
           "K": K_sel}
    if window:
        rec["local_branch"] = f"sliding window of {window} keys"
    del graph
    return rec, didx


# ---------------------------------------------------------------- CPU baselines
def cpu_prefill(oracle, x, w, nrows, seed):
    """All landmark summaries, then nrows sampled (row, head) queries scored, selected
    and attended; scaled to the full step."""
    rng = np.random.default_rng(seed)
    rows_total = w.B * w.T * w.H
    rows = np.sort(rng.choice(rows_total, size=nrows, replace=False))
    X = {k: x[k].astype(np.float64) for k in ("Q", "K", "V", "Ql")}
    t0 = time.perf_counter()
    oks, oent, _ = oracle.summarize(X["K"], X["Ql"], w.S)
    t_sum = time.perf_counter() - t0
    t0 = time.perf_counter()
    oidx, osc, _ = oracle.score_topk(X["Q"], oks, oent, w.S, w.K, rows=rows)
    oracle.attend_fuse(X["Q"], X["K"], X["V"], oidx, osc, w.S, rows=rows)
    t_rows = time.perf_counter() - t0
    t_full = t_sum + t_rows * rows_total / nrows
    return {"value": w.B * w.T / t_full, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"all {w.B * w.NC * w.H} landmark summaries ({t_sum:.2f} s) + {nrows} of "
                      f"{rows_total} (row, head) queries scored, selected and attended "
                      f"({t_rows:.2f} s), scaled to the full step"}


def cpu_decode(oracle, xd, wd, K_sel, nsteps):
    """Every step of the decode sequence: scoring, selection and attention of the
    step's query, plus the summary of each chunk that completes (the initial
    summaries of the cache are made before the timed region, as on the GPU)."""
    p0, S = wd.q_pos0, wd.S
    K64, V64 = xd["K"].astype(np.float64), xd["V"].astype(np.float64)
    Ql64 = xd["Ql"].astype(np.float64)
    oks, oent, _ = oracle.summarize(K64[:, :p0], Ql64[:, :p0 // S], S)
    NC = wd.T // S
    ks = np.zeros((1, NC, wd.H, wd.d))
    en = np.zeros((1, NC, wd.H))
    ks[:, :p0 // S], en[:, :p0 // S] = oks, oent
    t0 = time.perf_counter()
    for s in range(nsteps):
        p = p0 + s
        if p % S == 0 and p > p0:
            c = p // S - 1
            a, b_, _ = oracle.summarize(K64[:, c * S:(c + 1) * S], Ql64[:, c:c + 1], S)
            ks[:, c], en[:, c] = a[:, 0], b_[:, 0]
        q = xd["Q"][:, s:s + 1].astype(np.float64)
        oidx, osc, _ = oracle.score_topk(q, ks, en, S, K_sel, q_pos0=p)
        oracle.attend_fuse(q, K64[:, :p + 1], V64[:, :p + 1], oidx, osc, S, q_pos0=p)
    t = time.perf_counter() - t0
    return {"value": t / nsteps * 1e6, "unit": "us/token", "cores": 1, "kind": "oracle",
            "sample": f"all {nsteps} decode steps on the {wd.T}-token cache ({t:.2f} s)"}


def cpu_train(oracle, x, w):
    """Forward and backward of batch element 0, head 0 in full (heads and batch
    elements are independent at G = 1), scaled by B * H."""
    assert w.H == w.Hkv
    sl = {k: x[k][:1, :, :1].astype(np.float64) for k in ("Q", "K", "V", "Ql", "dO")}
    t0 = time.perf_counter()
    f = oracle.forward(sl["Q"], sl["K"], sl["V"], sl["Ql"], w.S, w.K)
    oracle.backward(sl["Q"], sl["K"], sl["V"], sl["Ql"], f["idx"], sl["dO"], w.S)
    t = time.perf_counter() - t0
    t_full = t * w.B * w.H
    return {"value": w.B * w.T / t_full, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"forward + backward of one (batch element, head) of {w.B * w.H} in full "
                      f"({t:.2f} s), scaled by {w.B * w.H}"}


# ---------------------------------------------------------------- main
def main():
    args = parse()
    if args.traffic:
        write_traffic_record(*args.traffic)
        return
    if args.counters:
        write_counter_summary(*args.counters)
        return
    if args.trace:
        write_trace_summary(*args.trace)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the HiLS path here runs on a single MI355X).", file=sys.stderr)
        sys.exit(2)
    import torch
    import hierarchical_sparse_attention_amd as hsa
    import synth

    dev = "cuda:0"
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    ev_ms, wall_ms = make_timers(torch, stream)

    if args.pmc_run:
        wname = args.pmc_run
        if wname == "decode_128k":
            wd = synth.workloads()[wname]
            xd = synth.make_inputs(wd)
            td = {k: torch.from_numpy(xd[k]).to(dev, torch.bfloat16) for k in ("Q", "K", "V", "Ql")}
            del xd
            measure_decode(torch, hsa, stream, td, wd, wd.K, 0, td["K"], td["V"], 16, dev)
        else:
            w, x, t, f, calls = prefill_setup(torch, hsa, synth, dev, wname)
            for _ in range(3):
                for fn in calls.values():
                    fn()
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)  # one elementwise kernel: COPY_BYTES read, COPY_BYTES written
        torch.cuda.synchronize()
        log("pmc run done")
        return

    extra = {}
    cpu_extra = {}
    oracle = None
    if not args.no_cpu_baseline:
        import oracle as oracle_mod
        oracle = oracle_mod
        path = oracle.use_native_build(tempfile.mkdtemp(prefix="hils_oracle_"))
        extra["cpu_host"] = {"nproc": os.cpu_count(), "oracle_build": "g++ -O3 -march=native, "
                             "one thread", "library": os.path.basename(path)}

    # ---------------------------------------------- headline: the 7B-class GQA prefill
    hw, hx, ht, hf, hcalls = prefill_setup(torch, hsa, synth, dev, "prefill_7b_gqa")

    def step():
        hcalls["summarize"]()
        hcalls["score_topk"]()
        hcalls["attend_fuse"]()

    log("warmup")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    ms = wall_ms(step, args.steps)
    head = measure_prefill(torch, ev_ms, hw, hf, {k: hcalls[k] for k in
                                                   ("summarize", "score_topk", "attend_fuse")},
                           args.steps, "prefill_7b_gqa", stream=stream)
    head["step_ms_wallclock"] = ms
    dominant = max(head["kernels_ms"], key=head["kernels_ms"].get)
    roof = dict(head["roofline"][dominant])
    extra["prefill_7b_gqa"] = head
    cpu = None
    if oracle is not None:
        log("cpu baseline: 7B GQA prefill")
        cpu = cpu_prefill(oracle, hx, hw, 8192, 0)
    del hx, ht, hf, hcalls
    torch.cuda.empty_cache()

    # ---------------------------------------------- 128K decode
    wd = synth.workloads()["decode_128k"]
    log("generating decode_128k inputs")
    xd = synth.make_inputs(wd)
    td = {k: torch.from_numpy(xd[k]).to(dev, torch.bfloat16) for k in ("Q", "K", "V", "Ql")}
    nsteps = min(args.decode_steps, wd.rows_q)
    rec, didx = measure_decode(torch, hsa, stream, td, wd, wd.K, 0, td["K"], td["V"], nsteps, dev,
                               traffic=call_traffic("decode_128k", "decode"))
    extra["decode_128k"] = rec
    if not args.no_extra_configs:
        rec, _ = measure_decode(torch, hsa, stream, td, wd, 32, 512, td["K"], td["V"], nsteps, dev)
        extra["decode_128k_main"] = rec
        Kh = torch.empty(td["K"].shape, dtype=torch.bfloat16, pin_memory=True)
        Vh = torch.empty(td["V"].shape, dtype=torch.bfloat16, pin_memory=True)
        Kh.copy_(td["K"])
        Vh.copy_(td["V"])
        torch.cuda.synchronize()
        rec, _ = measure_decode(torch, hsa, stream, td, wd, wd.K, 0, Kh, Vh, nsteps, dev)
        rec["cache"] = "K and V in pinned host memory, read through their device mapping"
        rec["host_link_gbs"] = ((wd.K + 1) * wd.S * wd.H * wd.d * 2 * 2
                                / (rec["us_per_token"] * 1e-6) / 1e9)
        extra["decode_128k_host_cache"] = rec
        del Kh, Vh
        rec, _ = measure_decode(torch, hsa, stream, td, wd, wd.K, 0, td["K"], td["V"], nsteps,
                                dev, nb=16)
        rec["rows"] = ("16 consecutive query positions of the one sequence per call (as in "
                       "speculative or chunked decoding); bytes are the call's unique ones: the "
                       "summaries once, each selected (head, chunk) once")
        extra["decode_128k_16_positions"] = rec
        # 16 sequences decoding together, each with its own 128K cache (8.6 GB of K and V,
        # drawn on the GPU from a seeded generator: a timing input, not a parity case)
        nbat = 16
        log("generating decode_128k batch-16 inputs")
        gen = torch.Generator(device=dev).manual_seed(wd.seed + 1000)
        tb = {"Q": torch.randn(nbat, wd.rows_q, wd.H, wd.d, device=dev, generator=gen),
              "Ql": torch.randn(nbat, wd.T // wd.S, wd.H, wd.d, device=dev, generator=gen)}
        tb = {k: v.to(torch.bfloat16) for k, v in tb.items()}
        for k in ("K", "V"):
            x = torch.empty(nbat, wd.T, wd.Hkv, wd.d, dtype=torch.bfloat16, device=dev)
            for i in range(nbat):
                x[i] = torch.randn(wd.T, wd.Hkv, wd.d, device=dev, generator=gen)
            tb[k] = x
        rec, _ = measure_decode(torch, hsa, stream, tb, wd, wd.K, 0, tb["K"], tb["V"], nsteps,
                                dev)
        rec["batch"] = nbat
        rec["inputs"] = ("16 independent 128K caches, N(0,1) from a seeded GPU generator; "
                         "each sequence moves its own summaries and chunks")
        extra["decode_128k_batch16"] = rec
        del tb
        torch.cuda.empty_cache()
    if oracle is not None:
        log("cpu baseline: 128K decode")
        cpu_extra["decode_128k"] = cpu_decode(oracle, xd, wd, wd.K, nsteps)
    del xd, td
    torch.cuda.empty_cache()

    # ---------------------------------------------- the other prefill and training workloads
    runs = [("prefill_345m", "prefill_345m", {})]
    if not args.no_extra_configs:
        runs += [("prefill_7b_gqa_group_max", "prefill_7b_gqa", {"group": True}),
                 ("prefill_345m_main", "prefill_345m", {"K": 32, "window": 512}),
                 ("train_345m", "train_345m", {}),
                 ("train_345m_qcal", "train_345m", {"qcal": True}),
                 ("train_345m_main", "train_345m", {"K": 32, "window": 512})]
    for rname, wname, opt in runs:
        w, x, t, f, calls = prefill_setup(torch, hsa, synth, dev, wname, **opt)
        rec = measure_prefill(torch, ev_ms, w, f, calls, 5, rname if not opt else "-",
                              opt.get("window", 0), stream=stream)
        if opt.get("group"):
            rec["selection"] = "group max over the 4 query heads of each kv head"
        if opt.get("qcal"):
            rec["scoring_query"] = "Q-Cal: separate scoring query, dQs returned apart"
        if opt.get("window"):
            rec["local_branch"] = f"sliding window of {opt['window']} keys"
        extra[rname] = rec
        if oracle is not None and rname == "prefill_345m":
            log("cpu baseline: 345M prefill")
            cpu_extra["prefill_345m"] = cpu_prefill(oracle, x, w, 4096, 1)
        if oracle is not None and rname == "train_345m":
            log("cpu baseline: training step")
            cpu_extra["train_345m"] = cpu_train(oracle, x, w)
        del x, t, f, calls
        torch.cuda.empty_cache()
    if cpu_extra:
        extra["cpu_baselines"] = cpu_extra

    out = {
        "metric": "HiLS prefill tokens/s + 128K decode us/token; % of HBM BW / bf16 MFMA peak",
        "value": hw.B * hw.T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill_7b_gqa: B=1 H=32 Hkv=8 d=128 T=32768 S=64 K=16, N(0,1) "
                               "+ 3 planted-peak and 26 near-uniform chunks, per-head selection",
                   "global_batch": hw.B, "seq_len": hw.T, "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
