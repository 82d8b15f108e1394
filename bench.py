#!/usr/bin/env python3
"""Decode-attention benchmark over a prefix-shared KV tree on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config c3] [--gpus 1]

One step = one pass of the hot path over one decode batch: one call of
pkvt_attn_decode (phase 1 + phase 2 in the attention kernel, then the merge
kernel) on one layer's K/V pools.  Steps rotate over L distinct layer pools,
L = max(2, ceil(2 GiB / unique KV bytes)), so the 256 MiB Infinity Cache
cannot serve a layer from the previous step.  The tree is static during the
run, so the plan is built and uploaded once (lazy context copy); host plan
time is reported separately.

Prints one JSON line.  value = effective KV GB/s: distinct stored KV bytes of
the batch (every shared chunk counted once, valid tokens only, K and V, fp16)
divided by the mean step time.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0     # MI355X dense fp16 matrix peak
SIMDS = 256 * 4                   # MI355X: 256 compute units x 4 SIMDs
METRIC = "decode attn µs/layer + effective KV GB/s (% HBM peak), shared prefix 1K–4K"
ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


class HipEvents:
    """hipEvent_t timing on an explicit stream (the one the kernels run on)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")      # the runtime torch already loaded
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(e))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed: {rc}")
            out.append(e.value)
        return out

    def record(self, ev, stream):
        rc = self.hip.hipEventRecord(ev, stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed: {rc}")

    def ms(self, a, b):
        self.hip.hipEventSynchronize(b)
        f = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(f), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return f.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


def time_region(ds, B, ev, stream, steps, warmup, per_kernel):
    """Run warmup + steps decode steps rotating layers; return per-step
    times (ms) and, with per_kernel, the attention-kernel times (ms)."""
    torch = ds.torch
    L = ds.layers
    for i in range(warmup):
        ds.decode(i % L, stream=stream)
    torch.cuda.synchronize()
    n_ev = steps + 1
    ends = ev.create(n_ev)
    mids = ev.create(steps) if per_kernel else [0] * steps       # after each attention kernel
    starts = ev.create(steps) if per_kernel else [0] * steps     # before each attention kernel
    ws = ds.ws.data_ptr() if ds.ws_bytes else 0
    t0 = time.perf_counter()
    ev.record(ends[0], stream)
    for i in range(steps):
        layer = i % L
        B.pkvt_attn_decode_ex(ds.tree, ds.meta.data_ptr(), ds.q.data_ptr(),
                              ds.k_pools[layer].data_ptr(), ds.v_pools[layer].data_ptr(),
                              ds.out.data_ptr(), ws, ds.ws_bytes, ds.scale, stream, starts[i],
                              mids[i])
        if per_kernel:
            ev.record(ends[i + 1], stream)
    if not per_kernel:
        ev.record(ends[steps], stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total = ev.ms(ends[0], ends[steps])
    step_ms, attn_ms = [], []
    if per_kernel:
        for i in range(steps):
            step_ms.append(ev.ms(ends[i], ends[i + 1]))
            attn_ms.append(ev.ms(starts[i], mids[i]))
    ev.destroy(ends)
    if per_kernel:
        ev.destroy(mids)
        ev.destroy(starts)
    return total, wall, step_ms, attn_ms


def _oracle_worker(args):
    """One worker of the all-cores oracle run: the oracle on its share of the
    sequences of layer 0 (the workload is inherited from the parent)."""
    from oracle import attention as A
    w, seqs = _ORACLE_JOB["w"], args
    A.attention_batch(w, layer=0, seqs=seqs)
    return len(seqs)


_ORACLE_JOB = {}


def oracle_cores():
    """CPU threads the all-cores oracle run may use: the CPUs this process
    may run on, at most 16 (a one-GPU share of a GPU host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def cpu_baseline(w, unique_bytes, budget_s):
    """The fp64 oracle, as it stands, on the same layer, twice:
      * single thread, on a bounded sample: sequences one by one until the
        time budget is spent, scaled to the whole layer;
      * on all the host cores this process may use (at most 16): every
        sequence of the layer, spread over that many forked worker processes
        (the oracle itself is unchanged; numpy runs one thread per worker),
        best of two runs.
    Must run before the GPU is initialised (the workers are forked)."""
    import multiprocessing as mp
    from oracle import attention as A
    t0 = time.perf_counter()
    done = 0
    for u in range(w.b):
        A.attention_batch(w, layer=0, seqs=[u])
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    per_layer_1 = el * w.b / done
    cores = oracle_cores()
    _ORACLE_JOB["w"] = w
    parts = [list(range(k, w.b, cores)) for k in range(cores) if k < w.b]
    runs = []
    with mp.get_context("fork").Pool(len(parts)) as pool:
        for _ in range(2):
            t1 = time.perf_counter()
            assert sum(pool.map(_oracle_worker, parts, chunksize=1)) == w.b
            runs.append(time.perf_counter() - t1)
    _ORACLE_JOB.clear()
    per_layer_n = min(runs)
    return {
        "value": round(unique_bytes / per_layer_n / 1e9, 4),
        "unit": "GB/s",
        "cores": len(parts),
        "kind": "oracle",
        "sample": f"all {w.b} sequences of layer 0 over {len(parts)} worker processes "
                  f"(numpy fp64, one thread each), best of 2 runs = {per_layer_n * 1e3:.0f} ms/layer; "
                  f"single thread: {done} of {w.b} sequences in {el:.1f} s, scaled to one layer = "
                  f"{per_layer_1 * 1e3:.0f} ms/layer",
        "single_thread_value": round(unique_bytes / per_layer_1 / 1e9, 4),
        "ms_per_layer": round(per_layer_n * 1e3, 1),
        "single_thread_ms_per_layer": round(per_layer_1 * 1e3, 1),
    }


# the sources that decide what the attention kernel reads and writes per launch:
# the kernels and the planner that cuts the work
KERNEL_SRCS = [os.path.join(ROOT, "prefix_shared_kv_tree_amd", "csrc", f)
               for f in ("attn.hip", "kernels.h", "shapes.h", "plan.cpp", "plan.h")]
PROFILES = os.path.join(ROOT, "profiles")
ATTN_KERNEL = "attn_kernel"
UNIT_KERNEL = "unit_kernel"


def kernel_of(info):
    """Name of the kernel that runs a decode plan: the units-only kernel for
    plans whose rows are all shared (plan info "kernel" = 1), else the
    two-phase attention kernel."""
    return UNIT_KERNEL if info.get("kernel") == 1 else ATTN_KERNEL


def kernel_source_sha256():
    """Identifies the attention kernel and planner code the counters were
    taken on: the SHA-256 of those sources with comments and blank space
    removed, so that a comment edit does not void the committed counters."""
    import hashlib
    import re
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        text = open(path).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def algorithmic_bytes(w, info):
    """Bytes one launch must move at least: the batch's distinct stored KV
    (every shared chunk once, valid tokens only), Q, and the attention
    kernel's outputs (partials for merged rows, O for rows finalised in
    place).  Returns (unique KV bytes, attention-kernel bytes)."""
    H, D = w.h, w.d
    unique = info["unique_tokens"] * H * D * 2 * 2
    q_bytes = w.b * H * D * 2
    direct_rows = w.b - info["merge_rows"]
    out_bytes = info["slots"] * H * (D + 2) * 4 + direct_rows * H * D * 2
    return unique, unique + q_bytes + out_bytes


def profile_traffic(config):
    """HBM bytes per attention launch from the committed counter summary of
    this workload, or None when there is none or the kernel source changed
    since the counters were taken."""
    for name in (ATTN_KERNEL, UNIT_KERNEL):
        path = os.path.join(PROFILES, f"{name}_{config}_pmc.md")
        if os.path.exists(path):
            break
    else:
        return None
    text = open(path).read()
    start = text.find("```json pmc-summary")
    if start < 0:
        return None
    body = text[text.index("\n", start) + 1:text.index("```", start + 3)]
    rec = json.loads(body)
    if rec.get("kernel_source_sha256") != kernel_source_sha256():
        return None
    return rec


def _counter_means(csv_path, kernel_substr):
    import csv as _csv
    from collections import defaultdict
    acc = defaultdict(list)
    for r in _csv.DictReader(open(csv_path)):
        if kernel_substr in r["Kernel_Name"]:
            acc[r["Counter_Name"]].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}, {k: len(v) for k, v in acc.items()}


def summarize_pmc(args):
    """Turn rocprofv3 counter CSVs of one bench run per counter set into the
    committed summary (markdown with a machine-readable JSON block)."""
    from prefix_shared_kv_tree_amd import binding as B
    from prefix_shared_kv_tree_amd import workloads as W
    w = W.make_config(args.config, with_kv=False)
    t = B.pkvt_tree_create(w.h, w.d, w.c, 1 << 20)
    ids, _ = B.pkvt_tree_build(t, w.all_seq_tokens())
    B.pkvt_plan(t, ids)
    info = B.pkvt_plan_info_get(t)
    B.pkvt_tree_destroy(t)
    kname = kernel_of(info)
    unique, attn_bytes = algorithmic_bytes(w, info)
    fetch, n_fetch = _counter_means(args.fetch_csv, kname)
    write, n_write = _counter_means(args.write_csv, kname)
    copy_bytes = args.copy_mib * 2 ** 20
    cf, ncf = _counter_means(args.fetch_csv, "neg_kernel")
    cw, ncw = _counter_means(args.write_csv, "neg_kernel")
    if ncf.get("FETCH_SIZE") != 3 or ncw.get("WRITE_SIZE") != 3:
        raise SystemExit(f"summarize-pmc: expected the 3 calibration copies, found "
                         f"{ncf.get('FETCH_SIZE')} / {ncw.get('WRITE_SIZE')} neg_kernel dispatches")
    # the copy runs three times after a fill: take the copies' own rows
    f_fetch = copy_bytes / (cf["FETCH_SIZE"] * 1024)
    f_write = copy_bytes / (cw["WRITE_SIZE"] * 1024)
    fetch_b = fetch["FETCH_SIZE"] * 1024 * f_fetch
    write_b = write["WRITE_SIZE"] * 1024 * f_write
    rec = {
        "workload": args.config,
        "kernel": f"{kname}<{w.d},{w.c}>",
        "kernel_source_sha256": kernel_source_sha256(),
        "dispatches": {"fetch": n_fetch.get("FETCH_SIZE", 0), "write": n_write.get("WRITE_SIZE", 0)},
        "fetch_kib_raw": round(fetch["FETCH_SIZE"], 1),
        "write_kib_raw": round(write["WRITE_SIZE"], 1),
        "copy_fetch_factor": round(f_fetch, 4),
        "copy_write_factor": round(f_write, 4),
        "fetch_bytes": int(fetch_b),
        "write_bytes": int(write_b),
        "traffic_bytes": int(fetch_b + write_b),
        "algorithmic_bytes": int(attn_bytes),
        "traffic_over_algorithmic": round((fetch_b + write_b) / attn_bytes, 4),
    }
    kernel_ns = None
    if args.trace_csv:
        import csv as _csv
        for r in _csv.DictReader(open(args.trace_csv)):
            if kname in r["Name"]:
                kernel_ns = float(r["AverageNs"])
                rec["kernel_avg_us_trace"] = round(kernel_ns / 1e3, 2)
                rec["traffic_gbps_at_trace_avg"] = round(rec["traffic_bytes"] / kernel_ns, 1)
    if args.mfma_csv:
        m, _ = _counter_means(args.mfma_csv, kname)
        rec["mfma_counters"] = {k: round(v, 1) for k, v in m.items()}
        if "SQ_INSTS_VALU_MFMA_MOPS_F16" in m:
            # the counter counts f16 MFMA math operations divided by 512
            flops = m["SQ_INSTS_VALU_MFMA_MOPS_F16"] * 512
            rec["mfma_f16_flops_issued"] = int(flops)
            if kernel_ns:
                rec["mfma_tflops"] = round(flops / kernel_ns / 1e3, 2)
                rec["mfma_frac_of_dense_f16_peak"] = round(flops / kernel_ns / 1e3 / MFMA_F16_PEAK_TFLOPS, 4)
        if "SQ_VALU_MFMA_BUSY_CYCLES" in m and "GRBM_GUI_ACTIVE" in m:
            # busy cycles summed over all SIMDs; GRBM_GUI_ACTIVE summed over the 8 XCDs
            cycles = m["GRBM_GUI_ACTIVE"] / 8
            rec["mfma_busy_frac"] = round(m["SQ_VALU_MFMA_BUSY_CYCLES"] / (cycles * SIMDS), 4)
    out = [f"# {rec['kernel']} -- HBM traffic per launch, workload {args.config}", "",
           f"Workload: {W.CONFIG_DESCRIPTIONS[args.config]}.", "",
           "Commands (repository root as $R):", "", "```"]
    out += [c for c in args.command]
    out += ["```", "",
            "FETCH_SIZE and WRITE_SIZE are read in KiB per dispatch and scaled by what",
            f"the same counters read for a plain elementwise copy of {args.copy_mib} MiB",
            "(torch.neg: that many bytes read and written) in the same run:",
            f"fetch factor {rec['copy_fetch_factor']}, write factor {rec['copy_write_factor']}.", "",
            "| quantity | value |", "|---|---|",
            f"| FETCH_SIZE (KiB, mean of {rec['dispatches']['fetch']} dispatches) | {rec['fetch_kib_raw']} |",
            f"| WRITE_SIZE (KiB, mean of {rec['dispatches']['write']} dispatches) | {rec['write_kib_raw']} |",
            f"| HBM bytes read per launch | {rec['fetch_bytes']:,} |",
            f"| HBM bytes written per launch | {rec['write_bytes']:,} |",
            f"| traffic per launch | {rec['traffic_bytes']:,} |",
            f"| algorithmic bytes per launch | {rec['algorithmic_bytes']:,} |",
            f"| traffic / algorithmic | {rec['traffic_over_algorithmic']} |"]
    if kernel_ns:
        out += [f"| attention kernel average, kernel trace (us) | {rec['kernel_avg_us_trace']} |",
                f"| traffic / average duration (GB/s) | {rec['traffic_gbps_at_trace_avg']} |"]
    if "mfma_counters" in rec:
        out += ["", "MFMA counters (mean per dispatch): " +
                ", ".join(f"{k} = {v}" for k, v in rec["mfma_counters"].items())]
        if "mfma_tflops" in rec:
            out += [f"MFMA f16 FLOPs issued per launch: {rec['mfma_f16_flops_issued']:,} "
                    f"(SQ_INSTS_VALU_MFMA_MOPS_F16 x 512) = {rec['mfma_tflops']} TFLOP/s over the "
                    f"traced average duration = {rec['mfma_frac_of_dense_f16_peak'] * 100:.2f} % of the "
                    f"{MFMA_F16_PEAK_TFLOPS:.0f} TFLOP/s dense f16 peak."]
        if "mfma_busy_frac" in rec:
            out += [f"SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x {SIMDS} SIMDs) = "
                    f"{rec['mfma_busy_frac'] * 100:.2f} % of SIMD cycles with the MFMA unit busy."]
    out += ["", "```json pmc-summary", json.dumps(rec, indent=1), "```", ""]
    print("\n".join(out))


def summarize_trace(args):
    """Turn a rocprofv3 --kernel-trace --stats CSV (and the bench JSON line
    printed by the same run) into the committed kernel-trace summary."""
    import csv as _csv
    from prefix_shared_kv_tree_amd import binding as B
    from prefix_shared_kv_tree_amd import workloads as W
    w = W.make_config(args.config, with_kv=False)
    t = B.pkvt_tree_create(w.h, w.d, w.c, 1 << 20)
    ids, _ = B.pkvt_tree_build(t, w.all_seq_tokens())
    B.pkvt_plan(t, ids)
    kname = kernel_of(B.pkvt_plan_info_get(t))
    B.pkvt_tree_destroy(t)
    rows = list(_csv.DictReader(open(args.trace_csv)))
    bench = None
    if args.bench_log:
        for line in open(args.bench_log):
            if line.startswith('{"metric"'):
                bench = json.loads(line)
    out = [f"# {kname} -- kernel trace, workload {args.config}", "",
           f"Workload: {W.CONFIG_DESCRIPTIONS[args.config]}.", "",
           "Commands (repository root as $R):", "", "```"] + list(args.command) + [
           "```", "",
           "| kernel | calls | total ns | avg ns | % | min ns | max ns | stddev |",
           "|---|---|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"].replace("pkvt::(anonymous namespace)::", "")
        name = name if len(name) <= 70 else name[:67] + "..."
        out.append(f"| `{name}` | {r['Calls']} | {r['TotalDurationNs']} | {float(r['AverageNs']):.0f} | "
                   f"{r['Percentage']} | {r['MinNs']} | {r['MaxNs']} | {float(r['StdDev']):.0f} |")
    attn = [r for r in rows if kname in r["Name"]][0]
    avg = float(attn["AverageNs"]) / 1e3
    if bench:
        out += ["", f"Same run, bench.py's own HIP-event figures: us_per_layer = {bench['us_per_layer']}, "
                f"attention kernel (events recorded right before and after it on its stream) = "
                f"{bench['attn_kernel_us']} us, roofline achieved = {bench['roofline']['achieved']} GB/s "
                f"of {bench['roofline']['peak']} GB/s.",
                f"rocprofv3 average for {kname}: {avg:.2f} us; the event figure is within "
                f"{abs(bench['attn_kernel_us'] - avg) / avg * 100:.1f} % of it."]
    print("\n".join(out + [""]))


def summarize_loop_trace(args):
    """Turn the rocprofv3 --kernel-trace --memory-copy-trace --stats output of
    a `bench.py --loop-only` run (and that run's JSON line) into the
    committed decode-loop summary: per-kernel stats and the GPU time of one
    pipelined step split by kernel."""
    import csv as _csv
    from collections import defaultdict
    from prefix_shared_kv_tree_amd import workloads as W
    d = args.trace_dir
    stats = list(_csv.DictReader(open(os.path.join(d, "run_kernel_stats.csv"))))
    trace = list(_csv.DictReader(open(os.path.join(d, "run_kernel_trace.csv"))))
    loop = None
    for line in open(args.bench_log):
        if line.startswith('{"config"'):
            loop = json.loads(line)["decode_loop"]

    def short(n):
        n = n.replace("pkvt::(anonymous namespace)::", "").replace("void ", "")
        return n.split("(")[0]

    ev = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), short(r["Kernel_Name"]))
                for r in trace)
    attn = [e for e in ev if e[2].startswith("attn_kernel")]
    L, T, warm = loop["layers"], loop["steps_pipelined"], loop["warmup"]
    t0, t1 = attn[warm * L][0], attn[(warm + T) * L - 1][1]
    region = [e for e in ev if t0 <= e[0] <= t1]
    tot, cnt = defaultdict(float), defaultdict(int)
    for s_, e_, n in region:
        tot[n] += (e_ - s_) / 1e3
        cnt[n] += 1
    span = (t1 - t0) / 1e3 / T
    busy = sum(tot.values()) / T
    out = [f"# Decode loop -- kernel trace, workload {args.config}", "",
           f"Workload: {W.CONFIG_DESCRIPTIONS[args.config]}; {L} layers, decoded for "
           f"{warm} + {T} (pipelined) + {loop['steps_synced']} (synchronised) steps, a row "
           f"replaced every {loop['churn_every']} steps.", "",
           "Commands (repository root as $R):", "", "```"] + list(args.command) + [
           "```", "",
           "| kernel | calls | total ns | avg ns | % | min ns | max ns |",
           "|---|---|---|---|---|---|---|"]
    for r in stats:
        name = short(r["Name"])
        out.append(f"| `{name[:70]}` | {r['Calls']} | {r['TotalDurationNs']} | "
                   f"{float(r['AverageNs']):.0f} | {r['Percentage']} | {r['MinNs']} | {r['MaxNs']} |")
    out += ["", f"GPU time per pipelined step (from the first attention launch of step {warm} to "
            f"the end of the last of step {warm + T - 1}): {span:.1f} us, of which kernels "
            f"busy {busy:.1f} us:", "",
            "| kernel | launches per step | us per step | avg us |", "|---|---|---|---|"]
    for n in sorted(tot, key=lambda k: -tot[k]):
        out.append(f"| `{n}` | {cnt[n] / T:.2f} | {tot[n] / T:.1f} | {tot[n] / cnt[n]:.1f} |")
    out += ["", f"Same run, bench.py's own figures: us_per_step_pipelined = "
            f"{loop['us_per_step_pipelined']}, attn_us_per_layer (events around the attention "
            f"calls) = {loop['attn_us_per_layer']}, host us per step (pipelined) = "
            f"{loop['host_us_pipelined']['per_step']}, of which tree and plan = "
            f"{loop['host_us_pipelined']['tree_and_plan_per_step']}; full plan "
            f"{loop['host_us_pipelined']['plan_full']} us, length refresh "
            f"{loop['host_us_pipelined']['plan_refresh']} us."]
    print("\n".join(out + [""]))


def summarize_prefill(args):
    """Kernel trace (--trace-csv) and MFMA counters (--mfma-csv) of a
    `bench.py --prefill --prefill-case N` run, with that run's JSON line
    (--bench-log), as the committed prefill-kernel summary."""
    import csv as _csv
    bench_row, steps = None, 0
    for line in open(args.bench_log):
        if line.startswith('{"prefill"'):
            bench_row = json.loads(line)["prefill"][0]
            steps = json.loads(line)["steps"]
    stats = list(_csv.DictReader(open(args.trace_csv)))
    kname = "prefill_kernel"
    kern = [r for r in stats if kname in r["Name"]][0]
    avg_ns = float(kern["AverageNs"])
    # the timed launches: the last `steps` dispatches in the per-dispatch trace
    # beside the statistics file (the warm-up launches come first)
    per = os.path.join(os.path.dirname(args.trace_csv), os.path.basename(args.trace_csv).replace(
        "kernel_stats", "kernel_trace"))
    timed_ns = None
    if os.path.exists(per):
        durs = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
                for r in _csv.DictReader(open(per)) if kname in r["Kernel_Name"]]
        if len(durs) >= steps:
            timed_ns = float(np.mean(durs[-steps:]))
    m, n = _counter_means(args.mfma_csv, kname)
    flops_issued = m["SQ_INSTS_VALU_MFMA_MOPS_F16"] * 512
    useful = bench_row["useful_gflop"] * 1e9
    busy = m["SQ_VALU_MFMA_BUSY_CYCLES"] / (m["GRBM_GUI_ACTIVE"] / 8 * SIMDS)
    out = [f"# prefill_kernel<{bench_row['d']},{bench_row['c']}> -- workload {bench_row['workload']}", "",
           f"Prefill of {bench_row['b']} sequences over a stored {bench_row['prefix']}-token prefix "
           f"({bench_row['rows']} query rows; h = {bench_row['h']}, d = {bench_row['d']}, c = {bench_row['c']}; "
           "Q, K/V drawn on the device).", "",
           "Commands (repository root as $R):", "", "```"] + list(args.command) + [
           "```", "",
           "| kernel | calls | avg ns | min ns | max ns |", "|---|---|---|---|---|"]
    for r in stats:
        nm = r["Name"].replace("pkvt::(anonymous namespace)::", "").replace("void ", "").split("(")[0]
        out.append(f"| `{nm[:70]}` | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | {r['MaxNs']} |")
    out += ["", "| quantity | value |", "|---|---|",
            f"| useful FLOPs per launch (4 d per row, head, visible key) | {useful:,.0f} |",
            f"| MFMA f16 FLOPs issued per launch (SQ_INSTS_VALU_MFMA_MOPS_F16 x 512, mean of "
            f"{n.get('SQ_INSTS_VALU_MFMA_MOPS_F16', 0)} dispatches) | {flops_issued:,.0f} |",
            f"| issued / useful (masked keys, padded tiles) | {flops_issued / useful:.3f} |",
            f"| prefill_kernel average (us, kernel trace) | {avg_ns / 1e3:.1f} |",
            f"| useful TFLOP/s over that average | {useful / avg_ns / 1e3:.1f} |",
            f"| useful fraction of the {MFMA_F16_PEAK_TFLOPS:.0f} TFLOP/s dense f16 peak | "
            f"{useful / avg_ns / 1e3 / MFMA_F16_PEAK_TFLOPS * 100:.1f} % |"]
    if timed_ns:
        out += [f"| prefill_kernel average over the {steps} timed launches (us, kernel trace) | "
                f"{timed_ns / 1e3:.1f} |",
                f"| useful fraction of the dense f16 peak over the timed launches | "
                f"{useful / timed_ns / 1e3 / MFMA_F16_PEAK_TFLOPS * 100:.1f} % |"]
    if args.fetch_csv and args.write_csv:
        # HBM traffic per launch, scaled by the calibration copy of the same runs
        # (as for the decode kernels), against the distinct K/V bytes
        fetch, nf = _counter_means(args.fetch_csv, kname)
        write, nw = _counter_means(args.write_csv, kname)
        cf, _ = _counter_means(args.fetch_csv, "neg_kernel")
        cw, _ = _counter_means(args.write_csv, "neg_kernel")
        copy_bytes = args.copy_mib * 2 ** 20
        fetch_b = fetch["FETCH_SIZE"] * 1024 * copy_bytes / (cf["FETCH_SIZE"] * 1024)
        write_b = write["WRITE_SIZE"] * 1024 * copy_bytes / (cw["WRITE_SIZE"] * 1024)
        kv = bench_row["distinct_kv_bytes"]
        out += [f"| HBM bytes read per launch (FETCH_SIZE, mean of {nf.get('FETCH_SIZE', 0)} dispatches, "
                f"copy-calibrated) | {fetch_b:,.0f} |",
                f"| HBM bytes written per launch (WRITE_SIZE, mean of {nw.get('WRITE_SIZE', 0)}) | "
                f"{write_b:,.0f} |",
                f"| distinct K/V bytes of the batch | {kv:,.0f} |",
                f"| bytes read / distinct K/V bytes | {fetch_b / kv:.2f} |",
                f"| Q read + O written (algorithmic) | {bench_row['q_o_bytes']:,.0f} |"]
    out += [
            f"| MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x {SIMDS})) | {busy * 100:.1f} % |",
            "", f"Same run, bench.py: {bench_row['shared_us_per_layer']} us per layer "
            f"(prefill kernel + merge, HIP events), {bench_row['shared_tflops']} TFLOP/s.", ""]
    print("\n".join(out))


def copy_probe(torch, mib):
    """A plain copy of known size (torch's elementwise kernel: `mib` MiB read,
    `mib` MiB written), launched three times.  Under a counter-collection run
    its FETCH_SIZE / WRITE_SIZE give the factor that converts those counters
    to bytes on this machine."""
    n = mib * 2 ** 20 // 2
    src = torch.ones(n, dtype=torch.float16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def copy_probe_gbps(torch, gib: int = 2, reps: int = 10) -> float:
    """HBM bandwidth a plain library copy reaches on this device, as context
    for the roofline (whose peak is the published 8 TB/s): torch's
    elementwise negation of a `gib` GiB fp16 tensor into another, counted as
    the bytes read plus the bytes written."""
    x = torch.ones(gib * 2 ** 30 // 2, dtype=torch.float16, device="cuda")
    y = torch.empty_like(x)
    for _ in range(2):
        torch.neg(x, out=y)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.neg(x, out=y)
    e1.record()
    torch.cuda.synchronize()
    gbps = 2 * gib * 2 ** 30 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del x, y
    return round(gbps, 1)


def decode_loop(args, name, layers, static_us_layer):
    """Decoding iterations with the tree changing under the kernels: per step
    a token appended to every row (K/V written by pkvt_kv_scatter), the plan
    refreshed -- rebuilt only when a leaf chunk filled or a sequence left or
    arrived -- and uploaded lazily, then attention on every layer.  A row
    gets a new sequence every --loop-churn steps.  Timed twice: pipelined
    (the host queues steps ahead of the GPU, as a serving loop that does not
    wait for sampled tokens between layers) and synchronised after every
    step (host work fully exposed)."""
    import torch
    from oracle import attention as A
    from prefix_shared_kv_tree_amd import workloads as W
    from prefix_shared_kv_tree_amd.harness import DecodeLoop, DecodeSetup, loop_pool_chunks

    w = W.make_config(name, layers=layers)
    tails = [len(w.segments[p[-1]]) for p in w.seq_paths if len(p) > 1]
    suffix = (min(tails), max(tails)) if tails else None
    warm, t1, t2 = args.loop_warmup, args.loop_steps, args.loop_steps // 2
    idx = (W.CONFIG_NAMES + W.DIAGNOSTIC_NAMES).index(name)
    tr = W.decode_trace(w, warm + t1 + t2, seed=2000 + idx, churn_every=args.loop_churn,
                        suffix=suffix)
    ds = DecodeSetup(w, layers=layers, pool_chunks=loop_pool_chunks(tr))
    loop = DecodeLoop(ds, tr)
    for t in range(warm):
        loop.step(t)
    torch.cuda.synchronize()

    def snapshot():
        return dict(loop.host.us), dict(loop.host.count), loop.us_total

    # pipelined
    h0 = snapshot()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    attn_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(t1)]
    e0.record()
    for k in range(t1):
        loop.step(warm + k, events=attn_ev[k])
    e1.record()
    torch.cuda.synchronize()
    pipe_us = e0.elapsed_time(e1) * 1e3 / t1
    attn_us = [a.elapsed_time(b) * 1e3 for a, b in attn_ev]
    h1 = snapshot()
    # synchronised after every step
    sync_us = []
    for k in range(t2):
        s0 = time.perf_counter()
        loop.step(warm + t1 + k)
        torch.cuda.synchronize()
        sync_us.append((time.perf_counter() - s0) * 1e6)
    t_last = warm + t1 + t2 - 1
    h2 = snapshot()

    def host_means(a, b, n_steps):
        us = {k: (b[0][k] - a[0][k]) for k in b[0]}
        cnt = {k: (b[1][k] - a[1][k]) for k in b[1]}
        tree_plan = sum(us.values())
        return {
            "per_step": round((b[2] - a[2]) / n_steps, 1),
            "tree_and_plan_per_step": round(tree_plan / n_steps, 1),
            "append": round(us["append"] / max(cnt["append"], 1), 1),
            "plan_full": round(us["plan_full"] / max(cnt["plan_full"], 1), 1),
            "plan_patch": round(us["plan_patch"] / max(cnt["plan_patch"], 1), 1),
            "plan_refresh": round(us["plan_refresh"] / max(cnt["plan_refresh"], 1), 1),
            "join": round(us["join"] / max(cnt["join"], 1), 1),
            "full_replans": cnt["plan_full"], "patches": cnt["plan_patch"],
            "refreshes": cnt["plan_refresh"], "joins": cnt["join"],
        }

    # parity on sampled rows (every replaced row among them) at the last step
    got = loop.out.float().cpu().numpy()
    rows = sorted(set([0, w.b // 2, w.b - 1] + [j.row for j in tr.joins]))[:12]
    wt = tr.workload_at(t_last)
    err = 0.0
    for l in range(layers):
        ref = A.attention_batch(wt, layer=l, seqs=rows)
        err = max(err, float(max(np.abs(got[l][u] - ref[u]).max() for u in rows)))
    ctx = [wt.seq_len(u) for u in range(w.b)]
    res = {
        "layers": layers, "steps_pipelined": t1, "steps_synced": t2, "warmup": warm,
        "churn_every": args.loop_churn, "join_suffix_tokens": list(suffix) if suffix else None,
        "context_tokens_at_end": {"min": int(min(ctx)), "max": int(max(ctx)),
                                  "mean": round(float(np.mean(ctx)), 1)},
        "us_per_step_pipelined": round(pipe_us, 1),
        "us_per_step_synced": round(float(np.median(sync_us)), 1),
        "attn_us_per_layer": round(float(np.mean(attn_us)) / layers, 2),
        "static_attn_us_per_layer": None if static_us_layer is None else round(static_us_layer, 2),
        "host_us_pipelined": host_means(h0, h1, t1),
        "host_us_synced": host_means(h1, h2, t2),
        "meta_regrow": loop.regrow,
        "parity_max_abs_err_sampled": err,
    }
    ds.close()
    return res


# ChunkAttention page, Knowl 8 (b = 32, c = 64, fp16, A100): decode throughput in
# 10^3 tokens/s while completions of n_c tokens grow after n_s shared prompt
# tokens -- (ChunkAttn, PagedAttn).  Context only: other hardware.
PAGE_DIVERGENCE = {
    (1024, 256): (241.93, 76.35), (1024, 512): (186.44, 69.15), (1024, 1024): (127.85, 58.12),
    (2048, 512): (145.41, 39.85), (2048, 1024): (107.37, 36.18), (2048, 2048): (70.33, 30.17),
    (4096, 512): (101.69, 21.04), (4096, 4096): (37.05, 15.12),
}
# Knowl 6 (b = 32, h = 32, d = 128, c = 64, fp16, A100): µs per attention kernel for n_p
# context tokens of which the first n_s are shared -- (ChunkAttn, PagedAttn).  Context only.
PAGE_KNOWL6 = {
    (1024, 0): (332.50, 356.17), (1024, 512): (198.87, 355.88), (1024, 768): (131.21, 356.02),
    (1024, 1024): (56.00, 355.44), (2048, 0): (655.44, 702.98), (2048, 1024): (384.37, 703.35),
    (2048, 1536): (247.14, 702.90), (2048, 2048): (110.48, 703.72), (4096, 0): (1301.78, 1400.61),
    (4096, 2048): (747.56, 1400.99), (4096, 3072): (477.66, 1400.30), (4096, 4096): (206.22, 1399.51),
}
# Knowl 9 (n_s = 2048, n_c = 64): ChunkAttn 10^3 tokens/s at the two ends of b in [16, 96].
PAGE_BATCH = {16: 155.0, 96: 224.0}


def sweep_time(torch, B, W, b, n_s, private, seed, variant, steps, warmup, ev, h=32, d=128, c=64,
               match="chunks"):
    """µs per layer of one decode batch: b sequences sharing n_s prompt
    tokens, each with `private` tokens of its own (a count, or one per
    sequence), K/V and Q drawn on the device; steps rotate over enough layer
    pools to defeat the Infinity Cache.  `match`: the tree's prefix matching;
    under "chunks" a prefix that ends inside a chunk leaves that chunk's
    tokens private to every sequence."""
    from prefix_shared_kv_tree_amd.harness import DecodeSetup
    w = W.unique_segment_starts(W.one_prefix(seed, b, n_s, private, h=h, d=d, c=c, with_kv=False))
    b_tok = w.h * w.d * 2 * 2
    unique = (n_s + int(np.sum(np.broadcast_to(private, (b,))))) * b_tok
    layers = max(2, math.ceil(2 * 2 ** 30 / unique))
    ds = DecodeSetup(w, layers=layers, device_random_seed=seed, match=match,
                     min_share=(1 << 20) if variant == "plain" else 0)
    stream = torch.cuda.current_stream().cuda_stream
    total_ms, _, _, _ = time_region(ds, B, ev, stream, steps, warmup, per_kernel=False)
    info = dict(ds.info)
    info["used_chunks"] = B.pkvt_tree_stats(ds.tree)["used_chunks"]
    ds.close()
    del ds
    return total_ms / steps * 1e3, info, unique


def run_sweep(args):
    """Knowl 8 (divergence) and Knowl 9 (batch) shapes.  A point's
    throughput is b / (mean step latency while the completions grow from 0
    to n_c tokens); the mean is taken with the midpoint rule over 4 equal
    panels of n_c (private lengths n_c/8, 3n_c/8, 5n_c/8, 7n_c/8), exact for a
    latency affine in the context length."""
    import torch
    from prefix_shared_kv_tree_amd import binding as B
    from prefix_shared_kv_tree_amd import workloads as W
    B.load()
    ev = HipEvents()
    if args.sweep == "shapes":
        # the long-shared-prompt batch (b = 64, 4096 shared tokens, private
        # suffixes uniform in [256, 1024]) at every supported head_dim and
        # chunk size, with h * d = 4096 so that a token's K/V bytes stay fixed
        rng = np.random.Generator(np.random.PCG64(1002))
        priv = [int(x) for x in rng.integers(256, 1025, size=64)]
        points = []
        for d in (64, 128, 256):
            for c in (16, 32, 64, 128):
                row = {"d": d, "c": c, "h": 4096 // d}
                for variant in ("tpp", "plain"):
                    t, info, unique = sweep_time(torch, B, W, 64, 4096, priv, 3100 + d + c, variant,
                                                 args.sweep_steps, 10, ev, h=4096 // d, d=d, c=c)
                    row[f"{variant}_us_per_layer"] = round(t, 2)
                    if variant == "tpp":
                        row["effective_gbps"] = round(unique / (t * 1e-6) / 1e9, 1)
                        row["frac_hbm_peak"] = round(unique / (t * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)
                row["speedup"] = round(row["plain_us_per_layer"] / row["tpp_us_per_layer"], 3)
                print(json.dumps(row), file=sys.stderr, flush=True)
                points.append(row)
        print(json.dumps({"sweep": "shapes", "b": 64, "n_s": 4096, "private": "uniform [256, 1024]",
                          "dtype": "f16", "data": "synthetic, device N(0,1)",
                          "steps_per_point": args.sweep_steps, "points": points}), flush=True)
        return
    if args.sweep == "tokens":
        # shared prompts that end inside a chunk: whole-chunk matching keeps the
        # prompt's last partial chunk private (one copy per sequence, read per
        # sequence); token-granular matching stores and reads it once
        rng = np.random.Generator(np.random.PCG64(1002))
        priv = [int(x) for x in rng.integers(256, 1025, size=64)]
        points = []
        for n_s in (40, 1000, 2000, 4000):
            row = {"n_s": n_s, "n_s_mod_c": n_s % 64}
            for match in ("chunks", "tokens"):
                t, info, unique = sweep_time(torch, B, W, 64, n_s, priv, 3400 + n_s, "tpp",
                                             args.sweep_steps, 10, ev, match=match)
                stored = info["unique_tokens"] * 32 * 128 * 4
                row[match] = {"us_per_layer": round(t, 2), "stored_tokens": info["unique_tokens"],
                              "used_chunks": info["used_chunks"],
                              "stored_kv_gbps": round(stored / (t * 1e-6) / 1e9, 1),
                              "frac_hbm_peak": round(stored / (t * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                              "phase1_items": info["phase1_items"], "wg_units": info["wg_units"]}
            row["speedup_tokens_vs_chunks"] = round(row["chunks"]["us_per_layer"] /
                                                    row["tokens"]["us_per_layer"], 3)
            print(json.dumps(row), file=sys.stderr, flush=True)
            points.append(row)
        print(json.dumps({"sweep": "tokens", "b": 64, "private": "uniform [256, 1024]", "h": 32,
                          "d": 128, "c": 64, "dtype": "f16", "data": "synthetic, device N(0,1)",
                          "points": points}), flush=True)
        return
    if args.sweep == "knowl6":
        # the pages' microkernel grid: 32 sequences of n_p context tokens, the
        # first n_s shared by all, one decode query each
        points = []
        for i, (n_p, n_s) in enumerate(sorted(PAGE_KNOWL6)):
            row = {"n_p": n_p, "n_s": n_s}
            for variant in ("tpp", "plain"):
                t, info, unique = sweep_time(torch, B, W, 32, n_s, n_p - n_s, 3600 + i, variant,
                                             args.sweep_steps, 10, ev)
                row[f"{variant}_us_per_layer"] = round(t, 2)
                if variant == "tpp":
                    row["unique_kv_bytes"] = int(unique)
                    row["effective_gbps"] = round(unique / (t * 1e-6) / 1e9, 1)
                    row["frac_hbm_peak"] = round(unique / (t * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)
                    row["plan"] = {k: info[k] for k in ("phase1_items", "wg_units", "tasks", "slots")}
            row["speedup_vs_plain"] = round(row["plain_us_per_layer"] / row["tpp_us_per_layer"], 3)
            ca, pa = PAGE_KNOWL6[(n_p, n_s)]
            row["page_a100_us"] = {"chunkattn": ca, "pagedattn": pa}
            print(json.dumps(row), file=sys.stderr, flush=True)
            points.append(row)
        print(json.dumps({"sweep": "knowl6", "b": 32, "h": 32, "d": 128, "c": 64, "dtype": "f16",
                          "data": "synthetic, device N(0,1)", "steps_per_point": args.sweep_steps,
                          "points": points}), flush=True)
        return
    if args.sweep == "shard":
        # one GPU's share of the long-shared-prompt batch when G GPUs split the
        # 32 heads (h = 32 / G at the real b, d, c): the work per GPU shrinks G
        # times and so does the number of (item, head) pieces to spread over
        # the 512 workgroups
        rng = np.random.Generator(np.random.PCG64(1002))
        priv = [int(x) for x in rng.integers(256, 1025, size=64)]
        points = []
        for g in (1, 2, 4, 8):
            h = 32 // g
            row = {"gpus_sharing_heads": g, "h": h}
            for variant in ("tpp", "plain"):
                t, info, unique = sweep_time(torch, B, W, 64, 4096, priv, 3200 + g, variant,
                                             args.sweep_steps, 10, ev, h=h, d=128, c=64)
                row[f"{variant}_us_per_layer"] = round(t, 2)
                if variant == "tpp":
                    row["effective_gbps"] = round(unique / (t * 1e-6) / 1e9, 1)
                    row["frac_hbm_peak"] = round(unique / (t * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)
                    row["plan"] = {k: info[k] for k in ("wg_units", "tasks", "phase1_split", "phase2_split")}
            print(json.dumps(row), file=sys.stderr, flush=True)
            points.append(row)
        print(json.dumps({"sweep": "shard", "b": 64, "n_s": 4096, "private": "uniform [256, 1024]",
                          "d": 128, "c": 64, "dtype": "f16", "data": "synthetic, device N(0,1)",
                          "points": points}), flush=True)
        return
    if args.sweep == "divergence":
        grid = [(32, n_s, n_c) for n_s, n_c in sorted(PAGE_DIVERGENCE)]
        grid += [(32, n_s, 0) for n_s in (1024, 2048, 4096)]
    else:
        grid = [(b, 2048, 64) for b in (16, 32, 48, 64, 80, 96)]
    points = []
    for i, (b, n_s, n_c) in enumerate(grid):
        privs = [max(1, (2 * k + 1) * n_c // 8) for k in range(4)] if n_c else [1]
        row = {"b": b, "n_s": n_s, "n_c": n_c, "private_tokens": privs}
        for variant in ("tpp", "plain"):
            us = []
            for k, p in enumerate(privs):
                t, info, _ = sweep_time(torch, B, W, b, n_s, p, 3000 + 10 * i + k, variant,
                                        args.sweep_steps, 10, ev)
                us.append(t)
            mean_us = float(np.mean(us))
            row[f"{variant}_us_per_layer"] = [round(x, 2) for x in us]
            row[f"{variant}_ktok_per_s"] = round(b / (mean_us * 1e-6) / 1e3, 2)
        row["speedup"] = round(row["tpp_ktok_per_s"] / row["plain_ktok_per_s"], 3)
        page = PAGE_DIVERGENCE.get((n_s, n_c)) if args.sweep == "divergence" else None
        if page:
            row["page_a100_ktok_per_s"] = {"chunkattn": page[0], "pagedattn": page[1]}
        if args.sweep == "batch" and b in PAGE_BATCH:
            row["page_a100_ktok_per_s"] = {"chunkattn": PAGE_BATCH[b]}
        print(json.dumps(row), file=sys.stderr, flush=True)
        points.append(row)
    print(json.dumps({"sweep": args.sweep, "h": 32, "d": 128, "c": 64, "dtype": "f16",
                      "data": "synthetic, device N(0,1)", "steps_per_point": args.sweep_steps,
                      "points": points}), flush=True)


def prefill_flops(pb):
    """Useful FLOPs of a prefill: 4 d per (row, head, visible key); the row
    at position p sees p + 1 keys."""
    n = 0
    for u, a in zip(pb.seqs, pb.q_from):
        L = pb.w.seq_len(u)
        n += (L * (L + 1) - a * (a + 1)) // 2
    return 4 * pb.w.d * pb.w.h * n


def run_prefill(args):
    """Prefix-aware prefill of arriving sequences over a stored shared
    prefix: µs per layer and useful TFLOP/s (against the dense f16 matrix
    peak), and the same rows with every sequence holding its own copy of the
    prefix (nothing shared: each sequence's rows read the prefix for
    themselves).  K/V and Q are drawn on the device."""
    import torch
    from prefix_shared_kv_tree_amd import binding as B
    from prefix_shared_kv_tree_amd import workloads as W
    from prefix_shared_kv_tree_amd.harness import PrefillSetup
    B.load()
    rng = np.random.Generator(np.random.PCG64(1002))
    cases = [("b32_prefix1024_new512", 32, 1024, 512),
             ("b64_prefix4096_new256-1024", 64, 4096, [int(x) for x in rng.integers(256, 1025, 64)]),
             ("b64_prefix2048_new64", 64, 2048, 64)]
    if args.prefill_case is not None:
        cases = [cases[args.prefill_case]]
    out = []
    d = args.prefill_head_dim
    for name, b, prefix, new in cases:
        row = {"workload": name, "b": b, "prefix": prefix, "h": 32, "d": d, "c": 64}
        for variant in ("shared",) if args.prefill_case is not None else ("shared", "unshared"):
            pb = W.prefill_batch(4242, b, prefix, new, h=32, d=d, c=64, with_kv=False)
            if variant == "unshared":
                pb = W.prefill_unshared(pb)
            ps = PrefillSetup(pb, layers=2, device_random_seed=4242)
            stream = torch.cuda.current_stream().cuda_stream
            for i in range(args.prefill_warmup):
                ps.run(i % 2, stream=stream)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            steps = args.prefill_steps
            e0.record()
            for i in range(steps):
                ps.run(i % 2, stream=stream)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / steps
            fl = prefill_flops(pb)
            row[f"{variant}_us_per_layer"] = round(us, 1)
            row[f"{variant}_tflops"] = round(fl / (us * 1e-6) / 1e12, 1)
            if variant == "shared":
                row["rows"] = pb.n_rows
                row["distinct_kv_bytes"] = W.unique_tokens(pb.w) * pb.w.h * pb.w.d * 2 * 2
                row["q_o_bytes"] = 2 * pb.n_rows * pb.w.h * pb.w.d * 2
                row["useful_gflop"] = round(fl / 1e9, 2)
                row["frac_mfma_f16_peak"] = round(fl / (us * 1e-6) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)
                row["plan"] = {k: ps.info[k] for k in ("wg_units", "slots", "phase1_items")}
            ps.close()
            del ps
        if "unshared_us_per_layer" in row:
            row["speedup_vs_unshared"] = round(row["unshared_us_per_layer"] / row["shared_us_per_layer"], 3)
        print(json.dumps(row), file=sys.stderr, flush=True)
        out.append(row)
    if args.copy_probe_mib:
        copy_probe(torch, args.copy_probe_mib)     # calibrates FETCH_SIZE / WRITE_SIZE
    print(json.dumps({"prefill": out, "dtype": "f16", "data": "synthetic, device N(0,1)",
                      "steps": args.prefill_steps}), flush=True)


def config_entry(name, args, ev, stream):
    """One more configuration at the bench's own protocol: layer 0 holds the
    workload's K/V (checked against the oracle on sampled rows), the other
    rotated layers are drawn on the device; TPP and the plain per-sequence
    schedule (phase 1 off) are each timed over --config-steps steps; the
    attention kernel alone is timed with events around it."""
    import torch
    from oracle import attention as A
    from prefix_shared_kv_tree_amd import binding as B
    from prefix_shared_kv_tree_amd import workloads as W
    from prefix_shared_kv_tree_amd.harness import DecodeSetup
    w = W.make_config(name, layers=1)
    b_tok = w.h * w.d * 2 * 2
    unique = W.unique_tokens(w) * b_tok
    layers = max(2, math.ceil(2 * 2 ** 30 / unique))
    ds = DecodeSetup(w, layers=layers, extra_layers_seed=5000 + W.CONFIG_NAMES.index(name))
    info = dict(ds.info)
    assert info["unique_tokens"] * b_tok == unique
    out = ds.decode(0)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    rows = sorted({0, 1, w.b // 2, w.b - 2, w.b - 1})
    ref = A.attention_batch(w, layer=0, seqs=rows)
    parity = float(max(np.abs(got[u] - ref[u]).max() for u in rows))
    steps, warm = args.config_steps, 10
    t_ms, _, _, _ = time_region(ds, B, ev, stream, steps, warm, per_kernel=False)
    _, _, _, attn_ms = time_region(ds, B, ev, stream, steps, warm, per_kernel=True)
    us = t_ms / steps * 1e3
    attn_us = float(np.mean(attn_ms)) * 1e3
    _, attn_bytes = algorithmic_bytes(w, info)
    ds.replan(0, 0, 1 << 20)
    p_ms, _, _, _ = time_region(ds, B, ev, stream, steps, warm, per_kernel=False)
    p_us = p_ms / steps * 1e3
    plain_plan = dict(ds.info)
    ds.close()
    del ds
    gbps = unique / (us * 1e-6) / 1e9
    res = {
        "workload": W.CONFIG_DESCRIPTIONS[name],
        "layers_rotated": layers, "steps": steps,
        "unique_kv_bytes": int(unique),
        "tpp_us_per_layer": round(us, 2),
        "effective_gbps": round(gbps, 1),
        "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
        "attn_kernel_us": round(attn_us, 2),
        "kernel_frac_unique_kv": round(unique / (attn_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        "kernel_frac_algorithmic": round(attn_bytes / (attn_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        "plain_us_per_layer": round(p_us, 2),
        "speedup_vs_plain": round(p_us / us, 3),
        "tpp_over_plain_time": round(us / p_us, 4),
        "same_plan_as_plain": info["tasks"] == plain_plan["tasks"] and info["wg_units"] == plain_plan["wg_units"]
                           and info["phase1_items"] == 0,
        "kernel": kernel_of(info),
        "plan": {k: info[k] for k in ("phase1_items", "phase2_items", "wg_units", "tasks", "slots",
                                       "merge_rows")},
        "parity_max_abs_err_sampled": parity,
        "parity_rows": rows,
    }
    traffic = profile_traffic(name)
    if traffic:
        res["rocprof_kernel_avg_us"] = traffic.get("kernel_avg_us_trace")
        res["traffic_bytes"] = traffic["traffic_bytes"]
    print(json.dumps({name: res}), file=sys.stderr, flush=True)
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=600)
    ap.add_argument("--warmup", type=int, default=60)
    ap.add_argument("--config", default="c3", choices=["tiny", "c2", "c3", "c4", "c5", "phase1"])
    ap.add_argument("--phase1-chunks", type=int, default=0)
    ap.add_argument("--phase2-chunks", type=int, default=0)
    ap.add_argument("--unit-rows", type=int, default=0,
                    help="smallest phase-1 row block run as a workgroup unit (0 = default; "
                         "above 64 runs every phase-1 row group as single-wave tasks)")
    ap.add_argument("--layers", type=int, default=0,
                    help="layer pools rotated (0 = max(2, ceil(2 GiB / unique KV bytes)))")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-plain", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the run, launch a plain elementwise copy of this many MiB "
                         "(reads and writes that many bytes) to calibrate HBM byte counters")
    ap.add_argument("--summarize-pmc", action="store_true",
                    help="(no GPU) print the counter summary of --config from rocprofv3 CSVs")
    ap.add_argument("--fetch-csv")
    ap.add_argument("--write-csv")
    ap.add_argument("--mfma-csv")
    ap.add_argument("--trace-csv")
    ap.add_argument("--summarize-trace", action="store_true",
                    help="(no GPU) print the kernel-trace summary of --config from a rocprofv3 stats CSV")
    ap.add_argument("--bench-log")
    ap.add_argument("--trace-dir")
    ap.add_argument("--summarize-prefill", action="store_true",
                    help="(no GPU) print the prefill-kernel summary from --trace-csv, --mfma-csv "
                         "and --bench-log")
    ap.add_argument("--summarize-loop-trace", action="store_true",
                    help="(no GPU) print the decode-loop trace summary from a rocprofv3 output "
                         "directory (--trace-dir) and the run's log (--bench-log)")
    ap.add_argument("--copy-mib", type=int, default=1024)
    ap.add_argument("--command", action="append", default=[])
    ap.add_argument("--loop-steps", type=int, default=128,
                    help="decode-loop steps timed pipelined (half as many again synchronised)")
    ap.add_argument("--loop-warmup", type=int, default=8)
    ap.add_argument("--loop-churn", type=int, default=16,
                    help="a row gets a new sequence every this many decode-loop steps")
    ap.add_argument("--no-loop", action="store_true")
    ap.add_argument("--sweep", choices=["divergence", "batch", "shapes", "shard", "tokens", "knowl6"],
                    help="time the pages' microkernel grid (Knowl 6), the decode-throughput sweeps "
                         "of the divergence (Knowl 8) or batch-size (Knowl 9) experiments, or the "
                         "shape / head-share / token-matching sweeps instead of the benchmark")
    ap.add_argument("--sweep-steps", type=int, default=60)
    ap.add_argument("--prefill", action="store_true",
                    help="time prefix-aware prefill attention instead of the decode benchmark")
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--prefill-warmup", type=int, default=10,
                    help="untimed prefill launches first (the first few run up to 20 %% slower)")
    ap.add_argument("--prefill-head-dim", type=int, default=128, choices=[64, 128, 256],
                    help="head_dim of the --prefill batches")
    ap.add_argument("--prefill-case", type=int, default=None,
                    help="time only this prefill workload (index), shared variant only")
    ap.add_argument("--loop-only", action="store_true",
                    help="run only the decode loop (for profiling it)")
    ap.add_argument("--other-configs", default="c2,c4,c5",
                    help="comma-separated configurations also timed (TPP and plain, sampled "
                         "parity) and reported in the line's `configs` object; '' for none")
    ap.add_argument("--config-steps", type=int, default=100,
                    help="timed steps per variant for each of --other-configs")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(args)
        return
    if args.summarize_trace:
        summarize_trace(args)
        return
    if args.summarize_loop_trace:
        summarize_loop_trace(args)
        return
    if args.summarize_prefill:
        summarize_prefill(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: it runs the decode attention of one "
              "GPU's share and has no multi-GPU path; run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    from prefix_shared_kv_tree_amd import workloads as W
    bench_run = not (args.sweep or args.prefill or args.loop_only)
    if bench_run:
        # host-side work first: the workload draws, and the oracle's CPU
        # baseline (its worker processes are forked before the GPU is touched)
        probe = W.make_config(args.config, with_kv=False)
        b_tok = probe.h * probe.d * 2 * 2
        unique_bytes_est = W.unique_tokens(probe) * b_tok
        layers = max(2, math.ceil(2 * 2 ** 30 / unique_bytes_est))
        if args.layers:
            layers = args.layers            # diagnostic: fewer or more layer pools
        t0 = time.perf_counter()
        w = W.make_config(args.config, layers=layers)
        gen_s = time.perf_counter() - t0
        cpu = None if args.no_cpu_baseline else cpu_baseline(w, unique_bytes_est, args.cpu_budget)

    import torch
    from prefix_shared_kv_tree_amd import binding as B
    from prefix_shared_kv_tree_amd.harness import DecodeSetup
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    B.load()
    if args.sweep:
        run_sweep(args)
        return
    if args.prefill:
        run_prefill(args)
        return
    if args.loop_only:
        probe = W.make_config(args.config, with_kv=False)
        layers = max(2, math.ceil(2 * 2 ** 30 / (W.unique_tokens(probe) * probe.h * probe.d * 4)))
        print(json.dumps({"config": args.config,
                          "decode_loop": decode_loop(args, args.config, layers, None)}), flush=True)
        return
    ds = DecodeSetup(w, phase1_chunks=args.phase1_chunks, phase2_chunks=args.phase2_chunks,
                     unit_rows=args.unit_rows)
    info = dict(ds.info)
    unique_bytes = info["unique_tokens"] * b_tok
    assert unique_bytes == unique_bytes_est, "tree and workload disagree on the stored tokens"
    logical_bytes = info["logical_tokens"] * b_tok
    stream = torch.cuda.current_stream().cuda_stream

    # host plan cost (structure rebuild, then the lazy length-only refresh)
    t0 = time.perf_counter()
    for _ in range(20):
        B.pkvt_plan(ds.tree, ds.seq_ids, args.phase1_chunks, args.phase2_chunks, 0)
    plan_refresh_us = (time.perf_counter() - t0) / 20 * 1e6
    plan_full_us = []
    for k in range(5):
        t0 = time.perf_counter()
        B.pkvt_plan(ds.tree, ds.seq_ids, args.phase1_chunks + (k % 2) * 0, args.phase2_chunks,
                    2 + (k % 2))                     # alternate options to force a rebuild
        plan_full_us.append((time.perf_counter() - t0) * 1e6)
    ds.replan(args.phase1_chunks, args.phase2_chunks, 0, unit_rows=args.unit_rows)

    # quick parity guard on a few sequences of layer 0
    from oracle import attention as A
    out = ds.decode(0)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    seqs = sorted({0, w.b // 2, w.b - 1})
    ref = A.attention_batch(w, layer=0, seqs=seqs)
    parity = float(max(np.abs(got[u] - ref[u]).max() for u in seqs))

    # The timed region: K steps back to back, events only at its two ends.
    ev = HipEvents()
    clean_ms, wall_s, _, _ = time_region(ds, B, ev, stream, args.steps, args.warmup,
                                         per_kernel=False)
    # Per-kernel split: the same K steps again with an event after each
    # attention launch and after each step (the extra events cost a few us).
    total_ms, _, step_ms, attn_ms = time_region(ds, B, ev, stream, args.steps,
                                                args.warmup // 2 + 1, per_kernel=True)
    us_layer = clean_ms / args.steps * 1e3
    us_layer_events = total_ms / args.steps * 1e3
    step_us = np.array(step_ms) * 1e3
    attn_us = np.array(attn_ms) * 1e3
    attn_avg_us = float(attn_us.mean())

    # algorithmic bytes of one attention-kernel launch
    H, D = w.h, w.d
    _, attn_bytes = algorithmic_bytes(w, info)
    achieved = attn_bytes / (attn_avg_us * 1e-6) / 1e9
    traffic = profile_traffic(args.config)

    res = {
        "metric": METRIC,
        "value": round(unique_bytes / (us_layer * 1e-6) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us_layer / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": f"{args.config}: {W.CONFIG_DESCRIPTIONS[args.config]}",
            "b": w.b, "h": H, "d": D, "c": w.c,
            "layers_rotated": layers,
            "variant": "two-phase partition",
            "phase1_chunks": args.phase1_chunks, "phase2_chunks": args.phase2_chunks,
        },
        "us_per_layer": round(us_layer, 2),
        # a second timed region with HIP events around every step (their
        # overhead included): the spread of single steps, not of us_per_layer
        "step_events_us_p10": round(float(np.percentile(step_us, 10)), 2),
        "step_events_us_p90": round(float(np.percentile(step_us, 90)), 2),
        "step_events_us_mean": round(us_layer_events, 2),
        "frac_hbm_peak": round(unique_bytes / (us_layer * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        "unique_kv_bytes": int(unique_bytes),
        "logical_kv_bytes": int(logical_bytes),
        "logical_kv_gbps": round(logical_bytes / (us_layer * 1e-6) / 1e9, 1),
        "attn_kernel_us": round(attn_avg_us, 2),
        "merge_and_gap_us": round(float((step_us - attn_us).mean()), 2),
        "host_wall_us_per_step": round(wall_s / args.steps * 1e6, 2),
        "plan": {k: info[k] for k in ("phase1_items", "phase2_items", "waves", "workgroups",
                                       "tasks", "slots", "merge_rows", "shared_chunks",
                                       "phase1_split", "phase2_split")},
        "host_plan_us": {"full": round(float(np.median(plan_full_us)), 1),
                         "length_refresh": round(plan_refresh_us, 1)},
        "parity_max_abs_err_sampled": parity,
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic["traffic_bytes"] if traffic else None,
            "kernel": f"{kernel_of(info)}<{D},{w.c}>",
            # achieved = algorithmic_bytes_per_launch / duration_us: the distinct
            # stored KV bytes plus Q and the kernel's partial / O writes, over the
            # mean HIP-event time of the attention kernel alone (events recorded
            # on its stream right before and after it, K launches)
            "algorithmic_bytes_per_launch": int(attn_bytes),
            "duration_us": round(attn_avg_us, 2),
            "duration": "mean of K HIP-event intervals around the attention kernel alone, on its stream",
            # the same duration with only the distinct stored KV bytes counted
            "unique_kv_bytes": int(unique_bytes),
            "frac_unique_kv": round(unique_bytes / (attn_avg_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "rocprof_avg_us": traffic.get("kernel_avg_us_trace") if traffic else None,
            # frac over the committed rocprofv3 kernel average instead of the events
            "frac_at_rocprof_avg": (round(attn_bytes / (traffic["kernel_avg_us_trace"] * 1e-6) / 1e9
                                          / HBM_PEAK_GBPS, 4)
                                    if traffic and traffic.get("kernel_avg_us_trace") else None),
        },
        "workload_gen_s": round(gen_s, 1),
        # a counter-collection run calibrates on its own copy's dispatches
        # alone, so it leaves this (differently sized) copy out
        "hbm_copy_probe_gbps": None if args.copy_probe_mib else copy_probe_gbps(torch),
    }

    if not args.no_plain:
        ds.replan(args.phase1_chunks, args.phase2_chunks, 1 << 20)
        p_ms, _, _, _ = time_region(ds, B, ev, stream, args.steps, args.warmup, per_kernel=False)
        p_us = p_ms / args.steps * 1e3
        res["plain_us_per_layer"] = round(p_us, 2)
        res["speedup_vs_plain"] = round(p_us / us_layer, 3)
        ds.replan(args.phase1_chunks, args.phase2_chunks, 0, unit_rows=args.unit_rows)

    if cpu is not None:
        res["cpu_baseline"] = cpu
    ds.close()
    del ds
    if args.other_configs:
        res["configs"] = {name: config_entry(name, args, ev, stream)
                          for name in args.other_configs.split(",") if name}
        probe_gbps = res["hbm_copy_probe_gbps"]
        for entry in res["configs"].values():
            entry["effective_over_copy_probe"] = (round(entry["effective_gbps"] / probe_gbps, 3)
                                                  if probe_gbps else None)
    if not args.no_loop:
        res["decode_loop"] = decode_loop(args, args.config, layers, us_layer)
    if args.copy_probe_mib:
        copy_probe(torch, args.copy_probe_mib)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
