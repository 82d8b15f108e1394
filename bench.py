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
    mids = ev.create(steps) if per_kernel else [0] * steps
    ws = ds.ws.data_ptr() if ds.ws_bytes else 0
    t0 = time.perf_counter()
    ev.record(ends[0], stream)
    for i in range(steps):
        layer = i % L
        B.pkvt_attn_decode_ex(ds.tree, ds.meta.data_ptr(), ds.q.data_ptr(),
                              ds.k_pools[layer].data_ptr(), ds.v_pools[layer].data_ptr(),
                              ds.out.data_ptr(), ws, ds.ws_bytes, ds.scale, stream, mids[i])
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
            attn_ms.append(ev.ms(ends[i], mids[i]))
    ev.destroy(ends)
    if per_kernel:
        ev.destroy(mids)
    return total, wall, step_ms, attn_ms


def cpu_baseline(w, unique_bytes, budget_s):
    """The fp64 oracle, as it stands, on a bounded sample of the same layer:
    sequences are evaluated one by one until the time budget is spent."""
    from oracle import attention as A
    t0 = time.perf_counter()
    done = 0
    for u in range(w.b):
        A.attention_batch(w, layer=0, seqs=[u])
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    per_layer_s = el * w.b / done
    return {
        "value": round(unique_bytes / per_layer_s / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{done} of {w.b} sequences of layer 0 ({el:.1f} s, numpy fp64 single thread); "
                  f"scaled to one layer = {per_layer_s * 1e3:.0f} ms/layer",
    }


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=600)
    ap.add_argument("--warmup", type=int, default=60)
    ap.add_argument("--config", default="c3", choices=["tiny", "c2", "c3", "c4", "c5"])
    ap.add_argument("--phase1-chunks", type=int, default=0)
    ap.add_argument("--phase2-chunks", type=int, default=0)
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-plain", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the run, launch a plain elementwise copy of this many MiB "
                         "(reads and writes that many bytes) to calibrate HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build runs the decode attention of one "
              "GPU's share and has no multi-GPU path; run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from prefix_shared_kv_tree_amd import binding as B
    from prefix_shared_kv_tree_amd import workloads as W
    from prefix_shared_kv_tree_amd.harness import DecodeSetup
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    B.load()

    probe = W.make_config(args.config, with_kv=False)
    b_tok = probe.h * probe.d * 2 * 2
    unique_bytes_est = W.unique_tokens(probe) * b_tok
    layers = max(2, math.ceil(2 * 2 ** 30 / unique_bytes_est))
    t0 = time.perf_counter()
    w = W.make_config(args.config, layers=layers)
    gen_s = time.perf_counter() - t0
    ds = DecodeSetup(w, phase1_chunks=args.phase1_chunks, phase2_chunks=args.phase2_chunks)
    info = dict(ds.info)
    unique_bytes = info["unique_tokens"] * b_tok
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
    ds.replan(args.phase1_chunks, args.phase2_chunks, 0)

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
    q_bytes = w.b * H * D * 2
    n_slots = info["slots"]
    direct_rows = w.b - info["merge_rows"]
    out_bytes = n_slots * H * (D + 2) * 4 + direct_rows * H * D * 2
    attn_bytes = unique_bytes + q_bytes + out_bytes
    achieved = attn_bytes / (attn_avg_us * 1e-6) / 1e9

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
        "us_per_layer_p10": round(float(np.percentile(step_us, 10)), 2),
        "us_per_layer_p90": round(float(np.percentile(step_us, 90)), 2),
        "us_per_layer_with_step_events": round(us_layer_events, 2),
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
            "traffic": None,
            "kernel": "attn_kernel<128,64>",
            "algorithmic_bytes_per_launch": int(attn_bytes),
        },
        "workload_gen_s": round(gen_s, 1),
    }

    if not args.no_plain:
        ds.replan(args.phase1_chunks, args.phase2_chunks, 1 << 20)
        p_ms, _, _, _ = time_region(ds, B, ev, stream, args.steps, args.warmup, per_kernel=False)
        p_us = p_ms / args.steps * 1e3
        res["plain_us_per_layer"] = round(p_us, 2)
        res["speedup_vs_plain"] = round(p_us / us_layer, 3)
        ds.replan(args.phase1_chunks, args.phase2_chunks, 0)

    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, unique_bytes, args.cpu_budget)
    ds.close()
    if args.copy_probe_mib:
        copy_probe(torch, args.copy_probe_mib)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
