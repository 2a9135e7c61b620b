#!/usr/bin/env python3
"""Benchmark: top-K decode-attention steps/sec at 128K context on one MI355X.

One step is the whole decode-attention hot path of one Llama-3-8B-shaped
layer (32 query heads, 8 KV heads, d=128, 131,072 cached rows, bf16 K/V):
  1. top-K attention (K=2048) of every query head over the dynamic rows
     [128, 130560): exact QK scan, per-head top-K select, softmax.V;
  2. dense attention over the 640 static rows (first 128, last 512);
  3. log-sum-exp merge of the two partial outputs.
By default the step is one call of topk_attn_decode_static: the scan scores
the static rows beside the dynamic ones, the select appends them to every
chosen-row list, and one softmax.V pass plus one combine produce the merged
output (Eq. 4-5 applied to the partials). --path three-calls runs the same
step as topk_attn_decode (dynamic) + topk_attn_decode (static, dense) +
attn_merge_lse. Inputs are synthetic and resident in HBM before timing starts.

Prints ONE JSON line. `value` is steps/s over --steps timed steps bracketed
by stream events (--graph on replays the step captured in a HIP graph
instead of launching it from the host; slower on this stack). The `roofline` object reports the K-cache scan kernel
(k_scan): algorithmic bytes per launch (every scanned key row once, 256 B)
over its average duration, measured over a second pass of --steps steps in
which the library attaches HIP start/stop events to every dispatch on the
launch stream (kernels_avg_us lists every kernel from the same pass).

Options for profiling runs: --copy-calibration runs only a plain device copy
of known size (to calibrate rocprofv3's FETCH_SIZE / WRITE_SIZE counters);
--no-cpu skips the oracle baseline.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
SCAN_SOURCES = ["sparse_top_decode_amd/csrc/scan_kernels.h", "sparse_top_decode_amd/csrc/device.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_scan_c2_hbm_traffic.md")


def scan_source_hash() -> str:
    h = hashlib.sha256()
    for p in SCAN_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def committed_traffic():
    """HBM bytes per k_scan launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            txt = f.read()
    except OSError:
        return None
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", txt)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m_hash or not m_bytes or m_hash.group(1) != scan_source_hash():
        return None
    return float(m_bytes.group(1))


def copy_calibration(nbytes: int):
    import torch
    x = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(5):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "launches": 5}), flush=True)


def cpu_baseline(w, budget_s: float = 12.0):
    """The oracle (untuned) on the host: whole decode steps of the same
    workload, repeated until about budget_s of CPU time has passed."""
    from oracle import reference as ref
    t0 = time.perf_counter()
    reps = 0
    while True:
        dyn = ref.topk_attn_decode(w.q, w.k, w.v, w.ranges, w.top_k, w.scale)
        stat = ref.topk_attn_decode(w.q, w.k, w.v, w.static_ranges, w.top_k, w.scale)
        ref.attn_merge_lse(stat["o"], stat["lse"], dyn["o"], dyn["lse"])
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 20:
            break
    return dict(value=reps / el, unit="steps/s", cores=1, kind="oracle",
                sample=f"{reps} full decode step(s) of the timed workload (all 32 query heads: dynamic top-K, "
                       f"static dense, merge), {el:.1f} s on one host thread (numpy fp64, no BLAS)")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--L", type=int, default=131072)
    ap.add_argument("--graph", choices=["on", "off"], default="off",
                    help="on: the timed steps replay the step captured in a HIP graph (measured slower than "
                         "direct launches for this five-kernel step)")
    ap.add_argument("--path", choices=["one-pass", "three-calls"], default="one-pass",
                    help="one-pass: topk_attn_decode_static; three-calls: topk_attn_decode over the dynamic "
                         "rows, topk_attn_decode over the static rows, attn_merge_lse")
    ap.add_argument("--kernel-events", choices=["on", "off"], default="on",
                    help="record per-kernel HIP events during the timed region (needed for the roofline)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path has no multi-GPU mode.",
              file=sys.stderr, flush=True)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import numpy as np
    import torch

    from sparse_top_decode_amd import ops
    from workloads import make_workload

    w = make_workload(2, L=args.L)
    dev = torch.device("cuda:0")
    q = torch.from_numpy(w.q).to(dev)
    k = torch.from_numpy(w.k.view(np.int16)).to(dev).view(torch.bfloat16)
    v = torch.from_numpy(w.v.view(np.int16)).to(dev).view(torch.bfloat16)
    lay = ops.make_layout(k, w.H_q)
    K = w.top_k
    n_dyn = sum(e - b for b, e in w.ranges)
    n_stat = sum(e - b for b, e in w.static_ranges)
    idx = torch.empty((1, w.H_q, K), dtype=torch.int32, device=dev)
    o_m = torch.empty((1, w.H_q, 128), dtype=torch.float32, device=dev)
    l_m = torch.empty((1, w.H_q), dtype=torch.float32, device=dev)
    if args.path == "one-pass":
        ws_f = ops.new_workspace(ops.topk_attn_decode_static_workspace_size(lay, n_dyn, n_stat, K), dev)

        def step():
            # static rows scored by the same scan and appended to the chosen
            # rows; one softmax.V pass and one combine give the merged output
            ops.topk_attn_decode_static(q, k, v, w.ranges, w.static_ranges, K, w.scale, idx_out=idx, o_out=o_m,
                                        lse_out=l_m, workspace=ws_f, layout=lay)
    else:
        ws_d = ops.new_workspace(ops.topk_attn_decode_workspace_size(lay, n_dyn, K), dev)
        ws_s = ops.new_workspace(ops.topk_attn_decode_workspace_size(lay, n_stat, K), dev)
        o_d = torch.empty_like(o_m)
        l_d = torch.empty_like(l_m)
        o_s = torch.empty_like(o_m)
        l_s = torch.empty_like(l_m)

        def step():
            ops.topk_attn_decode(q, k, v, w.ranges, K, w.scale, idx_out=idx, o_out=o_d, lse_out=l_d,
                                 workspace=ws_d, layout=lay)
            ops.topk_attn_decode(q, k, v, w.static_ranges, K, w.scale, o_out=o_s, lse_out=l_s, workspace=ws_s,
                                 want_idx=False, layout=lay)
            ops.attn_merge_lse(o_s, l_s, o_d, l_d, o_out=o_m, lse_out=l_m)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # The step captured once in a HIP graph, replayed in the timed pass (no
    # host work or launch gaps between its kernels). Falls back to eager
    # launches if capture is unavailable.
    graph = None
    if args.graph == "on":
        try:
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                step()
            torch.cuda.current_stream().wait_stream(side)
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                step()
            torch.cuda.synchronize()
            for _ in range(3):
                graph.replay()
            torch.cuda.synchronize()
        except Exception as e:  # capture unsupported: time eager launches
            print(f"graph capture failed ({e}); timing eager launches", file=sys.stderr)
            graph = None
    run_step = graph.replay if graph is not None else step

    # Pass A: the timed steps, bracketed by stream events only (a timing
    # event attached to a dispatch costs several microseconds of step time).
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(args.steps):
        run_step()
    ev1.record()
    torch.cuda.synchronize()
    total_ms = ev0.elapsed_time(ev1)
    # Pass B: the same number of steps again with HIP start/stop events
    # attached by the library to every dispatch, on the launch stream. These
    # give each kernel's average duration, the scan's included; with events on
    # every dispatch each start stamp follows the previous kernel's end, so
    # the durations agree with a rocprofv3 kernel trace.
    scan_bytes = w.H_kv * n_dyn * 256  # every dynamic key row once, bf16 d=128
    achieved = scan_avg_s = None
    kern = {}
    names = ("k_scan", "topk_filter", "topk_select", "sparse_sv", "dense_attn", "combine", "attn_merge")
    if args.kernel_events == "on":
        t_all = ops.KernelTimer(capacity=16 * (args.steps + 4))
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        for name in names:
            ms, n = t_all.read(name)
            if n:
                kern[name] = round(1000.0 * ms / n, 2)
        scan_ms, scan_n = t_all.read("k_scan")
        t_all.close()
        scan_avg_s = scan_ms / scan_n / 1000.0
        achieved = scan_bytes / scan_avg_s / 1e9
    traffic = committed_traffic()

    ms_per_step = total_ms / args.steps
    value = 1000.0 / ms_per_step
    out = {
        "metric": "top-K decode-attention steps/sec at 128K ctx; K-scan HBM GB/s vs peak",
        "value": round(value, 1),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"Llama-3-8B-shaped decode attention layer: 32 q / 8 KV heads, d=128, L={w.L}, bf16 K/V, "
                        f"top-K={K} over the {n_dyn} dynamic rows + dense over the {n_stat} static rows + LSE merge",
            "batch": 1, "seq_len": w.L, "top_k": K, "kv_cache": "bf16", "parallelism": "none (1 GPU)",
            "path": args.path, "hip_graph": graph is not None,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": None if achieved is None else round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": None if achieved is None else round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": "k_scan",
            "algorithmic_bytes_per_launch": scan_bytes,
            "avg_launch_us": None if scan_avg_s is None else round(scan_avg_s * 1e6, 2),
        },
        "kernels_avg_us": kern,
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
