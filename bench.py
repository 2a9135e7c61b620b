#!/usr/bin/env python3
"""Benchmark: top-K decode-attention steps/sec at 128K context on one MI355X.

Default workload (--config 2): one step is the whole decode-attention hot
path of one Llama-3-8B-shaped layer (32 query heads, 8 KV heads, d=128,
131,072 cached rows, bf16 K/V):
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

The other workloads are measured the same way when asked for:
  --config 3  ReTopK, Qwen2.5-7B-shaped (28 q / 4 KV heads), 65,536 initial
              rows, K=512, C=32, R=4, W=32, tau=0.85, refresh 128: the cache
              is warmed with 32 exact queries, then every timed pass runs the
              256 decode steps (one row appended per step) from that state.
              --requests B serves B independent requests per step (their own
              caches); --tau and --top-k select the pages' variants (0.90,
              1024); --budget N caps the voted candidates of the reuse path
              at N rows (confidence votes over the recalled supports);
  --config 4  batch of 16 sequences x 32,768 rows, K=1024, one
              topk_attn_decode call per step;
  --config 5  1,048,576 rows, K=8192, static window of 640 rows, one-pass step.
  --int8-recall K'  (workloads 2 and 5) the dynamic rows go through the int8
              recall stage instead: a scan of per-row int8 key codes (made
              before timing, one set per layer cache) picks K' rows, the
              exact keys choose K among them; the same exact-scoring pass
              scores the static window, whose rows join the chosen ones in
              one softmax.V pass (one topk_attn_decode_int8_static call).
              Not exact; the line reports the share of the exact top-K rows
              that the step chose.
  --config 6  multi-query exact top-K of the c3 prefill block: the 32 warm-up
              queries of all 28 query heads over the 65,536 initial rows,
              K=512, one topk_multi_query call per step (the products run on
              the bf16 matrix cores; the roofline is in TFLOP/s).
  --config 1  the small exact case: 1 query head, 1 KV head, fp32 cache of
              4,096 rows, K=64, one topk_attn_decode call per step
              (launch-bound; reported for completeness).

Workload 2 steps through --layers distinct copies of the K/V cache in turn
(default 4), as a model's decode does layer after layer: with a single copy
the 268 MB scanned per step would partly stay in the 256 MB last-level cache
between steps, and the scan would not be bound by HBM alone.

Prints ONE JSON line. `value` is steps/s over --steps timed steps bracketed
by stream events (--graph on replays the step captured in a HIP graph
instead of launching it from the host; slower on this stack). The
`roofline` object reports the kernel that dominates the step: algorithmic
bytes per launch over its average duration, measured over a second pass of
the same steps in which the library attaches HIP start/stop events to every
dispatch on the launch stream (kernels_avg_us lists every kernel from the
same pass).

Options for profiling runs: --copy-calibration runs only a plain device copy
of known size (to calibrate rocprofv3's FETCH_SIZE / WRITE_SIZE counters);
--plain-read runs only the library's plain-read kernel (stdk_hbm_read) over
the headline scan's partition of four rotating 268 MB key caches and prints
its rate, the ceiling the scan's HBM rate is compared against; --no-cpu skips
the oracle baseline.

The CPU baseline (cpu_baseline) is the oracle as it stands, timed on a
bounded sample of the same workload twice: on one host thread and on one
thread per available core (query heads split over a thread pool; numpy
releases the interpreter lock in its loops). `value` and `cores` are the
multi-thread leg's, `single_thread` the other's, `cpu_model` the host's.
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
BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix-core peak of MI355X
SCAN_SOURCES = ["sparse_top_decode_amd/csrc/scan_kernels.h", "sparse_top_decode_amd/csrc/device.h"]
METRIC = "top-K decode-attention steps/sec at 128K ctx; K-scan HBM GB/s vs peak"
TOPK_KERNELS = ("k_scan", "topk_filter_select", "topk_filter_select_sv", "topk_filter_lds_sv", "topk_select_lds",
                "topk_select_lds_sv", "sparse_sv", "dense_attn", "combine", "attn_merge")
MQ_KERNELS = ("mq_blockmax", "mq_threshold", "mq_collect", "mq_select")
RETOPK_KERNELS = ("retopk_reuse", "retopk_select", "retopk_vote", "retopk_attend", "retopk_rerank", "retopk_rerank_select",
                  "k_scan", "topk_filter_select", "topk_select_lds", "sparse_sv", "combine")


def scan_source_hash() -> str:
    h = hashlib.sha256()
    for p in SCAN_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def committed_traffic(cfg: int):
    """HBM bytes per k_scan launch from the committed rocprofv3 counter
    summary of this workload, if it was taken on the current kernel source."""
    try:
        with open(os.path.join(ROOT, "profiles", f"k_scan_c{cfg}_hbm_traffic.md")) as f:
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


# ---------------------------------------------------------------------------
# CPU baselines: the oracle as it stands, on a bounded sample of the workload
# ---------------------------------------------------------------------------
def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_threads() -> int:
    """Threads for the multi-thread leg: the cores this process may run on,
    capped by OMP_NUM_THREADS where it is set (the host's CPU share)."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def run_legs(one_rep, units, budget_s: float, max_reps: int = 20):
    """Times one_rep(list of units) repeated until budget_s has passed (at
    most max_reps times), first on one thread, then with the units split over
    cpu_threads() threads. Returns [(reps, seconds, threads), ...]."""
    from concurrent.futures import ThreadPoolExecutor
    legs = []
    for threads in (1, min(cpu_threads(), len(units))):
        parts = [units[i::threads] for i in range(threads)]
        ex = ThreadPoolExecutor(threads) if threads > 1 else None
        t0 = time.perf_counter()
        reps = 0
        while True:
            if ex is None:
                one_rep(units)
            else:
                list(ex.map(one_rep, parts))
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget_s or reps >= max_reps:
                break
        if ex is not None:
            ex.shutdown()
        legs.append((reps, el, threads))
    return legs


def baseline_record(legs, scale: float, what: str):
    """cpu_baseline: the multi-thread leg's rate (steps/s, scaled to whole
    steps by `scale`), the single-thread leg beside it, the host CPU model."""
    (r1, e1, _), (rn, en, tn) = legs
    return dict(value=rn * scale / en, unit="steps/s", cores=tn, kind="oracle",
                sample=f"{what}; multi-thread leg: {rn} rep(s) in {en:.1f} s on {tn} host threads (query heads "
                       f"split over a thread pool), single-thread leg: {r1} rep(s) in {e1:.1f} s (numpy fp64, no "
                       f"BLAS); values scaled to whole steps",
                single_thread=dict(value=r1 * scale / e1, cores=1), cpu_model=cpu_model())


def cpu_baseline_topk(w, budget_s: float = 10.0, seqs=None, heads=None):
    """Whole decode steps of the workload (or a stated sample of its
    sequences / query heads, scaled to whole steps)."""
    from oracle import reference as ref
    B, Hq = w.q.shape[0], w.q.shape[1]
    seqs = list(range(B)) if seqs is None else list(seqs)
    heads = list(range(Hq)) if heads is None else list(heads)
    sel = [(b, h) for b in seqs for h in heads]
    frac = len(sel) / float(B * Hq)

    def one_rep(part):
        dyn = ref.topk_attn_decode(w.q, w.k, w.v, w.ranges, w.top_k, w.scale, heads=part)
        if w.static_ranges:
            stat = ref.topk_attn_decode(w.q, w.k, w.v, w.static_ranges, w.top_k, w.scale, heads=part)
            ref.attn_merge_lse(stat["o"], stat["lse"], dyn["o"], dyn["lse"])

    legs = run_legs(one_rep, sel, budget_s)
    what = "dynamic top-K, static dense, merge" if w.static_ranges else "top-K attention"
    scope = ("all" if frac == 1.0 else f"{len(sel)} of {B * Hq}") + " (sequence, query head) pairs"
    return baseline_record(legs, frac, f"decode steps of the timed workload on {scope} ({what})")


def cpu_baseline_int8(w, K2: int, heads, budget_s: float = 10.0):
    """The oracle's int8-recall decode step (quantization of the dynamic rows
    included) on a stated sample of query heads, scaled to whole steps."""
    import numpy as np
    from oracle import reference as ref
    B, Hq = w.q.shape[0], w.q.shape[1]
    sel = [(0, h) for h in heads]
    rows = ref.range_rows(w.ranges)

    def one_rep(part):
        kvh = sorted({h // (Hq // w.H_kv) for _, h in part})
        codes = np.zeros(w.k.shape, dtype=np.int8)
        scales = np.zeros(w.k.shape[:3], dtype=np.float32)
        for hk in kvh:
            codes[0, hk, rows], scales[0, hk, rows] = ref.quantize_keys_int8(w.k[0, hk, rows])
        dyn = ref.topk_attn_decode_int8(w.q, w.k, w.v, codes, scales, w.ranges, w.top_k, K2, w.scale, heads=part)
        stat = ref.topk_attn_decode(w.q, w.k, w.v, w.static_ranges, w.top_k, w.scale, heads=part)
        ref.attn_merge_lse(stat["o"], stat["lse"], dyn["o"], dyn["lse"])

    legs = run_legs(one_rep, sel, budget_s)
    frac = len(sel) / float(B * Hq)
    return baseline_record(legs, frac, f"int8-recall decode steps on {len(sel)} of {B * Hq} query heads "
                                       f"(quantization of their KV heads' dynamic rows, int8 top-{K2}, exact top-K "
                                       f"inside, static dense, merge)")


def cpu_baseline_retopk(w, p, q_hist, sup_hist, budget_s: float = 10.0):
    """The oracle's ReTopK steps from the same warmed cache, in step order,
    until about budget_s of CPU time has passed; the multi-thread leg splits
    every step's (request, query head) pairs over the threads (each pair's
    cache is its own, so the split steps equal whole ones)."""
    from concurrent.futures import ThreadPoolExecutor
    from oracle import reference as ref
    rp = ref.RetopkParams(p["top_k"], p["cache_cap"], p["top_r"], p["recent"], p["tau"], p["refresh"],
                          p.get("budget", 0))
    warm, L0 = p["warmup"], p["L0"]
    B, Hq = w.q.shape[0], w.q.shape[1]
    pairs = [(b, h) for b in range(B) for h in range(Hq)]
    legs = []
    for threads in (1, min(cpu_threads(), len(pairs))):
        parts = [pairs[i::threads] for i in range(threads)]
        ex = ThreadPoolExecutor(threads) if threads > 1 else None
        st = ref.retopk_state_init(rp, q_hist, sup_hist)
        t0 = time.perf_counter()
        steps = 0
        for t in range(p["steps"]):
            qt = w.q[:, :, warm + t]
            if ex is None:
                _, st, _ = ref.retopk_step(rp, st, qt, w.k, w.v, L0 + t + 1, t, w.scale)
            else:
                cur = st
                outs = list(ex.map(lambda part: ref.retopk_step(rp, cur, qt, w.k, w.v, L0 + t + 1, t, w.scale,
                                                                heads=part)[1], parts))
                st = outs[0].copy()  # each thread's state holds the step of its own pairs
                for o_st, part in zip(outs, parts):
                    for b, h in part:
                        st.q_hat[b, h], st.support[b, h] = o_st.q_hat[b, h], o_st.support[b, h]
                        st.head[b, h], st.count[b, h] = o_st.head[b, h], o_st.count[b, h]
            steps += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        el = time.perf_counter() - t0
        if ex is not None:
            ex.shutdown()
        legs.append((steps, el, threads))
    (s1, e1, _), (sn, en, tn) = legs
    return dict(value=sn / en, unit="steps/s", cores=tn, kind="oracle",
                sample=f"the first timed ReTopK steps (all {B} x {Hq} (request, query head) pairs, from the same "
                       f"warmed cache): multi-thread leg {sn} step(s) in {en:.1f} s on {tn} host threads (pairs split "
                       f"over a thread pool), single-thread leg {s1} step(s) in {e1:.1f} s (numpy fp64, no BLAS)",
                single_thread=dict(value=s1 / e1, cores=1), cpu_model=cpu_model())


def cpu_baseline_mq(w, K: int, budget_s: float = 10.0):
    """The oracle's multi-query top-K on a seeded sample of the block's
    queries (scaled to whole blocks)."""
    import numpy as np
    from oracle import reference as ref
    B, Hq, M = w.q.shape[:3]
    rng = np.random.default_rng(5)
    perm = rng.permutation(Hq * M)
    n_sample = min(len(perm), 4 * cpu_threads())
    order = [(0, int(j // M), int(j % M)) for j in perm[:n_sample]]

    def one_rep(part):
        ref.topk_multi_query(w.q, w.k, w.ranges, K, w.scale, queries=part)

    legs = run_legs(one_rep, order, budget_s)
    return baseline_record(legs, n_sample / float(B * Hq * M),
                           f"{n_sample} of the block's {B * Hq * M} queries (seeded sample)")


# ---------------------------------------------------------------------------
# timing
# ---------------------------------------------------------------------------
def timed_passes(step, steps, names, reset=None, graph=None, graph_steps=1):
    """Pass A: `steps` steps bracketed by stream events only (a timing event
    attached to a dispatch costs several microseconds of step time). Pass B:
    the same number of steps again with HIP start/stop events attached by the
    library to every dispatch, on the launch stream; these give each kernel's
    average duration, and because every dispatch carries them each start
    stamp follows the previous kernel's end, so they agree with a rocprofv3
    kernel trace. `reset` (if given) restores the starting state before each
    pass. A `graph` holds `graph_steps` consecutive steps; pass A replays it
    until at least `steps` steps have run. Returns (ms per step, {kernel:
    (avg_us, launches)})."""
    import torch
    from sparse_top_decode_amd import ops
    run = graph.replay if graph is not None else step
    per_run = graph_steps if graph is not None else 1
    runs = -(-steps // per_run)
    if reset:
        reset()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(runs):
        run()
    ev1.record()
    torch.cuda.synchronize()
    total_ms = ev0.elapsed_time(ev1) * steps / (runs * per_run)
    kern = {}
    if names:
        if reset:
            reset()
        t_all = ops.KernelTimer(capacity=24 * (steps + 4))
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        for name in names:
            try:
                ms, n = t_all.read(name)
            except ops.native.StdkError:  # a family this library build does not have
                continue
            if n:
                kern[name] = (1000.0 * ms / n, n)
        t_all.close()
    return total_ms / steps, kern


def capture(step, n=1):
    """n consecutive steps captured once in a HIP graph (None if capture
    fails). With rotating layer caches n is a multiple of their number, so
    that each replay scans every cache equally often, as the direct
    launches do."""
    import torch
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n):
                step()
        torch.cuda.synchronize()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        return g
    except Exception as e:  # capture unsupported: time direct launches
        print(f"graph capture failed ({e}); timing direct launches", file=sys.stderr)
        return None


def roofline_mfma(kern, kernel, flops_per_launch):
    avg = kern.get(kernel, (None, 0))[0]
    achieved = None if not avg else flops_per_launch / (avg * 1e-6) / 1e12
    return {
        "bound": "mfma",
        "achieved": None if achieved is None else round(achieved, 1),
        "peak": BF16_PEAK_TFLOPS,
        "unit": "TFLOP/s",
        "frac": None if achieved is None else round(achieved / BF16_PEAK_TFLOPS, 4),
        "traffic": None,
        "kernel": kernel,
        "algorithmic_flops_per_launch": int(flops_per_launch),
        "avg_launch_us": None if not avg else round(avg, 2),
    }


def roofline(kern, kernel, bytes_per_launch, traffic):
    avg = kern.get(kernel, (None, 0))[0]
    achieved = None if not avg else bytes_per_launch / (avg * 1e-6) / 1e9
    return {
        "bound": "hbm",
        "achieved": None if achieved is None else round(achieved, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": None if achieved is None else round(achieved / HBM_PEAK_GBS, 4),
        "traffic": traffic,
        "kernel": kernel,
        "algorithmic_bytes_per_launch": int(bytes_per_launch),
        "avg_launch_us": None if not avg else round(avg, 2),
    }


def line(args, ms_per_step, workload, cfg_extra, roof, kern, cpu, dtype="bf16"):
    """The bench record. `dtype` is the type the path computes from (the key
    and value cache's: products and sums are accumulated in fp32)."""
    value = 1000.0 / ms_per_step
    config = {"workload": workload}
    config.update(cfg_extra)
    return {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": config,
        "roofline": roof,
        "kernels_avg_us": {k: round(v[0], 2) for k, v in kern.items()},
        "cpu_baseline": cpu,
    }


def to_dev(w):
    import numpy as np
    import torch
    dev = torch.device("cuda:0")
    if w.kv_dtype == "f32":
        return dev, torch.from_numpy(w.k).to(dev), torch.from_numpy(w.v).to(dev)
    k = torch.from_numpy(w.k.view(np.int16)).to(dev).view(torch.bfloat16)
    v = torch.from_numpy(w.v.view(np.int16)).to(dev).view(torch.bfloat16)
    return dev, k, v


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------
def bench_topk(args, cfg):
    """c2 / c5: dynamic top-K + static window + merge; c4: batched top-K;
    c1: the small fp32 case."""
    import torch
    from sparse_top_decode_amd import ops
    from workloads import make_workload

    w = make_workload(cfg, L=args.L if cfg == 2 else None)
    dev, k0, v0 = to_dev(w)
    # one cache per layer, used in turn (a decode step reads each layer's
    # cache once per token); with several layers no layer's 268 MB stays in
    # the 256 MB last-level cache between its steps, so the scan streams
    # from HBM as it would in a model
    n_layers = max(1, args.layers if cfg == 2 else 1)
    caches = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(n_layers - 1)]
    k, v = k0, v0
    layer = {"i": 0}
    q = torch.from_numpy(w.q).to(dev)
    lay = ops.make_layout(k, w.H_q)
    K = w.top_k
    B = w.q.shape[0]
    n_dyn = sum(e - b for b, e in w.ranges)
    n_stat = sum(e - b for b, e in w.static_ranges) if w.static_ranges else 0
    idx = torch.empty((B, w.H_q, K), dtype=torch.int32, device=dev)
    o_m = torch.empty((B, w.H_q, 128), dtype=torch.float32, device=dev)
    l_m = torch.empty((B, w.H_q), dtype=torch.float32, device=dev)
    path = args.path if n_stat else "top-k only"
    q8 = None
    if args.int8_recall and cfg in (2, 5):
        path = f"int8 recall K'={args.int8_recall}, static rows in the same softmax.V pass"
        q8 = [ops.quantize_keys_int8(kc, w.ranges, w.H_q, layout=lay) for kc, _ in caches]
        ws_q = ops.new_workspace(ops.topk_attn_decode_int8_static_workspace_size(lay, n_dyn, n_stat, K,
                                                                                 args.int8_recall), dev)

        def step():
            i = layer["i"]
            k, v = caches[i]
            codes, scales = q8[i]
            layer["i"] = (i + 1) % n_layers
            ops.topk_attn_decode_int8_static(q, k, v, codes, scales, w.ranges, w.static_ranges, K, args.int8_recall,
                                             w.scale, idx_out=idx, o_out=o_m, lse_out=l_m, workspace=ws_q,
                                             layout=lay)
    elif n_stat and args.path == "one-pass":
        ws_f = ops.new_workspace(ops.topk_attn_decode_static_workspace_size(lay, n_dyn, n_stat, K), dev)

        def step():
            # static rows scored by the same scan and appended to the chosen
            # rows; one softmax.V pass and one combine give the merged output
            k, v = caches[layer["i"]]
            layer["i"] = (layer["i"] + 1) % n_layers
            ops.topk_attn_decode_static(q, k, v, w.ranges, w.static_ranges, K, w.scale, idx_out=idx, o_out=o_m,
                                        lse_out=l_m, workspace=ws_f, layout=lay)
    elif n_stat:
        ws_d = ops.new_workspace(ops.topk_attn_decode_workspace_size(lay, n_dyn, K), dev)
        ws_s = ops.new_workspace(ops.topk_attn_decode_workspace_size(lay, n_stat, K), dev)
        o_d, l_d, o_s, l_s = (torch.empty_like(o_m), torch.empty_like(l_m), torch.empty_like(o_m),
                              torch.empty_like(l_m))

        def step():
            k, v = caches[layer["i"]]
            layer["i"] = (layer["i"] + 1) % n_layers
            ops.topk_attn_decode(q, k, v, w.ranges, K, w.scale, idx_out=idx, o_out=o_d, lse_out=l_d,
                                 workspace=ws_d, layout=lay)
            ops.topk_attn_decode(q, k, v, w.static_ranges, K, w.scale, o_out=o_s, lse_out=l_s, workspace=ws_s,
                                 want_idx=False, layout=lay)
            ops.attn_merge_lse(o_s, l_s, o_d, l_d, o_out=o_m, lse_out=l_m)
    else:
        ws_d = ops.new_workspace(ops.topk_attn_decode_workspace_size(lay, n_dyn, K), dev)

        def step():
            ops.topk_attn_decode(q, k, v, w.ranges, K, w.scale, idx_out=idx, o_out=o_m, lse_out=l_m,
                                 workspace=ws_d, layout=lay)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # a graph holds whole rounds of the layer caches, at least 8 steps, so
    # that a replay's own launch cost is spread over them
    graph_steps = n_layers * -(-8 // n_layers)
    graph = capture(step, graph_steps) if args.graph == "on" else None
    names = TOPK_KERNELS if args.kernel_events == "on" else ()
    if q8 is not None:
        names = names + ("retopk_rerank", "retopk_rerank_select") if names else ()
    ms, kern = timed_passes(step, args.steps, names, graph=graph, graph_steps=graph_steps)
    row_bytes = 128 * (4 if w.kv_dtype == "f32" else 2)
    if q8 is None:
        scan_bytes = B * w.H_kv * n_dyn * row_bytes  # every dynamic key row once, d=128
        roof = roofline(kern, "k_scan", scan_bytes, committed_traffic(cfg))
    else:
        # the scan reads the int8 codes (128 B) and the scale (4 B) of every
        # dynamic row; the static window is scored by the rerank, not k_scan
        scan_bytes = B * w.H_kv * n_dyn * (128 + 4)
        roof = roofline(kern, "k_scan", scan_bytes, None)
    if cfg == 1:
        workload = (f"small exact case: 1 q / 1 KV head, d=128, L={w.L}, fp32 K/V, top-K={K} over all rows "
                    f"(query rotated away from the key distribution)")
        cpu = None if args.no_cpu else cpu_baseline_topk(w)
    elif cfg == 4:
        workload = (f"batched decode attention: {B} sequences x {w.L} rows, 32 q / 8 KV heads (Llama-3-8B layout), "
                    f"d=128, bf16 K/V with per-sequence key offsets, top-K={K} per (sequence, query head)")
        cpu = None if args.no_cpu else cpu_baseline_topk(w, seqs=[0])
    else:
        workload = (f"Llama-3-8B-shaped decode attention layer: 32 q / 8 KV heads, d=128, L={w.L}, bf16 K/V, "
                    f"top-K={K} over the {n_dyn} dynamic rows + dense over the {n_stat} static rows + LSE merge")
        if cfg == 5:
            workload += " (64 planted rows per query head)"
        sample_heads = None if cfg == 2 else [0, 9, 18, 27]
        cpu = None if args.no_cpu or q8 is not None else cpu_baseline_topk(w, heads=sample_heads)
    extra = {"batch": B, "seq_len": w.L, "top_k": K, "kv_cache": w.kv_dtype, "accumulation": "f32",
             "parallelism": "none (1 GPU)", "path": path, "hip_graph": graph is not None, "layer_caches": n_layers}
    if cfg == 5 and w.planted is not None and q8 is None:
        # context: how many of each query head's 64 planted rows the last
        # timed step's top-K holds
        import numpy as np
        got = idx.cpu().numpy()
        rec = [int(np.isin(w.planted[h], got[0, h]).sum()) for h in range(w.H_q)]
        extra["planted_rows_recovered"] = {"mean": round(float(np.mean(rec)), 2), "min": int(min(rec)),
                                           "of": int(w.planted.shape[1])}
    if q8 is not None:
        # share of the exact top-K rows the int8 step chose (layer 0's cache)
        k0c, v0c = caches[0]
        ex_idx, _, _ = ops.topk_attn_decode(q, k0c, v0c, w.ranges, K, w.scale, layout=lay)
        q8_idx, _, _, _ = ops.topk_attn_decode_int8(q, k0c, v0c, q8[0][0], q8[0][1], w.ranges, K, args.int8_recall,
                                                    w.scale, layout=lay)
        torch.cuda.synchronize()
        a_ = ex_idx.cpu().numpy()
        b_ = q8_idx.cpu().numpy()
        import numpy as np
        rec = np.mean([np.isin(a_[0, h][a_[0, h] >= 0], b_[0, h]).mean() for h in range(a_.shape[1])])
        extra["recall_vs_exact"] = round(float(rec), 5)
        extra["int8_recall_k"] = args.int8_recall
        workload += f"; dynamic rows through the int8 recall stage (K'={args.int8_recall}), not exact"
        cpu = None if args.no_cpu else cpu_baseline_int8(w, args.int8_recall, [0, 9, 18, 27])
    return line(args, ms, workload, extra, roof, kern, cpu, dtype=w.kv_dtype)


def bench_retopk(args):
    """c3: 256 ReTopK decode steps from a warmed cache, per timed pass."""
    import numpy as np
    import torch
    from sparse_top_decode_amd import ops
    from workloads import make_workload

    w = make_workload(3, B=args.requests)
    p = dict(w.retopk)
    if args.tau is not None:
        p["tau"] = args.tau
    if args.top_k is not None:
        p["top_k"] = args.top_k
    p["budget"] = args.budget
    dev, k, v = to_dev(w)
    K, warm, n_steps, L0 = p["top_k"], p["warmup"], p["steps"], p["L0"]
    rt = ops.Retopk(k, w.H_q, top_k=K, cache_cap=p["cache_cap"], top_r=p["top_r"], recent=p["recent"],
                    tau=p["tau"], refresh=p["refresh"], scale=w.scale, budget=p["budget"])
    qall = torch.from_numpy(np.ascontiguousarray(w.q)).to(dev)
    qs = [qall[:, :, j].contiguous() for j in range(warm + n_steps)]
    # the cache starts from the last 32 exact-path queries over the initial rows
    sups = [ops.topk_attn_decode(qs[j], k, v, [(0, L0)], K, w.scale, layout=rt.layout)[0] for j in range(warm)]
    q_hist = torch.stack(qs[:warm], dim=2).contiguous()
    sup_hist = torch.stack(sups, dim=2).contiguous()
    B = w.q.shape[0]
    support = torch.empty((B, w.H_q, K), dtype=torch.int32, device=dev)
    o = torch.empty((B, w.H_q, 128), dtype=torch.float32, device=dev)
    lse = torch.empty((B, w.H_q), dtype=torch.float32, device=dev)
    paths = [torch.empty((B, w.H_q), dtype=torch.int32, device=dev) for _ in range(n_steps)]
    ncands = [torch.empty((B, w.H_q), dtype=torch.int32, device=dev) for _ in range(n_steps)]
    state = {"t": 0}

    def reset():
        rt.init(q_hist, sup_hist)
        state["t"] = 0

    def step():
        t = state["t"]
        rt.step(qs[warm + t], k, v, L0 + t + 1, t,
                out=dict(support=support, o=o, lse=lse, path=paths[t], n_cand=ncands[t]))
        state["t"] = (t + 1) % n_steps

    reset()
    for _ in range(n_steps):  # warm-up pass over the whole sequence
        step()
    torch.cuda.synchronize()
    args.steps = n_steps
    args.warmup = n_steps
    names = RETOPK_KERNELS if args.kernel_events == "on" else ()
    step_api = "retopk_step"
    if args.graph == "on":
        # retopk_step_device: [L_t, t] in device memory, advanced by every
        # step; the whole pass (one call per step, each with its own query
        # and per-step outputs) captured once in a HIP graph and replayed
        step_api = "retopk_step_device, the timed pass replayed from one HIP graph"
        step_t = torch.tensor([L0 + 1, 0], dtype=torch.int64, device=dev)
        start = torch.tensor([L0 + 1, 0], dtype=torch.int64, device=dev)

        def reset_dev():
            rt.init(q_hist, sup_hist)
            step_t.copy_(start)
            state["t"] = 0

        def step_dev():
            t = state["t"]
            rt.step_device(qs[warm + t], k, v, step_t,
                           out=dict(support=support, o=o, lse=lse, path=paths[t], n_cand=ncands[t]))
            state["t"] = (t + 1) % n_steps

        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n_steps):
                step_dev()
        torch.cuda.synchronize()
        reset_dev()
        g.replay()  # warm-up replay
        torch.cuda.synchronize()
        reset_dev()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record()
        g.replay()
        ev1.record()
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / n_steps
        # per-kernel durations from a pass of the same calls launched directly
        _, kern = timed_passes(step_dev, n_steps, names, reset=reset_dev) if names else (None, {})
        reset_dev()
        for _ in range(n_steps):  # the per-step paths and counts of one pass, for the statistics below
            step_dev()
        torch.cuda.synchronize()
    else:
        ms, kern = timed_passes(step, n_steps, names, reset=reset)
    pth = torch.stack(paths, dim=-1).cpu().numpy()
    nc = torch.stack(ncands, dim=-1).cpu().numpy()
    reuse = pth == 0
    mean_m = float(nc[reuse].mean()) if reuse.any() else 0.0
    # reuse heads: every candidate key row is read once (256 B) and, where
    # one workgroup also forms softmax . V (retopk_reuse, retopk_attend), the
    # value rows of the min(K, M) kept candidates; retopk_reuse also reads
    # every head's C cached unit queries (512 B each) and a reuse head's R
    # picked supports (4 B per row). Averaged over that kernel's launches.
    n_rr = int(kern.get("retopk_rerank", (0, 0))[1])
    n_att = int(kern.get("retopk_attend", (0, 0))[1])
    n_ru = int(kern.get("retopk_reuse", (0, 0))[1])
    att_rows = float(nc[reuse].sum()) + float(np.minimum(nc[reuse], K).sum())
    if n_ru:
        ru_bytes = (att_rows * 256 + float(pth.size) * p["cache_cap"] * 512
                    + float(reuse.sum()) * p["top_r"] * K * 4)
        roof = roofline(kern, "retopk_reuse", ru_bytes / n_ru, None)
    elif n_att:
        roof = roofline(kern, "retopk_attend", att_rows * 256 / n_att, None)
    else:
        roof = roofline(kern, "retopk_rerank", float(nc[reuse].sum()) * 256 / max(1, n_rr), None)
    vs_exact = free_running_vs_exact(rt, reset, qs, k, v, w, p, support, o, lse)
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline_retopk(w, p, q_hist.cpu().numpy(), sup_hist.cpu().numpy())
    workload = (f"ReTopK decode, Qwen2.5-7B-shaped layer: {B} request(s) per step, 28 q / 4 KV heads, d=128, "
                f"{L0} initial rows + 1 per step, "
                f"bf16 K/V, K={K}, C={p['cache_cap']}, R={p['top_r']}, W={p['recent']}, tau={p['tau']}, "
                f"refresh every {p['refresh']} steps, AR(1) queries; {n_steps} steps per timed pass"
                + (f"; voted candidates capped at {p['budget']}" if p["budget"] else ""))
    extra = {"batch": B, "seq_len": L0, "top_k": K, "kv_cache": "bf16", "parallelism": "none (1 GPU)",
             "reuse_fraction": round(float(reuse.mean()), 4), "mean_candidates_reuse": round(mean_m, 1),
             "rerank_launches": n_rr, "attend_launches": n_att, "reuse_launches": n_ru, "step_api": step_api, "hip_graph": args.graph == "on",
             "vs_exact_free_running": vs_exact}
    return line(args, ms, workload, extra, roof, kern, cpu)


def free_running_vs_exact(rt, reset, qs, k, v, w, p, support, o, lse):
    """Context, not a parity check: the ReTopK run, free-running from the
    warmed cache over the timed steps, against exact top-K attention of the
    same queries at every step (the ReTopK review's point that index recall
    and attention quality differ). Per (request, query head, step): recall =
    share of the exact top-K rows that ReTopK's support holds; output error =
    ||o_retopk - o_exact|| / ||o_exact||; lse difference."""
    import numpy as np
    import torch
    from sparse_top_decode_amd import ops
    K, warm, n_steps, L0 = p["top_k"], p["warmup"], p["steps"], p["L0"]
    reset()
    rec, rel, dl = [], [], []
    path = torch.empty_like(lse, dtype=torch.int32)
    ncand = torch.empty_like(lse, dtype=torch.int32)
    for t in range(n_steps):
        rt.step(qs[warm + t], k, v, L0 + t + 1, t, out=dict(support=support, o=o, lse=lse, path=path, n_cand=ncand))
        ex_idx, ex_o, ex_l = ops.topk_attn_decode(qs[warm + t], k, v, [(0, L0 + t + 1)], K, w.scale,
                                                  layout=rt.layout)
        a = support.cpu().numpy()
        e = ex_idx.cpu().numpy()
        for b in range(a.shape[0]):
            for h in range(a.shape[1]):
                rows = e[b, h][e[b, h] >= 0]
                rec.append(float(np.isin(rows, a[b, h]).mean()) if rows.size else 1.0)
        oo, eo = o.double(), ex_o.double()
        rel.append((torch.linalg.vector_norm(oo - eo, dim=-1) / torch.linalg.vector_norm(eo, dim=-1)).cpu().numpy())
        dl.append((lse.double() - ex_l.double()).abs().cpu().numpy())
    rel = np.concatenate([x.ravel() for x in rel])
    dl = np.concatenate([x.ravel() for x in dl])
    return {"steps": n_steps, "recall_mean": round(float(np.mean(rec)), 4), "recall_min": round(float(np.min(rec)), 4),
            "o_rel_l2_mean": round(float(rel.mean()), 5), "o_rel_l2_max": round(float(rel.max()), 5),
            "lse_abs_diff_mean": round(float(dl.mean()), 5)}


def bench_multi_query(args):
    """c3 prefill block: one topk_multi_query call (28 x 32 queries over
    65,536 rows, K=512) per step."""
    import torch
    from sparse_top_decode_amd import ops
    from workloads import c3_prefill_block

    w = c3_prefill_block()
    K = 512 if args.top_k is None else args.top_k
    dev, k, _ = to_dev(w)
    q = torch.from_numpy(w.q).to(dev)
    B, Hq, M = w.q.shape[:3]
    lay = ops.make_layout(k, Hq)
    n = w.L
    idx = torch.empty((B, Hq, M, K), dtype=torch.int32, device=dev)
    ws = ops.new_workspace(ops.topk_multi_query_workspace_size(lay, M, n, K), dev)

    def step():
        ops.topk_multi_query(q, k, w.ranges, K, w.scale, idx_out=idx, workspace=ws, layout=lay)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    names = MQ_KERNELS if args.kernel_events == "on" else ()
    ms, kern = timed_passes(step, args.steps, names)
    flops = 2.0 * B * Hq * M * n * 128  # one pass: every (query, row) product once
    dom = max(("mq_blockmax", "mq_collect"), key=lambda x: kern.get(x, (0.0, 0))[0])
    roof = roofline_mfma(kern, dom, flops)
    cpu = None if args.no_cpu else cpu_baseline_mq(w, K)
    workload = (f"multi-query exact top-K (prefill block): {M} queries x {Hq} q heads / {w.H_kv} KV heads "
                f"(Qwen2.5-7B layout), d=128, {n} bf16 key rows, K={K} per query")
    extra = {"batch": B, "seq_len": n, "top_k": K, "queries_per_head": M, "kv_cache": "bf16",
             "parallelism": "none (1 GPU)"}
    return line(args, ms, workload, extra, roof, kern, cpu)


def bench_plain_read(args):
    """The plain-read reference: stdk_hbm_read over the headline scan's
    partition (8 KV heads, the 130,432 dynamic rows of 256 B each, one
    workgroup per CU split evenly over the KV heads) of four rotating
    268 MB key caches; the same bytes k_scan reads per launch."""
    import torch
    from sparse_top_decode_amd import ops
    dev = torch.device("cuda:0")
    L, Hkv, row0, n_dyn, row_b, n_bufs = 131072, 8, 128, 130432, 256, 4
    bufs = [torch.empty(Hkv * L * row_b, dtype=torch.uint8, device=dev).random_(0, 256) for _ in range(n_bufs)]
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    wpg = max(1, torch.cuda.get_device_properties(dev).multi_processor_count // Hkv)
    nbytes = Hkv * n_dyn * row_b
    state = {"i": 0}

    def step():
        buf = bufs[state["i"]]
        state["i"] = (state["i"] + 1) % n_bufs
        ops.hbm_read(buf[row0 * row_b:], L * row_b, Hkv, n_dyn * row_b, wpg, sink)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ms, kern = timed_passes(step, args.steps, ("hbm_read",))
    avg = kern.get("hbm_read", (None, 0))[0]
    gbs = nbytes / (avg * 1e-6) / 1e9 if avg else None
    return {"metric": "plain HBM read rate over the key-scan partition (reference ceiling)",
            "value": None if gbs is None else round(gbs, 1), "unit": "GB/s", "peak": HBM_PEAK_GBS,
            "frac": None if gbs is None else round(gbs / HBM_PEAK_GBS, 4), "bytes_per_launch": nbytes,
            "avg_launch_us": None if avg is None else round(avg, 2), "steps": args.steps, "warmup": args.warmup,
            "config": {"workload": f"{Hkv} regions of {n_dyn} rows x {row_b} B (the c2 layer's dynamic key rows), "
                                   f"{wpg} workgroups of 512 threads per region, {n_bufs} rotating caches"}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, choices=[1, 2, 3, 4, 5, 6], default=2,
                    help="workload: 2 (default, the headline), 1 small fp32 case, 3 ReTopK, 4 batched, 5 1M rows, "
                         "6 multi-query top-K of the prefill block")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES")
    ap.add_argument("--plain-read", action="store_true",
                    help="only the plain-read reference over the headline scan's partition (prints its own line)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--requests", type=int, default=1, help="workload 3: requests served per step, each with its own caches")
    ap.add_argument("--tau", type=float, default=None, help="workload 3: similarity threshold (default 0.85)")
    ap.add_argument("--top-k", type=int, default=None, help="workloads 3 and 6: K (default 512)")
    ap.add_argument("--int8-recall", type=int, default=0, metavar="K2",
                    help="workloads 2 and 5: top-K' superset from int8 key codes, exact top-K inside it (0 = off)")
    ap.add_argument("--budget", type=int, default=0,
                    help="workload 3: voted candidates kept on the reuse path (0 = the whole union)")
    ap.add_argument("--L", type=int, default=131072, help="cache length of workload 2")
    ap.add_argument("--layers", type=int, default=4,
                    help="workload 2: distinct K/V caches used in turn, one per layer (1 = the same cache every "
                         "step, partly served by the last-level cache)")
    ap.add_argument("--graph", choices=["on", "off"], default="off",
                    help="on: the timed steps replay the step captured in a HIP graph (workload 3: the 256 steps "
                         "of a pass through retopk_step_device, captured as one graph)")
    ap.add_argument("--path", choices=["one-pass", "three-calls"], default="one-pass",
                    help="one-pass: topk_attn_decode_static; three-calls: topk_attn_decode over the dynamic "
                         "rows, topk_attn_decode over the static rows, attn_merge_lse")
    ap.add_argument("--kernel-events", choices=["on", "off"], default="on",
                    help="the second, evented pass that gives per-kernel durations and the roofline")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path has no multi-GPU mode.",
              file=sys.stderr, flush=True)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.plain_read:
        print(json.dumps(bench_plain_read(args)), flush=True)
        return
    if args.config == 3:
        out = bench_retopk(args)
    elif args.config == 6:
        out = bench_multi_query(args)
    else:
        out = bench_topk(args, args.config)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
