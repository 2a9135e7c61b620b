"""GPU parity of the ReTopK step, in lock-step with the oracle: before every
step the GPU's cache state is copied to the host, the oracle runs the same
step from it, and path, candidate set, support, o, lse and the pushed state
are compared. A step whose decision is within 1e-6 of a tie (best cosine vs
tau, the R-th vs (R+1)-th cosine, or, with a candidate budget, two different
vote sums at the cut) is flagged, not failed."""

import numpy as np
import pytest
import torch

from gpu_util import BAND, check_index_set, check_out, dev_kv, log, pmap
from oracle import reference as ref
from workloads import make_workload

pytestmark = pytest.mark.gpu

NEAR = 1e-6


@pytest.fixture(scope="module")
def ops(stdk):
    from sparse_top_decode_amd import ops
    return ops


def host_state(rt):
    return ref.RetopkState(rt.q_hat.cpu().numpy(), rt.support.cpu().numpy(), rt.head.cpu().numpy(),
                           rt.count.cpu().numpy())


def warm_cache(ops, w, rt, k, v, n_warm, K):
    """The first n_warm queries go through the exact path over the initial
    rows and fill the caches (oldest first); n_warm = 0 leaves them empty."""
    L0 = w.retopk["L0"]
    qs = torch.from_numpy(np.ascontiguousarray(w.q[:, :, :n_warm])).cuda()
    if n_warm == 0:
        sup = torch.zeros((w.q.shape[0], w.H_q, 0, K), dtype=torch.int32, device="cuda")
    else:
        sups = []
        for j in range(n_warm):
            idx, _, _ = ops.topk_attn_decode(qs[:, :, j].contiguous(), k, v, [(0, L0)], K, w.scale,
                                             layout=rt.layout)
            sups.append(idx)
        sup = torch.stack(sups, dim=2).contiguous()
    rt.init(qs, sup)
    torch.cuda.synchronize()
    return qs.cpu().numpy(), sup.cpu().numpy()


def oracle_step(p, before, qt, w, L_t, t, heads):
    """The oracle's step for the listed heads from the pre-step state
    `before`, one head per thread. Returns {(b, h): trace}; a trace's "new"
    holds the head's state after the push."""
    G = w.H_q // w.H_kv

    def one(bh):
        b, h = bh
        return ref.retopk_head_step(p, before.q_hat[b, h], before.support[b, h], int(before.head[b, h]),
                                    int(before.count[b, h]), qt[b, h], w.k[b, h // G], w.v[b, h // G], L_t, t,
                                    w.scale)

    heads = list(heads)
    return dict(zip(heads, pmap(one, heads)))


def run_lockstep(ops, w, p, n_steps, heads, n_warm, check_every=1, mode="host"):
    """mode "host": retopk_step with L_t, t from the host; "device":
    retopk_step_device with [L_t, t] in device memory, advanced by the step;
    "graph": that call captured once in a HIP graph and replayed for every
    step (the query copied into the captured input buffer before each
    replay, the host-side state copies between replays)."""
    L0 = w.retopk["L0"]
    k, v = dev_kv(w)
    rt = ops.Retopk(k, w.H_q, top_k=p.top_k, cache_cap=p.cache_cap, top_r=p.top_r, recent=p.recent, tau=p.tau,
                    refresh=p.refresh, scale=w.scale, budget=p.budget)
    qh, sh = warm_cache(ops, w, rt, k, v, n_warm, p.top_k)
    # the cache after init equals the oracle's init from the same history
    st0 = ref.retopk_state_init(p, qh, sh)
    g0 = host_state(rt)
    assert np.array_equal(g0.support, st0.support)
    assert np.array_equal(g0.head, st0.head) and np.array_equal(g0.count, st0.count)
    assert np.max(np.abs(g0.q_hat - st0.q_hat)) < 1e-6
    stats = dict(reuse=0, exact=0, fallback=0, refresh=0, mixed_steps=0, flagged=0, cand=[], swaps=0, capped=0)
    if mode != "host":
        B, K = w.q.shape[0], p.top_k
        i32 = dict(dtype=torch.int32, device="cuda")
        fixed = dict(support=torch.empty((B, w.H_q, K), **i32),
                     o=torch.empty((B, w.H_q, 128), dtype=torch.float32, device="cuda"),
                     lse=torch.empty((B, w.H_q), dtype=torch.float32, device="cuda"),
                     path=torch.empty((B, w.H_q), **i32), n_cand=torch.empty((B, w.H_q), **i32),
                     cand=torch.empty((B, w.H_q, rt.cand_cap), **i32))
        q_buf = torch.empty((B, w.H_q, 128), dtype=torch.float32, device="cuda")
        step_t = torch.tensor([L0 + 1, 0], dtype=torch.int64, device="cuda")
        graph = None
        if mode == "graph":
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                rt.step_device(q_buf, k, v, step_t, fixed)
            torch.cuda.synchronize()
            assert step_t.cpu().tolist() == [L0 + 1, 0], "capture must not run the step"
    for t in range(n_steps):
        L_t = L0 + t + 1
        qt = np.ascontiguousarray(w.q[:, :, n_warm + t])
        checking = (t % check_every) == 0
        before = host_state(rt) if checking else None
        if mode == "host":
            out = rt.step(torch.from_numpy(qt).cuda(), k, v, L_t, t, want_cand=True)
        else:
            q_buf.copy_(torch.from_numpy(qt).cuda())
            if graph is not None:
                graph.replay()
            else:
                rt.step_device(q_buf, k, v, step_t, fixed)
            out = fixed
            torch.cuda.synchronize()
            assert step_t.cpu().tolist() == [L_t + 1, t + 1], (t, step_t.cpu().tolist())
        torch.cuda.synchronize()
        if not checking:
            continue
        g = {kk: vv.cpu().numpy() for kk, vv in out.items()}
        after = host_state(rt)
        tr = oracle_step(p, before, qt, w, L_t, t, heads)
        paths_checked = set()
        for b, h in heads:
            r = tr[(b, h)]
            rs = r["rho_sorted"]
            near = rs.size > 0 and (abs(float(rs[0]) - p.tau) < NEAR or
                                    (rs.size > p.top_r and abs(float(rs[p.top_r - 1]) - float(rs[p.top_r])) < NEAR))
            vt = r.get("vote")
            if vt is not None and vt["cut"] is not None:
                fc, mc = vt["cut"]
                near = near or bool(np.any((np.abs(vt["f"].astype(np.float64) - fc) < NEAR) & (vt["mask"] != mc)))
                stats["capped"] += 1
            if near:
                stats["flagged"] += 1
                continue
            assert int(g["path"][b, h]) == r["path"], (t, b, h, int(g["path"][b, h]), r["path"])
            paths_checked.add(r["path"])
            if r["path"] == 1:
                stats["fallback"] += 1
            elif r["path"] == 2:
                stats["refresh"] += 1
            if r["path"] == 0:
                stats["reuse"] += 1
                M = r["cand"].shape[0]
                stats["cand"].append(M)
                assert int(g["n_cand"][b, h]) == M
                assert np.array_equal(g["cand"][b, h][:M], r["cand"]), (t, b, h)
                assert np.all(g["cand"][b, h][M:] == -1)
            else:
                stats["exact"] += 1
                assert int(g["n_cand"][b, h]) == L_t
            stats["swaps"] += check_index_set(g["support"][b, h], r["rows"], r["z"], r["zk"], p.top_k)
            check_out(g["o"][b, h], g["lse"][b, h], r["o"], r["lse"], w.kv_dtype == "f32", f"t={t} ({b},{h})")
            # the pushed entry: unit query and the GPU's own support
            C = p.cache_cap
            slot = (int(before.head[b, h]) + 1) % C
            assert int(after.head[b, h]) == slot
            assert int(after.count[b, h]) == min(int(before.count[b, h]) + 1, C)
            assert np.max(np.abs(after.q_hat[b, h, slot] - r["new"][0][slot])) < 1e-6
            assert np.array_equal(after.support[b, h, slot], g["support"][b, h])
        if 0 in paths_checked and 1 in paths_checked:
            stats["mixed_steps"] += 1
    return stats


def test_retopk_lockstep_small(ops):
    """c3 head layout (28 q / 4 KV, G = 7) at reduced length and parameters,
    with a refresh every 8 steps and a threshold that gives both paths."""
    w = make_workload(3, L=4096, steps=40, warm=8)
    p = ref.RetopkParams(top_k=64, cache_cap=8, top_r=2, recent=16, tau=0.85, refresh=8)
    heads = [(0, h) for h in range(28)]
    s = run_lockstep(ops, w, p, 40, heads, n_warm=8)
    log(f"retopk small: reuse {s['reuse']} exact {s['exact']} flagged {s['flagged']} "
        f"mean M {np.mean(s['cand']) if s['cand'] else 0:.0f} band swaps {s['swaps']}")
    assert s["reuse"] > 0 and s["exact"] > 0


@pytest.mark.parametrize("mode", ["device", "graph"])
def test_retopk_device_step_lockstep(ops, mode):
    """retopk_step_device (L_t and t in device memory, advanced by the step)
    on the small c3-shaped case, called directly and replayed from one
    captured HIP graph: every step of every head against the oracle, with
    refreshes, fallbacks and reuse."""
    w = make_workload(3, L=4096, steps=40, warm=8)
    p = ref.RetopkParams(top_k=64, cache_cap=8, top_r=2, recent=16, tau=0.9, refresh=8)
    heads = [(0, h) for h in range(28)]
    s = run_lockstep(ops, w, p, 40, heads, n_warm=8, mode=mode)
    log(f"retopk {mode} step: reuse {s['reuse']} fallback {s['fallback']} refresh {s['refresh']} "
        f"flagged {s['flagged']}")
    assert s["reuse"] > 0 and s["refresh"] > 0


@pytest.mark.slow
def test_retopk_c3_graph_replay_lockstep(ops):
    """c3 at full size (L0 = 65536, K=512, C=32, R=4, W=32, tau=0.85,
    T_r=128): the step captured once in a HIP graph and replayed for all 256
    steps, every head compared with the oracle at every step."""
    w = make_workload(3)
    P = w.retopk
    p = ref.RetopkParams(top_k=P["top_k"], cache_cap=P["cache_cap"], top_r=P["top_r"], recent=P["recent"],
                         tau=P["tau"], refresh=P["refresh"])
    heads = [(0, h) for h in range(w.H_q)]
    s = run_lockstep(ops, w, p, P["steps"], heads, n_warm=P["warmup"], mode="graph")
    log(f"retopk c3 graph replay: {len(heads)} heads x {P['steps']} steps: reuse {s['reuse']} "
        f"refresh {s['refresh']} flagged {s['flagged']}")
    assert s["reuse"] + s["exact"] + s["flagged"] == len(heads) * P["steps"]
    assert s["refresh"] == 2 * len(heads)


def test_retopk_tiny_cache_all_paths(ops):
    """L_t <= K on the exact path and M <= K on the reuse path (tiny caches)."""
    w = make_workload(3, L=100, steps=12, warm=3)
    p = ref.RetopkParams(top_k=128, cache_cap=4, top_r=2, recent=8, tau=0.5, refresh=5)
    s = run_lockstep(ops, w, p, 12, [(0, h) for h in range(28)], n_warm=3)
    log(f"retopk tiny: reuse {s['reuse']} exact {s['exact']} flagged {s['flagged']}")


def test_retopk_always_exact_equals_topk(ops):
    """tau > 1: every step takes the exact path: the same rows as
    topk_attn_decode, and o and lse equal up to the order in which the fp32
    softmax . V sums are formed (topk_attn_decode may fuse them into its
    select launch; the ReTopK exact step keeps them separate)."""
    w = make_workload(3, L=2048, steps=6, warm=4)
    k, v = dev_kv(w)
    rt = ops.Retopk(k, 28, top_k=32, cache_cap=4, top_r=2, recent=8, tau=1.5, refresh=0, scale=w.scale)
    warm_cache(ops, w, rt, k, v, 4, 32)
    for t in range(6):
        L_t = 2048 + t + 1
        qt = torch.from_numpy(np.ascontiguousarray(w.q[:, :, 4 + t])).cuda()
        out = rt.step(qt, k, v, L_t, t)
        idx, o, lse = ops.topk_attn_decode(qt, k, v, [(0, L_t)], 32, w.scale)
        torch.cuda.synchronize()
        assert np.all(out["path"].cpu().numpy() == 1)
        assert torch.equal(out["support"], idx)
        assert torch.max(torch.abs(out["o"] - o)).item() < 1e-5
        assert torch.max(torch.abs(out["lse"] - lse)).item() < 1e-5


@pytest.mark.parametrize("B,tau,K,L", [(3, 0.90, 128, 8192), (1, 0.85, 1024, 16384), (5, 0.85, 1100, 8192)])
def test_retopk_serving_variants(ops, B, tau, K, L):
    """Serving-shaped steps: several requests in one call, each with its own
    caches, at the pages' stricter threshold (tau = 0.90), and the K = 1024
    budget of the cross-model runs; c3's head layout, C=32, R=4, W=32. The
    last case (140 heads, K = 1100) takes the row-split softmax . V, whose
    split-0 workgroups push the cache."""
    w = make_workload(3, L=L, steps=24, warm=32, B=B)
    p = ref.RetopkParams(top_k=K, cache_cap=32, top_r=4, recent=32, tau=tau, refresh=16)
    heads = [(b, h) for b in range(B) for h in (0, 6, 13, 20, 27)]
    s = run_lockstep(ops, w, p, 24, heads, n_warm=32)
    log(f"retopk B={B} tau={tau} K={K}: reuse {s['reuse']} exact {s['exact']} flagged {s['flagged']} "
        f"mean M {np.mean(s['cand']) if s['cand'] else 0:.0f} band swaps {s['swaps']}")
    assert s["reuse"] + s["exact"] > 0


@pytest.mark.parametrize("K", [3072, 4096])
def test_retopk_rerank_path_lockstep(ops, K):
    """Candidate sets too large for one workgroup's LDS (R*K + W = 12,320 and
    16,416 slots): the reuse heads take retopk_select, retopk_rerank and the
    rerank select (staged in LDS for the first size, from global memory for
    the second), then the row-split softmax . V that pushes the cache; every
    head against the oracle, refreshes included."""
    log(f"case retopk rerank path K={K} L=32768")
    w = make_workload(3, L=32768, steps=12, warm=8)
    p = ref.RetopkParams(top_k=K, cache_cap=8, top_r=4, recent=32, tau=0.85, refresh=4)
    heads = [(0, h) for h in range(28)]
    s = run_lockstep(ops, w, p, 12, heads, n_warm=8)
    log(f"retopk rerank path K={K}: reuse {s['reuse']} exact {s['exact']} flagged {s['flagged']} "
        f"mean M {np.mean(s['cand']) if s['cand'] else 0:.0f} band swaps {s['swaps']}")
    assert s["reuse"] > 0 and s["exact"] > 0


@pytest.mark.slow
def test_retopk_c3_full_lockstep(ops):
    """c3 at full size (L0 = 65536, K=512, C=32, R=4, W=32, tau=0.85,
    T_r=128), all 256 steps, every one of the 28 heads compared every step."""
    w = make_workload(3)
    P = w.retopk
    p = ref.RetopkParams(top_k=P["top_k"], cache_cap=P["cache_cap"], top_r=P["top_r"], recent=P["recent"],
                         tau=P["tau"], refresh=P["refresh"])
    heads = [(0, h) for h in range(w.H_q)]
    s = run_lockstep(ops, w, p, P["steps"], heads, n_warm=P["warmup"])
    log(f"retopk c3 full: {len(heads)} heads x {P['steps']} steps: reuse {s['reuse']} fallback {s['fallback']} "
        f"refresh {s['refresh']} flagged {s['flagged']} mean M {np.mean(s['cand']) if s['cand'] else 0:.0f} "
        f"(parity unpinned: context only) band swaps {s['swaps']}")
    assert s["reuse"] + s["exact"] + s["flagged"] == len(heads) * P["steps"]


def test_retopk_fallback_mixed_with_reuse(ops):
    """Similarity fallback (ReTopK review, 核心方法 5) on some heads while the
    others reuse the cache in the same step: no periodic refresh, and tau at
    the lag-1 cosine of the AR(1) queries (about 0.95), so about half of the
    heads fall back at each step. The exact kernels then run on the fallback
    heads only (per-head masks), the rerank on the others; every head is
    compared with the oracle."""
    w = make_workload(3, L=4096, steps=40, warm=8)
    p = ref.RetopkParams(top_k=64, cache_cap=8, top_r=2, recent=16, tau=0.95, refresh=0)
    heads = [(0, h) for h in range(28)]
    s = run_lockstep(ops, w, p, 40, heads, n_warm=8)
    log(f"retopk fallback mix: reuse {s['reuse']} fallback {s['fallback']} refresh {s['refresh']} "
        f"steps with both paths checked {s['mixed_steps']} flagged {s['flagged']}")
    assert s["refresh"] == 0
    assert s["fallback"] > 0 and s["reuse"] > 0
    assert s["mixed_steps"] >= 10


def test_retopk_empty_cache_start(ops):
    """retopk_state_init with no history: the first step falls back on every
    head (count = 0), the cache then fills one entry per step; reuse and
    fallback both occur afterwards (no refresh)."""
    w = make_workload(3, L=4096, steps=24, warm=0)
    p = ref.RetopkParams(top_k=64, cache_cap=8, top_r=2, recent=16, tau=0.9, refresh=0)
    heads = [(0, h) for h in range(28)]
    s = run_lockstep(ops, w, p, 24, heads, n_warm=0)
    log(f"retopk empty start: reuse {s['reuse']} fallback {s['fallback']} flagged {s['flagged']}")
    assert s["fallback"] >= 28 and s["reuse"] > 0


def test_retopk_checkpoint_resume_bit_exact(ops):
    """128 steps, the state (q_hat, support, head, count) copied to the host
    and restored into a fresh state and workspace, 128 more steps: every
    output of the resumed run equals the uninterrupted run's bit for bit."""
    w = make_workload(3, L=16384, steps=256, warm=32)
    P = w.retopk
    kw = dict(top_k=256, cache_cap=32, top_r=4, recent=32, tau=0.85, refresh=64, scale=w.scale)
    k, v = dev_kv(w)
    L0 = P["L0"]
    qs = torch.from_numpy(np.ascontiguousarray(w.q)).cuda()

    def run(rt, t0, t1):
        outs = []
        for t in range(t0, t1):
            o = rt.step(qs[:, :, 32 + t].contiguous(), k, v, L0 + t + 1, t, want_cand=True)
            outs.append({kk: vv.clone() for kk, vv in o.items()})
        return outs

    rt = ops.Retopk(k, w.H_q, **kw)
    warm_cache(ops, w, rt, k, v, 32, kw["top_k"])
    whole = run(rt, 0, 256)
    torch.cuda.synchronize()

    rt1 = ops.Retopk(k, w.H_q, **kw)
    warm_cache(ops, w, rt1, k, v, 32, kw["top_k"])
    run(rt1, 0, 128)
    torch.cuda.synchronize()
    saved = {name: getattr(rt1, name).cpu().numpy().copy() for name in ("q_hat", "support", "head", "count")}
    del rt1
    rt2 = ops.Retopk(k, w.H_q, **kw)
    for name, arr in saved.items():
        getattr(rt2, name).copy_(torch.from_numpy(arr))
    resumed = run(rt2, 128, 256)
    torch.cuda.synchronize()
    paths = set()
    for i, o in enumerate(resumed):
        ref_o = whole[128 + i]
        for name in ("support", "o", "lse", "path", "n_cand", "cand"):
            assert torch.equal(o[name], ref_o[name]), (128 + i, name)
        paths |= set(np.unique(o["path"].cpu().numpy()).tolist())
    for name in ("q_hat", "support", "head", "count"):
        assert torch.equal(getattr(rt2, name), getattr(rt, name)), name
    log(f"retopk resume: 128 resumed steps bit-exact, paths seen {sorted(paths)}")
    assert 0 in paths and 2 in paths


def test_retopk_nan_query_propagates(ops):
    """A NaN in one head's query: the call succeeds, that head's o and lse are
    not finite, and every other head's outputs and state equal those of the
    same step without the NaN, bit for bit (heads never mix)."""
    w = make_workload(3, L=4096, steps=4, warm=8)
    p = dict(top_k=64, cache_cap=8, top_r=2, recent=16, tau=0.85, refresh=0, scale=w.scale)
    k, v = dev_kv(w)
    outs, states = [], []
    for poison in (False, True):
        rt = ops.Retopk(k, w.H_q, **p)
        warm_cache(ops, w, rt, k, v, 8, 64)
        res = []
        for t in range(3):
            q = np.ascontiguousarray(w.q[:, :, 8 + t]).copy()
            if poison:
                q[0, 5, 17] = np.nan
            res.append(rt.step(torch.from_numpy(q).cuda(), k, v, 4096 + t + 1, t + 1))
        torch.cuda.synchronize()
        outs.append([{kk: vv.cpu().numpy() for kk, vv in r.items()} for r in res])
        states.append({n: getattr(rt, n).cpu().numpy() for n in ("q_hat", "support", "head", "count")})
    others = [h for h in range(w.H_q) if h != 5]
    for clean, bad in zip(*outs):
        assert not np.all(np.isfinite(bad["o"][0, 5])) and not np.isfinite(bad["lse"][0, 5])
        for name in ("support", "o", "lse", "path", "n_cand"):
            assert np.array_equal(clean[name][0, others], bad[name][0, others]), name
    for name in ("q_hat", "support", "head", "count"):
        assert np.array_equal(states[0][name][0, others], states[1][name][0, others]), name


@pytest.mark.parametrize("budget", [100, 40])
def test_retopk_vote_lockstep(ops, budget):
    """Confidence-voted candidates (R = 4): the union outside the recent
    window is capped at the budget by vote confidence; 40 leaves fewer
    candidates than K = 64 (padded supports)."""
    w = make_workload(3, L=4096, steps=30, warm=8)
    p = ref.RetopkParams(top_k=64, cache_cap=8, top_r=4, recent=16, tau=0.85, refresh=10, budget=budget)
    heads = [(0, h) for h in range(28)]
    s = run_lockstep(ops, w, p, 30, heads, n_warm=8)
    log(f"retopk vote budget {budget}: reuse {s['reuse']} exact {s['exact']} capped {s['capped']} "
        f"flagged {s['flagged']} mean M {np.mean(s['cand']) if s['cand'] else 0:.0f}")
    assert s["reuse"] > 0 and s["capped"] > 0


def test_retopk_vote_full_size_sampled(ops):
    """The c3 layout at full size (65,536 rows, K = 512, R = 4, W = 32) with a
    budget of 600 voted rows, 6 steps checked on 8 heads."""
    w = make_workload(3, steps=6, warm=32)
    p = ref.RetopkParams(top_k=512, cache_cap=32, top_r=4, recent=32, tau=0.85, refresh=128, budget=600)
    heads = [(0, h) for h in (0, 3, 7, 11, 15, 19, 23, 27)]
    s = run_lockstep(ops, w, p, 6, heads, n_warm=32)
    log(f"retopk vote full size: reuse {s['reuse']} capped {s['capped']} flagged {s['flagged']} "
        f"mean M {np.mean(s['cand']) if s['cand'] else 0:.0f}")
    assert s["reuse"] > 0
