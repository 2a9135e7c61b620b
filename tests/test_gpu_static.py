"""GPU parity of topk_attn_decode_static (static window W plus top-K over the
dynamic rows, one pass) against the CPU oracle's merge of the two parts."""

import numpy as np
import pytest
import torch

from gpu_util import check_index_set, check_out, dev_kv, log, oracle_head
from oracle import reference as ref
from workloads import make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops(stdk):
    from sparse_top_decode_amd import ops
    return ops


def oracle_step(w, b, h, ranges, static_ranges, K, q=None):
    """The pages' decode step on one head: merge(dense(W), topk(Omega))."""
    r, rows = oracle_head(w, b, h, ranges, K, q=q) if ranges else (None, None)
    n_st = sum(e - s for s, e in static_ranges)
    rs, _ = oracle_head(w, b, h, static_ranges, max(n_st, 1), q=q)
    if r is None:
        return None, None, rs["o"], rs["lse"]
    om, lm = ref.attn_merge_lse(rs["o"], np.float64(rs["lse"]), r["o"], np.float64(r["lse"]))
    return r, rows, om, float(lm)


def run_static(ops, w, ranges, static_ranges, K, q=None):
    qa = w.q if q is None else q
    qt = torch.from_numpy(np.ascontiguousarray(qa)).cuda()
    k, v = dev_kv(w)
    idx, o, lse = ops.topk_attn_decode_static(qt, k, v, ranges, static_ranges, K, w.scale)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), o.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("L,K", [(16384, 2048), (8192, 300), (3000, 1)])
def test_c2_decode_step_reduced(ops, L, K):
    """Llama-3-8B layout (bf16, G = 4): W = first 128 + last 512 rows, top-K
    over the rest; every head against the oracle's merge."""
    log(f"case static c2 L={L} K={K}")
    w = make_workload(2, L=L)
    idx, o, lse = run_static(ops, w, w.ranges, w.static_ranges, K)
    worst = 0.0
    for h in range(w.H_q):
        r, rows, om, lm = oracle_step(w, 0, h, w.ranges, w.static_ranges, K)
        check_index_set(idx[0, h], rows, r["z"], r["zk"], K)
        eo, _ = check_out(o[0, h], lse[0, h], om, lm, False, f"static c2 head {h}")
        worst = max(worst, eo)
    log(f"[static c2 L={L} K={K}] {w.H_q} heads ok, worst o err {worst:.2e}")


def test_matches_three_calls(ops):
    """The one-pass result equals topk_attn_decode(W, dense) +
    topk_attn_decode(Omega) + attn_merge_lse on the GPU (same chosen rows)."""
    log("case static vs three calls c2 L=20000")
    w = make_workload(2, L=20000)
    K = 1500
    q = torch.from_numpy(w.q).cuda()
    k, v = dev_kv(w)
    idx_f, o_f, l_f = ops.topk_attn_decode_static(q, k, v, w.ranges, w.static_ranges, K, w.scale)
    idx_d, o_d, l_d = ops.topk_attn_decode(q, k, v, w.ranges, K, w.scale)
    _, o_s, l_s = ops.topk_attn_decode(q, k, v, w.static_ranges, K, w.scale)
    o_m, l_m = ops.attn_merge_lse(o_s, l_s, o_d, l_d)
    torch.cuda.synchronize()
    assert torch.equal(idx_f, idx_d)
    assert torch.max(torch.abs(o_f - o_m)).item() < 1e-5
    assert torch.max(torch.abs(l_f - l_m)).item() < 1e-5


def test_no_static_rows_is_topk(ops):
    """Without static rows the call is topk_attn_decode, bit for bit."""
    w = make_workload(2, L=8192)
    q = torch.from_numpy(w.q).cuda()
    k, v = dev_kv(w)
    a = ops.topk_attn_decode_static(q, k, v, w.ranges, [], 700, w.scale)
    b = ops.topk_attn_decode(q, k, v, w.ranges, 700, w.scale)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("K", [7552, 9000])
def test_all_dynamic_rows_chosen(ops, K):
    """top_k >= |Omega|: dense attention over W and all of Omega; idx_out lists
    the dynamic rows then -1."""
    L = 8192
    w = make_workload(2, L=L)
    n_dyn = sum(e - b for b, e in w.ranges)
    idx, o, lse = run_static(ops, w, w.ranges, w.static_ranges, K)
    rows = ref.range_rows(w.ranges)
    m = min(K, n_dyn)
    assert np.all(idx[:, :, :m] == rows[None, None, :m]) and np.all(idx[:, :, m:] == -1)
    for h in (0, 13, 31):
        _, _, om, lm = oracle_step(w, 0, h, w.ranges, w.static_ranges, K)
        check_out(o[0, h], lse[0, h], om, lm, False, f"dense union head {h}")


def test_only_static_rows(ops):
    w = make_workload(2, L=4096)
    idx, o, lse = run_static(ops, w, [], w.static_ranges, 64)
    assert np.all(idx == -1)
    for h in (0, 31):
        _, _, om, lm = oracle_step(w, 0, h, [], w.static_ranges, 64)
        check_out(o[0, h], lse[0, h], om, lm, False, f"static only head {h}")


def test_fp32_single_head(ops):
    """fp32 cache, 1 q / 1 KV head (the c1 shapes) with a static window."""
    w = make_workload(1)
    ranges = [(64, 3900)]
    static = [(0, 64), (3900, 4096)]
    idx, o, lse = run_static(ops, w, ranges, static, w.top_k)
    r, rows, om, lm = oracle_step(w, 0, 0, ranges, static, w.top_k)
    check_index_set(idx[0, 0], rows, r["z"], r["zk"], w.top_k)
    check_out(o[0, 0], lse[0, 0], om, lm, True, "fp32 static")


def test_batch_and_ragged_static(ops):
    """c4 layout (B = 16, 512 heads: softmax . V fused into the select
    launch), static ranges on both sides of several dynamic ranges; every
    (b, h) against the oracle."""
    log("case ragged static c4 layout B=16 L=4096 K=256")
    w = make_workload(4, L=4096)
    ranges = [(100, 1000), (1200, 3000), (3100, 4000)]
    static = [(0, 100), (1000, 1200), (4000, 4096)]
    idx, o, lse = run_static(ops, w, ranges, static, 256)
    for b in range(w.q.shape[0]):
        for h in range(w.H_q):
            r, rows, om, lm = oracle_step(w, b, h, ranges, static, 256)
            check_index_set(idx[b, h], rows, r["z"], r["zk"], 256)
            check_out(o[b, h], lse[b, h], om, lm, False, f"ragged static ({b},{h})")
    log(f"[ragged static] {w.q.shape[0] * w.H_q} heads ok")


def test_batch_static_half_workgroups(ops):
    """c4 layout over 12,288 rows with a 640-row static window: 512 heads of
    11,648 dynamic positions, each filtered, selected and attended (its
    static slots included) in a half-size workgroup, two per CU; every
    (b, h) against the oracle."""
    if 2 * torch.cuda.get_device_properties(0).multi_processor_count > 512:
        pytest.skip("half-size workgroups need at least twice as many heads as CUs")
    log("case static c4 layout B=16 L=12288 K=1024, half-size workgroups")
    w = make_workload(4, L=12288)
    ranges = [(128, 11776)]
    static = [(0, 128), (11776, 12288)]
    timer = ops.KernelTimer()
    try:
        idx, o, lse = run_static(ops, w, ranges, static, 1024)
        assert timer.read("topk_filter_lds_sv")[1] == 1
    finally:
        timer.close()
    for b in range(w.q.shape[0]):
        for h in range(w.H_q):
            r, rows, om, lm = oracle_step(w, b, h, ranges, static, 1024)
            check_index_set(idx[b, h], rows, r["z"], r["zk"], 1024)
            check_out(o[b, h], lse[b, h], om, lm, False, f"half static ({b},{h})")
    log(f"[half static] {w.q.shape[0] * w.H_q} heads ok")


def test_graph_replays_match_eager(ops):
    """The one-pass step captured in a HIP graph: several replays, with eager
    calls and synchronisations between them, each equal to the eager result
    (the workspace counters must be back at zero after every replay)."""
    log("case graph replay c2 L=16384")
    w = make_workload(2, L=16384)
    K = 2048
    q = torch.from_numpy(w.q).cuda()
    k, v = dev_kv(w)
    lay = ops.make_layout(k, w.H_q)
    n = sum(e - b for b, e in w.ranges)
    n_st = sum(e - b for b, e in w.static_ranges)
    ws = ops.new_workspace(ops.topk_attn_decode_static_workspace_size(lay, n, n_st, K), q.device)
    idx = torch.empty((1, w.H_q, K), dtype=torch.int32, device=q.device)
    o = torch.empty((1, w.H_q, 128), dtype=torch.float32, device=q.device)
    lse = torch.empty((1, w.H_q), dtype=torch.float32, device=q.device)

    def step():
        ops.topk_attn_decode_static(q, k, v, w.ranges, w.static_ranges, K, w.scale, idx_out=idx, o_out=o,
                                    lse_out=lse, workspace=ws, layout=lay)

    step()
    torch.cuda.synchronize()
    want = [t.clone() for t in (idx, o, lse)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    counters = w.B * w.H_q * ops.COUNTER_BYTES_PER_HEAD
    for rep in range(4):
        for t in (idx, o, lse):
            t.fill_(-7)
        graph.replay()
        torch.cuda.synchronize()
        for t, ref_t in zip((idx, o, lse), want):
            assert torch.equal(t, ref_t), f"replay {rep} differs from the eager result"
        assert int(torch.count_nonzero(ws[:counters]).item()) == 0
        step()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(o, want[1])
