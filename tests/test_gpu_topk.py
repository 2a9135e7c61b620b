"""GPU parity of topk_attn_decode and attn_merge_lse against the CPU oracle."""

import math

import numpy as np
import pytest
import torch

from gpu_util import check_heads, check_index_set, check_out, dev_kv, log, oracle_head
from oracle import reference as ref
from workloads import make_workload, static_window_ranges

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops(stdk):
    from sparse_top_decode_amd import ops
    return ops


def run(ops, w, ranges, K, q=None, **kw):
    qa = w.q if q is None else q
    q = torch.from_numpy(np.ascontiguousarray(qa if qa.ndim == 3 else qa[:, :, 0])).cuda()
    k, v = dev_kv(w)
    idx, o, lse = ops.topk_attn_decode(q, k, v, ranges, K, w.scale, **kw)
    torch.cuda.synchronize()
    return (None if idx is None else idx.cpu().numpy()), o.cpu().numpy(), lse.cpu().numpy()


def test_c1_exact_fp32(ops):
    """1 q / 1 KV head, fp32 cache, L=4096, K=64: index set exact, o/lse 1e-4."""
    log("case c1 fp32 L=4096 K=64")
    w = make_workload(1)
    idx, o, lse = run(ops, w, w.ranges, w.top_k)
    want = ref.topk_attn_decode(w.q, w.k, w.v, w.ranges, w.top_k, w.scale)
    check_heads(w, [(0, 0)], idx, o, lse, w.ranges, w.top_k, fp32=True, label="c1")
    assert np.array_equal(idx, want["idx"])


@pytest.mark.parametrize("K", [64, 5000])
def test_long_head_filter_batches(ops, K):
    """One head over 1.2M rows (fp32): more positions than 64 filter
    workgroups take in one pass, so each takes several batches; the index
    set equals the oracle's, o/lse to the fp32 bar."""
    log(f"case c1 fp32 L=1200000 K={K} (several filter batches per workgroup)")
    w = make_workload(1, L=1_200_000)
    idx, o, lse = run(ops, w, w.ranges, K)
    want = ref.topk_attn_decode(w.q, w.k, w.v, w.ranges, K, w.scale)
    check_heads(w, [(0, 0)], idx, o, lse, w.ranges, K, fp32=True, label=f"c1 L=1.2M K={K}")
    assert np.array_equal(idx, want["idx"])


def test_c2_shape_two_filter_batches(ops):
    """The c2 head layout over 200,000 rows: each filter workgroup takes two
    batches of wave slices; every head against the oracle."""
    log("case c2 layout L=200000 K=3000 (two filter batches per workgroup)")
    w = make_workload(2, L=200_000)
    idx, o, lse = run(ops, w, w.ranges, 3000)
    heads = [(0, h) for h in range(w.H_q)]
    check_heads(w, heads, idx, o, lse, w.ranges, 3000, label="c2 L=200000 K=3000")


@pytest.mark.parametrize("L,K", [(8192, 2048), (8192, 97), (20000, 1), (3000, 2047)])
def test_c2_shape_reduced(ops, L, K):
    """Llama-3-8B head layout (32 q / 8 KV, bf16) at reduced length: the
    dynamic-set top-K call on every head, several tiles and a ragged tail."""
    log(f"case c2 reduced L={L} K={K}")
    w = make_workload(2, L=L)
    idx, o, lse = run(ops, w, w.ranges, K)
    heads = [(0, h) for h in range(w.H_q)]
    check_heads(w, heads, idx, o, lse, w.ranges, K, label=f"c2 L={L} K={K}")


def test_c2_static_dense_and_merge(ops):
    """The pages' decode step at reduced length: dense attention over the static
    rows (first 128 + last 512), top-K over the rest, LSE merge; equals the
    oracle's attention over the union of both row sets."""
    log("case c2 static+dynamic+merge L=16384")
    w = make_workload(2, L=16384)
    K = 2048
    q = torch.from_numpy(w.q).cuda()
    k, v = dev_kv(w)
    idx_d, o_d, l_d = ops.topk_attn_decode(q, k, v, w.ranges, K, w.scale)
    idx_s, o_s, l_s = ops.topk_attn_decode(q, k, v, w.static_ranges, K, w.scale)
    o_m, l_m = ops.attn_merge_lse(o_s, l_s, o_d, l_d)
    torch.cuda.synchronize()
    idx_s = idx_s.cpu().numpy()
    srows = ref.range_rows(w.static_ranges)
    assert np.all(idx_s[:, :, :srows.shape[0]] == srows[None, None, :])
    assert np.all(idx_s[:, :, srows.shape[0]:] == -1)
    idx_d = idx_d.cpu().numpy()
    for h in range(w.H_q):
        r, rows = oracle_head(w, 0, h, w.ranges, K)
        check_index_set(idx_d[0, h], rows, r["z"], r["zk"], K)
        rs, _ = oracle_head(w, 0, h, w.static_ranges, K)
        om, lm = ref.attn_merge_lse(rs["o"], np.float64(rs["lse"]), r["o"], np.float64(r["lse"]))
        check_out(o_s.cpu().numpy()[0, h], l_s.cpu().numpy()[0, h], rs["o"], rs["lse"], False, "static")
        check_out(o_m.cpu().numpy()[0, h], l_m.cpu().numpy()[0, h], om, float(lm), False, "merged")
        # the merged result is attention over W u S computed directly
        union = np.union1d(srows, idx_d[0, h][idx_d[0, h] >= 0])
        direct = ref.attend_rows(w.q[0, h], w.k[0, h // 4], w.v[0, h // 4], union, union.shape[0], w.scale)
        check_out(o_m.cpu().numpy()[0, h], l_m.cpu().numpy()[0, h], direct["o"], direct["lse"], False, "union")


def test_ragged_ranges_and_edges(ops):
    """Several odd-sized ranges, K at 1, n-1, n and above n, fp32 and bf16."""
    for cfg in (1, 2):
        w = make_workload(cfg, L=4096) if cfg == 2 else make_workload(1)
        ranges = [(3, 1000), (1500, 1501), (2000, 2777), (4000, 4096)]
        n = sum(e - b for b, e in ranges)
        for K in (1, 5, n - 1, n, n + 7):
            log(f"case ragged cfg={cfg} K={K} n={n}")
            idx, o, lse = run(ops, w, ranges, K)
            heads = [(0, h) for h in range(w.H_q)][:8]
            check_heads(w, heads, idx, o, lse, ranges, K, fp32=(cfg == 1), label=f"ragged c{cfg} K={K}")


def test_empty_range(ops):
    w = make_workload(2, L=1024)
    idx, o, lse = run(ops, w, [], 16)
    assert np.all(idx == -1) and np.all(o == 0) and np.all(np.isneginf(lse))


def test_exact_ties_lowest_row_wins(ops):
    """Duplicated key rows give bit-equal scores; the lowest rows must win."""
    rng = np.random.default_rng(5)
    L, K = 3000, 40
    w = make_workload(2, L=L)
    k = w.k.copy()
    # 30 copies of one strong row and 30 of another, scattered
    src = rng.choice(L, 2, replace=False)
    for g in range(w.H_kv):
        for j, s in enumerate(src):
            dst = rng.choice(L, 30, replace=False)
            k[0, g, dst] = k[0, g, s]
    w.k = k
    idx, o, lse = run(ops, w, [(0, L)], K)
    want = ref.topk_attn_decode(w.q, w.k, w.v, [(0, L)], K, w.scale)
    n_exact = 0
    for h in range(w.H_q):
        r, rows = oracle_head(w, 0, h, [(0, L)], K)
        check_index_set(idx[0, h], rows, r["z"], r["zk"], K)
        # where the K-th score is an exact tie among duplicates, the choice
        # among the tied rows must be the lowest ones
        tied = rows[r["z"] == r["zk"]]
        if tied.shape[0] > 1:
            n_exact += 1
            got = set(int(x) for x in idx[0, h] if x >= 0) & set(int(x) for x in tied)
            exp = set(int(x) for x in want["idx"][0, h] if x >= 0) & set(int(x) for x in tied)
            assert got == exp, (h, sorted(got), sorted(exp))
    log(f"tie heads checked exactly: {n_exact}")


@pytest.mark.parametrize("L", [8192, 8193])
def test_short_segment_boundary(ops, L):
    """Segments of up to 8192 positions are selected by one workgroup per
    head (all scores in LDS), longer ones by the filter-select: both sides of
    the boundary, every head checked."""
    w = make_workload(2, L=L)
    K = 100
    log(f"case short-segment boundary L={L}")
    idx, o, lse = run(ops, w, [(0, L)], K)
    heads = [(0, h) for h in range(w.H_q)]
    check_heads(w, heads, idx, o, lse, [(0, L)], K, label=f"boundary L={L}")


def test_short_segment_codebook_ties(ops):
    """A short segment whose scores take 6 values: the K-th score's bin holds
    about a thousand scores, too many for the one-pass histogram cut, so the
    radix cut decides; the set must equal the oracle's (lowest rows first)."""
    from workloads import make_multi_query
    w = make_multi_query(1, 4, 2, 1, 6000, "bf16", codebook=6, tag=44)
    w.q = np.ascontiguousarray(w.q[:, :, 0])
    ranges = [(0, 2500), (3000, 6000)]
    for K in (1, 300, 5499):
        log(f"case short codebook ties K={K}")
        idx, o, lse = run(ops, w, ranges, K)
        want = ref.topk_attn_decode(w.q, w.k, w.v, ranges, K, w.scale)
        assert np.array_equal(idx, want["idx"])
        for h in range(w.H_q):
            check_out(o[0, h], lse[0, h], want["o"][0, h], want["lse"][0, h], False, f"short codebook K={K} head {h}")


@pytest.mark.parametrize("K", [300, 5000])
def test_one_workgroup_per_head_ties_and_nan(ops, K):
    """256 heads of 9,000 positions: one filter workgroup per head, which
    selects in its own LDS (one-pass cut, radix passes when the K-th score's
    bin is crowded or a score is NaN). Keys from a 6-row codebook, so every
    score ties with about 1,500 others: the index sets must equal the
    oracle's exactly (lowest rows first). A NaN in one head's query makes
    that head's o and lse NaN and leaves every other head bit-identical."""
    from workloads import make_multi_query
    w = make_multi_query(8, 32, 4, 1, 9000, "bf16", codebook=6, tag=45)
    w.q = np.ascontiguousarray(w.q[:, :, 0])
    ranges = [(0, 9000)]
    log(f"case one workgroup per head, codebook ties K={K}")
    idx, o, lse = run(ops, w, ranges, K)
    want = ref.topk_attn_decode(w.q, w.k, w.v, ranges, K, w.scale)
    assert np.array_equal(idx, want["idx"])
    for b in range(w.B):
        for h in range(w.H_q):
            check_out(o[b, h], lse[b, h], want["o"][b, h], want["lse"][b, h], False, f"ties K={K} ({b},{h})")
    qn = w.q.copy()
    qn[3, 5, 17] = np.nan
    qt = torch.from_numpy(qn).cuda()
    k, v = dev_kv(w)
    idx2, o2, lse2 = ops.topk_attn_decode(qt, k, v, ranges, K, w.scale)
    torch.cuda.synchronize()
    idx2, o2, lse2 = idx2.cpu().numpy(), o2.cpu().numpy(), lse2.cpu().numpy()
    assert np.all(np.isnan(o2[3, 5])) and np.isnan(lse2[3, 5])
    sel = idx2[3, 5][idx2[3, 5] >= 0]
    assert sel.shape[0] == K and np.all(np.diff(sel) > 0)
    keep = np.ones((w.B, w.H_q), bool)
    keep[3, 5] = False
    for x, y in ((idx, idx2), (o, o2), (lse, lse2)):
        assert np.array_equal(x[keep], y[keep])


@pytest.mark.parametrize("K", [64, 3000])
def test_half_workgroups_ties_nan_overflow(ops, K):
    """512 heads of 9,000 positions, twice as many heads as CUs: each head
    is filtered, selected and attended in a half-size workgroup (two per
    CU) with its candidates in LDS. Keys from a 6-row codebook (every score
    ties with about 1,500 others): the index sets must equal the oracle's
    exactly. A NaN in one query makes all 9,000 positions its head's
    candidates, more than that LDS holds: the head is flagged and taken by
    the full-size kernel, its o and lse are NaN, and every other head is
    bit-identical to the run without the NaN."""
    from workloads import make_multi_query
    if 2 * torch.cuda.get_device_properties(0).multi_processor_count > 512:
        pytest.skip("half-size workgroups need at least twice as many heads as CUs")
    w = make_multi_query(16, 32, 4, 1, 9000, "bf16", codebook=6, tag=46)
    w.q = np.ascontiguousarray(w.q[:, :, 0])
    ranges = [(0, 9000)]
    log(f"case half-size workgroups, codebook ties K={K}")
    qn = w.q.copy()
    qn[11, 7, 40] = np.nan
    timer = ops.KernelTimer()
    try:
        idx, o, lse = run(ops, w, ranges, K)
        idx2, o2, lse2 = run(ops, w, ranges, K, q=qn)
        assert timer.read("topk_filter_lds_sv")[1] == 2
        assert timer.read("topk_filter_select_sv")[1] == 2
    finally:
        timer.close()
    want = ref.topk_attn_decode(w.q, w.k, w.v, ranges, K, w.scale)
    assert np.array_equal(idx, want["idx"])
    for b in range(w.B):
        for h in range(w.H_q):
            check_out(o[b, h], lse[b, h], want["o"][b, h], want["lse"][b, h], False, f"half K={K} ({b},{h})")
    assert np.all(np.isnan(o2[11, 7])) and np.isnan(lse2[11, 7])
    sel = idx2[11, 7][idx2[11, 7] >= 0]
    assert sel.shape[0] == K and np.all(np.diff(sel) > 0)
    keep = np.ones((w.B, w.H_q), bool)
    keep[11, 7] = False
    for x, y in ((idx, idx2), (o, o2), (lse, lse2)):
        assert np.array_equal(x[keep], y[keep])


@pytest.mark.parametrize("K", [300, 9000])
def test_codebook_ties_many_candidates(ops, K):
    """Keys from a 6-row codebook over 24,000 rows: every score ties with
    thousands of others. K = 9000 puts more than 8 candidates per select
    thread into the tied bin (the wave-segment compaction), K = 300 fewer;
    both sets must equal the oracle's exactly (lowest rows first)."""
    from workloads import make_multi_query
    w = make_multi_query(1, 4, 2, 1, 24000, "bf16", codebook=6, tag=43)
    w.q = np.ascontiguousarray(w.q[:, :, 0])
    ranges = [(0, 11000), (12000, 24000)]
    log(f"case codebook ties K={K}")
    idx, o, lse = run(ops, w, ranges, K)
    want = ref.topk_attn_decode(w.q, w.k, w.v, ranges, K, w.scale)
    assert np.array_equal(idx, want["idx"])
    for h in range(w.H_q):
        check_out(o[0, h], lse[0, h], want["o"][0, h], want["lse"][0, h], False, f"codebook K={K} head {h}")


def test_c4_batch_reduced(ops):
    """Batch of 16 sequences with per-sequence key offsets, K=1024."""
    log("case c4 reduced B=16 L=4096 K=1024")
    w = make_workload(4, L=4096)
    idx, o, lse = run(ops, w, w.ranges, 1024)
    heads = [(b, h) for b in range(16) for h in (0, 5, 31)]
    check_heads(w, heads, idx, o, lse, w.ranges, 1024, label="c4 reduced")


def test_merge_kernel(ops):
    rng = np.random.default_rng(9)
    rows, d = 37, 128
    oa = rng.standard_normal((rows, d)).astype(np.float32)
    ob = rng.standard_normal((rows, d)).astype(np.float32)
    la = (rng.standard_normal(rows) * 5).astype(np.float32)
    lb = (rng.standard_normal(rows) * 5).astype(np.float32)
    la[3] = -np.inf
    lb[4] = -np.inf
    la[5] = lb[5] = -np.inf
    oa[3] = np.nan  # an empty operand's o must not leak
    want_o, want_l = ref.attn_merge_lse(oa.astype(np.float64), la.astype(np.float64), ob.astype(np.float64),
                                        lb.astype(np.float64))
    ta, tb = torch.from_numpy(oa).cuda(), torch.from_numpy(ob).cuda()
    tla, tlb = torch.from_numpy(la).cuda(), torch.from_numpy(lb).cuda()
    o, l = ops.attn_merge_lse(ta, tla, tb, tlb)
    torch.cuda.synchronize()
    assert np.max(np.abs(o.cpu().numpy() - want_o)) < 1e-5
    lg = l.cpu().numpy()
    fin = np.isfinite(want_l)
    assert np.max(np.abs(lg[fin] - want_l[fin])) < 1e-5 and np.all(np.isneginf(lg[~fin]))
    # in place (outputs alias the first operand)
    ops.attn_merge_lse(ta, tla, tb, tlb, o_out=ta, lse_out=tla)
    torch.cuda.synchronize()
    assert np.max(np.abs(ta.cpu().numpy() - want_o)) < 1e-5


def test_deterministic_repeats_and_grids(ops):
    """Ten calls give bit-identical outputs; so does the same sequence inside a
    batch of three, where the scan splits its rows over a different number
    of workgroups per KV head (the results do not depend on the grid)."""
    w = make_workload(2, L=8192)
    first = run(ops, w, w.ranges, 1000)
    for _ in range(9):
        again = run(ops, w, w.ranges, 1000)
        for x, y in zip(first, again):
            assert np.array_equal(x, y)
    q = torch.from_numpy(np.repeat(w.q, 3, axis=0)).cuda()
    k, v = dev_kv(w)
    k3, v3 = k.repeat(3, 1, 1, 1).contiguous(), v.repeat(3, 1, 1, 1).contiguous()
    idx, o, lse = ops.topk_attn_decode(q, k3, v3, w.ranges, 1000, w.scale)
    torch.cuda.synchronize()
    for b in range(3):
        for x, y in zip(first, (idx[b:b + 1].cpu().numpy(), o[b:b + 1].cpu().numpy(), lse[b:b + 1].cpu().numpy())):
            assert np.array_equal(x, y), f"sequence {b} of the batch differs"


@pytest.mark.parametrize("K", [500, 10000])
def test_nan_query_propagates(ops, K):
    """A NaN in one head's query makes every score of that head NaN: the call
    returns STDK_OK, that head's o and lse are NaN, and every other head
    (including the other heads of its KV group, which share the scan) equals
    the clean call bit for bit. K = 10000 >= n takes the dense path."""
    w = make_workload(2, L=8192 if K < 8192 else 7000)
    clean = run(ops, w, w.ranges, K)
    qn = w.q.copy()
    qn[0, 5, 17] = np.nan
    qt = torch.from_numpy(qn).cuda()
    k, v = dev_kv(w)
    idx, o, lse = ops.topk_attn_decode(qt, k, v, w.ranges, K, w.scale)
    torch.cuda.synchronize()
    idx, o, lse = idx.cpu().numpy(), o.cpu().numpy(), lse.cpu().numpy()
    assert np.all(np.isnan(o[0, 5])) and np.isnan(lse[0, 5])
    sel = idx[0, 5][idx[0, 5] >= 0]
    assert sel.shape[0] == min(K, sum(e - b for b, e in w.ranges)) and np.all(np.diff(sel) > 0)
    others = [h for h in range(w.H_q) if h != 5]
    for x, y in zip(clean, (idx, o, lse)):
        assert np.array_equal(x[0, others], y[0, others])


def test_workspace_reuse_counters_return_to_zero(ops):
    """One workspace serves several calls of one layout with different n and
    K: each call leaves the counters (the first B*H_q*16448 bytes) zero,
    and every result equals the result with a fresh zero-filled workspace."""
    log("case workspace reuse c2 layout L=20000")
    w = make_workload(2, L=20000)
    q = torch.from_numpy(w.q).cuda()
    k, v = dev_kv(w)
    lay = ops.make_layout(k, w.H_q)
    n_full = sum(e - b for b, e in w.ranges)
    ws = ops.new_workspace(ops.topk_attn_decode_workspace_size(lay, n_full, 2048), q.device)
    counters = w.B * w.H_q * ops.COUNTER_BYTES_PER_HEAD
    cases = [(w.ranges, 2048), ([(0, 5000)], 100), (w.ranges, 7), ([(100, 300), (9000, 19000)], 512)]
    for ranges, K in cases:
        got = ops.topk_attn_decode(q, k, v, ranges, K, w.scale, workspace=ws, layout=lay)
        fresh = ops.topk_attn_decode(q, k, v, ranges, K, w.scale, layout=lay)
        torch.cuda.synchronize()
        assert int(torch.count_nonzero(ws[:counters]).item()) == 0, f"counters left dirty after K={K}"
        for x, y in zip(got, fresh):
            assert torch.equal(x, y), f"reused workspace differs for K={K}"


def test_workspace_shared_with_multi_query(ops):
    """topk_multi_query leaves the decode calls' counter region alone: a
    buffer used by it and then by topk_attn_decode gives the result of a
    fresh zero-filled buffer, with the counters zero afterwards."""
    w = make_workload(2, L=8192)
    q = torch.from_numpy(w.q).cuda()
    k, v = dev_kv(w)
    lay = ops.make_layout(k, w.H_q)
    n = sum(e - b for b, e in w.ranges)
    qm = torch.from_numpy(np.random.default_rng(3).standard_normal((1, w.H_q, 3, 128), dtype=np.float32)).cuda()
    size = max(ops.topk_attn_decode_workspace_size(lay, n, 500), ops.topk_multi_query_workspace_size(lay, 3, n, 500))
    ws = ops.new_workspace(size, q.device)
    ops.topk_multi_query(qm, k, w.ranges, 500, w.scale, workspace=ws, layout=lay)
    got = ops.topk_attn_decode(q, k, v, w.ranges, 500, w.scale, workspace=ws, layout=lay)
    fresh = ops.topk_attn_decode(q, k, v, w.ranges, 500, w.scale, layout=lay)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(ws[:w.B * w.H_q * ops.COUNTER_BYTES_PER_HEAD]).item()) == 0
    for x, y in zip(got, fresh):
        assert torch.equal(x, y)


@pytest.mark.parametrize("entry", ["topk", "static", "retopk"])
def test_failed_call_leaves_workspace_usable(ops, entry):
    """A launch failure forced from the host right after the scan (the
    select is never enqueued) leaves the workspace's counters non-zero; the
    call returns STDK_EHIP, and the next call on the same buffer repairs them
    first: its results equal those of a fresh buffer."""
    from sparse_top_decode_amd.native import STDK_EHIP, StdkError
    w = make_workload(2, L=8192)
    q = torch.from_numpy(w.q).cuda()
    k, v = dev_kv(w)
    lay = ops.make_layout(k, w.H_q)
    n = sum(e - b for b, e in w.ranges)
    counters = w.B * w.H_q * ops.COUNTER_BYTES_PER_HEAD
    if entry == "retopk":
        rt = ops.Retopk(k, w.H_q, top_k=300, cache_cap=4, top_r=2, recent=8, tau=0.5, refresh=1, scale=w.scale)
        ws = rt.workspace
        first = 1  # retopk_select, then the scan
        call = lambda: rt.step(q, k, v, 8192, 0)
        fresh_rt = ops.Retopk(k, w.H_q, top_k=300, cache_cap=4, top_r=2, recent=8, tau=0.5, refresh=1, scale=w.scale)
        fresh_call = lambda: fresh_rt.step(q, k, v, 8192, 0)
    else:
        size = (ops.topk_attn_decode_workspace_size(lay, n, 500) if entry == "topk" else
                ops.topk_attn_decode_static_workspace_size(lay, n, 640, 500))
        ws = ops.new_workspace(size, q.device)
        first = 0
        if entry == "topk":
            call = lambda: ops.topk_attn_decode(q, k, v, w.ranges, 500, w.scale, workspace=ws, layout=lay)
            fresh_call = lambda: ops.topk_attn_decode(q, k, v, w.ranges, 500, w.scale, layout=lay)
        else:
            call = lambda: ops.topk_attn_decode_static(q, k, v, w.ranges, w.static_ranges, 500, w.scale,
                                                       workspace=ws, layout=lay)
            fresh_call = lambda: ops.topk_attn_decode_static(q, k, v, w.ranges, w.static_ranges, 500, w.scale,
                                                             layout=lay)
    ops.inject_launch_failure(first + 1)
    with pytest.raises(StdkError) as ei:
        call()
    assert ei.value.code == STDK_EHIP
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(ws[:counters]).item()) > 0, "the forced failure should leave counters set"
    got = call()
    want = fresh_call()
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(ws[:counters]).item()) == 0
    for name in (got if isinstance(got, dict) else range(len(got))):
        x, y = got[name], want[name]
        if x is not None:
            assert torch.equal(x, y), name


@pytest.mark.parametrize("cfg,n_rows", [(2, 640), (2, 1280), (2, 1281), (2, 3000), (1, 640), (1, 641), (3, 300), (3, 900)])
def test_dense_path_sizes(ops, cfg, n_rows):
    """K >= n is dense attention over the whole row set. Short sets run in one
    workgroup per KV head, longer ones split over workgroups and combine;
    sizes on both sides of the switch, bf16 (G = 4 and G = 7) and fp32."""
    L = 4096
    w = make_workload(cfg, L=L) if cfg != 1 else make_workload(1)
    # two ranges so that positions map to rows through the range table
    first = n_rows // 3
    ranges = [(5, 5 + first), (L - (n_rows - first), L)]
    K = n_rows + 3
    log(f"case dense cfg={cfg} n={n_rows} K={K}")
    q = w.q if w.q.ndim == 3 else w.q[:, :, 0]
    qt = torch.from_numpy(np.ascontiguousarray(q)).cuda()
    k, v = dev_kv(w)
    idx, o, lse = ops.topk_attn_decode(qt, k, v, ranges, K, w.scale)
    torch.cuda.synchronize()
    idx, o, lse = idx.cpu().numpy(), o.cpu().numpy(), lse.cpu().numpy()
    rows = ref.range_rows(ranges)
    assert np.all(idx[:, :, :n_rows] == rows[None, None, :]) and np.all(idx[:, :, n_rows:] == -1)
    heads = [(0, h) for h in range(w.H_q)]
    check_heads(w, heads, None, o, lse, ranges, K, fp32=(cfg == 1), q=q, label=f"dense c{cfg} n={n_rows}")
