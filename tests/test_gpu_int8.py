"""GPU parity of the int8 recall stage: quantize_keys_int8 against the
oracle's codes (bit-exact: the codes are integers decided by one fp32
division each, taken in fp32 on both sides), and topk_attn_decode_int8
against the oracle's two-stage definition: the superset is the top-K' of the
int8 scores (index-set band 1e-3 around the oracle's K'-th int8 score), the
final set is the exact top-K inside the GPU's own superset (same band on the
exact scores), and o / lse are the oracle's attention over that set."""

import numpy as np
import pytest
import torch

from gpu_util import check_index_set, check_out, dev_kv, log
from oracle import reference as ref
from workloads import make_multi_query, make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops(stdk):
    from sparse_top_decode_amd import ops
    return ops


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_bit_exact(ops, dtype):
    w = make_multi_query(2, 4, 2, 1, 3000, dtype, tag=31)
    ranges = [(0, 1000), (1500, 2713)]
    log(f"case quantize {dtype}")
    k, _ = dev_kv(w)
    codes, scales = ops.quantize_keys_int8(k, ranges, w.H_q)
    torch.cuda.synchronize()
    c = codes.cpu().numpy()
    s = scales.cpu().numpy()
    rows = ref.range_rows(ranges)
    want_c, want_s = ref.quantize_keys_int8(w.k[:, :, rows])
    assert np.array_equal(s[:, :, rows], want_s)
    assert np.array_equal(c[:, :, rows], want_c)
    outside = np.setdiff1d(np.arange(3000), rows)
    assert not np.any(c[:, :, outside]) and not np.any(s[:, :, outside])


def run_int8(ops, w, ranges, K, K2):
    q = torch.from_numpy(w.q if w.q.ndim == 3 else np.ascontiguousarray(w.q[:, :, 0])).cuda()
    k, v = dev_kv(w)
    codes, scales = ops.quantize_keys_int8(k, ranges, w.H_q)
    idx, sup, o, lse = ops.topk_attn_decode_int8(q, k, v, codes, scales, ranges, K, K2, w.scale, want_sup=True)
    torch.cuda.synchronize()
    return (q.cpu().numpy(), codes.cpu().numpy(), scales.cpu().numpy(), idx.cpu().numpy(), sup.cpu().numpy(),
            o.cpu().numpy(), lse.cpu().numpy())


def oracle_codes(w, codes, scales, rows, label):
    """The oracle's codes and scales of every KV head's rows (zero outside
    them), after checking that the GPU's equal them bit for bit; the int8
    scores are then formed from the oracle's own codes, so no oracle input
    comes from the GPU."""
    want_c, want_s = ref.quantize_keys_int8(w.k[:, :, rows])
    assert np.array_equal(codes[:, :, rows], want_c), f"{label}: int8 codes differ from the oracle's"
    assert np.array_equal(scales[:, :, rows], want_s), f"{label}: row scales differ from the oracle's"
    oc = np.zeros(codes.shape, np.int8)
    osc = np.zeros(scales.shape, np.float32)
    oc[:, :, rows], osc[:, :, rows] = want_c, want_s
    return oc, osc


def check_int8_heads(w, q, codes, scales, ranges, K, K2, idx, sup, o, lse, heads, label):
    G = w.H_q // w.H_kv
    rows = ref.range_rows(ranges)
    codes, scales = oracle_codes(w, codes, scales, rows, label)
    recall = []
    for b, h in heads:
        hk = h // G
        z8 = ref.int8_scores(q[b, h], codes[b, hk], scales[b, hk], rows, w.scale)
        _, zk8 = ref.select_topk(z8, rows, K2)
        check_index_set(sup[b, h], rows, z8, zk8, K2)
        srows = sup[b, h][sup[b, h] >= 0].astype(np.int64)
        r = ref.attend_rows(q[b, h], w.k[b, hk], w.v[b, hk], srows, K, w.scale)
        check_index_set(idx[b, h], srows, r["z"], r["zk"], K)
        check_out(o[b, h], lse[b, h], r["o"], r["lse"], w.kv_dtype == "f32", f"{label} ({b},{h})")
        ex = ref.attend_rows(q[b, h], w.k[b, hk], w.v[b, hk], rows, K, w.scale)
        recall.append(np.isin(ex["rows"], srows).mean())
    return float(np.mean(recall))


@pytest.mark.parametrize("L,K,K2", [(8192, 256, 512), (8192, 256, 256), (5000, 100, 1500),
                                    (30000, 2000, 17000)])
def test_int8_recall_c2_shape(ops, L, K, K2):
    """Llama-3-8B head layout (32 q / 8 KV, bf16) at reduced length; the last
    case has more superset rows than the staged top-K keeps in LDS."""
    w = make_workload(2, L=L)
    log(f"case int8 recall c2 L={L} K={K} K'={K2}")
    q, codes, scales, idx, sup, o, lse = run_int8(ops, w, w.ranges, K, K2)
    rec = check_int8_heads(w, q, codes, scales, w.ranges, K, K2, idx, sup, o, lse,
                           [(0, h) for h in range(w.H_q)], f"int8 L={L}")
    log(f"[int8 L={L} K={K} K'={K2}] exact top-K rows inside the superset: {rec:.4f}")
    if K2 >= 2 * K:
        assert rec > 0.9


def test_int8_recall_fp32_cache_and_ranges(ops):
    w = make_multi_query(1, 4, 2, 1, 3000, "f32", tag=33)
    w.q = np.ascontiguousarray(w.q[:, :, 0])
    ranges = [(10, 900), (1200, 2999)]
    log("case int8 recall fp32 cache")
    q, codes, scales, idx, sup, o, lse = run_int8(ops, w, ranges, 40, 120)
    check_int8_heads(w, q, codes, scales, ranges, 40, 120, idx, sup, o, lse, [(0, h) for h in range(4)], "int8 f32")


def test_int8_superset_of_everything_is_exact(ops):
    """recall_k >= n: the superset is every row and the result is
    topk_attn_decode's, bit for bit."""
    w = make_workload(2, L=4096)
    log("case int8 recall_k >= n")
    q = torch.from_numpy(w.q).cuda()
    k, v = dev_kv(w)
    codes, scales = ops.quantize_keys_int8(k, w.ranges, w.H_q)
    n = sum(e - b for b, e in w.ranges)
    idx, sup, o, lse = ops.topk_attn_decode_int8(q, k, v, codes, scales, w.ranges, 300, n + 5, w.scale, want_sup=True)
    idx2, o2, lse2 = ops.topk_attn_decode(q, k, v, w.ranges, 300, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(o, o2) and torch.equal(lse, lse2)
    rows = torch.from_numpy(ref.range_rows(w.ranges).astype(np.int32)).cuda()
    assert torch.equal(sup[:, :, :n], rows.expand(sup.shape[0], sup.shape[1], n))
    assert torch.all(sup[:, :, n:] == -1)


def test_int8_empty_ranges(ops):
    w = make_workload(2, L=1024)
    q = torch.from_numpy(w.q).cuda()
    k, v = dev_kv(w)
    codes = torch.zeros(k.shape, dtype=torch.int8, device="cuda")
    scales = torch.zeros(k.shape[:3], dtype=torch.float32, device="cuda")
    idx, sup, o, lse = ops.topk_attn_decode_int8(q, k, v, codes, scales, [], 8, 16, w.scale, want_sup=True)
    torch.cuda.synchronize()
    assert torch.all(idx == -1) and torch.all(sup == -1) and torch.all(o == 0) and torch.all(torch.isneginf(lse))


# ---------------------------------------------------------------------------
# int8 recall with a static window in one pass
# ---------------------------------------------------------------------------
def run_int8_static(ops, w, ranges, static, K, K2):
    q = torch.from_numpy(w.q if w.q.ndim == 3 else np.ascontiguousarray(w.q[:, :, 0])).cuda()
    k, v = dev_kv(w)
    codes, scales = ops.quantize_keys_int8(k, ranges, w.H_q)
    idx, sup, o, lse = ops.topk_attn_decode_int8_static(q, k, v, codes, scales, ranges, static, K, K2, w.scale,
                                                        want_sup=True)
    torch.cuda.synchronize()
    return (q.cpu().numpy(), codes.cpu().numpy(), scales.cpu().numpy(), idx.cpu().numpy(), sup.cpu().numpy(),
            o.cpu().numpy(), lse.cpu().numpy())


def check_int8_static_heads(w, q, codes, scales, ranges, static, K, K2, idx, sup, o, lse, heads, label):
    """Superset and chosen set as check_int8_heads; o / lse are the oracle's
    attention over the chosen rows united with the static rows, and equal the
    oracle's LSE merge of the two partial attentions."""
    G = w.H_q // w.H_kv
    rows = ref.range_rows(ranges)
    srows_static = ref.range_rows(static)
    codes, scales = oracle_codes(w, codes, scales, rows, label)
    for b, h in heads:
        hk = h // G
        z8 = ref.int8_scores(q[b, h], codes[b, hk], scales[b, hk], rows, w.scale)
        _, zk8 = ref.select_topk(z8, rows, K2)
        check_index_set(sup[b, h], rows, z8, zk8, K2)
        srows = sup[b, h][sup[b, h] >= 0].astype(np.int64)
        r = ref.attend_rows(q[b, h], w.k[b, hk], w.v[b, hk], srows, K, w.scale)
        check_index_set(idx[b, h], srows, r["z"], r["zk"], K)
        chosen = idx[b, h][idx[b, h] >= 0].astype(np.int64)
        union = np.union1d(chosen, srows_static)
        u = ref.attend_rows(q[b, h], w.k[b, hk], w.v[b, hk], union, union.shape[0], w.scale)
        check_out(o[b, h], lse[b, h], u["o"], u["lse"], w.kv_dtype == "f32", f"{label} ({b},{h})")
        if srows_static.shape[0] and chosen.shape[0]:
            st = ref.attend_rows(q[b, h], w.k[b, hk], w.v[b, hk], srows_static, srows_static.shape[0], w.scale)
            dy = ref.attend_rows(q[b, h], w.k[b, hk], w.v[b, hk], chosen, chosen.shape[0], w.scale)
            mo, ml = ref.attn_merge_lse(st["o"][None], np.array([st["lse"]]), dy["o"][None], np.array([dy["lse"]]))
            assert np.allclose(mo[0], u["o"], atol=1e-12) and abs(ml[0] - u["lse"]) < 1e-12


@pytest.mark.parametrize("L,K,K2", [(8192, 256, 1024), (6000, 100, 700), (8192, 300, 300)])
def test_int8_static_c2_shape(ops, L, K, K2):
    """Llama-3-8B head layout, static window of the first 128 and last 512
    rows, int8 recall over the rest."""
    w = make_workload(2, L=L)
    log(f"case int8 static c2 L={L} K={K} K'={K2}")
    q, codes, scales, idx, sup, o, lse = run_int8_static(ops, w, w.ranges, w.static_ranges, K, K2)
    check_int8_static_heads(w, q, codes, scales, w.ranges, w.static_ranges, K, K2, idx, sup, o, lse,
                            [(0, h) for h in range(w.H_q)], f"int8 static L={L}")


def test_int8_static_fp32_ragged(ops):
    """fp32 cache, two dynamic and two static ranges, ragged lengths."""
    w = make_multi_query(1, 4, 2, 1, 3000, "f32", tag=35)
    w.q = np.ascontiguousarray(w.q[:, :, 0])
    ranges = [(40, 900), (1000, 2811)]
    static = [(0, 37), (2900, 3000)]
    log("case int8 static fp32 ragged")
    q, codes, scales, idx, sup, o, lse = run_int8_static(ops, w, ranges, static, 33, 130)
    check_int8_static_heads(w, q, codes, scales, ranges, static, 33, 130, idx, sup, o, lse,
                            [(0, h) for h in range(4)], "int8 static f32")


def test_int8_static_equals_merge_of_calls(ops):
    """The one pass against the dense static call, topk_attn_decode_int8 and
    attn_merge_lse on the GPU: same chosen rows, outputs within fp32 rounding."""
    w = make_workload(2, L=8192)
    log("case int8 static vs merge of calls")
    q = torch.from_numpy(w.q).cuda()
    k, v = dev_kv(w)
    codes, scales = ops.quantize_keys_int8(k, w.ranges, w.H_q)
    K, K2 = 256, 1024
    idx, sup, o, lse = ops.topk_attn_decode_int8_static(q, k, v, codes, scales, w.ranges, w.static_ranges, K, K2,
                                                        w.scale, want_sup=True)
    idx2, sup2, o_d, l_d = ops.topk_attn_decode_int8(q, k, v, codes, scales, w.ranges, K, K2, w.scale, want_sup=True)
    n_st = sum(e - b for b, e in w.static_ranges)
    _, o_s, l_s = ops.topk_attn_decode(q, k, v, w.static_ranges, n_st, w.scale)
    o_m, l_m = ops.attn_merge_lse(o_s, l_s, o_d, l_d)
    torch.cuda.synchronize()
    assert torch.equal(sup, sup2) and torch.equal(idx, idx2)
    assert torch.allclose(o, o_m, atol=1e-5, rtol=1e-4) and torch.allclose(lse, l_m, atol=1e-5, rtol=1e-5)


def test_int8_static_full_superset_is_static_path(ops):
    """recall_k >= |Omega|: topk_attn_decode_static's result, bit for bit, and
    the superset lists every dynamic row; likewise with top_k >= |Omega|."""
    w = make_workload(2, L=3000)
    log("case int8 static recall_k >= n")
    q = torch.from_numpy(w.q).cuda()
    k, v = dev_kv(w)
    codes, scales = ops.quantize_keys_int8(k, w.ranges, w.H_q)
    n = sum(e - b for b, e in w.ranges)
    for K in (200, n + 3):
        idx, sup, o, lse = ops.topk_attn_decode_int8_static(q, k, v, codes, scales, w.ranges, w.static_ranges, K,
                                                            max(K, n), w.scale, want_sup=True)
        idx2, o2, lse2 = ops.topk_attn_decode_static(q, k, v, w.ranges, w.static_ranges, K, w.scale)
        torch.cuda.synchronize()
        assert torch.equal(idx, idx2) and torch.equal(o, o2) and torch.equal(lse, lse2)
        rows = torch.from_numpy(ref.range_rows(w.ranges).astype(np.int32)).cuda()
        assert torch.equal(sup[:, :, :n], rows.expand(sup.shape[0], sup.shape[1], n))
        assert torch.all(sup[:, :, n:] == -1)


def test_int8_static_only_static_rows(ops):
    """No dynamic rows: dense attention over the static window; idx and the
    superset are all -1."""
    w = make_workload(2, L=2048)
    q = torch.from_numpy(w.q).cuda()
    k, v = dev_kv(w)
    codes = torch.zeros(k.shape, dtype=torch.int8, device="cuda")
    scales = torch.zeros(k.shape[:3], dtype=torch.float32, device="cuda")
    static = [(0, 128), (1536, 2048)]
    idx, sup, o, lse = ops.topk_attn_decode_int8_static(q, k, v, codes, scales, [], static, 8, 16, w.scale,
                                                        want_sup=True)
    n_st = 640
    _, o2, l2 = ops.topk_attn_decode(q, k, v, static, n_st, w.scale)
    torch.cuda.synchronize()
    assert torch.all(idx == -1) and torch.all(sup == -1)
    assert torch.allclose(o, o2, atol=1e-6) and torch.allclose(lse, l2, atol=1e-6)


def test_int8_static_equal_recall_without_sup(ops):
    """recall_k == top_k with and without the superset output: the same
    chosen rows, o and lse (the superset is then the chosen set)."""
    w = make_workload(2, L=8192)
    q = torch.from_numpy(w.q).cuda()
    k, v = dev_kv(w)
    codes, scales = ops.quantize_keys_int8(k, w.ranges, w.H_q)
    a = ops.topk_attn_decode_int8_static(q, k, v, codes, scales, w.ranges, w.static_ranges, 300, 300, w.scale,
                                         want_sup=True)
    b = ops.topk_attn_decode_int8_static(q, k, v, codes, scales, w.ranges, w.static_ranges, 300, 300, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(a[0], a[1]) and torch.equal(a[0], b[0])
    assert torch.equal(a[2], b[2]) and torch.equal(a[3], b[3])


@pytest.mark.parametrize("K,K2", [(100, 700), (300, 300), (64, 5000)])
def test_int8_exact_ties_codebook(ops, K, K2):
    """Keys drawn from a 6-row codebook: int8 and exact scores tie in groups
    of thousands, so both the superset and the final set are decided by the
    lowest-row rule. Both must equal the oracle's exactly (with a static
    window in the same call)."""
    w = make_multi_query(1, 4, 2, 1, 12000, "bf16", codebook=6, tag=41)
    w.q = np.ascontiguousarray(w.q[:, :, 0])
    ranges = [(100, 7000), (7500, 11800)]
    static = [(0, 100), (11800, 12000)]
    log(f"case int8 codebook ties K={K} K'={K2}")
    q, codes, scales, idx, sup, o, lse = run_int8_static(ops, w, ranges, static, K, K2)
    codes, scales = oracle_codes(w, codes, scales, ref.range_rows(ranges), "codebook")
    want = ref.topk_attn_decode_int8(q, w.k, w.v, codes, scales, ranges, K, K2, w.scale)
    assert np.array_equal(sup, want["sup"]), "superset differs from the oracle's"
    assert np.array_equal(idx, want["idx"]), "chosen rows differ from the oracle's"
    check_int8_static_heads(w, q, codes, scales, ranges, static, K, K2, idx, sup, o, lse,
                            [(0, h) for h in range(4)], f"int8 ties K={K}")


@pytest.mark.parametrize("K", [150, 333, 512, 599])
def test_rerank_select_near_ties_exact(ops, K):
    """The exact top-K inside a superset whose scores crowd into a few
    thousand fp32 ulps above 1.0 (640 rows at 1.0 + u ulps, u < 4000, with
    repeats) plus 60 negative rows that widen the key range: the radix
    passes then narrow to 1024-key bins that hold many rows each, and the
    last pass must count only the chosen bin (keys above it were counted
    already). q = e_0, scale 1 and an fp32 cache make every score exactly
    the row's first element on both sides, so the chosen rows (ties to the
    lowest row) must equal the oracle's bit for bit. A window twice the bin
    counted the next bin's rows twice and chose K - 1 rows here."""
    rng = np.random.default_rng(77)
    n, d = 700, 128
    one = np.float32(1.0).view(np.uint32)
    pos = (one + rng.integers(0, 4000, 640)).astype(np.uint32).view(np.float32)
    neg = -rng.uniform(1, 5, 60).astype(np.float32)
    x = np.empty(n, np.float32)
    perm = rng.permutation(n)
    x[perm[:640]], x[perm[640:]] = pos, neg
    kc = np.zeros((1, 1, n, d), np.float32)
    kc[0, 0, :, 0] = x
    vc = rng.standard_normal((1, 1, n, d), dtype=np.float32)
    q = np.zeros((1, 1, d), np.float32)
    q[0, 0, 0] = 1.0
    K2 = 650
    log(f"case rerank select near ties K={K}")
    k, v = torch.from_numpy(kc).cuda(), torch.from_numpy(vc).cuda()
    codes, scales = ops.quantize_keys_int8(k, [(0, n)], 1)
    idx, sup, o, lse = ops.topk_attn_decode_int8(torch.from_numpy(q).cuda(), k, v, codes, scales, [(0, n)], K, K2,
                                                 1.0, want_sup=True)
    torch.cuda.synchronize()

    class W:  # the oracle's view of this input
        pass
    w = W()
    w.k, w.v = kc, vc
    oc, osc = oracle_codes(w, codes.cpu().numpy(), scales.cpu().numpy(), np.arange(n), "near ties")
    want = ref.topk_attn_decode_int8(q, kc, vc, oc, osc, [(0, n)], K, K2, 1.0)
    assert np.array_equal(sup.cpu().numpy(), want["sup"])
    assert np.array_equal(idx.cpu().numpy(), want["idx"]), "chosen rows differ from the oracle's"
    check_out(o.cpu().numpy()[0, 0], lse.cpu().numpy()[0, 0], want["o"][0, 0], want["lse"][0, 0], True, "near ties")
