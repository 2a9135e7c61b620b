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


def check_int8_heads(w, q, codes, scales, ranges, K, K2, idx, sup, o, lse, heads, label):
    G = w.H_q // w.H_kv
    rows = ref.range_rows(ranges)
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


@pytest.mark.parametrize("L,K,K2", [(8192, 256, 512), (8192, 256, 256), (5000, 100, 1500)])
def test_int8_recall_c2_shape(ops, L, K, K2):
    """Llama-3-8B head layout (32 q / 8 KV, bf16) at reduced length."""
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
