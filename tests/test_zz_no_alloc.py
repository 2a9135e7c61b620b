"""GPU test of topk_attn_decode_static_noalloc (the allocation-free variant
of the one-pass decode step): through the C ABI, against
topk_attn_decode_static with a caller-owned workspace, on consecutive calls
of different sizes that share the library's scratch array."""

import numpy as np
import pytest
import torch

from gpu_util import dev_kv, log
from workloads import make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops(stdk):
    from sparse_top_decode_amd import ops
    return ops


def both(ops, w, K):
    q = torch.from_numpy(w.q).cuda()
    k, v = dev_kv(w)
    lay = ops.make_layout(k, w.H_q)
    got = ops.topk_attn_decode_static_noalloc(q, k, v, w.ranges, w.static_ranges, K, w.scale, layout=lay)
    want = ops.topk_attn_decode_static(q, k, v, w.ranges, w.static_ranges, K, w.scale, layout=lay)
    torch.cuda.synchronize()
    return [x.cpu().numpy() for x in got], [x.cpu().numpy() for x in want]


def test_noalloc_matches_workspace_entry_point(ops):
    """The headline layer (131,072 rows, K = 2048, 640 static rows), then a
    smaller one (20,000 rows, K = 512), then the large one again: each call's
    chosen rows, o and lse equal topk_attn_decode_static's bit for bit (same
    kernels; the scratch keeps the previous call's contents, so this also
    checks that each call clears what must start at zero)."""
    big = make_workload(2)
    small = make_workload(2, L=20000)
    for w, K in ((big, 2048), (small, 512), (big, 2048)):
        log(f"case noalloc L={w.L} K={K}")
        got, want = both(ops, w, K)
        for name, x, y in zip(("idx", "o", "lse"), got, want):
            assert np.array_equal(x, y), f"L={w.L} K={K}: {name} differs"
        assert np.all(got[0] >= 0) and np.all(np.isfinite(got[1]))


def test_noalloc_dense_and_empty(ops):
    """Every dynamic row chosen (dense path) and no rows at all."""
    w = make_workload(2, L=3000)
    n = sum(e - b for b, e in w.ranges)
    got, want = both(ops, w, n + 7)
    for x, y in zip(got, want):
        assert np.array_equal(x, y)
    q = torch.from_numpy(w.q).cuda()
    k, v = dev_kv(w)
    idx, o, lse = ops.topk_attn_decode_static_noalloc(q, k, v, [], [], 8, w.scale)
    torch.cuda.synchronize()
    assert torch.all(idx == -1) and torch.all(o == 0) and torch.all(torch.isneginf(lse))
