"""The seeded input generators: reproducible, chunk-addressable, right shapes."""

import numpy as np

from workloads import make_workload, static_window_ranges, bf16_bits_from_f32, f32_from_bf16_bits


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e38, 1e-40], np.float32)
    b = bf16_bits_from_f32(x)
    back = f32_from_bf16_bits(b)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: goes to the even mantissa (1.0)
    assert back[1] == 1.0
    # 1 + 3*2^-8 is a tie between 1+2^-7 and 1+2^-6: even is 1+2^-6
    assert back[2] == np.float32(1.015625)
    assert back[3] == -2.5
    assert np.all(np.abs(back[:4] - x[:4]) <= np.abs(x[:4]) * 2.0 ** -8)


def test_static_window_ranges():
    s, d = static_window_ranges(131072)
    assert s == [(0, 128), (130560, 131072)] and d == [(128, 130560)]
    s, d = static_window_ranges(600)
    assert s == [(0, 128), (128, 600)] and d == []
    s, d = static_window_ranges(700)
    assert s == [(0, 128), (188, 700)] and d == [(128, 188)]


def test_reproducible_and_shapes():
    a = make_workload(2, L=2048)
    b = make_workload(2, L=2048)
    assert a.k.shape == (1, 8, 2048, 128) and a.k.dtype == np.uint16
    assert a.q.shape == (1, 32, 128) and a.q.dtype == np.float32
    assert np.array_equal(a.k, b.k) and np.array_equal(a.v, b.v) and np.array_equal(a.q, b.q)
    c1 = make_workload(1)
    assert c1.k.dtype == np.float32 and c1.k.shape == (1, 1, 4096, 128) and c1.top_k == 64
    c3 = make_workload(3, L=1024, steps=8, warm=4)
    assert c3.q.shape == (1, 28, 12, 128) and c3.L_max == 1032
    c4 = make_workload(4, L=512, B=3)
    assert c4.k.shape == (3, 8, 512, 128)


def test_c5_planted_rows_are_in_dynamic_set_and_disjoint():
    w = make_workload(5, L=8192, top_k=256)
    lo, hi = w.ranges[0]
    for h in range(8):
        rows = np.concatenate([w.planted[h * 4 + g] for g in range(4)])
        assert len(set(rows.tolist())) == rows.size
        assert rows.min() >= lo and rows.max() < hi
