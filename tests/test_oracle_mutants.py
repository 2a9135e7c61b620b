"""Planted mistakes in the CPU oracle must be caught by at least one pin.

Each mutant replaces one oracle function (on the CPU, inside this test only)
with a plausible wrong version; the test passes when some pin fails.
"""

import math

import numpy as np
import pytest

import pins
from oracle import reference as ref


def _caught(monkeypatch, name, fn):
    monkeypatch.setattr(ref, name, fn)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(ref)
        except AssertionError:
            failed.append(pin.__name__)
        except Exception as e:  # a crash also counts as detection
            failed.append(pin.__name__ + ":" + type(e).__name__)
    return failed


_orig_softmax_v = ref.softmax_v
_orig_select = ref.select_topk
_orig_scores = ref.scores
_orig_merge = ref.attn_merge_lse
_orig_head_step = ref.retopk_head_step
_orig_unit = ref.unit_query_f32


def m_no_renormalisation(z, v):
    o, lse = _orig_softmax_v(z, v)
    if z.shape[0] == 0:
        return o, lse
    m = float(np.max(z))
    return o * float(np.sum(np.exp(z - m))), lse


def m_ties_to_highest(z, rows, k):
    if z.shape[0] == 0 or k <= 0:
        return np.zeros(0, np.int64), float("-inf")
    order = np.lexsort((-rows, -z))
    take = order[:min(k, z.shape[0])]
    return np.sort(rows[take]), float(z[take[-1]])


def m_off_by_one_k(z, rows, k):
    return _orig_select(z, rows, k + 1)


def m_dropped_scale(q, kc, rows, scale):
    return _orig_scores(q, kc, rows, 1.0)


def m_last_coordinate_dropped(q, kc, rows, scale):
    q2 = np.array(q, dtype=np.float64).copy()
    q2[-1] = 0.0
    return _orig_scores(q2, kc, rows, scale)


def m_merge_wrong_weight(o_a, lse_a, o_b, lse_b):
    o, lse = _orig_merge(o_a, lse_a, o_b, lse_b)
    la = np.asarray(lse_a, dtype=np.float64)
    lb = np.asarray(lse_b, dtype=np.float64)
    # forget to rescale the second operand
    ga = np.where(np.isneginf(la), 0.0, np.exp(la - lse))
    return ga[..., None] * np.asarray(o_a) + np.asarray(o_b), lse


def m_merge_lse_max_only(o_a, lse_a, o_b, lse_b):
    o, lse = _orig_merge(o_a, lse_a, o_b, lse_b)
    return o, np.maximum(lse_a, lse_b)


def m_no_recent_window(p, *a, **kw):
    p2 = ref.RetopkParams(p.top_k, p.cache_cap, p.top_r, 0, p.tau, p.refresh)
    return _orig_head_step(p2, *a, **kw)


def m_topr_least_similar(p, q_hat, support, head, count, q, *a, **kw):
    return _orig_head_step(p, -q_hat, support, head, count, q, *a, **kw) if count else \
        _orig_head_step(p, q_hat, support, head, count, q, *a, **kw)


def m_no_normalisation(q):
    return np.asarray(q, dtype=np.float32)


_orig_multi = ref.topk_multi_query


def m_multi_head_mapping(q, k_cache, ranges, top_k, scale, queries=None):
    """query head h read against KV head h mod H_kv instead of h // G"""
    B, Hq, M, d = q.shape
    Hkv = k_cache.shape[1]
    perm = np.concatenate([k_cache[:, [h % Hkv]] for h in range(Hq)], axis=1)
    return _orig_multi(q, np.ascontiguousarray(perm), ranges, top_k, scale, queries)


def m_multi_first_query_only(q, k_cache, ranges, top_k, scale, queries=None):
    """every query of the block gets the first query's set"""
    q0 = np.repeat(q[:, :, :1], q.shape[2], axis=2)
    return _orig_multi(q0, k_cache, ranges, top_k, scale, queries)


_orig_vote = ref.vote_candidates


def m_vote_count_only(union_rows, recent_rows, supports, weights, budget):
    """votes counted without the similarity weights"""
    return _orig_vote(union_rows, recent_rows, supports, [np.float32(1.0)] * len(weights), budget)


def m_vote_ties_to_highest(union_rows, recent_rows, supports, weights, budget):
    """equal confidence resolved towards the highest row"""
    flip = lambda x: 10 ** 6 - np.asarray(x, dtype=np.int64)
    rows, tr = _orig_vote(flip(union_rows), flip(recent_rows), [flip(s) for s in supports], weights, budget)
    return np.sort(flip(rows)), tr


_orig_int8_scores = ref.int8_scores
_orig_quant = ref.quantize_keys_int8


def m_int8_no_row_scale(q, codes_head, scales_head, rows, scale):
    """int8 scores without the per-row scale"""
    return _orig_int8_scores(q, codes_head, np.ones_like(scales_head), rows, scale)


def m_int8_truncating_codes(rows):
    """codes truncated towards zero instead of rounded"""
    k = ref.widen(rows).astype(np.float32)
    c, s = _orig_quant(rows)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    t = np.trunc((k / safe[..., None]).astype(np.float32))
    return np.where((s > 0)[..., None], np.clip(t, -127, 127), 0).astype(np.int8), s


MUTANTS = [
    ("softmax_v", m_no_renormalisation),
    ("select_topk", m_ties_to_highest),
    ("select_topk", m_off_by_one_k),
    ("scores", m_dropped_scale),
    ("scores", m_last_coordinate_dropped),
    ("attn_merge_lse", m_merge_wrong_weight),
    ("attn_merge_lse", m_merge_lse_max_only),
    ("retopk_head_step", m_no_recent_window),
    ("retopk_head_step", m_topr_least_similar),
    ("unit_query_f32", m_no_normalisation),
    ("topk_multi_query", m_multi_head_mapping),
    ("topk_multi_query", m_multi_first_query_only),
    ("vote_candidates", m_vote_count_only),
    ("vote_candidates", m_vote_ties_to_highest),
    ("int8_scores", m_int8_no_row_scale),
    ("quantize_keys_int8", m_int8_truncating_codes),
]


@pytest.mark.parametrize("name,fn", MUTANTS, ids=[f.__name__ for _, f in MUTANTS])
def test_mutant_is_caught(monkeypatch, name, fn):
    failed = _caught(monkeypatch, name, fn)
    assert failed, f"no pin caught mutant {fn.__name__}"
