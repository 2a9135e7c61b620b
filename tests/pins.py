"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each ``pin_*`` function raises AssertionError when the oracle (passed in as a
module-like object) disagrees with a fact that does not come from the oracle
itself: a hand-derived worked example (``tests/golden``), a library routine
for the dense special case, an algebraic identity, or the independent
pure-Python brute force. ``test_oracle_pins.py`` runs them on the real oracle
and ``test_oracle_mutants.py`` checks that planted mistakes make them fail.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

from oracle import brute

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _golden_topk_cache():
    g = _load("closed_form_topk.json")
    a = g["a"]
    n = len(a)
    k = np.zeros((1, 1, n, g["d"]), np.float32)
    v = np.zeros((1, 1, n, g["d"]), np.float32)
    kk = np.zeros((n, g["d"]), np.float64)
    for i, ai in enumerate(a):
        kk[i] = [math.log(ai), 0.5 * i, -1.0, 2.0]
        v[0, 0, i] = [i, 1, (-1) ** i, i * i]
    # fp64 keys: the oracle widens fp32, so keep them as a float64-capable store
    q = np.array(g["q"], np.float32)[None, None, :]
    return g, q, kk[None, None], v.astype(np.float64)


def pin_golden_topk(ref):
    g, q, k, v = _golden_topk_cache()
    for case in g["cases"]:
        out = ref.topk_attn_decode(q, k, v, [tuple(r) for r in case["ranges"]], case["top_k"], g["scale"])
        K = case["top_k"]
        want_idx = case["idx"] + [-1] * (K - len(case["idx"]))
        assert list(out["idx"][0, 0]) == want_idx, (case["name"], out["idx"][0, 0], want_idx)
        np.testing.assert_allclose(out["o"][0, 0], case["o"], rtol=0, atol=1e-12, err_msg=case["name"])
        assert abs(out["lse"][0, 0] - math.log(case["lse_exp"])) < 1e-12, case["name"]


def pin_golden_merge(ref):
    g, q, k, v = _golden_topk_cache()
    a = ref.topk_attn_decode(q, k, v, [(0, 1), (2, 3)], 2, 1.0)
    b = ref.topk_attn_decode(q, k, v, [(1, 2), (3, 7)], 3, 1.0)
    o, lse = ref.attn_merge_lse(a["o"], a["lse"], b["o"], b["lse"])
    np.testing.assert_allclose(o[0, 0], g["merge"]["o"], rtol=0, atol=1e-12)
    assert abs(lse[0, 0] - math.log(g["merge"]["lse_exp"])) < 1e-12
    # the operand order must not matter
    o2, lse2 = ref.attn_merge_lse(b["o"], b["lse"], a["o"], a["lse"])
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-13)


def pin_golden_retopk(ref):
    g = _load("closed_form_retopk.json")
    p = ref.RetopkParams(**g["params"])
    n = len(g["b"])
    k = np.zeros((1, 1, n, g["d"]), np.float64)
    v = np.zeros((1, 1, n, g["d"]), np.float64)
    for i, bi in enumerate(g["b"]):
        k[0, 0, i] = [math.log(bi) / 2.0, 1.0]
        v[0, 0, i] = [i, 10 - i]
    ents = g["cache_oldest_first"]
    qh = np.array([[e["q_hat"] for e in ents]], np.float32)[None]
    sp = np.array([[e["support"] for e in ents]], np.int32)[None]
    st = ref.retopk_state_init(p, qh, sp)
    q = np.array(g["q"], np.float32)[None, None]
    out, new, tr = ref.retopk_step(p, st, q, k, v, g["L_t"], g["t"], g["scale"])
    e = g["expected"]
    assert int(out["path"][0, 0]) == e["path"]
    assert list(tr[(0, 0)]["cand"]) == e["cand"]
    assert list(out["support"][0, 0]) == e["support"]
    np.testing.assert_allclose(out["o"][0, 0], e["o"], rtol=0, atol=1e-12)
    assert abs(out["lse"][0, 0] - math.log(e["lse_exp"])) < 1e-12
    C = p.cache_cap
    h, c = int(new.head[0, 0]), int(new.count[0, 0])
    oldest_first = [((h - (c - 1) + j) % C) for j in range(c)]
    got = [(list(new.q_hat[0, 0, s]), list(new.support[0, 0, s])) for s in oldest_first]
    want = [(x["q_hat"], x["support"]) for x in e["cache_after_oldest_first"]]
    assert got == want, (got, want)


def pin_dense_matches_library_attention(ref, seed=0):
    """K >= n: the oracle must equal torch's scaled_dot_product_attention and
    torch.logsumexp (library routines) in fp64."""
    import torch
    rng = np.random.default_rng([77, seed])
    for (n, d, sc) in [(37, 16, 0.37), (64, 8, 1.0 / math.sqrt(8)), (5, 128, 1.0 / math.sqrt(128))]:
        q = rng.standard_normal((1, 2, d)).astype(np.float32)
        k = rng.standard_normal((1, 1, n, d)).astype(np.float32)
        v = rng.standard_normal((1, 1, n, d)).astype(np.float32)
        out = ref.topk_attn_decode(q, k, v, [(0, n)], n + 3, sc)
        for h in range(2):
            tq = torch.tensor(q[0, h], dtype=torch.float64)[None, None, None, :]
            tk = torch.tensor(k[0, 0], dtype=torch.float64)[None, None]
            tv = torch.tensor(v[0, 0], dtype=torch.float64)[None, None]
            o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=sc)[0, 0, 0].numpy()
            z = (tk[0, 0] @ tq[0, 0, 0]) * sc
            lse = float(torch.logsumexp(z, 0))
            np.testing.assert_allclose(out["o"][0, h], o, rtol=1e-12, atol=1e-12)
            assert abs(out["lse"][0, h] - lse) < 1e-12
            assert list(out["idx"][0, h][:n]) == list(range(n))
            assert all(x == -1 for x in out["idx"][0, h][n:])


def pin_split_merge_identity(ref, seed=0):
    """Any split of the rows into two disjoint sets, each attended in full and
    combined, equals attention over their union (RetrievalAttention review,
    Eq. 3-5)."""
    rng = np.random.default_rng([78, seed])
    n, d = 300, 16
    q = rng.standard_normal((1, 1, d)).astype(np.float32)
    k = rng.standard_normal((1, 1, n, d)).astype(np.float32)
    v = rng.standard_normal((1, 1, n, d)).astype(np.float32)
    full = ref.topk_attn_decode(q, k, v, [(0, n)], n, 0.3)
    for trial in range(4):
        colour = rng.integers(0, 2, n)
        def runs(c):
            rr, start = [], None
            for i in range(n + 1):
                inside = i < n and colour[i] == c
                if inside and start is None:
                    start = i
                if not inside and start is not None:
                    rr.append((start, i))
                    start = None
            return rr
        a = ref.topk_attn_decode(q, k, v, runs(0), n, 0.3)
        b = ref.topk_attn_decode(q, k, v, runs(1), n, 0.3)
        o, lse = ref.attn_merge_lse(a["o"], a["lse"], b["o"], b["lse"])
        np.testing.assert_allclose(o, full["o"], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(lse, full["lse"], rtol=1e-12, atol=1e-12)
    # static window + top-K over the rest = attention over W u S (the pages'
    # decode step), checked against dense attention over that explicit set
    K = 20
    w_ranges = [(0, 8), (n - 24, n)]
    dyn = ref.topk_attn_decode(q, k, v, [(8, n - 24)], K, 0.3)
    stat = ref.topk_attn_decode(q, k, v, w_ranges, n, 0.3)
    o, lse = ref.attn_merge_lse(stat["o"], stat["lse"], dyn["o"], dyn["lse"])
    rows = sorted(list(range(8)) + list(range(n - 24, n)) + [int(x) for x in dyn["idx"][0, 0]])
    explicit = ref.topk_attn_decode(q, k, v, [(r, r + 1) for r in rows], n, 0.3)
    np.testing.assert_allclose(o, explicit["o"], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, explicit["lse"], rtol=1e-12, atol=1e-12)


def pin_shift_invariance(ref, seed=0):
    """Adding one vector c to every key shifts every logit by scale*q.c: the
    chosen rows and the output stay, lse moves by exactly that amount
    (RetrievalAttention review, local-maximum subtraction). Dyadic values keep
    every product and sum exact."""
    rng = np.random.default_rng([79, seed])
    n, d, K = 200, 16, 17
    q = (rng.integers(-8, 9, (1, 1, d)) / 4.0).astype(np.float32)
    k = (rng.integers(-32, 33, (1, 1, n, d)) / 8.0).astype(np.float32)
    v = rng.standard_normal((1, 1, n, d)).astype(np.float32)
    c = (rng.integers(-16, 17, d) / 8.0).astype(np.float32)
    a = ref.topk_attn_decode(q, k, v, [(0, n)], K, 0.25)
    b = ref.topk_attn_decode(q, (k + c).astype(np.float32), v, [(0, n)], K, 0.25)
    assert np.array_equal(a["idx"], b["idx"])
    np.testing.assert_allclose(b["o"], a["o"], rtol=0, atol=1e-12)
    shift = 0.25 * float(np.dot(q[0, 0].astype(np.float64), c.astype(np.float64)))
    assert abs((b["lse"][0, 0] - a["lse"][0, 0]) - shift) < 1e-10


def pin_argmax_and_weights(ref, seed=0):
    """K = 1 returns the value row of the largest logit and lse = that logit;
    with one-hot values the output is the weight vector itself, whose ratios
    are e^{z_i - z_j} (RetrievalAttention review, Eq. 2 keeps the ratios)."""
    rng = np.random.default_rng([80, seed])
    n = 40
    d = n
    q = rng.standard_normal((1, 1, d)).astype(np.float32)
    k = rng.standard_normal((1, 1, n, d)).astype(np.float32)
    v = np.eye(n, d, dtype=np.float32)[None, None]
    sc = 0.4
    z = np.array([sc * float(np.dot(q[0, 0].astype(np.float64), k[0, 0, i].astype(np.float64))) for i in range(n)])
    one = ref.topk_attn_decode(q, k, v, [(0, n)], 1, sc)
    j = int(np.argmax(z))
    assert one["idx"][0, 0, 0] == j
    np.testing.assert_allclose(one["o"][0, 0], v[0, 0, j], atol=1e-15)
    assert abs(one["lse"][0, 0] - z[j]) < 1e-12
    K = 9
    out = ref.topk_attn_decode(q, k, v, [(0, n)], K, sc)
    w = out["o"][0, 0]
    sel = [int(x) for x in out["idx"][0, 0]]
    assert abs(w.sum() - 1.0) < 1e-12
    assert all(abs(w[i]) == 0.0 for i in range(n) if i not in sel)
    for i in sel:
        for jj in sel:
            assert abs(w[i] / w[jj] - math.exp(z[i] - z[jj])) < 1e-9 * math.exp(z[i] - z[jj])
    assert abs(out["lse"][0, 0] - math.log(sum(math.exp(z[i]) for i in sel))) < 1e-12


def pin_brute_topk(ref, seed=0):
    """Oracle == pure-Python brute force on tiny inputs, with duplicated key
    rows (exact ties) and several range layouts."""
    rng = np.random.default_rng([81, seed])
    for trial in range(12):
        n = int(rng.integers(1, 40))
        d = int(rng.integers(1, 9))
        k = rng.standard_normal((1, 1, n, d)).astype(np.float32)
        for _ in range(int(rng.integers(0, 6))):
            i, j = rng.integers(0, n, 2)
            k[0, 0, i] = k[0, 0, j]
        v = rng.standard_normal((1, 1, n, d)).astype(np.float32)
        q = rng.standard_normal((1, 1, d)).astype(np.float32)
        cuts = sorted(set(int(x) for x in rng.integers(0, n + 1, 4)))
        ranges = [(cuts[i], cuts[i + 1]) for i in range(0, len(cuts) - 1, 2) if cuts[i + 1] > cuts[i]] or [(0, n)]
        K = int(rng.integers(1, n + 3))
        sc = float(rng.uniform(0.1, 1.0))
        out = ref.topk_attn_decode(q, k, v, ranges, K, sc)
        rows = [r for b, e in ranges for r in range(b, e)]
        kk = [[float(x) for x in row] for row in k[0, 0]]
        vv = [[float(x) for x in row] for row in v[0, 0]]
        bf = brute.topk_attention([float(x) for x in q[0, 0]], kk, vv, rows, K, sc)
        got = [int(x) for x in out["idx"][0, 0] if x >= 0]
        assert got == bf["rows"], (trial, got, bf["rows"])
        np.testing.assert_allclose(out["o"][0, 0], bf["o"], rtol=1e-10, atol=1e-12)
        if bf["lse"] == float("-inf"):
            assert out["lse"][0, 0] == float("-inf")
        else:
            assert abs(out["lse"][0, 0] - bf["lse"]) < 1e-10


def pin_brute_multi_query(ref, seed=0):
    """Multi-query top-K == pure-Python brute force per (b, h_q, m), on tiny
    inputs with two KV heads (G = 2), several queries, duplicated key rows
    (exact ties) and split ranges."""
    rng = np.random.default_rng([83, seed])
    for trial in range(6):
        B, Hkv, G, M = int(rng.integers(1, 3)), 2, 2, 3
        n = int(rng.integers(2, 30))
        d = int(rng.integers(1, 7))
        k = rng.standard_normal((B, Hkv, n, d)).astype(np.float32)
        for _ in range(int(rng.integers(0, 5))):
            b, h = int(rng.integers(0, B)), int(rng.integers(0, Hkv))
            i, j = rng.integers(0, n, 2)
            k[b, h, i] = k[b, h, j]
        q = rng.standard_normal((B, Hkv * G, M, d)).astype(np.float32)
        cut = int(rng.integers(0, n + 1))
        ranges = [(0, cut), (cut + 1, n)] if 0 < cut < n - 1 else [(0, n)]
        K = int(rng.integers(1, n + 2))
        sc = float(rng.uniform(0.1, 1.0))
        out = ref.topk_multi_query(q, k, ranges, K, sc)
        rows = [r for b0, e in ranges for r in range(b0, e)]
        for b in range(B):
            for h in range(Hkv * G):
                for m in range(M):
                    kk = [[float(x) for x in k[b, h // G, r]] for r in rows]
                    z = [brute.dot([float(x) for x in q[b, h, m]], row) * sc for row in kk]
                    want = brute.topk_members(z, rows, K)
                    got = [int(x) for x in out["idx"][b, h, m] if x >= 0]
                    assert got == want, (trial, b, h, m, got, want)
                    assert all(int(x) == -1 for x in out["idx"][b, h, m][len(want):])


def pin_brute_gamma(ref, seed=0):
    """The (o, lse) combination equals the pages' gamma_1 o_W + gamma_2 o_Omega
    computed from the raw scores (brute force of Eq. 3-5)."""
    rng = np.random.default_rng([82, seed])
    for trial in range(6):
        n, d = 30, 6
        q = rng.standard_normal((1, 1, d)).astype(np.float32)
        k = (rng.standard_normal((1, 1, n, d)) * 2).astype(np.float32)
        v = rng.standard_normal((1, 1, n, d)).astype(np.float32)
        split = int(rng.integers(1, n))
        a = ref.topk_attn_decode(q, k, v, [(0, split)], n, 0.5)
        b = ref.topk_attn_decode(q, k, v, [(split, n)], n, 0.5)
        o, lse = ref.attn_merge_lse(a["o"], a["lse"], b["o"], b["lse"])
        qq = [float(x) for x in q[0, 0]]
        z = [0.5 * brute.dot(qq, [float(x) for x in k[0, 0, i]]) for i in range(n)]
        vv = [[float(x) for x in v[0, 0, i]] for i in range(n)]
        og, ow, oo, g1, g2 = brute.gamma_combine(z[:split], vv[:split], z[split:], vv[split:], d)
        np.testing.assert_allclose(o[0, 0], og, rtol=1e-10, atol=1e-12)
        assert abs(g1 - math.exp(a["lse"][0, 0] - lse[0, 0])) < 1e-12
        assert abs(g2 - math.exp(b["lse"][0, 0] - lse[0, 0])) < 1e-12


def pin_merge_algebra(ref, seed=0):
    rng = np.random.default_rng([83, seed])
    d = 8
    o = [rng.standard_normal((3, d)) for _ in range(3)]
    l = [rng.standard_normal(3) * 3 for _ in range(3)]
    ninf = np.full(3, -np.inf)
    z = np.zeros((3, d))
    # -inf is the identity
    om, lm = ref.attn_merge_lse(o[0], l[0], z, ninf)
    np.testing.assert_allclose(om, o[0], atol=1e-15)
    np.testing.assert_allclose(lm, l[0], atol=1e-15)
    om, lm = ref.attn_merge_lse(z, ninf, o[1], l[1])
    np.testing.assert_allclose(om, o[1], atol=1e-15)
    # an empty operand is not read: its o may hold anything
    junk = np.full((3, d), np.nan)
    om, lm = ref.attn_merge_lse(junk, ninf, o[1], l[1])
    np.testing.assert_allclose(om, o[1], atol=1e-15)
    # both empty
    om, lm = ref.attn_merge_lse(z, ninf, z, ninf)
    assert np.all(om == 0) and np.all(np.isneginf(lm))
    # commutative, associative
    a1, b1 = ref.attn_merge_lse(*ref.attn_merge_lse(o[0], l[0], o[1], l[1]), o[2], l[2])
    a2, b2 = ref.attn_merge_lse(o[0], l[0], *ref.attn_merge_lse(o[1], l[1], o[2], l[2]))
    np.testing.assert_allclose(a1, a2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(b1, b2, rtol=1e-12, atol=1e-13)
    c1, e1 = ref.attn_merge_lse(o[1], l[1], o[0], l[0])
    c0, e0 = ref.attn_merge_lse(o[0], l[0], o[1], l[1])
    np.testing.assert_allclose(c1, c0, rtol=1e-13, atol=1e-14)
    # lse of the merge is the log-sum-exp of the two (library routine)
    np.testing.assert_allclose(e0, np.logaddexp(l[0], l[1]), rtol=1e-13)


# ---------------------------------------------------------------------------
# ReTopK pins
# ---------------------------------------------------------------------------
def _ar1_setup(seed, n_steps=24, L0=160, d=16, Hq=2, Hkv=1):
    rng = np.random.default_rng([84, seed])
    L_max = L0 + n_steps
    k = rng.standard_normal((1, Hkv, L_max, d)).astype(np.float32)
    v = rng.standard_normal((1, Hkv, L_max, d)).astype(np.float32)
    qs = np.empty((n_steps + 8, 1, Hq, d), np.float32)
    cur = rng.standard_normal((1, Hq, d)).astype(np.float32)
    for t in range(n_steps + 8):
        cur = (0.9 * cur + 0.44 * rng.standard_normal((1, Hq, d))).astype(np.float32)
        qs[t] = cur
    return k, v, qs, L0


def _warm_state(ref, p, k, v, qs, L0, n_warm, sc):
    Hq = qs.shape[2]
    sups = np.stack([ref.topk_attn_decode(qs[j], k, v, [(0, L0)], p.top_k, sc)["idx"] for j in range(n_warm)], axis=2)
    qh = np.stack([qs[j] for j in range(n_warm)], axis=2)
    return ref.retopk_state_init(p, qh, sups)


def pin_retopk_invariants(ref, seed=0):
    """Over an AR(1) query run: the candidate set is ascending, inside
    [0, L_t), holds the recent window and has at most R*K + W rows; every
    step pushes one entry; when the exact top-K is inside the candidates the
    rerank returns it (ReTopK review, 核心方法 1, 3, 4)."""
    k, v, qs, L0 = _ar1_setup(seed)
    sc = 0.25
    p = ref.RetopkParams(top_k=8, cache_cap=6, top_r=2, recent=4, tau=0.2, refresh=10)
    st = _warm_state(ref, p, k, v, qs, L0, 6, sc)
    seen_reuse = 0
    for t in range(20):
        L_t = L0 + t + 1
        out, new, tr = ref.retopk_step(p, st, qs[8 + t], k, v, L_t, t, sc)
        for (b, h), r in tr.items():
            assert int(new.count[b, h]) == min(int(st.count[b, h]) + 1, p.cache_cap)
            assert int(new.head[b, h]) == (int(st.head[b, h]) + 1) % p.cache_cap
            if r["path"] == 0:
                seen_reuse += 1
                c = r["cand"]
                assert np.all(np.diff(c) > 0) and c[0] >= 0 and c[-1] < L_t
                assert c.shape[0] <= p.top_r * p.top_k + p.recent
                assert set(range(L_t - p.recent, L_t)) <= set(int(x) for x in c)
                ex = ref.topk_attn_decode(qs[8 + t][:, h:h + 1], k[:, :1], v[:, :1], [(0, L_t)], p.top_k, sc)
                exact = set(int(x) for x in ex["idx"][0, 0] if x >= 0)
                if exact <= set(int(x) for x in c):
                    assert set(int(x) for x in out["support"][b, h] if x >= 0) == exact
            else:
                assert r["path"] == (2 if t % p.refresh == 0 else 1)
        st = new
    assert seen_reuse > 0


def pin_retopk_special_cases(ref, seed=0):
    """tau > 1 or T_r = 1: every step is exact and equals top-K attention over
    [0, L_t). tau = -2 with no refresh: every step reuses. A recent window
    that covers the whole cache makes reuse equal to exact. After C+1 pushes
    the first entry is gone."""
    k, v, qs, L0 = _ar1_setup(seed, n_steps=8)
    sc = 0.25
    for p in [ref.RetopkParams(top_k=8, cache_cap=4, top_r=2, recent=4, tau=1.5, refresh=0),
              ref.RetopkParams(top_k=8, cache_cap=4, top_r=2, recent=4, tau=-2.0, refresh=1)]:
        st = _warm_state(ref, p, k, v, qs, L0, 4, sc)
        for t in range(5):
            L_t = L0 + t + 1
            out, st, tr = ref.retopk_step(p, st, qs[8 + t], k, v, L_t, t, sc)
            ex = ref.topk_attn_decode(qs[8 + t], k, v, [(0, L_t)], p.top_k, sc)
            assert np.all(out["path"] != 0)
            assert np.array_equal(out["support"], ex["idx"])
            np.testing.assert_allclose(out["o"], ex["o"], rtol=0, atol=1e-14)
    p = ref.RetopkParams(top_k=8, cache_cap=4, top_r=2, recent=4, tau=-2.0, refresh=0)
    st = _warm_state(ref, p, k, v, qs, L0, 4, sc)
    for t in range(5):
        out, st, tr = ref.retopk_step(p, st, qs[8 + t], k, v, L0 + t + 1, t, sc)
        assert np.all(out["path"] == 0)
    p = ref.RetopkParams(top_k=8, cache_cap=4, top_r=1, recent=10 ** 6, tau=-2.0, refresh=0)
    st = _warm_state(ref, p, k, v, qs, L0, 4, sc)
    for t in range(3):
        L_t = L0 + t + 1
        out, st, tr = ref.retopk_step(p, st, qs[8 + t], k, v, L_t, t, sc)
        ex = ref.topk_attn_decode(qs[8 + t], k, v, [(0, L_t)], p.top_k, sc)
        assert np.all(out["path"] == 0)
        assert np.array_equal(out["support"], ex["idx"])
    # FIFO eviction
    p = ref.RetopkParams(top_k=8, cache_cap=3, top_r=1, recent=2, tau=-2.0, refresh=0)
    st = _warm_state(ref, p, k, v, qs, L0, 1, sc)
    first = st.q_hat[0, 0, 0].copy()
    pushed = []
    for t in range(3):
        out, st, tr = ref.retopk_step(p, st, qs[8 + t], k, v, L0 + t + 1, t, sc)
        pushed.append(tr[(0, 0)]["new"][0][tr[(0, 0)]["new"][2]].copy())
    C = p.cache_cap
    live = [st.q_hat[0, 0, (int(st.head[0, 0]) - a) % C] for a in range(int(st.count[0, 0]))]
    assert int(st.count[0, 0]) == C
    assert not any(np.array_equal(x, first) for x in live)
    assert np.array_equal(live[0], pushed[-1])


def pin_retopk_brute(ref, seed=0):
    """Oracle == pure-Python brute force over multi-step runs with every
    combination of refresh / fallback / reuse, skipping steps whose decision
    is within 1e-6 of a tie (the two compute the fp32 cosine in different
    orders)."""
    for variant in range(4):
        k, v, qs, L0 = _ar1_setup(seed * 10 + variant, n_steps=10, L0=40, d=6, Hq=1)
        sc = 0.5
        tau = [0.3, 0.9, -2.0, 0.6][variant]
        T_r = [4, 0, 0, 3][variant]
        p = ref.RetopkParams(top_k=5, cache_cap=4, top_r=2, recent=3, tau=tau, refresh=T_r)
        st = _warm_state(ref, p, k, v, qs, L0, 3, sc)
        C = p.cache_cap
        cache = []
        cnt, hd = int(st.count[0, 0]), int(st.head[0, 0])
        for a in range(cnt - 1, -1, -1):
            s = (hd - a) % C
            cache.append(([float(x) for x in st.q_hat[0, 0, s]], [int(x) for x in st.support[0, 0, s]]))
        kk = [[float(x) for x in row] for row in k[0, 0]]
        vv = [[float(x) for x in row] for row in v[0, 0]]
        for t in range(10):
            L_t = L0 + t + 1
            out, st2, tr = ref.retopk_step(p, st, qs[8 + t], k, v, L_t, t, sc)
            r = tr[(0, 0)]
            bf = brute.retopk_head_step(cache, [float(x) for x in qs[8 + t][0, 0]], kk, vv, L_t, t,
                                        p.top_k, C, p.top_r, p.recent, p.tau, p.refresh, sc)
            rs = r["rho_sorted"]
            near = rs.size and (abs(float(rs[0]) - tau) < 1e-6 or
                                (rs.size > p.top_r and abs(float(rs[p.top_r - 1]) - float(rs[p.top_r])) < 1e-6))
            if not near:
                assert bf["path"] == r["path"], (variant, t)
                if r["path"] == 0:
                    assert bf["cand"] == [int(x) for x in r["cand"]]
                assert bf["support"] == [int(x) for x in out["support"][0, 0]]
                np.testing.assert_allclose(out["o"][0, 0], bf["o"], rtol=1e-10, atol=1e-12)
            st = st2
            # keep the brute cache equal to the oracle's (lock-step)
            C = p.cache_cap
            cnt, hd = int(st.count[0, 0]), int(st.head[0, 0])
            cache[:] = [([float(x) for x in st.q_hat[0, 0, (hd - a) % C]],
                         [int(x) for x in st.support[0, 0, (hd - a) % C]]) for a in range(cnt - 1, -1, -1)]


def pin_retopk_vote(ref):
    """Confidence-voted candidates (ReTopK review, 启发 4-5), worked by hand.
    The current query is 3*e0, so its unit query is e0. Cached unit queries
    (oldest first): e2, (e0+e1)/sqrt2, e0, with cosines 0, 1/sqrt2 and 1; R=2
    recalls the last two. Supports: S_A = {5, 13, 21, 29} (cosine 1) and
    S_B = {2, 5, 8, 13} (cosine 1/sqrt2), so f = 1 + 1/sqrt2 for rows 5 and 13,
    1 for 21 and 29, 1/sqrt2 for 2 and 8. The recent window is {38, 39}.
      budget 3 -> 5, 13, then the lowest of the f = 1 rows: {5, 13, 21};
      budget 5 -> {5, 13, 21, 29, 2} (2 before 8);
      budget 0 or >= 6 -> the whole union."""
    d, L_t, K = 4, 40, 4
    e = np.eye(d, dtype=np.float32)
    q_hist = np.stack([e[2], e[0] + e[1], e[0]])[None, None]  # [1, 1, 3, d]
    sup = np.array([[[30, 31, 32, 33], [2, 5, 8, 13], [5, 13, 21, 29]]], dtype=np.int32)[None]
    rng = np.random.default_rng(3)
    k = rng.standard_normal((1, 1, L_t, d)).astype(np.float32)
    v = rng.standard_normal((1, 1, L_t, d)).astype(np.float32)
    q = (3.0 * e[0])[None, None]
    union = [2, 5, 8, 13, 21, 29, 38, 39]
    want = {3: [5, 13, 21, 38, 39], 5: [2, 5, 13, 21, 29, 38, 39], 0: union, 6: union, 9: union}
    for budget, rows in want.items():
        p = ref.RetopkParams(top_k=K, cache_cap=3, top_r=2, recent=2, tau=-2.0, refresh=0, budget=budget)
        st = ref.retopk_state_init(p, q_hist, sup)
        out, new, tr = ref.retopk_step(p, st, q, k, v, L_t, 1, 0.5)
        r = tr[(0, 0)]
        assert r["path"] == 0
        assert [int(x) for x in r["cand"]] == rows, (budget, r["cand"])
        # the rerank stays exact inside the (capped) candidates
        z = ref.scores(q[0, 0], k[0, 0], np.asarray(rows, dtype=np.int64), 0.5)
        sel, _ = ref.select_topk(z, np.asarray(rows, dtype=np.int64), K)
        assert [int(x) for x in out["support"][0, 0] if x >= 0] == [int(x) for x in sel]


def pin_retopk_vote_brute(ref, seed=0):
    """Oracle == pure-Python brute force with a candidate budget, over
    multi-step runs (budgets below, at and above the union size), skipping
    steps whose recall or vote decision is within 1e-6 of a tie."""
    for variant in range(3):
        k, v, qs, L0 = _ar1_setup(seed * 10 + 5 + variant, n_steps=10, L0=40, d=6, Hq=1)
        sc = 0.5
        budget = [3, 6, 40][variant]
        p = ref.RetopkParams(top_k=5, cache_cap=4, top_r=3, recent=3, tau=-2.0, refresh=0, budget=budget)
        st = _warm_state(ref, p, k, v, qs, L0, 4, sc)
        C = p.cache_cap
        kk = [[float(x) for x in row] for row in k[0, 0]]
        vv = [[float(x) for x in row] for row in v[0, 0]]
        checked = 0
        for t in range(10):
            cnt, hd = int(st.count[0, 0]), int(st.head[0, 0])
            cache = [([float(x) for x in st.q_hat[0, 0, (hd - a) % C]],
                      [int(x) for x in st.support[0, 0, (hd - a) % C]]) for a in range(cnt - 1, -1, -1)]
            L_t = L0 + t + 1
            out, st2, tr = ref.retopk_step(p, st, qs[8 + t], k, v, L_t, t, sc)
            r = tr[(0, 0)]
            bf = brute.retopk_head_step(cache, [float(x) for x in qs[8 + t][0, 0]], kk, vv, L_t, t,
                                        p.top_k, C, p.top_r, p.recent, p.tau, p.refresh, sc, budget=budget)
            rs = r["rho_sorted"]
            near = rs.size > p.top_r and abs(float(rs[p.top_r - 1]) - float(rs[p.top_r])) < 1e-6
            vt = r["vote"]
            if vt is not None and vt["cut"] is not None:
                fc, mc = vt["cut"]
                near = near or bool(np.any((np.abs(vt["f"].astype(np.float64) - fc) < 1e-6) & (vt["mask"] != mc)))
            if not near:
                assert bf["path"] == r["path"] == 0
                assert bf["cand"] == [int(x) for x in r["cand"]], (variant, t)
                assert bf["support"] == [int(x) for x in out["support"][0, 0]]
                checked += 1
            st = st2
        assert checked >= 8


def pin_int8_quantization(ref):
    """Per-row symmetric int8 codes (RetrievalAttention review, "CPU memory
    minimization (Appendix C)"): a row on the integer grid of its scale comes
    back exactly (0.5 * [127, -64, 3, ...] -> scale 0.5 and those integers);
    a zero row gives scale 0; codes lie in [-127, 127], reach +-127 at the
    largest |k|, are odd under k -> -k, and dequantize within half a step;
    the pure-Python quantizer agrees code for code."""
    grid = np.array([127, -64, 3, 0, 1, -1, 2, 5, -127, 100, 64, -3], dtype=np.float32)
    c, s = ref.quantize_keys_int8((0.5 * grid)[None])
    assert float(s[0]) == 0.5 and np.array_equal(c[0].astype(np.int64), grid.astype(np.int64))
    c0, s0 = ref.quantize_keys_int8(np.zeros((1, 12), np.float32))
    assert float(s0[0]) == 0.0 and not np.any(c0)
    rng = np.random.default_rng(21)
    k = (rng.standard_normal((40, 16)) * rng.uniform(0.01, 30, (40, 1))).astype(np.float32)
    k[3, 5] = 0.0
    c, s = ref.quantize_keys_int8(k)
    cn, sn = ref.quantize_keys_int8(-k)
    assert np.array_equal(sn, s) and np.array_equal(cn, -c)
    ci = c.astype(np.int64)
    assert np.all(np.abs(ci) <= 127)
    am = np.argmax(np.abs(k), axis=1)
    assert np.all(np.abs(ci[np.arange(40), am]) == 127)
    err = np.abs(k.astype(np.float64) - s.astype(np.float64)[:, None] * ci)
    assert np.all(err <= 0.5 * s.astype(np.float64)[:, None] * (1 + 1e-6))
    for i in range(40):
        bc, bs = brute.quantize_row_int8([float(x) for x in k[i]])
        assert bs == float(s[i]) and bc == [int(x) for x in ci[i]], i
    # bf16 rows: the codes of the widened values
    kb = (k.view(np.uint32) >> 16).astype(np.uint16)
    cb, sb = ref.quantize_keys_int8(kb)
    cw, sw = ref.quantize_keys_int8((kb.astype(np.uint32) << 16).view(np.float32))
    assert np.array_equal(cb, cw) and np.array_equal(sb, sw)


def pin_int8_recall(ref):
    """The int8 recall stage: with recall_k >= n it is exact top-K attention;
    with keys on the int8 grid (k = s * c exactly) the int8 scores are the
    exact scores, so recall_k = K gives the exact set too; the final set lies
    in the superset and is the exact top-K of it; a pure-Python two-stage
    brute force agrees on small inputs."""
    rng = np.random.default_rng(22)
    d, L = 8, 60
    q = rng.standard_normal((1, 2, d)).astype(np.float32)
    k = rng.standard_normal((1, 1, L, d)).astype(np.float32)
    v = rng.standard_normal((1, 1, L, d)).astype(np.float32)
    ranges = [(3, 25), (30, 58)]
    codes, scales = ref.quantize_keys_int8(k)
    sc = 0.3
    ex = ref.topk_attn_decode(q, k, v, ranges, 6, sc)
    full = ref.topk_attn_decode_int8(q, k, v, codes, scales, ranges, 6, 100, sc)
    assert np.array_equal(full["idx"], ex["idx"])
    np.testing.assert_allclose(full["o"], ex["o"], rtol=0, atol=1e-12)
    # keys on the grid: codes times a power-of-two scale per row
    cg = rng.integers(-127, 128, (1, 1, L, d)).astype(np.float32)
    cg[..., 0] = 127.0
    kg = (cg * np.float32(2.0) ** rng.integers(-4, 3, (1, 1, L, 1))).astype(np.float32)
    cq, sq = ref.quantize_keys_int8(kg)
    assert np.array_equal(cq.astype(np.float32), cg)
    exg = ref.topk_attn_decode(q, kg, v, ranges, 6, sc)
    g6 = ref.topk_attn_decode_int8(q, kg, v, cq, sq, ranges, 6, 6, sc)
    assert np.array_equal(g6["idx"], exg["idx"])
    # nesting, and agreement with the brute force
    r = ref.topk_attn_decode_int8(q, k, v, codes, scales, ranges, 5, 9, sc)
    rows = ref.range_rows(ranges)
    kk = [[float(x) for x in row] for row in k[0, 0]]
    vv = [[float(x) for x in row] for row in v[0, 0]]
    for h in range(2):
        sup = [int(x) for x in r["sup"][0, h] if x >= 0]
        fin = [int(x) for x in r["idx"][0, h] if x >= 0]
        assert len(sup) == 9 and set(fin) <= set(sup)
        z = ref.scores(q[0, h], k[0, 0], np.asarray(sup, dtype=np.int64), sc)
        sel, _ = ref.select_topk(z, np.asarray(sup, dtype=np.int64), 5)
        assert [int(x) for x in sel] == fin
        bf = brute.int8_recall_attention([float(x) for x in q[0, h]], kk, vv, [int(x) for x in rows], 5, 9, sc)
        assert bf["sup"] == sup and bf["rows"] == fin
        np.testing.assert_allclose(r["o"][0, h], bf["o"], rtol=1e-10, atol=1e-12)


ALL_PINS = [
    pin_golden_topk, pin_golden_merge, pin_golden_retopk, pin_dense_matches_library_attention,
    pin_split_merge_identity, pin_shift_invariance, pin_argmax_and_weights, pin_brute_topk,
    pin_brute_gamma, pin_merge_algebra, pin_retopk_invariants, pin_retopk_special_cases,
    pin_retopk_brute, pin_brute_multi_query, pin_retopk_vote, pin_retopk_vote_brute,
    pin_int8_quantization, pin_int8_recall,
]
