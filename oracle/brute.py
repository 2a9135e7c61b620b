"""Pure-Python brute force for tiny shapes — TEST INFRASTRUCTURE ONLY.

An independent second derivation of the same definitions as
``oracle.reference``, written without numpy and in a different form, so that
the two can pin each other on inputs small enough for plain loops
(n <= a few hundred rows, d <= 16):

* membership in the top-K is decided by counting, for each row, how many rows
  beat it (a larger score, or an equal score at a lower row), instead of by
  sorting;
* the softmax uses ``math.fsum`` and the normaliser e^{lse};
* the two-set combination is written with the pages' gamma_1 / gamma_2 of
  RetrievalAttention ("CPU-GPU Co-Execution Architecture", Eq. 4-5), computed
  from the raw scores of both sets rather than from (o, lse) pairs;
* the ReTopK cache is a Python list ordered from oldest to newest instead of
  a ring of slots.

Sources: RetrievalAttention review, "Approximated Attention Formulation"
(Eq. 2) and "CPU-GPU Co-Execution Architecture" (Eq. 3-5); the ReTopK review
"Recall Before You Rank", "核心方法" 1-5.
"""

from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

NEG_INF = float("-inf")


def dot(a: Sequence[float], b: Sequence[float]) -> float:
    return math.fsum(x * y for x, y in zip(a, b))


def topk_members(z: Sequence[float], rows: Sequence[int], k: int) -> List[int]:
    """Rows whose number of 'better' rows is below k, ascending."""
    n = len(z)
    chosen = []
    for i in range(n):
        better = 0
        for j in range(n):
            if z[j] > z[i] or (z[j] == z[i] and rows[j] < rows[i]):
                better += 1
        if better < k:
            chosen.append(rows[i])
    return sorted(chosen)


def attention(zs: Sequence[float], vs: Sequence[Sequence[float]], d: int) -> Tuple[List[float], float]:
    """Softmax-weighted mean of ``vs`` with logits ``zs``; returns (o, lse)."""
    if not zs:
        return [0.0] * d, NEG_INF
    m = max(zs)
    lse = m + math.log(math.fsum(math.exp(z - m) for z in zs))
    o = [math.fsum(math.exp(z - lse) * v[j] for z, v in zip(zs, vs)) for j in range(d)]
    return o, lse


def topk_attention(q: Sequence[float], keys: Sequence[Sequence[float]], values: Sequence[Sequence[float]],
                   rows: Sequence[int], k: int, scale: float) -> Dict:
    """Top-K attention of one query over the listed rows of one head."""
    z = [scale * dot(q, keys[r]) for r in rows]
    chosen = topk_members(z, list(rows), k)
    zmap = {r: zz for r, zz in zip(rows, z)}
    o, lse = attention([zmap[r] for r in chosen], [values[r] for r in chosen], len(q))
    return dict(rows=chosen, o=o, lse=lse, z=z)


def gamma_combine(z_w: Sequence[float], v_w: Sequence[Sequence[float]],
                  z_o: Sequence[float], v_o: Sequence[Sequence[float]], d: int) -> Tuple[List[float], List[float], List[float], float, float]:
    """Eq. 3-5 of the RetrievalAttention review, literally: partial outputs
    with local maxima z~1, z~2, global maximum z~, scaling factors gamma_1,
    gamma_2 and o = gamma_1 o_W + gamma_2 o_Omega. Returns
    (o, o_W, o_Omega, gamma_1, gamma_2). Both sets must be non-empty."""
    z1, z2 = max(z_w), max(z_o)
    zt = max(z1, z2)
    s1 = math.fsum(math.exp(z - z1) for z in z_w)
    s2 = math.fsum(math.exp(z - z2) for z in z_o)
    o_w = [math.fsum(math.exp(z - z1) * v[j] for z, v in zip(z_w, v_w)) / s1 for j in range(d)]
    o_o = [math.fsum(math.exp(z - z2) * v[j] for z, v in zip(z_o, v_o)) / s2 for j in range(d)]
    den = math.fsum([math.exp(z - zt) for z in z_w] + [math.exp(z - zt) for z in z_o])
    g1 = math.exp(z1 - zt) * s1 / den
    g2 = math.exp(z2 - zt) * s2 / den
    return [g1 * a + g2 * b for a, b in zip(o_w, o_o)], o_w, o_o, g1, g2


def unit_f32(q: Sequence[float]):
    """fp32 unit vector, as the oracle and the kernel take this decision in
    fp32; uses numpy only for the fp32 rounding of each operation."""
    import numpy as np
    q32 = np.asarray(q, dtype=np.float32)
    nrm = np.float32(0.0)
    for x in q32:
        nrm = np.float32(nrm + np.float32(x * x))
    nrm = np.float32(np.sqrt(nrm))
    if nrm == 0:
        return [0.0] * len(q)
    return [float(np.float32(x / nrm)) for x in q32]


def retopk_head_step(cache: List[Tuple[List[float], List[int]]], q: Sequence[float],
                     keys: Sequence[Sequence[float]], values: Sequence[Sequence[float]],
                     L_t: int, t: int, K: int, C: int, R: int, W: int, tau: float, T_r: int,
                     scale: float, rho_fn=None, budget: int = 0) -> Dict:
    """One ReTopK step of one head. ``cache`` is a list of (unit query,
    support rows) from oldest to newest, at most C long; it is updated in
    place (append, drop the oldest beyond C)."""
    import numpy as np
    qbar = unit_f32(q)
    rhos = []
    for age, (qc, _) in enumerate(reversed(cache)):
        r = rho_fn(qbar, qc) if rho_fn else float(np.float32(math.fsum(a * b for a, b in zip(qbar, qc))))
        rhos.append((r, age))
    refresh = T_r > 0 and t % T_r == 0
    best = max((r for r, _ in rhos), default=None)
    if refresh:
        path = 2
    elif not cache or np.float32(best) < np.float32(tau):
        path = 1
    else:
        path = 0
    if path == 0:
        ranked = sorted(rhos, key=lambda ra: (-ra[0], ra[1]))[:R]
        newest_first = list(reversed(cache))
        pool = set()
        for _, age in ranked:
            for x in newest_first[age][1]:
                if 0 <= x < L_t:
                    pool.add(x)
        recent = set(range(max(0, L_t - W), L_t))
        if budget > 0:
            # confidence votes: each row of the union collects the cosines of
            # the recalled entries whose support holds it, added one by one
            # in fp32 in recall order
            voted = sorted(pool - recent)
            if len(voted) > budget:
                conf = {}
                for x in voted:
                    f = np.float32(0.0)
                    for r, age in ranked:
                        if x in set(newest_first[age][1]):
                            f = np.float32(f + np.float32(r))
                    conf[x] = float(f)
                best = sorted(voted, key=lambda x: (-conf[x], x))[:budget]
                pool = set(best)
        rows = sorted(pool | recent)
    else:
        rows = list(range(L_t))
    res = topk_attention(q, keys, values, rows, K, scale)
    sup = res["rows"] + [-1] * (K - len(res["rows"]))
    cache.append((qbar, sup))
    while len(cache) > C:
        cache.pop(0)
    return dict(path=path, cand=(rows if path == 0 else None), support=sup, o=res["o"], lse=res["lse"])


def quantize_row_int8(k: Sequence[float]) -> Tuple[List[int], float]:
    """One key row to symmetric int8: scale = max |k| / 127, code = the
    nearest integer to k / scale (halves to even), each step one fp32
    operation; a zero row gives scale 0 and zero codes."""
    import numpy as np
    big = np.float32(0.0)
    for x in k:
        ax = np.float32(abs(np.float32(x)))
        if ax > big:
            big = ax
    s = np.float32(big / np.float32(127.0))
    if s == 0:
        return [0] * len(k), 0.0
    codes = []
    for x in k:
        t = float(np.float32(np.float32(x) / s))
        f = math.floor(t)
        frac = t - f
        c = f + 1 if frac > 0.5 or (frac == 0.5 and f % 2 != 0) else f
        codes.append(int(max(-127, min(127, c))))
    return codes, float(s)


def int8_recall_attention(q: Sequence[float], keys: Sequence[Sequence[float]], values: Sequence[Sequence[float]],
                          rows: Sequence[int], k: int, recall_k: int, scale: float) -> Dict:
    """Two-stage top-K of one head: the recall_k rows of largest score on the
    int8 rows (scale_i * code_i), then top-K attention on the exact keys of
    those rows."""
    q8 = {r: quantize_row_int8(keys[r]) for r in rows}
    z8 = [scale * q8[r][1] * math.fsum(a * b for a, b in zip(q, q8[r][0])) for r in rows]
    sup = topk_members(z8, list(rows), recall_k)
    res = topk_attention(q, keys, values, sup, k, scale)
    res["sup"] = sup
    return res
