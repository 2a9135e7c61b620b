"""Plain fp64 CPU oracle for dynamic top-K sparse decode attention.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the ``cpu_baseline`` leg of ``bench.py``; never by the HIP library or
its binding. It shares no code with them.

Every function follows one passage of the pages and is written out in the
plainest way numpy allows: inputs are widened exactly to fp64, a dot product
is an elementwise product summed along the head dimension (the same summation
for every row, so identical key rows give identical scores), the top-K is a
full lexicographic sort, and the softmax is the textbook max-shifted one.

Sources (cited by page title and section):

* [RA] "RetrievalAttention: Accelerating Long-Context LLM Inference via Vector
  Retrieval" (paper-graph-ui review): section "Approximated Attention
  Formulation" (Eq. 2, renormalised attention over a subset) and section
  "CPU-GPU Co-Execution Architecture" (Eq. 3 partition W u Omega, partial
  outputs with local maxima, Eq. 4-5 rescaled combination).
* [RA-pc] the papercache summary of the same paper: "背景知识" (decode
  attention, Eq. 1) and appendix B.1 (merge formulas).
* [RT] "Recall Before You Rank: Similarity-Guided Top-K Reuse for Efficient
  Long-Context Attention" (blog review): "Exact Top-K 的隐藏成本" (full scan and
  global Top-K), "核心方法" 1-5 (query-support cache, similar-query recall,
  candidate union with the recent window, exact rerank, similarity fallback
  and periodic refresh).

Readings where the pages are silent:

* scale = 1/sqrt(d) with d the head dimension; passed explicitly.
* Top-K ties go to the lowest row index. Index sets are returned ascending,
  padded with -1 up to K.
* K >= n means every row of the range is used (dense attention).
* An empty range gives o = 0 and lse = -inf.
* Query-head h uses KV head h // G (consecutive query heads share a KV head).
* ReTopK's decisions that turn floats into integers (the query norm, the
  cosine rho, the comparison with tau and the top-R order) are taken in fp32,
  the precision of the kernel; the attention itself stays in fp64.
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

NEG_INF = float("-inf")
_ROW_CHUNK = 65536


# --------------------------------------------------------------------------
# exact widening of stored rows
# --------------------------------------------------------------------------
def widen(rows: np.ndarray) -> np.ndarray:
    """Stored key/value rows -> fp64. ``uint16`` arrays hold bf16 bit patterns
    (the upper half of an IEEE fp32); ``float32`` arrays are taken as is.
    Both widenings are exact."""
    if rows.dtype == np.uint16:
        return (rows.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return rows.astype(np.float64)


def range_rows(ranges: Sequence[Tuple[int, int]]) -> np.ndarray:
    """Row indices covered by the half-open ranges, in ascending order."""
    parts = [np.arange(b, e, dtype=np.int64) for b, e in ranges if e > b]
    if not parts:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate(parts)


# --------------------------------------------------------------------------
# step 1: scores  z_i = scale * q . k_i      ([RA-pc] Eq. 1; [RT] exact Top-K)
# --------------------------------------------------------------------------
def scores(q: np.ndarray, key_cache_head: np.ndarray, rows: np.ndarray, scale: float) -> np.ndarray:
    """Pre-softmax logits of query ``q`` (length d) against the given rows of
    one KV head's cache ``[L_max, d]``, in fp64."""
    qd = np.asarray(q, dtype=np.float64)
    out = np.empty(rows.shape[0], dtype=np.float64)
    for s in range(0, rows.shape[0], _ROW_CHUNK):
        r = rows[s:s + _ROW_CHUNK]
        kr = widen(key_cache_head[r])
        out[s:s + r.shape[0]] = (kr * qd[None, :]).sum(axis=1) * scale
    return out


# --------------------------------------------------------------------------
# step 2: top-K selection   ([RT] S_t = TopK(e, K); ties -> lowest index)
# --------------------------------------------------------------------------
def select_topk(z: np.ndarray, rows: np.ndarray, k: int) -> Tuple[np.ndarray, float]:
    """Rows of the K largest scores, ties broken towards the lowest row.

    Returns the chosen rows sorted ascending and the K-th largest score
    (-inf when nothing is chosen). With K >= n every row is chosen."""
    n = z.shape[0]
    if n == 0 or k <= 0:
        return np.zeros(0, dtype=np.int64), NEG_INF
    order = np.lexsort((rows, -z))  # primary: z descending, secondary: row ascending
    take = order[:min(k, n)]
    return np.sort(rows[take]), float(z[take[-1]])


# --------------------------------------------------------------------------
# step 3: renormalised softmax . V over the chosen rows    ([RA] Eq. 2)
# --------------------------------------------------------------------------
def softmax_v(z_sel: np.ndarray, v_sel: np.ndarray) -> Tuple[np.ndarray, float]:
    """o = sum_i e^{z_i - m} v_i / sum_i e^{z_i - m}, lse = m + ln sum_i e^{z_i - m}
    with m the largest chosen score ([RA] "CPU-GPU Co-Execution
    Architecture": partial output with a local maximum)."""
    d = v_sel.shape[1] if v_sel.ndim == 2 else 0
    if z_sel.shape[0] == 0:
        return np.zeros(d, dtype=np.float64), NEG_INF
    m = float(np.max(z_sel))
    w = np.exp(z_sel - m)
    s = float(np.sum(w))
    o = (w[:, None] * v_sel).sum(axis=0) / s
    return o, m + math.log(s)


def pad_rows(sel: np.ndarray, k: int) -> np.ndarray:
    out = np.full(k, -1, dtype=np.int32)
    out[:sel.shape[0]] = sel
    return out


def attend_rows(q: np.ndarray, kc_head: np.ndarray, vc_head: np.ndarray, rows: np.ndarray,
                top_k: int, scale: float) -> Dict:
    """One query head: scores over ``rows``, top-K, renormalised softmax . V."""
    z = scores(q, kc_head, rows, scale)
    sel, zk = select_topk(z, rows, top_k)
    pos = np.searchsorted(rows, sel) if rows.shape[0] and np.all(np.diff(rows) > 0) else None
    if pos is None:
        lut = {int(r): i for i, r in enumerate(rows)}
        pos = np.array([lut[int(r)] for r in sel], dtype=np.int64)
    z_sel = z[pos]
    v_sel = widen(vc_head[sel]) if sel.shape[0] else np.zeros((0, vc_head.shape[-1]))
    o, lse = softmax_v(z_sel, v_sel)
    return dict(rows=sel, z=z, zk=zk, o=o, lse=lse)


def topk_attn_decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                     ranges: Sequence[Tuple[int, int]], top_k: int, scale: float,
                     heads: Optional[Sequence[Tuple[int, int]]] = None) -> Dict:
    """Top-K attention of every query head over the union of ``ranges``.

    q: [B, H_q, d] fp32. k_cache/v_cache: [B, H_kv, L_max, d] (bf16 bits or
    fp32). Returns idx [B, H_q, K] (ascending rows, -1 padded), o [B, H_q, d],
    lse [B, H_q] (fp64) and zk [B, H_q] (the K-th score). ``heads`` restricts
    the work to the listed (b, h_q) pairs (the other entries stay NaN / -2).
    """
    B, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    rows = range_rows(ranges)
    K = int(top_k)
    idx = np.full((B, Hq, K), -2, dtype=np.int32)
    o = np.full((B, Hq, d), np.nan)
    lse = np.full((B, Hq), np.nan)
    zk = np.full((B, Hq), np.nan)
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    for b, h in todo:
        hk = h // G
        r = attend_rows(q[b, h], k_cache[b, hk], v_cache[b, hk], rows, K, scale)
        idx[b, h] = pad_rows(r["rows"], K)
        o[b, h] = r["o"]
        lse[b, h] = r["lse"]
        zk[b, h] = r["zk"]
    return dict(idx=idx, o=o, lse=lse, zk=zk)


# --------------------------------------------------------------------------
# int8 keys as a recall stage ([RA] "CPU memory minimization (Appendix C)":
# 8-bit scalar quantization of the key vectors, scheme left open; the review
# asks whether quantized keys shift the nearest-key rankings, so here the
# int8 scores only choose a superset and the exact scores decide inside it)
# --------------------------------------------------------------------------
def quantize_keys_int8(rows: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-row symmetric int8 codes of stored key rows [..., d] (bf16 bits or
    fp32). Reading (the pages give no scheme): s = max_j |k_j| / 127 and
    c_j = round-half-even(k_j / s), both one correctly rounded fp32 operation,
    clamped to [-127, 127]; a row of zeros has s = 0 and codes 0. Returns
    (codes int8 [..., d], scales float32 [...])."""
    k = widen(rows).astype(np.float32)  # exact: bf16 and fp32 values are fp32
    maxabs = np.max(np.abs(k), axis=-1).astype(np.float32)
    s = (maxabs / np.float32(127.0)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    c = np.rint((k / safe[..., None]).astype(np.float32))
    c = np.clip(c, -127, 127)
    c = np.where((s > 0)[..., None], c, 0)
    return c.astype(np.int8), s


def int8_scores(q: np.ndarray, codes_head: np.ndarray, scales_head: np.ndarray, rows: np.ndarray,
                scale: float) -> np.ndarray:
    """Scores of q against the dequantized rows s_i * c_i, in fp64."""
    qd = np.asarray(q, dtype=np.float64)
    out = np.empty(rows.shape[0], dtype=np.float64)
    for a in range(0, rows.shape[0], _ROW_CHUNK):
        r = rows[a:a + _ROW_CHUNK]
        c = codes_head[r].astype(np.float64)
        out[a:a + r.shape[0]] = (c * qd[None, :]).sum(axis=1) * scales_head[r].astype(np.float64) * scale
    return out


def topk_attn_decode_int8(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, codes: np.ndarray,
                          scales: np.ndarray, ranges: Sequence[Tuple[int, int]], top_k: int, recall_k: int,
                          scale: float, heads: Optional[Sequence[Tuple[int, int]]] = None) -> Dict:
    """Top-K attention with an int8 recall stage: S' = the recall_k rows of
    largest int8 score (ties to the lowest row), then S = the top_k rows of
    largest exact score inside S' (ties to the lowest row), then the
    renormalised softmax . V over S ([RA] Eq. 2). codes [B, H_kv, L_max, d]
    int8 and scales [B, H_kv, L_max] as quantize_keys_int8 gives them.
    Returns idx [B, H_q, K], the superset sup [B, H_q, K'] (both ascending,
    -1 padded), o, lse and zk8 (the K'-th int8 score)."""
    B, Hq, d = q.shape
    G = Hq // k_cache.shape[1]
    rows = range_rows(ranges)
    K, K2 = int(top_k), int(recall_k)
    idx = np.full((B, Hq, K), -2, dtype=np.int32)
    sup = np.full((B, Hq, K2), -2, dtype=np.int32)
    o = np.full((B, Hq, d), np.nan)
    lse = np.full((B, Hq), np.nan)
    zk8 = np.full((B, Hq), np.nan)
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    for b, h in todo:
        hk = h // G
        z8 = int8_scores(q[b, h], codes[b, hk], scales[b, hk], rows, scale)
        s8, zk8[b, h] = select_topk(z8, rows, K2)
        r = attend_rows(q[b, h], k_cache[b, hk], v_cache[b, hk], s8, K, scale)
        sup[b, h] = pad_rows(s8, K2)
        idx[b, h] = pad_rows(r["rows"], K)
        o[b, h] = r["o"]
        lse[b, h] = r["lse"]
    return dict(idx=idx, sup=sup, o=o, lse=lse, zk8=zk8)


# --------------------------------------------------------------------------
# multi-query exact top-K: the index sets of a block of queries, each the
# exact TopK of its own scores over the ranges ([RT] "Exact Top-K 的隐藏成本":
# S_t = TopK(e, K); "核心方法" 1: the cache holds the supports of the last
# prefill queries; [RA] "CPU-GPU Co-Execution Architecture": the key index is
# built from the prefill queries' nearest keys)
# --------------------------------------------------------------------------
def topk_multi_query(q: np.ndarray, k_cache: np.ndarray, ranges: Sequence[Tuple[int, int]], top_k: int,
                     scale: float, queries: Optional[Sequence[Tuple[int, int, int]]] = None) -> Dict:
    """q: [B, H_q, M, d] fp32. Returns idx [B, H_q, M, K] (ascending rows, -1
    padded) and zk [B, H_q, M] (the K-th score). ``queries`` restricts the
    work to the listed (b, h_q, m) triples (the other entries stay -2 / NaN)."""
    B, Hq, M, d = q.shape
    G = Hq // k_cache.shape[1]
    rows = range_rows(ranges)
    K = int(top_k)
    idx = np.full((B, Hq, M, K), -2, dtype=np.int32)
    zk = np.full((B, Hq, M), np.nan)
    todo = queries if queries is not None else [(b, h, m) for b in range(B) for h in range(Hq) for m in range(M)]
    for b, h, m in todo:
        z = scores(q[b, h, m], k_cache[b, h // G], rows, scale)
        sel, zk[b, h, m] = select_topk(z, rows, K)
        idx[b, h, m] = pad_rows(sel, K)
    return dict(idx=idx, zk=zk)


# --------------------------------------------------------------------------
# combination of two partial outputs   ([RA] Eq. 4-5; [RA-pc] appendix B.1)
# --------------------------------------------------------------------------
def attn_merge_lse(o_a: np.ndarray, lse_a: np.ndarray, o_b: np.ndarray, lse_b: np.ndarray):
    """o = g_a o_a + g_b o_b with g_j = e^{lse_j - lse} and
    lse = M + ln(e^{lse_a - M} + e^{lse_b - M}), M = max(lse_a, lse_b).

    g_j equals the pages' gamma_j: e^{z~_j - z~} times the set's partial
    denominator over the joint denominator, since lse_j = z~_j + ln(partial
    denominator). An operand with lse = -inf contributes nothing; two such
    operands give o = 0, lse = -inf. Rows are the leading dimensions."""
    o_a = np.asarray(o_a, dtype=np.float64)
    o_b = np.asarray(o_b, dtype=np.float64)
    la = np.asarray(lse_a, dtype=np.float64)
    lb = np.asarray(lse_b, dtype=np.float64)
    M = np.maximum(la, lb)
    both_empty = np.isneginf(M)
    Ms = np.where(both_empty, 0.0, M)
    ea = np.where(np.isneginf(la), 0.0, np.exp(la - Ms))
    eb = np.where(np.isneginf(lb), 0.0, np.exp(lb - Ms))
    tot = ea + eb
    lse = np.where(both_empty, NEG_INF, Ms + np.log(np.where(both_empty, 1.0, tot)))
    ga = np.where(both_empty, 0.0, ea / np.where(both_empty, 1.0, tot))
    gb = np.where(both_empty, 0.0, eb / np.where(both_empty, 1.0, tot))
    # a set with weight 0 (lse = -inf) is not used at all, whatever its o holds
    ta = np.where(ga[..., None] == 0.0, 0.0, ga[..., None] * o_a)
    tb = np.where(gb[..., None] == 0.0, 0.0, gb[..., None] * o_b)
    return ta + tb, lse


# --------------------------------------------------------------------------
# ReTopK   ([RT] 核心方法 1-5)
# --------------------------------------------------------------------------
PATH_REUSE, PATH_FALLBACK, PATH_REFRESH = 0, 1, 2


@dataclass
class RetopkParams:
    top_k: int = 512        # K
    cache_cap: int = 32     # C, FIFO capacity per query head
    top_r: int = 4          # R, recalled cache entries
    recent: int = 32        # W, recent rows always added to the candidates
    tau: float = 0.85       # similarity threshold of the fallback
    refresh: int = 128      # T_r; 0 disables the periodic refresh
    budget: int = 0         # voted rows kept on the reuse path; 0 = the whole union


@dataclass
class RetopkState:
    """Per query head FIFO: q_hat [B,H_q,C,d] fp32 (unit queries), support
    [B,H_q,C,K] int32 (ascending rows, -1 padded), head [B,H_q] (slot of the
    newest entry), count [B,H_q] (valid entries)."""
    q_hat: np.ndarray
    support: np.ndarray
    head: np.ndarray
    count: np.ndarray

    def copy(self) -> "RetopkState":
        return RetopkState(self.q_hat.copy(), self.support.copy(), self.head.copy(), self.count.copy())


def unit_query_f32(q: np.ndarray) -> np.ndarray:
    """q / ||q||_2 in fp32 (a zero query stays zero)."""
    q32 = np.asarray(q, dtype=np.float32)
    nrm = np.sqrt(np.sum(q32 * q32, dtype=np.float32), dtype=np.float32)
    if nrm == 0:
        return np.zeros_like(q32)
    return (q32 / nrm).astype(np.float32)


def retopk_state_init(p: RetopkParams, q_hist: np.ndarray, sup_hist: np.ndarray) -> RetopkState:
    """Fill each head's cache with its last min(n, C) exact-path (query,
    support) pairs, oldest first ([RT] 核心方法 1: the cache starts from the
    last C prefill queries). q_hist [B,H_q,n,d]; sup_hist [B,H_q,n,K]."""
    B, Hq, n, d = q_hist.shape
    C, K = p.cache_cap, p.top_k
    st = RetopkState(np.zeros((B, Hq, C, d), np.float32), np.full((B, Hq, C, K), -1, np.int32),
                     np.full((B, Hq), C - 1, np.int32), np.zeros((B, Hq), np.int32))
    m = min(n, C)
    for b in range(B):
        for h in range(Hq):
            for j in range(m):
                src = n - m + j
                st.q_hat[b, h, j] = unit_query_f32(q_hist[b, h, src])
                st.support[b, h, j] = sup_hist[b, h, src]
            st.head[b, h] = (m - 1) % C if m > 0 else C - 1
            st.count[b, h] = m
    return st


def vote_candidates(union_rows: np.ndarray, recent_rows: np.ndarray, supports: Sequence[np.ndarray],
                    weights: Sequence[np.float32], budget: int) -> Tuple[np.ndarray, Dict]:
    """Confidence-voted candidate set ([RT] "启发 4": the access confidence of
    row i is f(i) = sum over the recalled entries c of w_c * [i in S_c]; the
    high-confidence rows are read first under a candidate budget, 启发 5).

    Readings: w_c is the recalled entry's cosine rho_c; f is summed in fp32
    in recall-rank order (``supports`` / ``weights`` in that order); the
    recent window is always kept (the recent guard of 核心方法 3) and the
    budget applies to the other rows of the union: when more than ``budget``
    of them exist, the ``budget`` rows of largest f are kept, ties to the
    lowest row. Returns the ascending candidate rows and a trace (f and the
    membership mask of every voted row, in ascending row order)."""
    recent_rows = np.asarray(recent_rows, dtype=np.int64)
    voted = np.setdiff1d(np.asarray(union_rows, dtype=np.int64), recent_rows)
    f = np.zeros(voted.shape[0], dtype=np.float32)
    mask = np.zeros(voted.shape[0], dtype=np.int64)
    for r, (sup, w) in enumerate(zip(supports, weights)):
        mem = np.isin(voted, np.asarray(sup, dtype=np.int64))
        f = np.where(mem, (f + np.float32(w)).astype(np.float32), f)
        mask |= mem.astype(np.int64) << r
    trace = dict(voted=voted, f=f, mask=mask, cut=None)
    if budget <= 0 or voted.shape[0] <= budget:
        return np.union1d(voted, recent_rows), trace
    order = np.lexsort((voted, -f.astype(np.float64)))  # f descending, then row ascending
    keep = voted[order[:budget]]
    trace["cut"] = (float(f[order[budget - 1]]), int(mask[order[budget - 1]]))
    return np.union1d(keep, recent_rows), trace


def retopk_head_step(p: RetopkParams, q_hat: np.ndarray, support: np.ndarray, head: int, count: int,
                     q: np.ndarray, kc_head: np.ndarray, vc_head: np.ndarray, L_t: int, t: int,
                     scale: float) -> Dict:
    """One decode step of one query head, from the definitions of [RT]
    "核心方法": the cosines rho_{t,c} = qbar_t . qbar_c against the valid
    entries of the head's FIFO B_t (sections 1-2); the two guards of section
    5 (a refresh every T_r steps, or the best rho_{t,c} below tau) choose
    the exact path; otherwise the candidate set A_t = Unique(union of the
    supports S^_c of the R most similar entries, and the recent window L_t
    of the W newest rows), with M_t = |A_t| <= R*K + W (section 3); the
    support S^_t = TopK over A_t of e^_{t,i} = q_t . k_i / sqrt(d) (section
    4), or over all L_t rows on the exact path; renormalised softmax . V
    over S^_t ([RA] Eq. 2); and (qbar_t, S^_t) entering B_t on either path
    (section 1).

    Returns the outputs and the updated (q_hat, support, head, count)."""
    C, K, R, W = p.cache_cap, p.top_k, p.top_r, p.recent
    qbar = unit_query_f32(q)
    # rho_{t,c} = qbar_t . qbar_c over the valid entries of B_t ([RT] 核心方法 2), fp32
    ages = np.array([(head - s) % C for s in range(C)], dtype=np.int64)
    valid = np.nonzero(ages < count)[0]
    rho = (q_hat[valid].astype(np.float32) @ qbar.astype(np.float32)).astype(np.float32) if valid.size else np.zeros(0, np.float32)
    rho_of_slot = np.full(C, -np.inf, dtype=np.float32)
    rho_of_slot[valid] = rho
    order = valid[np.lexsort((ages[valid], -rho.astype(np.float64)))] if valid.size else valid
    rho_sorted = np.sort(rho)[::-1]
    max_rho = float(rho_sorted[0]) if rho_sorted.size else float("nan")
    # the two guards of [RT] 核心方法 5: periodic refresh, similarity fallback
    refresh = p.refresh > 0 and (t % p.refresh) == 0
    if refresh:
        path = PATH_REFRESH
    elif count == 0 or np.float32(max_rho) < np.float32(p.tau):
        path = PATH_FALLBACK
    else:
        path = PATH_REUSE
    cand = None
    vote = None
    if path == PATH_REUSE:
        picked = order[:min(R, count)]
        parts = [support[s][(support[s] >= 0) & (support[s] < L_t)].astype(np.int64) for s in picked]
        recent = np.arange(max(0, L_t - W), L_t, dtype=np.int64)  # L_t, the W newest rows ([RT] 核心方法 3)
        if p.budget > 0:
            union = np.unique(np.concatenate(parts)) if parts else np.zeros(0, np.int64)
            cand, vote = vote_candidates(union, recent, parts, [rho_of_slot[s] for s in picked], p.budget)
        else:
            cand = np.unique(np.concatenate(parts + [recent]))  # A_t ([RT] 核心方法 3)
        rows = cand
    else:
        rows = np.arange(0, L_t, dtype=np.int64)
    r = attend_rows(q, kc_head, vc_head, rows, K, scale)  # S^_t = TopK of e^_{t,i} over A_t ([RT] 核心方法 4), or over all rows
    sup = pad_rows(r["rows"], K)
    # (qbar_t, S^_t) enters the FIFO on either path ([RT] 核心方法 1)
    q_hat = q_hat.copy()
    support = support.copy()
    slot = (head + 1) % C
    q_hat[slot] = qbar
    support[slot] = sup
    return dict(path=path, cand=cand, n_cand=(cand.shape[0] if cand is not None else L_t),
                support=sup, o=r["o"], lse=r["lse"], zk=r["zk"], z=r["z"], rows=rows,
                rho_sorted=rho_sorted, max_rho=max_rho, picked=(order[:min(R, count)] if path == PATH_REUSE else None),
                vote=vote,
                new=(q_hat, support, slot, min(count + 1, C)))


def retopk_step(p: RetopkParams, st: RetopkState, q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                L_t: int, t: int, scale: float, heads: Optional[Sequence[Tuple[int, int]]] = None):
    """One ReTopK decode step for every (b, h_q). q: [B,H_q,d] fp32. Returns
    (outputs, new_state, per-head traces)."""
    B, Hq, d = q.shape
    G = Hq // k_cache.shape[1]
    K = p.top_k
    new = st.copy()
    out = dict(support=np.full((B, Hq, K), -2, np.int32), o=np.full((B, Hq, d), np.nan),
               lse=np.full((B, Hq), np.nan), path=np.full((B, Hq), -1, np.int32),
               n_cand=np.full((B, Hq), -1, np.int64))
    traces = {}
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    for b, h in todo:
        hk = h // G
        r = retopk_head_step(p, st.q_hat[b, h], st.support[b, h], int(st.head[b, h]), int(st.count[b, h]),
                             q[b, h], k_cache[b, hk], v_cache[b, hk], L_t, t, scale)
        out["support"][b, h] = r["support"]
        out["o"][b, h] = r["o"]
        out["lse"][b, h] = r["lse"]
        out["path"][b, h] = r["path"]
        out["n_cand"][b, h] = r["n_cand"]
        qh, sp, hd, ct = r["new"]
        new.q_hat[b, h], new.support[b, h], new.head[b, h], new.count[b, h] = qh, sp, hd, ct
        traces[(b, h)] = r
    return out, new, traces
