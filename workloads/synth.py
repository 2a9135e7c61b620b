"""Seeded synthetic workloads for dynamic top-K sparse decode attention.

Five workloads stand in for the pages' settings (no model weights or datasets
are used). Every tensor is drawn from ``numpy.random.default_rng`` with a seed
list ``[1000 + cfg, tensor_id, stream, chunk]`` so that any 65,536-row chunk
can be regenerated on its own, in bounded memory, and in parallel threads.

Tensor ids: 0 = keys, 1 = values, 2 = queries, 3 = per-head / per-sequence
offsets and other side draws.

bf16 tensors are returned as ``uint16`` bit patterns produced by
round-to-nearest-even from the fp32 draw; fp32 tensors as ``float32``.
Nothing here computes attention: the generator only draws and lays out data.

Workloads (sizes are the defaults; ``L`` may be overridden for reduced-size
parity runs, which keeps every distribution and only changes the length):

1. ``c1`` one query head / one KV head, d=128, L=4096, fp32, K=64. Keys and
   values N(0,1). The query is 0.3*x + 0.7*A*m with x ~ N(0,1), m the mean of
   16 distinct random keys and A a fixed random orthogonal matrix (Q factor of
   the QR of an N(0,1) matrix, signs fixed by diag(R)).
2. ``c2`` Llama-3-8B-shaped layer: 32 q heads, 8 KV heads, d=128, L=131072,
   bf16. Keys N(0,1) plus one mean offset per KV head drawn from N(0, 2 I)
   (variance 2). Values N(0,1). Queries N(0,1) fp32. K=2048. The static set is
   the first 128 and the last 512 rows; the dynamic set is the rest.
3. ``c3`` Qwen2.5-7B-shaped ReTopK run: 28 q heads, 4 KV heads, d=128,
   L0=65536, bf16 keys/values N(0,1); 32 warm-up + 256 step queries per head
   from the AR(1) chain q_t = 0.95 q_{t-1} + 0.31 eps_t, q_0 ~ N(0,1). The
   cache holds L0 + 256 rows; step t sees L_t = L0 + t + 1 rows.
4. ``c4`` batch 16 x 32768 rows, 32 q / 8 KV heads, bf16, keys N(0,1) plus one
   offset per sequence from N(0, I) shared by its KV heads, K=1024.
5. ``c5`` one 1,048,576-row sequence, 32 q / 8 KV heads, bf16 N(0,1). For
   every q head, 64 distinct rows of the dynamic set (disjoint between the
   heads of one KV group) are planted as 4*q_dir + N(0, 0.5 I) (variance 0.5),
   with q_dir the unit query direction. K=8192 plus the 640-row static set.

Blocks of queries for the multi-query top-K (``make_multi_query``): the c3
prefill block is c3's 32 warm-up queries of every head over its L0 rows
(K=512). Reduced shapes draw keys N(0,1) plus one offset per (sequence, KV
head) from N(0, I), queries N(0,1) fp32, with the seed id 6; ``codebook`` > 0
draws every key row from that many N(0,1) rows instead (exact score ties).
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

CHUNK_ROWS = 65536
HEAD_DIM = 128

T_KEY, T_VALUE, T_QUERY, T_SIDE = 0, 1, 2, 3


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even) and return the uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
    return r.astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def static_window_ranges(L: int, n_sink: int = 128, n_local: int = 512) -> Tuple[List[Tuple[int, int]], List[Tuple[int, int]]]:
    """Index ranges of the static set (first ``n_sink`` + last ``n_local`` rows)
    and of the dynamic set (everything else), as half-open [begin, end) pairs.

    For short caches the two static pieces are clipped so that they never
    overlap: static = [0, min(n_sink, L)) U [max(n_sink, L - n_local), L).
    """
    a_end = min(n_sink, L)
    b_beg = max(n_sink, L - n_local)
    static = [(0, a_end)]
    if b_beg < L:
        static.append((b_beg, L))
    dynamic = [(a_end, b_beg)] if b_beg > a_end else []
    static = [r for r in static if r[1] > r[0]]
    return static, dynamic


def _threads() -> int:
    n = os.cpu_count() or 4
    return max(1, min(16, n))


def _normal_rows(seed: List[int], rows: int, d: int = HEAD_DIM) -> np.ndarray:
    return np.random.default_rng(seed).standard_normal((rows, d), dtype=np.float32)


@dataclass
class Workload:
    """One synthetic workload, as host arrays.

    ``q``: float32 [B, H_q, d] (for c3: [B, H_q, 32 + steps, d], the query
    sequence). ``k``/``v``: [B, H_kv, L_max, d] as uint16 bf16 bits or float32.
    """

    name: str
    cfg: int
    B: int
    H_q: int
    H_kv: int
    d: int
    L: int
    L_max: int
    kv_dtype: str  # "bf16" or "f32"
    top_k: int
    scale: float
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    ranges: List[Tuple[int, int]]
    static_ranges: List[Tuple[int, int]] = field(default_factory=list)
    retopk: Optional[Dict] = None
    planted: Optional[np.ndarray] = None  # c5: [H_q, 64] planted row indices
    note: str = ""

    @property
    def G(self) -> int:
        return self.H_q // self.H_kv


def _fill_kv(cfg: int, B: int, H_kv: int, L_max: int, dtype: str,
             offsets: Optional[np.ndarray] = None,
             offset_per_batch: bool = False,
             planted: Optional[Dict[Tuple[int, int], Tuple[np.ndarray, np.ndarray]]] = None):
    """Draw keys and values chunk by chunk.

    ``offsets``: per (b, h_kv) or per b mean vectors added to the keys.
    ``planted``: {(b, h_kv): (rows, key_rows_f32)} rows overwritten after the
    offset is added.
    """
    store = np.uint16 if dtype == "bf16" else np.float32
    k = np.empty((B, H_kv, L_max, HEAD_DIM), dtype=store)
    v = np.empty((B, H_kv, L_max, HEAD_DIM), dtype=store)
    jobs = []
    for b in range(B):
        for h in range(H_kv):
            stream = b * H_kv + h
            for c0 in range(0, L_max, CHUNK_ROWS):
                jobs.append((b, h, stream, c0))

    def work(job):
        b, h, stream, c0 = job
        rows = min(CHUNK_ROWS, L_max - c0)
        chunk = c0 // CHUNK_ROWS
        kk = _normal_rows([1000 + cfg, T_KEY, stream, chunk], rows)
        if offsets is not None:
            kk += offsets[b] if offset_per_batch else offsets[b, h]
        if planted is not None and (b, h) in planted:
            prow, pval = planted[(b, h)]
            sel = (prow >= c0) & (prow < c0 + rows)
            if np.any(sel):
                kk[prow[sel] - c0] = pval[sel]
        vv = _normal_rows([1000 + cfg, T_VALUE, stream, chunk], rows)
        if dtype == "bf16":
            k[b, h, c0:c0 + rows] = bf16_bits_from_f32(kk)
            v[b, h, c0:c0 + rows] = bf16_bits_from_f32(vv)
        else:
            k[b, h, c0:c0 + rows] = kk
            v[b, h, c0:c0 + rows] = vv

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, jobs))
    return k, v


def _c1(L: int) -> Workload:
    cfg = 1
    side = np.random.default_rng([1000 + cfg, T_SIDE, 0, 0])
    k, v = _fill_kv(cfg, 1, 1, L, "f32")
    g = side.standard_normal((HEAD_DIM, HEAD_DIM))
    qm, rm = np.linalg.qr(g)
    qm = qm * np.sign(np.diag(rm))[None, :]
    picks = side.choice(L, size=16, replace=False)
    m = k[0, 0, picks].astype(np.float64).mean(axis=0)
    x = np.random.default_rng([1000 + cfg, T_QUERY, 0, 0]).standard_normal(HEAD_DIM)
    q = (0.3 * x + 0.7 * (qm @ m)).astype(np.float32)[None, None, :]
    return Workload("c1_fp32_L4096_K64", cfg, 1, 1, 1, HEAD_DIM, L, L, "f32", min(64, L),
                    1.0 / math.sqrt(HEAD_DIM), q, k, v, [(0, L)],
                    note="query shifted away from the key distribution by a fixed rotation")


def _c2(L: int) -> Workload:
    cfg, B, Hq, Hkv = 2, 1, 32, 8
    side = np.random.default_rng([1000 + cfg, T_SIDE, 0, 0])
    mu = (side.standard_normal((B, Hkv, HEAD_DIM)) * math.sqrt(2.0)).astype(np.float32)
    k, v = _fill_kv(cfg, B, Hkv, L, "bf16", offsets=mu)
    q = np.random.default_rng([1000 + cfg, T_QUERY, 0, 0]).standard_normal((B, Hq, HEAD_DIM), dtype=np.float32)
    static, dynamic = static_window_ranges(L)
    return Workload(f"c2_llama3_8b_L{L}_K2048", cfg, B, Hq, Hkv, HEAD_DIM, L, L, "bf16", 2048,
                    1.0 / math.sqrt(HEAD_DIM), q, k, v, dynamic, static_ranges=static)


def _c3(L: int, steps: int = 256, warm: int = 32, B: int = 1) -> Workload:
    """B > 1: independent requests (their own query streams and K/V rows),
    one ReTopK cache per (request, query head)."""
    cfg, Hq, Hkv = 3, 28, 4
    L_max = L + steps
    k, v = _fill_kv(cfg, B, Hkv, L_max, "bf16")
    rng = np.random.default_rng([1000 + cfg, T_QUERY, 0, 0])
    n = warm + steps
    eps = rng.standard_normal((n, B, Hq, HEAD_DIM), dtype=np.float32)
    seq = np.empty((B, Hq, n, HEAD_DIM), dtype=np.float32)
    cur = eps[0]
    seq[:, :, 0] = cur
    for t in range(1, n):
        cur = (np.float32(0.95) * cur + np.float32(0.31) * eps[t]).astype(np.float32)
        seq[:, :, t] = cur
    params = dict(top_k=512, cache_cap=32, top_r=4, recent=32, tau=0.85, refresh=128,
                  warmup=warm, steps=steps, L0=L)
    name = f"c3_qwen25_7b_retopk_L{L}" + (f"_B{B}" if B > 1 else "")
    return Workload(name, cfg, B, Hq, Hkv, HEAD_DIM, L, L_max, "bf16", 512,
                    1.0 / math.sqrt(HEAD_DIM), seq, k, v, [(0, L)], retopk=params)


def _c4(L: int, B: int = 16) -> Workload:
    cfg, Hq, Hkv = 4, 32, 8
    side = np.random.default_rng([1000 + cfg, T_SIDE, 0, 0])
    mu = side.standard_normal((B, HEAD_DIM)).astype(np.float32)
    k, v = _fill_kv(cfg, B, Hkv, L, "bf16", offsets=mu, offset_per_batch=True)
    q = np.random.default_rng([1000 + cfg, T_QUERY, 0, 0]).standard_normal((B, Hq, HEAD_DIM), dtype=np.float32)
    return Workload(f"c4_batch{B}_L{L}_K1024", cfg, B, Hq, Hkv, HEAD_DIM, L, L, "bf16", 1024,
                    1.0 / math.sqrt(HEAD_DIM), q, k, v, [(0, L)])


def _c5(L: int, top_k: int = 8192, n_plant: int = 64) -> Workload:
    cfg, B, Hq, Hkv = 5, 1, 32, 8
    G = Hq // Hkv
    q = np.random.default_rng([1000 + cfg, T_QUERY, 0, 0]).standard_normal((B, Hq, HEAD_DIM), dtype=np.float32)
    static, dynamic = static_window_ranges(L)
    lo, hi = dynamic[0]
    side = np.random.default_rng([1000 + cfg, T_SIDE, 0, 0])
    planted_rows = np.empty((Hq, n_plant), dtype=np.int64)
    planted: Dict[Tuple[int, int], Tuple[np.ndarray, np.ndarray]] = {}
    for h in range(Hkv):
        rows = lo + side.choice(hi - lo, size=G * n_plant, replace=False)
        vals = []
        for g in range(G):
            hq = h * G + g
            r = np.sort(rows[g * n_plant:(g + 1) * n_plant])
            planted_rows[hq] = r
            qd = q[0, hq].astype(np.float64)
            qd = qd / np.linalg.norm(qd)
            noise = side.standard_normal((n_plant, HEAD_DIM)) * math.sqrt(0.5)
            vals.append((4.0 * qd[None, :] + noise).astype(np.float32))
        allr = np.concatenate([planted_rows[h * G + g] for g in range(G)])
        allv = np.concatenate(vals)
        planted[(0, h)] = (allr, allv)
    k, v = _fill_kv(cfg, B, Hkv, L, "bf16", planted=planted)
    return Workload(f"c5_1M_L{L}_K{top_k}", cfg, B, Hq, Hkv, HEAD_DIM, L, L, "bf16", top_k,
                    1.0 / math.sqrt(HEAD_DIM), q, k, v, dynamic, static_ranges=static,
                    planted=planted_rows)


DEFAULT_L = {1: 4096, 2: 131072, 3: 65536, 4: 32768, 5: 1048576}


def make_workload(cfg: int, L: Optional[int] = None, **kw) -> Workload:
    """Build workload ``cfg`` (1..5). ``L`` overrides the cache length."""
    L = DEFAULT_L[cfg] if L is None else int(L)
    if cfg == 1:
        return _c1(L)
    if cfg == 2:
        return _c2(L)
    if cfg == 3:
        return _c3(L, **kw)
    if cfg == 4:
        return _c4(L, **kw)
    if cfg == 5:
        return _c5(L, **kw)
    raise ValueError(f"unknown workload {cfg}")


def make_multi_query(B: int, Hq: int, Hkv: int, M: int, L: int, dtype: str = "bf16", top_k: int = 64,
                     codebook: int = 0, tag: int = 0) -> Workload:
    """A block of M queries per query head over an L-row cache (``q`` is
    [B, Hq, M, d]); ``tag`` selects an independent draw."""
    cfg = 6
    side = np.random.default_rng([1000 + cfg, T_SIDE, tag, 0])
    if codebook > 0:
        store = np.uint16 if dtype == "bf16" else np.float32
        book = side.standard_normal((codebook, HEAD_DIM)).astype(np.float32)
        pick = side.integers(0, codebook, size=(B, Hkv, L))
        k = book[pick]
        k = bf16_bits_from_f32(k) if dtype == "bf16" else k.astype(store)
        v = np.zeros_like(k)
    else:
        mu = side.standard_normal((B, Hkv, HEAD_DIM)).astype(np.float32)
        k, v = _fill_kv(cfg, B, Hkv, L, dtype, offsets=mu)
    q = np.random.default_rng([1000 + cfg, T_QUERY, tag, 0]).standard_normal((B, Hq, M, HEAD_DIM),
                                                                            dtype=np.float32)
    return Workload(f"mq_B{B}_H{Hq}x{Hkv}_M{M}_L{L}_{dtype}", cfg, B, Hq, Hkv, HEAD_DIM, L, L, dtype, top_k,
                    1.0 / math.sqrt(HEAD_DIM), q, k, v, [(0, L)])


def c3_prefill_block(L: Optional[int] = None) -> Workload:
    """c3's warm-up queries [B, Hq, 32, d] over its first L0 rows."""
    w = _c3(DEFAULT_L[3] if L is None else int(L), steps=0, warm=32)
    w.q = np.ascontiguousarray(w.q[:, :, :32])
    w.name = f"c3_prefill_block_M32_L{w.L}_K512"
    return w
