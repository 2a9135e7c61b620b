"""Helpers for the GPU parity tests: device copies of workloads and the
acceptance checks against the oracle.

Acceptance (fixed before any kernel was written):
* index sets: every row whose fp64 oracle score exceeds the oracle's K-th
  score by more than 1e-3 must be chosen, every row below it by more than
  1e-3 must not; the set is ascending, unique, of size min(K, n), -1 padded;
* o and lse: max-abs 1e-4 when the cache is fp32, relative L2 1e-2 (per
  head) when it is bf16.
"""

from __future__ import annotations

import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from oracle import reference as ref

BAND = 1e-3


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_kv(w, device="cuda:0"):
    dt = torch.bfloat16 if w.kv_dtype == "bf16" else torch.float32
    if w.kv_dtype == "bf16":
        k = torch.from_numpy(w.k.view(np.int16)).to(device).view(torch.bfloat16)
        v = torch.from_numpy(w.v.view(np.int16)).to(device).view(torch.bfloat16)
    else:
        k = torch.from_numpy(w.k).to(device)
        v = torch.from_numpy(w.v).to(device)
    assert k.dtype == dt
    return k, v


def check_index_set(got_row: np.ndarray, rows: np.ndarray, z: np.ndarray, zk: float, K: int, band: float = BAND):
    """got_row: [K] int32 from the GPU. rows/z: the scanned rows and their fp64
    oracle scores. Returns the number of rows that differ from the oracle set
    (all inside the band)."""
    n = rows.shape[0]
    m = min(K, n)
    sel = got_row[got_row >= 0]
    assert sel.shape[0] == m, f"{sel.shape[0]} rows chosen, {m} expected"
    assert np.all(got_row[m:] == -1), "padding must be -1"
    assert np.all(np.diff(sel) > 0), "rows must be strictly ascending"
    pos = np.searchsorted(rows, sel)
    assert np.all(pos < n) and np.array_equal(rows[np.minimum(pos, n - 1)], sel), "row outside the scanned ranges"
    chosen = np.zeros(n, bool)
    chosen[pos] = True
    must = z > zk + band
    forbid = z < zk - band
    assert np.all(chosen[must]), f"{int(np.sum(must & ~chosen))} rows above the band were not chosen"
    assert not np.any(chosen[forbid]), f"{int(np.sum(forbid & chosen))} rows below the band were chosen"
    return int(np.sum(chosen & ~(z >= zk)))


def rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    nb = float(np.linalg.norm(b))
    return float(np.linalg.norm(a - b)) / (nb if nb > 0 else 1.0)


def check_out(o_gpu: np.ndarray, lse_gpu: np.ndarray, o_ref: np.ndarray, lse_ref: float, fp32: bool, what: str = ""):
    o_gpu = o_gpu.astype(np.float64)
    if fp32:
        eo = float(np.max(np.abs(o_gpu - o_ref)))
        el = abs(float(lse_gpu) - lse_ref) if np.isfinite(lse_ref) else (0.0 if lse_gpu == lse_ref else np.inf)
        assert eo <= 1e-4, f"{what} o max-abs {eo:.3g}"
        assert el <= 1e-4, f"{what} lse abs {el:.3g}"
        return eo, el
    eo = rel_l2(o_gpu, o_ref)
    el = abs(float(lse_gpu) - lse_ref) / max(1.0, abs(lse_ref)) if np.isfinite(lse_ref) else (0.0 if lse_gpu == lse_ref else np.inf)
    assert eo <= 1e-2, f"{what} o rel-L2 {eo:.3g}"
    assert el <= 1e-2, f"{what} lse rel {el:.3g}"
    return eo, el


def oracle_head(w, b: int, h: int, ranges, K: int, q=None):
    """Oracle scores, chosen rows, o and lse of one query head."""
    G = w.H_q // w.H_kv
    rows = ref.range_rows(ranges)
    qv = (w.q if q is None else q)[b, h]
    return ref.attend_rows(qv, w.k[b, h // G], w.v[b, h // G], rows, K, w.scale), rows


# Oracle work over many heads runs in a thread pool (numpy releases the GIL
# inside its array loops), at most 16 host threads.
ORACLE_THREADS = max(1, min(16, os.cpu_count() or 1))


def pmap(fn, items, threads: int = ORACLE_THREADS):
    """[fn(x) for x in items], evaluated in a thread pool, in order."""
    items = list(items)
    if threads <= 1 or len(items) <= 1:
        return [fn(x) for x in items]
    with ThreadPoolExecutor(min(threads, len(items))) as ex:
        return list(ex.map(fn, items))


def check_heads(w, heads, idx, o, lse, ranges, K, fp32=False, q=None, label=""):
    """Compares GPU outputs of the listed (b, h) heads with the oracle (the
    oracle's heads are computed in parallel threads, the checks in order)."""
    worst_o = worst_l = 0.0
    swaps = 0
    heads = list(heads)
    results = pmap(lambda bh: oracle_head(w, bh[0], bh[1], ranges, K, q=q), heads)
    for (b, h), (r, rows) in zip(heads, results):
        if idx is not None:
            swaps += check_index_set(idx[b, h], rows, r["z"], r["zk"], K)
        eo, el = check_out(o[b, h], lse[b, h], r["o"], r["lse"], fp32, f"{label} head ({b},{h})")
        worst_o, worst_l = max(worst_o, eo), max(worst_l, el)
    log(f"[{label}] {len(heads)} heads ok: worst o err {worst_o:.2e}, lse err {worst_l:.2e}, band swaps {swaps}")
    return worst_o, worst_l, swaps
