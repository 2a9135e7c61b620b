"""PyTorch-facing wrappers of the C ABI (include/stdk.h).

Tensors only supply device pointers, shapes and the current HIP stream;
every step of the computation runs in libstdk.so. Outputs that the caller
does not pass are allocated with torch (plumbing, not compute).
"""

from __future__ import annotations

import ctypes
import math
from typing import Optional, Sequence, Tuple

import torch

from . import native
from .native import Layout, RetopkParams, RetopkState, check, load


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtype=None, shape=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def make_layout(k_cache: torch.Tensor, n_q_heads: int) -> Layout:
    """Layout of a contiguous [B, H_kv, L_max, 128] cache (bf16 or fp32)."""
    if k_cache.dim() != 4:
        raise ValueError("k_cache must be [B, H_kv, L_max, head_dim]")
    B, Hkv, L, d = k_cache.shape
    if k_cache.dtype == torch.bfloat16:
        dt = native.STDK_BF16
    elif k_cache.dtype == torch.float32:
        dt = native.STDK_F32
    else:
        raise ValueError(f"unsupported KV dtype {k_cache.dtype}")
    return Layout(B, n_q_heads, Hkv, d, L, dt, 0, Hkv * L * d, L * d)


def _ranges_arr(ranges: Sequence[Tuple[int, int]]):
    flat = [int(x) for r in ranges for x in r]
    arr = (ctypes.c_int64 * max(1, len(flat)))(*flat) if flat else (ctypes.c_int64 * 1)(0)
    return arr, len(ranges)


# Bytes per query head of the counter region at the start of every decode
# workspace (two radix histograms and an arrival counter), zero between calls.
COUNTER_BYTES_PER_HEAD = 16448


def new_workspace(nbytes: int, device) -> torch.Tensor:
    """A zero-filled workspace buffer (the library keeps its counters zero
    between calls, so it must start that way)."""
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def topk_attn_decode_workspace_size(layout: Layout, n_scan: int, top_k: int) -> int:
    return int(load().topk_attn_decode_workspace_size(ctypes.byref(layout), int(n_scan), int(top_k)))


def topk_attn_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                     ranges: Sequence[Tuple[int, int]], top_k: int, scale: Optional[float] = None,
                     *, idx_out: Optional[torch.Tensor] = None, o_out: Optional[torch.Tensor] = None,
                     lse_out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                     want_idx: bool = True, layout: Optional[Layout] = None):
    """Top-K decode attention of every query head over the union of ``ranges``.

    q [B, H_q, 128] fp32; caches [B, H_kv, L_max, 128] (bf16 or fp32).
    Returns (idx [B, H_q, K] int32 or None, o [B, H_q, 128] fp32, lse [B, H_q] fp32).
    """
    lib = load()
    B, Hq, d = q.shape
    _need(q, "q", torch.float32)
    _need(k_cache, "k_cache")
    _need(v_cache, "v_cache", k_cache.dtype, k_cache.shape)
    lay = layout if layout is not None else make_layout(k_cache, Hq)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    n = sum(int(e) - int(b) for b, e in ranges)
    if o_out is None:
        o_out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if lse_out is None:
        lse_out = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if idx_out is None and want_idx:
        idx_out = torch.empty((B, Hq, top_k), dtype=torch.int32, device=q.device)
    if workspace is None:
        workspace = new_workspace(topk_attn_decode_workspace_size(lay, n, top_k), q.device)
    arr, nr = _ranges_arr(ranges)
    rc = lib.topk_attn_decode(ctypes.byref(lay), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), arr, nr,
                              int(top_k), ctypes.c_float(scale), _ptr(idx_out), o_out.data_ptr(), lse_out.data_ptr(),
                              workspace.data_ptr(), workspace.numel(), _stream())
    check(rc)
    return idx_out, o_out, lse_out


def topk_attn_decode_static_workspace_size(layout: Layout, n_scan: int, n_static: int, top_k: int) -> int:
    return int(load().topk_attn_decode_static_workspace_size(ctypes.byref(layout), int(n_scan), int(n_static),
                                                             int(top_k)))


def topk_attn_decode_static(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                            ranges: Sequence[Tuple[int, int]], static_ranges: Sequence[Tuple[int, int]], top_k: int,
                            scale: Optional[float] = None, *, idx_out: Optional[torch.Tensor] = None,
                            o_out: Optional[torch.Tensor] = None, lse_out: Optional[torch.Tensor] = None,
                            workspace: Optional[torch.Tensor] = None, want_idx: bool = True,
                            layout: Optional[Layout] = None):
    """Dense attention over ``static_ranges`` combined with top-K attention
    over ``ranges`` (one pass; equals attn_merge_lse of the two calls).
    Returns (idx of the chosen dynamic rows or None, o, lse)."""
    lib = load()
    B, Hq, d = q.shape
    _need(q, "q", torch.float32)
    _need(k_cache, "k_cache")
    _need(v_cache, "v_cache", k_cache.dtype, k_cache.shape)
    lay = layout if layout is not None else make_layout(k_cache, Hq)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    n = sum(int(e) - int(b) for b, e in ranges)
    n_st = sum(int(e) - int(b) for b, e in static_ranges)
    if o_out is None:
        o_out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if lse_out is None:
        lse_out = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if idx_out is None and want_idx:
        idx_out = torch.empty((B, Hq, top_k), dtype=torch.int32, device=q.device)
    if workspace is None:
        workspace = new_workspace(topk_attn_decode_static_workspace_size(lay, n, n_st, top_k), q.device)
    arr, nr = _ranges_arr(ranges)
    sarr, ns = _ranges_arr(static_ranges)
    rc = lib.topk_attn_decode_static(ctypes.byref(lay), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), arr,
                                     nr, sarr, ns, int(top_k), ctypes.c_float(scale), _ptr(idx_out),
                                     o_out.data_ptr(), lse_out.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                     _stream())
    check(rc)
    return idx_out, o_out, lse_out


def topk_attn_decode_static_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                    ranges: Sequence[Tuple[int, int]], static_ranges: Sequence[Tuple[int, int]],
                                    top_k: int, scale: Optional[float] = None, *,
                                    idx_out: Optional[torch.Tensor] = None, o_out: Optional[torch.Tensor] = None,
                                    lse_out: Optional[torch.Tensor] = None, want_idx: bool = True,
                                    layout: Optional[Layout] = None):
    """topk_attn_decode_static with the library's own scratch array instead of
    a workspace (no allocation inside the call when the outputs are given).
    Returns (idx or None, o, lse)."""
    lib = load()
    B, Hq, d = q.shape
    _need(q, "q", torch.float32)
    _need(k_cache, "k_cache")
    _need(v_cache, "v_cache", k_cache.dtype, k_cache.shape)
    lay = layout if layout is not None else make_layout(k_cache, Hq)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if o_out is None:
        o_out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if lse_out is None:
        lse_out = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if idx_out is None and want_idx:
        idx_out = torch.empty((B, Hq, top_k), dtype=torch.int32, device=q.device)
    arr, nr = _ranges_arr(ranges)
    sarr, ns = _ranges_arr(static_ranges)
    rc = lib.topk_attn_decode_static_noalloc(ctypes.byref(lay), q.data_ptr(), k_cache.data_ptr(),
                                             v_cache.data_ptr(), arr, nr, sarr, ns, int(top_k), ctypes.c_float(scale),
                                             _ptr(idx_out), o_out.data_ptr(), lse_out.data_ptr(), _stream())
    check(rc)
    return idx_out, o_out, lse_out


def attn_merge_lse(o_a: torch.Tensor, lse_a: torch.Tensor, o_b: torch.Tensor, lse_b: torch.Tensor,
                   o_out: Optional[torch.Tensor] = None, lse_out: Optional[torch.Tensor] = None):
    """Log-sum-exp combination of two partial attention outputs."""
    lib = load()
    d = o_a.shape[-1]
    rows = lse_a.numel()
    for t, nm in ((o_a, "o_a"), (o_b, "o_b")):
        _need(t, nm, torch.float32)
    for t, nm in ((lse_a, "lse_a"), (lse_b, "lse_b")):
        _need(t, nm, torch.float32)
    if o_out is None:
        o_out = torch.empty_like(o_a)
    if lse_out is None:
        lse_out = torch.empty_like(lse_a)
    rc = lib.attn_merge_lse(rows, d, o_a.data_ptr(), lse_a.data_ptr(), o_b.data_ptr(), lse_b.data_ptr(),
                            o_out.data_ptr(), lse_out.data_ptr(), _stream())
    check(rc)
    return o_out, lse_out


class Retopk:
    """Per-query-head ReTopK state (device tensors) and its step."""

    def __init__(self, k_cache: torch.Tensor, n_q_heads: int, top_k: int = 512, cache_cap: int = 32,
                 top_r: int = 4, recent: int = 32, tau: float = 0.85, refresh: int = 128,
                 scale: Optional[float] = None, max_len_t: Optional[int] = None, budget: int = 0):
        load()
        self.layout = make_layout(k_cache, n_q_heads)
        B, Hkv, L, d = k_cache.shape
        self.B, self.Hq, self.d = B, n_q_heads, d
        self.params = RetopkParams(top_k, cache_cap, top_r, recent, float(tau), refresh,
                                   float(1.0 / math.sqrt(d) if scale is None else scale), int(budget))
        dev = k_cache.device
        # one allocation of retopk_state_size bytes, carved at the offsets
        # stdk.h documents for it
        S, C = B * n_q_heads, cache_cap
        nbytes = int(load().retopk_state_size(ctypes.byref(self.layout), ctypes.byref(self.params)))
        if nbytes == 0:
            raise ValueError("invalid ReTopK parameters")
        self.state_buffer = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
        al = lambda x: (x + 255) // 256 * 256
        o_sup = al(S * C * d * 4)
        o_head = o_sup + al(S * C * top_k * 4)
        o_cnt = o_head + al(S * 4)
        buf = self.state_buffer
        self.q_hat = buf[:S * C * d * 4].view(torch.float32).view(B, n_q_heads, C, d)
        self.support = buf[o_sup:o_sup + S * C * top_k * 4].view(torch.int32).view(B, n_q_heads, C, top_k)
        self.head = buf[o_head:o_head + S * 4].view(torch.int32).view(B, n_q_heads)
        self.count = buf[o_cnt:o_cnt + S * 4].view(torch.int32).view(B, n_q_heads)
        self.support.fill_(-1)
        self.head.fill_(cache_cap - 1)
        self.state = RetopkState(self.q_hat.data_ptr(), self.support.data_ptr(), self.head.data_ptr(),
                                 self.count.data_ptr())
        self.cand_cap = top_r * top_k + recent
        mx = L if max_len_t is None else int(max_len_t)
        nbytes = int(load().retopk_workspace_size(ctypes.byref(self.layout), ctypes.byref(self.params), mx))
        self.workspace = new_workspace(nbytes, dev)
        # step_device sizes every launch for the cache's full length; the
        # workspace above serves it unless max_len_t was set lower
        need = int(load().retopk_workspace_size(ctypes.byref(self.layout), ctypes.byref(self.params), L))
        self.device_workspace = self.workspace if self.workspace.numel() >= need else new_workspace(need, dev)

    def init(self, q_hist: torch.Tensor, sup_hist: torch.Tensor):
        """Fill the caches from [B, H_q, n, 128] queries and [B, H_q, n, K] supports."""
        n = q_hist.shape[2]
        _need(q_hist, "q_hist", torch.float32)
        _need(sup_hist, "sup_hist", torch.int32)
        rc = load().retopk_state_init(ctypes.byref(self.layout), ctypes.byref(self.params), ctypes.byref(self.state),
                                      q_hist.data_ptr(), sup_hist.data_ptr(), n, _stream())
        check(rc)

    def step(self, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, L_t: int, t: int,
             *, out: Optional[dict] = None, want_cand: bool = False) -> dict:
        """One decode step; returns support, o, lse, path, n_cand (and cand)."""
        B, Hq, K = self.B, self.Hq, self.params.top_k
        dev = q.device
        _need(q, "q", torch.float32)
        if out is None:
            out = dict(support=torch.empty((B, Hq, K), dtype=torch.int32, device=dev),
                       o=torch.empty((B, Hq, self.d), dtype=torch.float32, device=dev),
                       lse=torch.empty((B, Hq), dtype=torch.float32, device=dev),
                       path=torch.empty((B, Hq), dtype=torch.int32, device=dev),
                       n_cand=torch.empty((B, Hq), dtype=torch.int32, device=dev))
            if want_cand:
                out["cand"] = torch.empty((B, Hq, self.cand_cap), dtype=torch.int32, device=dev)
        rc = load().retopk_step(ctypes.byref(self.layout), ctypes.byref(self.params), ctypes.byref(self.state),
                                q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), int(L_t), int(t),
                                out["support"].data_ptr(), out["o"].data_ptr(), out["lse"].data_ptr(),
                                _ptr(out.get("path")), _ptr(out.get("n_cand")), _ptr(out.get("cand")),
                                self.workspace.data_ptr(), self.workspace.numel(), _stream())
        check(rc)
        return out


    def step_device(self, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, step: torch.Tensor,
                    out: dict, want_cand: bool = False) -> dict:
        """One decode step with L_t and t read from the device tensor ``step``
        (int64 [L_t, t]) and advanced there by the step; nothing is allocated
        (``out`` holds support, o, lse and optionally path, n_cand, cand), so
        the call can be captured in a graph and replayed for later steps."""
        _need(q, "q", torch.float32)
        _need(step, "step", torch.int64, (2,))
        ws = self.device_workspace
        rc = load().retopk_step_device(ctypes.byref(self.layout), ctypes.byref(self.params),
                                       ctypes.byref(self.state), q.data_ptr(), k_cache.data_ptr(),
                                       v_cache.data_ptr(), step.data_ptr(), out["support"].data_ptr(),
                                       out["o"].data_ptr(), out["lse"].data_ptr(), _ptr(out.get("path")),
                                       _ptr(out.get("n_cand")), _ptr(out.get("cand")), ws.data_ptr(), ws.numel(),
                                       _stream())
        check(rc)
        return out


def hbm_read(buf: torch.Tensor, group_stride_bytes: int, n_groups: int, group_bytes: int, wg_per_group: int,
             sink: torch.Tensor):
    """Measurement aid: stream n_groups regions of ``buf`` once with the key
    scan's workgroup split (kernel family "hbm_read")."""
    _need(buf, "buf")
    _need(sink, "sink")
    check(load().stdk_hbm_read(buf.data_ptr(), int(group_stride_bytes), int(n_groups), int(group_bytes),
                               int(wg_per_group), sink.data_ptr(), _stream()))


def inject_launch_failure(after_launches: int):
    """Testing aid: the library launch numbered ``after_launches`` from now is
    not enqueued and its call fails with STDK_EHIP (-1 disarms)."""
    check(load().stdk_inject_launch_failure(int(after_launches)))


class KernelTimer:
    """Per-kernel durations from HIP events the library records around each
    of its launches (on the launch stream)."""

    def __init__(self, capacity: int = 1 << 16, only: Optional[str] = None):
        check(load().stdk_profile_enable(capacity, None if only is None else only.encode()))
        check(load().stdk_profile_reset())

    def read(self, name: str) -> Tuple[float, int]:
        ms = ctypes.c_double(0.0)
        n = ctypes.c_int64(0)
        check(load().stdk_profile_read(name.encode(), ctypes.byref(ms), ctypes.byref(n)))
        return ms.value, n.value

    def reset(self):
        check(load().stdk_profile_reset())

    def close(self):
        check(load().stdk_profile_disable())


def topk_multi_query_workspace_size(layout: Layout, n_queries: int, n_scan: int, top_k: int) -> int:
    return int(load().topk_multi_query_workspace_size(ctypes.byref(layout), int(n_queries), int(n_scan), int(top_k)))


def topk_multi_query(q: torch.Tensor, k_cache: torch.Tensor, ranges: Sequence[Tuple[int, int]], top_k: int,
                     scale: Optional[float] = None, *, idx_out: Optional[torch.Tensor] = None,
                     z_out: Optional[torch.Tensor] = None, want_z: bool = False,
                     workspace: Optional[torch.Tensor] = None, layout: Optional[Layout] = None):
    """Exact top-K index sets of a block of queries per head.

    q [B, H_q, M, 128] fp32; k_cache [B, H_kv, L_max, 128] (bf16 or fp32).
    Returns (idx [B, H_q, M, K] int32, z [B, H_q, M, K] fp32 or None).
    """
    lib = load()
    B, Hq, M, d = q.shape
    _need(q, "q", torch.float32)
    _need(k_cache, "k_cache")
    lay = layout if layout is not None else make_layout(k_cache, Hq)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    n = sum(int(e) - int(b) for b, e in ranges)
    if idx_out is None:
        idx_out = torch.empty((B, Hq, M, top_k), dtype=torch.int32, device=q.device)
    if z_out is None and want_z:
        z_out = torch.empty((B, Hq, M, top_k), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = new_workspace(topk_multi_query_workspace_size(lay, M, n, top_k), q.device)
    arr, nr = _ranges_arr(ranges)
    rc = lib.topk_multi_query(ctypes.byref(lay), q.data_ptr(), int(M), k_cache.data_ptr(), arr, nr, int(top_k),
                              ctypes.c_float(scale), idx_out.data_ptr(), _ptr(z_out), workspace.data_ptr(),
                              workspace.numel(), _stream())
    check(rc)
    return idx_out, z_out


def quantize_keys_int8(k_cache: torch.Tensor, ranges: Sequence[Tuple[int, int]], n_q_heads: int,
                       codes: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None,
                       layout: Optional[Layout] = None):
    """Per-row symmetric int8 codes of the rows in ``ranges`` (the int8 recall
    stage's keys). Returns (codes [B, H_kv, L_max, 128] int8, scales
    [B, H_kv, L_max] fp32); rows outside the ranges keep what they held."""
    _need(k_cache, "k_cache")
    B, Hkv, L, d = k_cache.shape
    lay = layout if layout is not None else make_layout(k_cache, n_q_heads)
    if codes is None:
        codes = torch.zeros((B, Hkv, L, d), dtype=torch.int8, device=k_cache.device)
    if scales is None:
        scales = torch.zeros((B, Hkv, L), dtype=torch.float32, device=k_cache.device)
    arr, nr = _ranges_arr(ranges)
    check(load().quantize_keys_int8(ctypes.byref(lay), k_cache.data_ptr(), arr, nr, codes.data_ptr(),
                                    scales.data_ptr(), _stream()))
    return codes, scales


def topk_attn_decode_int8_workspace_size(layout: Layout, n_scan: int, top_k: int, recall_k: int) -> int:
    return int(load().topk_attn_decode_int8_workspace_size(ctypes.byref(layout), int(n_scan), int(top_k),
                                                           int(recall_k)))


def topk_attn_decode_int8(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, codes: torch.Tensor,
                          scales: torch.Tensor, ranges: Sequence[Tuple[int, int]], top_k: int, recall_k: int,
                          scale: Optional[float] = None, *, idx_out: Optional[torch.Tensor] = None,
                          sup_out: Optional[torch.Tensor] = None, want_sup: bool = False,
                          o_out: Optional[torch.Tensor] = None, lse_out: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None, layout: Optional[Layout] = None):
    """Top-K attention with an int8 recall stage (superset of recall_k rows by
    the int8 scores, exact top-K inside it). Returns (idx, sup or None, o, lse)."""
    lib = load()
    B, Hq, d = q.shape
    _need(q, "q", torch.float32)
    _need(k_cache, "k_cache")
    _need(v_cache, "v_cache", k_cache.dtype, k_cache.shape)
    _need(codes, "codes", torch.int8, k_cache.shape)
    _need(scales, "scales", torch.float32, k_cache.shape[:3])
    lay = layout if layout is not None else make_layout(k_cache, Hq)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    n = sum(int(e) - int(b) for b, e in ranges)
    if o_out is None:
        o_out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if lse_out is None:
        lse_out = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if idx_out is None:
        idx_out = torch.empty((B, Hq, top_k), dtype=torch.int32, device=q.device)
    if sup_out is None and want_sup:
        sup_out = torch.empty((B, Hq, recall_k), dtype=torch.int32, device=q.device)
    if workspace is None:
        workspace = new_workspace(topk_attn_decode_int8_workspace_size(lay, n, top_k, recall_k), q.device)
    arr, nr = _ranges_arr(ranges)
    rc = lib.topk_attn_decode_int8(ctypes.byref(lay), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                   codes.data_ptr(), scales.data_ptr(), arr, nr, int(top_k), int(recall_k),
                                   ctypes.c_float(scale), _ptr(idx_out), _ptr(sup_out), o_out.data_ptr(),
                                   lse_out.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream())
    check(rc)
    return idx_out, sup_out, o_out, lse_out


def topk_attn_decode_int8_static_workspace_size(layout: Layout, n_scan: int, n_static: int, top_k: int,
                                                recall_k: int) -> int:
    return int(load().topk_attn_decode_int8_static_workspace_size(ctypes.byref(layout), int(n_scan), int(n_static),
                                                                  int(top_k), int(recall_k)))


def topk_attn_decode_int8_static(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, codes: torch.Tensor,
                                 scales: torch.Tensor, ranges: Sequence[Tuple[int, int]],
                                 static_ranges: Sequence[Tuple[int, int]], top_k: int, recall_k: int,
                                 scale: Optional[float] = None, *, idx_out: Optional[torch.Tensor] = None,
                                 sup_out: Optional[torch.Tensor] = None, want_sup: bool = False,
                                 o_out: Optional[torch.Tensor] = None, lse_out: Optional[torch.Tensor] = None,
                                 workspace: Optional[torch.Tensor] = None, layout: Optional[Layout] = None):
    """Dense attention over ``static_ranges`` together with the int8-recall
    top-K attention over ``ranges``, in one pass (equals attn_merge_lse of the
    dense call and topk_attn_decode_int8). Returns (idx, sup or None, o, lse)."""
    lib = load()
    B, Hq, d = q.shape
    _need(q, "q", torch.float32)
    _need(k_cache, "k_cache")
    _need(v_cache, "v_cache", k_cache.dtype, k_cache.shape)
    _need(codes, "codes", torch.int8, k_cache.shape)
    _need(scales, "scales", torch.float32, k_cache.shape[:3])
    lay = layout if layout is not None else make_layout(k_cache, Hq)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    n = sum(int(e) - int(b) for b, e in ranges)
    n_st = sum(int(e) - int(b) for b, e in static_ranges)
    if o_out is None:
        o_out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if lse_out is None:
        lse_out = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if idx_out is None:
        idx_out = torch.empty((B, Hq, top_k), dtype=torch.int32, device=q.device)
    if sup_out is None and want_sup:
        sup_out = torch.empty((B, Hq, recall_k), dtype=torch.int32, device=q.device)
    if workspace is None:
        workspace = new_workspace(topk_attn_decode_int8_static_workspace_size(lay, n, n_st, top_k, recall_k),
                                  q.device)
    arr, nr = _ranges_arr(ranges)
    sarr, ns = _ranges_arr(static_ranges)
    rc = lib.topk_attn_decode_int8_static(ctypes.byref(lay), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                          codes.data_ptr(), scales.data_ptr(), arr, nr, sarr, ns, int(top_k),
                                          int(recall_k), ctypes.c_float(scale), _ptr(idx_out), _ptr(sup_out),
                                          o_out.data_ptr(), lse_out.data_ptr(), workspace.data_ptr(),
                                          workspace.numel(), _stream())
    check(rc)
    return idx_out, sup_out, o_out, lse_out
