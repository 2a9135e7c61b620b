"""The C ABI without a GPU: the library loads, exports every symbol the header
declares, sizes workspaces, and rejects bad arguments on the host before any
HIP call (so these run on a machine with no GPU)."""

import ctypes
import os
import re

import pytest

from sparse_top_decode_amd import native
from sparse_top_decode_amd.native import Layout, RetopkParams, RetopkState

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x100000  # never dereferenced: every call below fails validation first


def header_functions():
    with open(os.path.join(ROOT, "include", "stdk.h")) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return native.load()


def test_exports_match_header(lib):
    declared = header_functions()
    assert sorted(native.EXPORTS) == declared
    for name in declared:
        assert hasattr(lib, name), name


def test_version(lib):
    assert lib.stdk_version() == 100


def lay(B=1, Hq=32, Hkv=8, d=128, L=4096, dt=native.STDK_BF16):
    return Layout(B, Hq, Hkv, d, L, dt, 0, Hkv * L * d, L * d)


def test_workspace_size(lib):
    a = lib.topk_attn_decode_workspace_size(ctypes.byref(lay()), 4000, 64)
    b = lib.topk_attn_decode_workspace_size(ctypes.byref(lay()), 8000, 64)
    assert a > 0 and b > a and a % 256 == 0
    assert lib.topk_attn_decode_workspace_size(ctypes.byref(lay(d=64)), 4000, 64) == 0
    p = RetopkParams(512, 32, 4, 32, 0.85, 128, 0.088)
    assert lib.retopk_workspace_size(ctypes.byref(lay(Hq=28, Hkv=4)), ctypes.byref(p), 65536) > 0


def test_retopk_state_size(lib):
    """One allocation for the four state arrays at the documented 256-byte
    aligned offsets: q_hat, support, head, count."""
    al = lambda x: (x + 255) // 256 * 256
    for B, Hq, Hkv, C, K in [(1, 28, 4, 32, 512), (3, 32, 8, 5, 1100), (2, 4, 4, 1, 1)]:
        p = RetopkParams(K, C, 1, 0, 0.85, 0, 0.088)
        S = B * Hq
        want = al(S * C * 128 * 4) + al(S * C * K * 4) + al(S * 4) + al(S * 4)
        assert lib.retopk_state_size(ctypes.byref(lay(B=B, Hq=Hq, Hkv=Hkv)), ctypes.byref(p)) == want
    bad = RetopkParams(0, 32, 4, 32, 0.85, 128, 0.088)
    assert lib.retopk_state_size(ctypes.byref(lay(Hq=28, Hkv=4)), ctypes.byref(bad)) == 0
    assert lib.retopk_state_size(ctypes.byref(lay(d=64)), ctypes.byref(RetopkParams(8, 2, 1, 0, 0.5, 0, 0.1))) == 0


def test_noalloc_rejects_before_launch(lib):
    """The allocation-free step rejects bad arguments like the workspace
    variant, and a call whose scratch need exceeds the library's array with
    STDK_EWORKSPACE, all before any HIP call."""
    def call(L, ranges, static, top_k=64, q=FAKE):
        flat = [x for r in ranges for x in r]
        sflat = [x for r in static for x in r]
        arr = (ctypes.c_int64 * max(1, len(flat)))(*flat)
        sarr = (ctypes.c_int64 * max(1, len(sflat)))(*sflat)
        return lib.topk_attn_decode_static_noalloc(ctypes.byref(L), q, FAKE, FAKE, arr, len(ranges), sarr,
                                                   len(static), top_k, ctypes.c_float(0.1), FAKE, FAKE, FAKE, None)
    big = lay(L=1 << 20)
    assert call(big, [(128, (1 << 20) - 512)], [(0, 128), ((1 << 20) - 512, 1 << 20)], 8192) == native.STDK_EWORKSPACE
    need = lib.topk_attn_decode_static_workspace_size(ctypes.byref(big), (1 << 20) - 640, 640, 8192)
    assert need > native.STDK_NOALLOC_SCRATCH_BYTES
    c2 = lay(L=131072)
    need2 = lib.topk_attn_decode_static_workspace_size(ctypes.byref(c2), 130432, 640, 2048)
    assert 0 < need2 <= native.STDK_NOALLOC_SCRATCH_BYTES
    assert call(c2, [(128, 130560)], [(0, 128), (130560, 131072)], 0) == native.STDK_EINVAL
    assert call(c2, [(128, 130560)], [(100, 200)], 64) == native.STDK_EINVAL  # overlap
    assert call(lay(d=64), [(0, 10)], [], 4) == native.STDK_EUNSUPPORTED
    assert call(c2, [(0, 10)], [], 4, q=0) == native.STDK_EINVAL


def test_inject_launch_failure_arguments(lib):
    assert lib.stdk_inject_launch_failure(-2) == native.STDK_EINVAL
    assert lib.stdk_inject_launch_failure(-1) == native.STDK_OK


def call_topk(lib, L=None, ranges=((0, 100),), top_k=8, ws_bytes=1 << 30, q=FAKE, scale=0.1, idx=FAKE):
    L = L or lay()
    flat = [x for r in ranges for x in r]
    arr = (ctypes.c_int64 * max(1, len(flat)))(*flat)
    return lib.topk_attn_decode(ctypes.byref(L), q, FAKE, FAKE, arr, len(ranges), top_k, ctypes.c_float(scale),
                                idx, FAKE, FAKE, FAKE, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(L=lay(d=64)), native.STDK_EUNSUPPORTED),
    (dict(L=lay(Hq=30, Hkv=8)), native.STDK_EUNSUPPORTED),
    (dict(L=lay(Hq=80, Hkv=8)), native.STDK_EUNSUPPORTED),
    (dict(L=lay(dt=7)), native.STDK_EUNSUPPORTED),
    (dict(top_k=0), native.STDK_EINVAL),
    (dict(ranges=((0, 5000),)), native.STDK_EINVAL),
    (dict(ranges=((10, 10),)), native.STDK_EINVAL),
    (dict(ranges=((0, 100), (50, 200))), native.STDK_EINVAL),
    (dict(ranges=((300, 400), (0, 100))), native.STDK_EINVAL),
    (dict(ranges=tuple((2 * i, 2 * i + 1) for i in range(17))), native.STDK_EINVAL),
    (dict(ws_bytes=16), native.STDK_EWORKSPACE),
    (dict(q=0), native.STDK_EINVAL),
    (dict(q=FAKE + 4), native.STDK_EINVAL),
    (dict(idx=FAKE + 2), native.STDK_EINVAL),
    (dict(scale=float("nan")), native.STDK_EINVAL),
])
def test_topk_rejects_before_launch(lib, kw, code):
    assert call_topk(lib, **kw) == code
    assert lib.stdk_last_error()


def call_static(lib, ranges=((128, 3584),), static=((0, 128), (3584, 4096)), top_k=8, ws_bytes=1 << 30, L=None):
    L = L or lay()
    flat = [x for r in ranges for x in r]
    sflat = [x for r in static for x in r]
    arr = (ctypes.c_int64 * max(1, len(flat)))(*flat)
    sarr = (ctypes.c_int64 * max(1, len(sflat)))(*sflat)
    return lib.topk_attn_decode_static(ctypes.byref(L), FAKE, FAKE, FAKE, arr, len(ranges), sarr, len(static),
                                       top_k, ctypes.c_float(0.1), FAKE, FAKE, FAKE, FAKE, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(static=((0, 200),)), native.STDK_EINVAL),                       # overlaps the dynamic range
    (dict(static=((3500, 3600),)), native.STDK_EINVAL),                   # overlaps at the end
    (dict(static=((3584, 4096), (0, 128))), native.STDK_EINVAL),          # not ascending
    (dict(static=((0, 128), (4000, 4097))), native.STDK_EINVAL),          # past max_len
    (dict(ranges=tuple((200 + 2 * i, 201 + 2 * i) for i in range(15))), native.STDK_EINVAL),  # 17 ranges in total
    (dict(top_k=0), native.STDK_EINVAL),
    (dict(ws_bytes=1024), native.STDK_EWORKSPACE),
])
def test_static_rejects_before_launch(lib, kw, code):
    assert call_static(lib, **kw) == code
    assert lib.stdk_last_error()


def test_static_rejects_too_many_attended_rows(lib):
    # the chosen rows plus the static rows exceed what one merge handles
    big = lay(L=200000)
    assert call_static(lib, ranges=((0, 150000),), static=((150000, 200000),), top_k=20000,
                       L=big) == native.STDK_EUNSUPPORTED
    assert lib.stdk_last_error()


def test_static_workspace_size(lib):
    a = lib.topk_attn_decode_static_workspace_size(ctypes.byref(lay()), 3456, 640, 64)
    b = lib.topk_attn_decode_workspace_size(ctypes.byref(lay()), 3456, 64)
    assert a > b > 0
    assert lib.topk_attn_decode_static_workspace_size(ctypes.byref(lay(d=64)), 3456, 640, 64) == 0


def test_merge_rejects(lib):
    assert lib.attn_merge_lse(4, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == native.STDK_EINVAL
    assert lib.attn_merge_lse(-1, 128, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == native.STDK_EINVAL
    assert lib.attn_merge_lse(4, 128, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None) == native.STDK_EINVAL
    assert lib.attn_merge_lse(0, 128, 0, 0, 0, 0, 0, 0, None) == native.STDK_OK  # nothing to do


def test_hbm_read_rejects(lib):
    E = native.STDK_EINVAL
    assert lib.stdk_hbm_read(0, 4096, 8, 4096, 32, FAKE, None) == E             # no buffer
    assert lib.stdk_hbm_read(FAKE + 4, 4096, 8, 4096, 32, FAKE, None) == E      # misaligned
    assert lib.stdk_hbm_read(FAKE, 4096, 0, 4096, 32, FAKE, None) == E          # no region
    assert lib.stdk_hbm_read(FAKE, 4096, 8, 4100, 32, FAKE, None) == E          # not whole 16-byte loads
    assert lib.stdk_hbm_read(FAKE, 4096, 8, 4096, 0, FAKE, None) == E           # no workgroup
    assert lib.stdk_hbm_read(FAKE, 4096, 8, 4096, 32, 0, None) == E             # no sink
    assert lib.stdk_hbm_read(FAKE, 4096, 1 << 20, 4096, 1 << 12, FAKE, None) == E  # grid too large


def step(lib, p, L_t=100, t=0, ws=1 << 30, L=None, st=None, sup=FAKE):
    L = L or lay(Hq=28, Hkv=4, L=4096)
    st = st or RetopkState(FAKE, FAKE, FAKE, FAKE)
    return lib.retopk_step(ctypes.byref(L), ctypes.byref(p), ctypes.byref(st), FAKE, FAKE, FAKE, L_t, t, sup, FAKE,
                           FAKE, None, None, None, FAKE, ws, None)


def test_retopk_rejects(lib):
    good = RetopkParams(64, 8, 2, 8, 0.85, 16, 0.088)
    assert step(lib, RetopkParams(0, 8, 2, 8, 0.85, 16, 0.088)) == native.STDK_EINVAL
    assert step(lib, RetopkParams(64, 0, 1, 8, 0.85, 16, 0.088)) == native.STDK_EINVAL
    assert step(lib, RetopkParams(64, 65, 2, 8, 0.85, 16, 0.088)) == native.STDK_EINVAL
    assert step(lib, RetopkParams(64, 8, 9, 8, 0.85, 16, 0.088)) == native.STDK_EINVAL
    assert step(lib, RetopkParams(64, 8, 2, -1, 0.85, 16, 0.088)) == native.STDK_EINVAL
    assert step(lib, RetopkParams(64, 8, 2, 8, float("nan"), 16, 0.088)) == native.STDK_EINVAL
    assert step(lib, RetopkParams(64, 8, 2, 8, 0.85, -3, 0.088)) == native.STDK_EINVAL
    assert step(lib, good, L_t=0) == native.STDK_EINVAL
    assert step(lib, good, L_t=5000) == native.STDK_EINVAL
    assert step(lib, good, t=-1) == native.STDK_EINVAL
    assert step(lib, good, ws=100) == native.STDK_EWORKSPACE
    assert step(lib, good, sup=0) == native.STDK_EINVAL
    assert step(lib, good, st=RetopkState(FAKE, 0, FAKE, FAKE)) == native.STDK_EINVAL
    assert step(lib, good, L=lay(Hq=28, Hkv=4, L=4096, d=96)) == native.STDK_EUNSUPPORTED
    big = lay(Hq=28, Hkv=4, L=2_000_000)
    assert step(lib, good, L=big, L_t=1_500_000) == native.STDK_EUNSUPPORTED
    # candidate budget: >= 0, at most 8 recalled entries, R*K + W within the vote's LDS
    assert step(lib, RetopkParams(64, 8, 2, 8, 0.85, 16, 0.088, -1)) == native.STDK_EINVAL
    assert step(lib, RetopkParams(64, 16, 9, 8, 0.85, 16, 0.088, 100)) == native.STDK_EUNSUPPORTED
    assert step(lib, RetopkParams(4096, 8, 4, 8, 0.85, 16, 0.088, 100), L=lay(Hq=28, Hkv=4, L=8192),
                L_t=5000) == native.STDK_EUNSUPPORTED


def test_retopk_device_rejects(lib):
    """retopk_step_device: the step words are required and 8-byte aligned;
    the workspace must cover L_t = max_len (every launch is sized for it)."""
    good = RetopkParams(64, 8, 2, 8, 0.85, 16, 0.088)
    L = lay(Hq=28, Hkv=4, L=4096)
    st = RetopkState(FAKE, FAKE, FAKE, FAKE)

    def dstep(step_ptr, ws=1 << 30):
        return lib.retopk_step_device(ctypes.byref(L), ctypes.byref(good), ctypes.byref(st), FAKE, FAKE, FAKE,
                                      step_ptr, FAKE, FAKE, FAKE, None, None, None, FAKE, ws, None)

    assert dstep(0) == native.STDK_EINVAL
    assert dstep(FAKE + 4) == native.STDK_EINVAL
    need = lib.retopk_workspace_size(ctypes.byref(L), ctypes.byref(good), 4096)
    assert need > lib.retopk_workspace_size(ctypes.byref(L), ctypes.byref(good), 100)
    assert dstep(FAKE, ws=need - 1) == native.STDK_EWORKSPACE


def call_mq(lib, L=None, M=4, ranges=((0, 100),), top_k=8, ws_bytes=1 << 30, q=FAKE, scale=0.1, idx=FAKE, z=None):
    L = L or lay()
    flat = [x for r in ranges for x in r]
    arr = (ctypes.c_int64 * max(1, len(flat)))(*flat)
    return lib.topk_multi_query(ctypes.byref(L), q, M, FAKE, arr, len(ranges), top_k, ctypes.c_float(scale), idx, z,
                                FAKE, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(L=lay(d=64)), native.STDK_EUNSUPPORTED),
    (dict(L=lay(Hq=30, Hkv=8)), native.STDK_EUNSUPPORTED),
    (dict(M=0), native.STDK_EINVAL),
    (dict(top_k=0), native.STDK_EINVAL),
    (dict(top_k=65537), native.STDK_EUNSUPPORTED),
    (dict(ranges=((0, 5000),)), native.STDK_EINVAL),
    (dict(ranges=((0, 100), (50, 200))), native.STDK_EINVAL),
    (dict(ws_bytes=16), native.STDK_EWORKSPACE),
    (dict(q=0), native.STDK_EINVAL),
    (dict(q=FAKE + 4), native.STDK_EINVAL),
    (dict(idx=0), native.STDK_EINVAL),
    (dict(idx=FAKE + 2), native.STDK_EINVAL),
    (dict(z=FAKE + 1), native.STDK_EINVAL),
    (dict(scale=float("inf")), native.STDK_EINVAL),
    (dict(L=lay(B=70000, Hq=8, Hkv=1)), native.STDK_EUNSUPPORTED),
    (dict(L=lay(Hq=8, Hkv=1), M=1048576), native.STDK_EUNSUPPORTED),
])
def test_multi_query_rejects_before_launch(lib, kw, code):
    assert call_mq(lib, **kw) == code


def test_multi_query_workspace_size(lib):
    L = lay(Hq=28, Hkv=4, L=65536)
    a = lib.topk_multi_query_workspace_size(ctypes.byref(L), 32, 65536, 512)
    b = lib.topk_multi_query_workspace_size(ctypes.byref(L), 16, 65536, 512)
    assert a > b > 0 and a % 256 == 0
    # the candidate list of every query has room for every row
    assert a >= 28 * 32 * 65536 * 8
    assert lib.topk_multi_query_workspace_size(ctypes.byref(L), 0, 65536, 512) == 0
    assert lib.topk_multi_query_workspace_size(ctypes.byref(lay(d=64)), 4, 100, 8) == 0


def test_int8_entry_points_reject(lib):
    L = lay()
    flat = (ctypes.c_int64 * 2)(0, 100)
    # quantize: bad pointers and ranges
    assert lib.quantize_keys_int8(ctypes.byref(L), FAKE, flat, 1, 0, FAKE, None) == native.STDK_EINVAL
    assert lib.quantize_keys_int8(ctypes.byref(L), FAKE, flat, 1, FAKE + 8, FAKE, None) == native.STDK_EINVAL
    bad = (ctypes.c_int64 * 2)(0, 5000)
    assert lib.quantize_keys_int8(ctypes.byref(L), FAKE, bad, 1, FAKE, FAKE, None) == native.STDK_EINVAL

    def dec(top_k=8, recall_k=16, codes=FAKE, ws=1 << 30, scale=0.1):
        return lib.topk_attn_decode_int8(ctypes.byref(L), FAKE, FAKE, FAKE, codes, FAKE, flat, 1, top_k, recall_k,
                                         ctypes.c_float(scale), None, None, FAKE, FAKE, FAKE, ws, None)
    assert dec(recall_k=4) == native.STDK_EINVAL
    assert dec(top_k=0) == native.STDK_EINVAL
    assert dec(codes=0) == native.STDK_EINVAL
    assert dec(scale=float("nan")) == native.STDK_EINVAL
    assert dec(ws=64) == native.STDK_EWORKSPACE
    assert lib.topk_attn_decode_int8_workspace_size(ctypes.byref(L), 4000, 64, 128) > \
        lib.topk_attn_decode_workspace_size(ctypes.byref(L), 4000, 64)
    assert lib.topk_attn_decode_int8_workspace_size(ctypes.byref(L), 4000, 64, 32) == 0


def test_int8_static_entry_point_rejects(lib):
    L = lay()
    dyn = (ctypes.c_int64 * 2)(128, 3000)
    st = (ctypes.c_int64 * 4)(0, 128, 3000, 3500)

    def dec(top_k=8, recall_k=16, codes=FAKE, ws=1 << 30, ranges=dyn, n_r=1, static=st, n_s=2):
        return lib.topk_attn_decode_int8_static(ctypes.byref(L), FAKE, FAKE, FAKE, codes, FAKE, ranges, n_r, static,
                                                n_s, top_k, recall_k, ctypes.c_float(0.1), None, None, FAKE, FAKE,
                                                FAKE, ws, None)
    assert dec(recall_k=4) == native.STDK_EINVAL
    assert dec(top_k=0) == native.STDK_EINVAL
    assert dec(codes=0) == native.STDK_EINVAL
    assert dec(ws=64) == native.STDK_EWORKSPACE
    # a static range that overlaps a dynamic one
    over = (ctypes.c_int64 * 4)(0, 130, 3000, 3500)
    assert dec(static=over) == native.STDK_EINVAL
    # too many ranges in total
    many = (ctypes.c_int64 * 32)(*[v for i in range(16) for v in (3000 + 10 * i, 3005 + 10 * i)])
    assert dec(static=many, n_s=16) == native.STDK_EINVAL
    # top_k + |W| beyond the slot limit while top_k is below |Omega|
    big = (ctypes.c_int64 * 2)(0, 70000)
    L2 = lay(L=200000)
    assert lib.topk_attn_decode_int8_static(ctypes.byref(L2), FAKE, FAKE, FAKE, FAKE, FAKE,
                                            (ctypes.c_int64 * 2)(70000, 190000), 1, big, 1, 8, 16,
                                            ctypes.c_float(0.1), None, None, FAKE, FAKE, FAKE, 1 << 40,
                                            None) == native.STDK_EUNSUPPORTED
    a = lib.topk_attn_decode_int8_static_workspace_size(ctypes.byref(L), 2872, 628, 64, 512)
    assert a >= lib.topk_attn_decode_int8_workspace_size(ctypes.byref(L), 2872, 64, 512)
    assert a >= lib.topk_attn_decode_static_workspace_size(ctypes.byref(L), 2872, 628, 64)
    assert lib.topk_attn_decode_int8_static_workspace_size(ctypes.byref(L), 2872, 628, 64, 32) == 0
