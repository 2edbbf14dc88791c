"""The C ABI on the host, without a GPU: the library loads, exports exactly the
functions include/wf.h declares, and every argument check returns its status
code before any device work (a failed call leaves the cache table unchanged)."""
import ctypes
import os

import pytest

import chunk_causal_dit_amd as wf

WF_OK, WF_E_NULL, WF_E_SHAPE, WF_E_DTYPE, WF_E_SLOT, WF_E_FULL, WF_E_EMPTY, WF_E_UNSUPPORTED, WF_E_HIP = \
    0, -1, -2, -3, -4, -5, -6, -7, -8


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(wf.library_path()):
        from chunk_causal_dit_amd.build import build
        build()
    return wf.lib()


class HostPools:
    """256-byte aligned host addresses standing in for device pools (never dereferenced)."""

    def __init__(self, nbytes=1 << 16):
        self.buf = ctypes.create_string_buffer(nbytes + 512)
        base = (ctypes.addressof(self.buf) + 255) // 256 * 256
        self.k = ctypes.c_void_p(base)
        self.v = ctypes.c_void_p(base + 256)


def make_cache(L, n_slots=6, C=64, H=2, D=64, dtype=wf.WF_BF16):
    pools = HostPools()
    h = ctypes.c_void_p()
    assert L.wf_kv_cache_create(ctypes.byref(h), pools.k, pools.v, n_slots, C, H, D, dtype, wf.WF_KV_ADOPT,
                                None) == WF_OK
    return h, pools


def table(L, h):
    arr = (ctypes.c_int * 64)()
    n = ctypes.c_int()
    assert L.wf_kv_get_table(h, arr, 64, ctypes.byref(n)) == WF_OK
    return list(arr[: n.value])


def set_table(L, h, slots):
    arr = (ctypes.c_int * max(1, len(slots)))(*slots)
    return L.wf_kv_set_table(h, arr, len(slots))


def test_exports_match_header(L):
    declared = wf.header_symbols()
    exported = wf.exported_symbols()
    assert declared == exported, (sorted(set(declared) - set(exported)), sorted(set(exported) - set(declared)))
    assert len(declared) == 27


def test_device_peak_info_argument_errors(L):
    n = ctypes.c_int()
    assert L.wf_device_peak_info(0, None, ctypes.byref(n)) == WF_E_NULL
    assert L.wf_device_peak_info(0, ctypes.byref(n), None) == WF_E_NULL


def test_version_and_status_strings(L):
    assert L.wf_version() == 100
    for code in (WF_OK, WF_E_NULL, WF_E_SHAPE, WF_E_DTYPE, WF_E_SLOT, WF_E_FULL, WF_E_EMPTY, WF_E_UNSUPPORTED,
                 WF_E_HIP):
        assert L.wf_status_str(code).decode().startswith("WF_")
    assert L.wf_status_str(-99) == b"unknown status"


def test_pool_bytes(L):
    # S_pad = chunk rounded up to 128 tokens; one pool = n_slots * H * S_pad * D * elem
    assert L.wf_kv_pool_bytes(7, 4680, 12, 128, wf.WF_BF16) == 7 * 12 * 4736 * 128 * 2
    assert L.wf_kv_pool_bytes(5, 64, 2, 64, wf.WF_F32) == 5 * 2 * 128 * 64 * 4
    assert L.wf_kv_pool_bytes(5, 64, 2, 96, wf.WF_F32) == 0
    assert b"head_dim" in L.wf_last_error()
    assert L.wf_kv_pool_bytes(0, 64, 2, 64, wf.WF_F32) == 0
    assert L.wf_kv_pool_bytes(65, 64, 2, 64, wf.WF_F32) == 0
    assert L.wf_kv_pool_bytes(5, 0, 2, 64, wf.WF_F32) == 0
    assert L.wf_kv_pool_bytes(5, 64, 2, 64, 7) == 0


def test_create_argument_errors(L):
    pools = HostPools()
    h = ctypes.c_void_p()
    args = lambda **kw: dict(dict(n=4, C=64, H=2, D=64, dt=wf.WF_BF16, fl=wf.WF_KV_ADOPT), **kw)

    def create(k=pools.k, v=pools.v, **kw):
        a = args(**kw)
        return L.wf_kv_cache_create(ctypes.byref(h), k, v, a["n"], a["C"], a["H"], a["D"], a["dt"], a["fl"], None)

    assert L.wf_kv_cache_create(None, pools.k, pools.v, 4, 64, 2, 64, 1, 0, None) == WF_E_NULL
    assert create(k=None) == WF_E_NULL
    assert create(D=80) == WF_E_UNSUPPORTED
    assert create(dt=2) == WF_E_DTYPE
    assert create(n=0) == WF_E_SHAPE
    assert create(C=(1 << 20) + 1) == WF_E_SHAPE
    assert create(H=0) == WF_E_SHAPE
    assert create(fl=5) == WF_E_SHAPE
    misaligned = ctypes.c_void_p(pools.k.value + 16)
    assert create(k=misaligned) == WF_E_SHAPE
    assert create() == WF_OK
    assert L.wf_kv_cache_destroy(h) == WF_OK
    assert L.wf_kv_cache_destroy(None) == WF_OK


def test_table_operations(L):
    h, pools = make_cache(L, n_slots=6)
    assert table(L, h) == []
    assert set_table(L, h, [4, 1, 3]) == WF_OK
    assert table(L, h) == [4, 1, 3]
    # invalid edits leave the table unchanged
    assert set_table(L, h, [0, 0]) == WF_E_SLOT
    assert set_table(L, h, [0, 6]) == WF_E_SLOT
    assert set_table(L, h, [-1]) == WF_E_SLOT
    assert set_table(L, h, list(range(7))) == WF_E_SHAPE
    assert table(L, h) == [4, 1, 3]
    assert L.wf_kv_evict(h, 4) == WF_E_EMPTY
    assert L.wf_kv_evict(h, -1) == WF_E_SHAPE
    assert table(L, h) == [4, 1, 3]
    assert L.wf_kv_evict(h, 1) == WF_OK
    assert table(L, h) == [1, 3]
    assert L.wf_kv_evict(h, 0) == WF_OK
    assert L.wf_kv_evict(None, 1) == WF_E_NULL
    # get_table with a small buffer still reports the full length
    arr = (ctypes.c_int * 1)()
    n = ctypes.c_int()
    assert L.wf_kv_get_table(h, arr, 1, ctypes.byref(n)) == WF_OK
    assert n.value == 2 and arr[0] == 1
    assert L.wf_kv_get_table(h, None, 0, ctypes.byref(n)) == WF_OK and n.value == 2
    assert L.wf_kv_get_table(h, None, 1, ctypes.byref(n)) == WF_E_NULL
    assert L.wf_kv_get_table(h, arr, 1, None) == WF_E_NULL
    L.wf_kv_cache_destroy(h)


def test_refresh_and_append_argument_errors(L):
    h, pools = make_cache(L, n_slots=2)
    k = ctypes.c_void_p(pools.k.value)
    assert L.wf_kv_refresh(h, 0, k, k, None) == WF_E_SLOT  # empty table
    assert L.wf_kv_append(h, None, k, None, None) == WF_E_NULL
    assert L.wf_kv_append(h, ctypes.c_void_p(k.value + 4), k, None, None) == WF_E_SHAPE
    assert set_table(L, h, [0, 1]) == WF_OK
    assert L.wf_kv_append(h, k, k, None, None) == WF_E_FULL  # every slot in use
    assert L.wf_kv_refresh(h, 2, k, k, None) == WF_E_SLOT
    assert L.wf_kv_refresh(h, -1, k, k, None) == WF_E_SLOT
    assert table(L, h) == [0, 1]
    L.wf_kv_cache_destroy(h)


def test_attention_argument_errors(L):
    h, pools = make_cache(L, n_slots=4)
    q = ctypes.c_void_p(pools.k.value)
    lse = ctypes.cast(ctypes.c_void_p(pools.v.value), ctypes.POINTER(ctypes.c_float))
    f = L.wf_chunk_causal_attn_fwd
    assert f(None, h, 1, 0.1, q, None, None) == WF_E_NULL
    assert f(q, None, 1, 0.1, q, None, None) == WF_E_NULL
    assert f(q, h, 1, 0.1, None, None, None) == WF_E_NULL
    assert f(q, h, 1, 0.1, q, None, None) == WF_E_EMPTY  # empty table
    assert set_table(L, h, [2, 0, 1]) == WF_OK
    assert f(q, h, 0, 0.1, q, None, None) == WF_E_SHAPE
    assert f(q, h, 4, 0.1, q, None, None) == WF_E_EMPTY
    assert f(q, h, 2, 0.0, q, None, None) == WF_E_SHAPE
    assert f(q, h, 2, -0.1, q, None, None) == WF_E_SHAPE
    assert f(q, h, 2, float("inf"), q, None, None) == WF_E_SHAPE
    assert f(ctypes.c_void_p(q.value + 2), h, 2, 0.1, q, None, None) == WF_E_SHAPE
    bad_lse = ctypes.cast(ctypes.c_void_p(pools.v.value + 2), ctypes.POINTER(ctypes.c_float))
    assert f(q, h, 2, 0.1, q, bad_lse, None) == WF_E_SHAPE
    # the workspace variant: same checks, plus a 256-byte aligned workspace (NULL allowed)
    fw = L.wf_chunk_causal_attn_fwd_ws
    ws = ctypes.c_void_p(pools.v.value)
    assert fw(None, h, 2, 0.1, ws, q, None, None) == WF_E_NULL
    assert fw(q, h, 4, 0.1, ws, q, None, None) == WF_E_EMPTY
    assert fw(q, h, 2, 0.0, None, q, None, None) == WF_E_SHAPE
    assert fw(q, h, 2, 0.1, ctypes.c_void_p(ws.value + 64), q, None, None) == WF_E_SHAPE
    # bf16 cache, H=2, C=64 (make_cache defaults), D=64: 2 halves x H x C rows of D fp32 + (max, sum)
    assert L.wf_attn_fwd_workspace_bytes(h) == 2 * 2 * 64 * 64 * 4 + 2 * 2 * 64 * 8
    assert L.wf_attn_fwd_workspace_bytes(None) == 0
    # the int8 variant: needs bf16 and head_dim 128
    g = L.wf_chunk_causal_attn_fwd_i8qk
    assert g(q, h, 2, 0.1, None, q, lse, None) == WF_E_NULL
    assert g(q, h, 2, 0.1, ws, q, lse, None) == WF_E_UNSUPPORTED  # head_dim 64
    assert L.wf_attn_i8qk_workspace_bytes(h, 2) == 0
    L.wf_kv_cache_destroy(h)
    h32, p32 = make_cache(L, n_slots=4, D=128, dtype=wf.WF_F32)
    assert g(q, h32, 2, 0.1, ws, q, lse, None) == WF_E_DTYPE
    assert L.wf_attn_fwd_workspace_bytes(h32) == 0  # fp32 rounds never split
    L.wf_kv_cache_destroy(h32)


def test_static_scratch_call_refuses_before_any_launch(L):
    """wf_chunk_causal_attn_fwd_static: the attention call's argument checks, and a cache
    whose key-split partials exceed the 64 MiB static scratch refused with WF_E_SHAPE."""
    fs = L.wf_chunk_causal_attn_fwd_static
    h, pools = make_cache(L, n_slots=4)
    q = ctypes.c_void_p(pools.k.value)
    assert fs(None, h, 1, 0.1, q, None, None) == WF_E_NULL
    assert fs(q, None, 1, 0.1, q, None, None) == WF_E_NULL
    assert fs(q, h, 1, 0.1, q, None, None) == WF_E_EMPTY
    assert set_table(L, h, [2, 0, 1]) == WF_OK
    assert fs(q, h, 4, 0.1, q, None, None) == WF_E_EMPTY
    assert fs(q, h, 2, 0.0, q, None, None) == WF_E_SHAPE
    L.wf_kv_cache_destroy(h)
    # 14 heads of 4680 tokens, head_dim 128: 2 x 14 x 4680 x (4 x 128 + 8) bytes > 64 MiB
    big, bp = make_cache(L, n_slots=3, C=4680, H=14, D=128)
    assert set_table(L, big, [0, 1, 2]) == WF_OK
    need = L.wf_attn_fwd_workspace_bytes(big)
    assert need > 64 << 20
    st = fs(ctypes.c_void_p(bp.k.value), big, 2, 0.1, ctypes.c_void_p(bp.k.value), None, None)
    assert st == WF_E_SHAPE and b"static" in L.wf_last_error()
    assert table(L, big) == [0, 1, 2]
    L.wf_kv_cache_destroy(big)


def test_workspace_overlap_refused(L):
    """A workspace that overlaps q, out, lse or a cache pool is refused before any launch."""
    import torch
    buf = ctypes.create_string_buffer((1 << 20) + 512)
    base = (ctypes.addressof(buf) + 255) // 256 * 256
    q, out = ctypes.c_void_p(base), ctypes.c_void_p(base + (64 << 10))
    lse_addr = base + (128 << 10)
    lse = ctypes.cast(ctypes.c_void_p(lse_addr), ctypes.POINTER(ctypes.c_float))
    fw = L.wf_chunk_causal_attn_fwd_ws
    h, pools = make_cache(L, n_slots=4)  # bf16, C = 64, H = 2, D = 64
    assert set_table(L, h, [2, 0, 1]) == WF_OK
    wsb = L.wf_attn_fwd_workspace_bytes(h)
    for ws in (q.value, out.value - 256, lse_addr, pools.k.value, pools.v.value + 256):
        assert fw(q, h, 2, 0.1, ctypes.c_void_p(ws), out, lse, None) == WF_E_SHAPE, hex(ws - base)
        assert b"overlaps" in L.wf_last_error()
    if not torch.cuda.is_available():  # disjoint (ending right where q starts): passes the checks, fails at launch
        ws_end_at_q = ctypes.c_void_p(base + (256 << 10))
        q2 = ctypes.c_void_p(ws_end_at_q.value + wsb)
        assert fw(q2, h, 2, 0.1, ws_end_at_q, out, lse, None) == WF_E_HIP
    L.wf_kv_cache_destroy(h)
    h, pools = make_cache(L, n_slots=4, D=128)  # the int8 variant
    assert set_table(L, h, [2, 0, 1]) == WF_OK
    g = L.wf_chunk_causal_attn_fwd_i8qk
    assert L.wf_attn_i8qk_workspace_bytes(h, 2) > 0
    for ws in (q.value, out.value - 256, lse_addr):
        assert g(q, h, 2, 0.1, ctypes.c_void_p(ws), out, lse, None) == WF_E_SHAPE, hex(ws - base)
    L.wf_kv_cache_destroy(h)


def test_i8qk_scale_table_limit(L):
    """The int8 call keeps the K block scales of every table entry in LDS: table length x
    128-token blocks per chunk must stay <= 16384. 64 entries of 257 blocks (C = 32,896)
    are refused on the host with WF_E_SHAPE; 64 x 256 blocks pass that check (and, with
    no GPU, fail only at the launch)."""
    h, pools = make_cache(L, n_slots=64, C=128 * 257, H=1, D=128)
    assert set_table(L, h, list(range(64))) == WF_OK
    q = ctypes.c_void_p(pools.k.value)
    ws = ctypes.c_void_p(pools.v.value + (1 << 20))
    g = L.wf_chunk_causal_attn_fwd_i8qk
    assert g(q, h, 2, 0.1, ws, q, None, None) == WF_E_SHAPE
    assert b"exceeds 16384" in L.wf_last_error()
    L.wf_kv_cache_destroy(h)
    import torch

    if not torch.cuda.is_available():  # the pointers are host stand-ins: launch only where it fails cleanly
        h, pools = make_cache(L, n_slots=64, C=128 * 256, H=1, D=128)
        assert set_table(L, h, list(range(64))) == WF_OK
        far = lambda gib: ctypes.c_void_p(pools.k.value + (gib << 30))  # past the 0.5 GiB pools, disjoint
        assert g(far(4), h, 2, 0.1, far(6), far(5), None, None) == WF_E_HIP, L.wf_last_error()
        assert b"exceeds 16384" not in L.wf_last_error()
        L.wf_kv_cache_destroy(h)


def test_attention_launch_size_limit(L):
    """A round whose launch would exceed 2^32 work-items is refused on the host:
    2^20-token chunks x 1024 heads (the largest shape a cache accepts)."""
    h, pools = make_cache(L, n_slots=2, C=1 << 20, H=1024, D=64)
    assert set_table(L, h, [0, 1]) == WF_OK
    q = ctypes.c_void_p(pools.k.value)
    assert L.wf_chunk_causal_attn_fwd(q, h, 1, 0.1, q, None, None) == WF_E_SHAPE
    assert b"exceed one launch" in L.wf_last_error()
    assert L.wf_chunk_causal_attn_fwd_ws(q, h, 1, 0.1, None, q, None, None) == WF_E_SHAPE
    L.wf_kv_cache_destroy(h)


def test_rope_argument_errors(L):
    pools = HostPools()
    x = pools.k
    r = L.wf_rope3d
    assert r(None, 4, 1, 128, 1, 0, 1, 2, 2, 44, 42, 42, 1e4, None) == WF_E_NULL
    assert r(x, 4, 1, 128, 1, 0, 1, 2, 2, 44, 42, 40, 1e4, None) == WF_E_SHAPE  # split sum
    assert r(x, 4, 1, 128, 1, 0, 1, 2, 2, 43, 43, 42, 1e4, None) == WF_E_SHAPE  # odd split
    assert r(x, 6, 1, 128, 1, 0, 1, 2, 2, 44, 42, 42, 1e4, None) == WF_E_SHAPE  # not whole chunks
    assert r(x, 4, 1, 128, 1, 0, 1, 2, 2, 44, 42, 42, -1.0, None) == WF_E_SHAPE
    assert r(x, 4, 1, 96, 1, 0, 1, 2, 2, 32, 32, 32, 1e4, None) == WF_E_UNSUPPORTED
    assert r(x, 4, 1, 128, 5, 0, 1, 2, 2, 44, 42, 42, 1e4, None) == WF_E_DTYPE
    assert r(x, 4, 1, 128, 1, -1, 1, 2, 2, 44, 42, 42, 1e4, None) == WF_E_SHAPE
    assert r(x, 0, 1, 128, 1, 0, 1, 2, 2, 44, 42, 42, 1e4, None) == WF_OK  # nothing to do
    assert r(x, (1 << 27) + 4, 1, 128, 1, 0, 1, 2, 2, 44, 42, 42, 1e4, None) == WF_E_SHAPE  # launch too large


def test_fused_rope_write_argument_errors(L):
    """set_rope geometry checks; append_rope/refresh_rope refuse before any launch and leave the table as is."""
    h, pools = make_cache(L, n_slots=3, C=60, H=2, D=128)
    k = ctypes.c_void_p(pools.k.value)
    slot = ctypes.c_int(-1)
    assert L.wf_kv_append_rope(h, k, k, 0, None, ctypes.byref(slot)) == WF_E_UNSUPPORTED  # no geometry yet
    assert L.wf_kv_set_rope(None, 3, 4, 5, 44, 42, 42, 1e4) == WF_E_NULL
    assert L.wf_kv_set_rope(h, 3, 4, 4, 44, 42, 42, 1e4) == WF_E_SHAPE   # 3*4*4 != 60 tokens
    assert L.wf_kv_set_rope(h, 3, 4, 5, 44, 42, 40, 1e4) == WF_E_SHAPE   # split does not sum to 128
    assert L.wf_kv_set_rope(h, 3, 4, 5, 44, 42, 42, 0.0) == WF_E_SHAPE
    assert L.wf_kv_set_rope(h, 3, 4, 5, 44, 42, 42, 1e4) == WF_OK
    assert L.wf_kv_append_rope(h, None, k, 0, None, ctypes.byref(slot)) == WF_E_NULL
    assert L.wf_kv_append_rope(h, ctypes.c_void_p(pools.k.value + 4), k, 0, None, None) == WF_E_SHAPE
    assert L.wf_kv_append_rope(h, k, k, -1, None, None) == WF_E_SHAPE  # negative chunk index
    assert L.wf_kv_append_rope(h, k, k, 1 << 23, None, None) == WF_E_SHAPE  # frames beyond exact fp32
    assert L.wf_kv_refresh_rope(h, 0, k, k, 0, None) == WF_E_SLOT  # empty table
    assert table(L, h) == [] and slot.value == -1
    L.wf_kv_cache_destroy(h)


def test_w8a8_argument_errors(L):
    """Row quantization and the W8A8 GEMM refuse bad arguments before any launch; zero rows are a no-op."""
    p = HostPools()
    a = ctypes.c_void_p(p.k.value)
    f = ctypes.cast(ctypes.c_void_p(p.v.value), ctypes.POINTER(ctypes.c_float))
    q = L.wf_quant_rows_i8
    assert q(None, 4, 64, wf.WF_BF16, a, f, None) == WF_E_NULL
    assert q(a, 4, 64, wf.WF_BF16, a, None, None) == WF_E_NULL
    assert q(a, 4, 64, wf.WF_F32, a, f, None) == WF_E_DTYPE
    assert q(a, 4, 60, wf.WF_BF16, a, f, None) == WF_E_SHAPE  # cols not a multiple of 8
    assert q(a, -1, 64, wf.WF_BF16, a, f, None) == WF_E_SHAPE
    assert q(a, (1 << 24) + 1, 64, wf.WF_BF16, a, f, None) == WF_E_SHAPE
    assert q(ctypes.c_void_p(a.value + 8), 4, 64, wf.WF_BF16, a, f, None) == WF_E_SHAPE  # misaligned x
    assert q(a, 0, 64, wf.WF_BF16, a, f, None) == WF_OK
    g = L.wf_gemm_w8a8
    assert g(None, f, a, f, None, 4, 8, 64, wf.WF_BF16, a, None) == WF_E_NULL
    assert g(a, None, a, f, None, 4, 8, 64, wf.WF_BF16, a, None) == WF_E_NULL  # bf16 output needs scales
    assert g(a, f, a, f, None, 4, 8, 64, wf.WF_F32, a, None) == WF_E_DTYPE
    assert g(a, f, a, f, None, 4, 12, 64, wf.WF_BF16, a, None) == WF_E_SHAPE  # N % 8
    assert g(a, f, a, f, None, 4, 8, 96, wf.WF_BF16, a, None) == WF_E_SHAPE   # K % 64
    assert g(a, f, a, f, None, 4, 8, 131072 + 64, wf.WF_BF16, a, None) == WF_E_SHAPE  # int32 range
    assert g(a, f, a, f, None, 1 << 30, 1 << 20, 64, wf.WF_BF16, a, None) == WF_E_SHAPE  # grid size
    assert g(ctypes.c_void_p(a.value + 4), f, a, f, None, 4, 8, 64, wf.WF_BF16, a, None) == WF_E_SHAPE
    assert g(a, None, a, None, None, 0, 8, 64, wf.WF_I32, a, None) == WF_OK


def test_no_gpu_launch_fails_cleanly(L):
    """Without a device a launch is refused: WF_E_HIP, and append leaves the table unchanged."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: launches would succeed")
    h, pools = make_cache(L, n_slots=3)
    k = ctypes.c_void_p(pools.k.value)
    slot = ctypes.c_int(-1)
    assert L.wf_kv_append(h, k, k, None, ctypes.byref(slot)) == WF_E_HIP
    assert b"HIP" in L.wf_last_error()
    assert table(L, h) == [] and slot.value == -1
    L.wf_kv_cache_destroy(h)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    """No silent fallback: a missing library raises at first use."""
    monkeypatch.setattr(wf, "_lib", None)
    monkeypatch.setenv("WF_LIBRARY", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        wf.lib()
