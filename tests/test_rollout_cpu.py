"""The native 1F1C planner and round runner on the host, without a GPU: every plan
equals the schedule oracle's, the table state carries from round to round, and the
runner refuses bad arguments before enqueuing anything."""
import ctypes

import pytest

import chunk_causal_dit_amd as wf
from oracle import schedule as SC
from test_abi_cpu import HostPools, L, make_cache, table  # noqa: F401  (fixture)

WF_OK, WF_E_NULL, WF_E_SHAPE, WF_E_FULL = 0, -1, -2, -5

LAYOUTS = [(1, 1, 0), (1, 9, 1), (2, 7, 0), (3, 2, 5), (4, 1, 2), (4, 3, 2), (4, 8, 2), (4, 20, 6),
           (5, 8, 3), (5, 40, 6), (6, 11, 4), (62, 3, 1), (4, 133, 57)]


@pytest.mark.parametrize("S,F,W", LAYOUTS)
def test_plans_equal_the_oracle(L, S, F, W):
    R = wf.rounds_1f1c(S, F)
    assert R == SC.n_rounds(S, F)
    for r in range(R):
        p = wf.plan_1f1c(S, F, W, r)
        ref = SC.round_plan(S, F, W, r)
        assert p.round == r
        assert p.inflight == ref["inflight"]
        assert p.hist == ref["hist"]
        assert p.new == ref["new"] and p.output == ref["output"]


@pytest.mark.parametrize("S,F,W", LAYOUTS)
def test_table_state_carries_between_rounds(L, S, F, W):
    """Append the new chunk, evict after attention: the entries held at each round's
    attention are exactly that round's history then its in-flight chunks."""
    held = []
    R = wf.rounds_1f1c(S, F)
    for r in range(R):
        p = wf.plan_1f1c(S, F, W, r)
        assert len(held) == p.n_hist + p.n_inflight - (p.new is not None)
        if p.new is not None:
            held.append(p.new)
        assert held == p.hist + [c for c, _ in p.inflight]
        assert len(held) <= W + S + 1
        assert 0 <= p.evict_after <= len(held)
        del held[:p.evict_after]
    assert wf.plan_1f1c(S, F, W, R - 1).evict_after == 0


def test_planner_argument_errors(L):
    p = wf.RoundPlan()
    assert L.wf_1f1c_rounds(0, 5) == WF_E_SHAPE
    assert L.wf_1f1c_rounds(4, 0) == WF_E_SHAPE
    assert L.wf_1f1c_rounds(wf.WF_MAX_TABLE, 5) == WF_E_SHAPE  # more stages than table entries
    assert L.wf_1f1c_plan(4, 6, 2, 0, None) == WF_E_NULL
    assert L.wf_1f1c_plan(4, 6, -1, 0, ctypes.byref(p)) == WF_E_SHAPE
    assert L.wf_1f1c_plan(4, 6, wf.WF_MAX_TABLE - 4, 0, ctypes.byref(p)) == WF_E_SHAPE  # window + stages > table
    assert L.wf_1f1c_plan(4, 6, 2, 9, ctypes.byref(p)) == WF_E_SHAPE  # past the last round
    assert L.wf_1f1c_plan(4, 6, 2, -1, ctypes.byref(p)) == WF_E_SHAPE
    assert L.wf_1f1c_plan(4, 6, 2, 8, ctypes.byref(p)) == WF_OK


def test_run_round_refuses_before_enqueuing(L):
    h, pools = make_cache(L, n_slots=8, C=64, H=2, D=64)
    a = ctypes.c_void_p(pools.k.value)
    plan = wf.plan_1f1c(4, 6, 2, 1)  # expects 1 entry held before the round (chunk 0), appends chunk 1
    ptrs = (ctypes.c_void_p * 2)(a.value, a.value)
    run = L.wf_1f1c_run_round
    assert run(None, ctypes.byref(plan), a, ptrs, ptrs, 0.1, None, a, None, None) == WF_E_NULL
    assert run(h, None, a, ptrs, ptrs, 0.1, None, a, None, None) == WF_E_NULL
    assert run(h, ctypes.byref(plan), a, ptrs, ptrs, 0.1, None, a, None, None) == WF_E_SHAPE  # table empty, 1 expected
    assert table(L, h) == []
    plan0 = wf.plan_1f1c(4, 6, 2, 0)
    bad = (ctypes.c_void_p * 1)(a.value + 8)
    assert run(h, ctypes.byref(plan0), a, bad, bad, 0.1, None, a, None, None) == WF_E_SHAPE  # misaligned K/V
    nul = (ctypes.c_void_p * 1)(None)
    assert run(h, ctypes.byref(plan0), a, nul, nul, 0.1, None, a, None, None) == WF_E_NULL
    one = (ctypes.c_void_p * 1)(a.value)
    assert run(h, ctypes.byref(plan0), a, one, one, 0.0, None, a, None, None) == WF_E_SHAPE  # scale
    assert run(h, ctypes.byref(plan0), ctypes.c_void_p(a.value + 4), one, one, 0.1, None, a, None, None) == WF_E_SHAPE
    wsb = ctypes.c_void_p(a.value + 128)  # workspace not 256-byte aligned
    assert run(h, ctypes.byref(plan0), a, one, one, 0.1, wsb, a, None, None) == WF_E_SHAPE
    assert run(h, ctypes.byref(plan0), a, one, one, 0.1, a, a, None, None) == WF_E_SHAPE  # workspace overlaps out
    assert b"overlaps" in L.wf_last_error()
    forged = wf.plan_1f1c(4, 6, 2, 0)
    forged.evict_after = 5
    assert run(h, ctypes.byref(forged), a, one, one, 0.1, None, a, None, None) == WF_E_SHAPE
    assert table(L, h) == []
    L.wf_kv_cache_destroy(h)


def test_run_round_too_large_for_one_launch(L):
    """A round whose attention launch would exceed 2^32 work-items (2^20-token chunks,
    1024 heads): WF_E_SHAPE before the append is enqueued, the table unchanged."""
    h, pools = make_cache(L, n_slots=4, C=1 << 20, H=1024, D=64)
    a = ctypes.c_void_p(pools.k.value)
    plan0 = wf.plan_1f1c(4, 6, 2, 0)  # round 0: appends chunk 0, one chunk in flight
    one = (ctypes.c_void_p * 1)(a.value)
    assert L.wf_1f1c_run_round(h, ctypes.byref(plan0), a, one, one, 0.1, None, a, None, None) == WF_E_SHAPE
    assert b"exceed one launch" in L.wf_last_error()
    assert table(L, h) == []
    L.wf_kv_cache_destroy(h)


def test_run_round_full_cache(L):
    """No free slot for the new chunk: WF_E_FULL before anything is enqueued."""
    h, pools = make_cache(L, n_slots=1, C=64, H=2, D=64)
    a = ctypes.c_void_p(pools.k.value)
    arr = (ctypes.c_int * 1)(0)
    assert L.wf_kv_set_table(h, arr, 1) == WF_OK  # the one slot holds chunk 0
    plan = wf.plan_1f1c(4, 6, 2, 1)
    ptrs = (ctypes.c_void_p * 2)(a.value, a.value)
    assert L.wf_1f1c_run_round(h, ctypes.byref(plan), a, ptrs, ptrs, 0.1, None, a, None, None) == WF_E_FULL
    assert table(L, h) == [0]
    L.wf_kv_cache_destroy(h)


def test_run_round_rope_checks(L):
    """With a RoPE geometry the in-flight chunk ids must be consecutive and their frame
    positions exact in fp32; both are refused before anything is enqueued."""
    h, pools = make_cache(L, n_slots=8, C=64, H=2, D=64)
    assert L.wf_kv_set_rope(h, 1, 8, 8, 22, 22, 20, 1e4) == WF_OK
    a = ctypes.c_void_p(pools.k.value)
    one = (ctypes.c_void_p * 1)(a.value)
    plan = wf.plan_1f1c(4, 6, 2, 0)
    plan.inflight_chunk[0] = 1 << 24  # frame position 2^24 and beyond: not exact in fp32
    assert L.wf_1f1c_run_round(h, ctypes.byref(plan), a, one, one, 0.1, None, a, None, None) == WF_E_SHAPE
    arr = (ctypes.c_int * 1)(0)
    assert L.wf_kv_set_table(h, arr, 1) == WF_OK
    plan1 = wf.plan_1f1c(4, 6, 2, 1)  # chunks 0, 1 in flight
    plan1.inflight_chunk[1] = 5  # not consecutive
    two = (ctypes.c_void_p * 2)(a.value, a.value)
    assert L.wf_1f1c_run_round(h, ctypes.byref(plan1), a, two, two, 0.1, None, a, None, None) == WF_E_SHAPE
    assert table(L, h) == [0]
    L.wf_kv_cache_destroy(h)
