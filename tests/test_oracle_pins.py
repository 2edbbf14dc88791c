"""Pins of the fp64 oracle against values fixed outside it (CPU only).

Each check compares the oracle with something it does not compute itself:
hand-derived golden values (tests/golden), an independent scalar brute force,
a second vectorised form, closed forms, and library special cases (torch CPU
scaled_dot_product_attention in float64). The mutation tests at the end plant
plausible mistakes in copies of the oracle and require that some pin fails.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle.attention as A
import oracle.quant as Q
import oracle.rope as R
from oracle.ring import RingModel

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _round_inputs(C, N, Hs, H, D, seed):
    q = _rand((N * C, H, D), seed)
    k = _rand(((Hs + N) * C, H, D), seed + 1)
    v = _rand(((Hs + N) * C, H, D), seed + 2)
    return q, k, v


# ---------------------------------------------------------------- checks
# Each check takes the attention function under test so that the mutation
# tests can run the very same checks against planted mistakes.

def check_hand_example(attn):
    rows = [l.split() for l in open(os.path.join(GOLDEN, "attn_hand_example.txt"))
            if l.strip() and not l.startswith("#")]
    q = np.array([[[math.log(2), math.log(3)]], [[math.log(2), math.log(3)]]])
    k = np.array([[[1, 0]], [[0, 1]], [[1, 1]], [[0, 0]]], dtype=np.float64)
    v = np.array([[[11, 0]], [[0, 11]], [[1, 1]], [[0, 0]]], dtype=np.float64)
    o, lse = attn(q, k, v, 2, 1, 1.0)
    for r in rows:
        i, a, b, c, d, e = map(int, r)
        np.testing.assert_allclose(o[i, 0], [a / b, c / d], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[0, i], math.log(e), rtol=0, atol=1e-13)


def check_mask_fixture(attn):
    mask = np.loadtxt(os.path.join(GOLDEN, "mask_c2_h1_n2.txt"))
    nq, nk = mask.shape
    q = np.zeros((nq, 1, nk))
    k = _rand((nk, 1, nk), 5)
    v = np.eye(nk)[:, None, :]
    o, lse = attn(q, k, v, 1, 2, 0.7)
    expect = mask / mask.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(o[:, 0, :], expect, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0], np.log(mask.sum(axis=1)), rtol=0, atol=1e-14)


def check_bruteforce(attn, C, N, Hs, H, D, seed):
    q, k, v = _round_inputs(C, N, Hs, H, D, seed)
    scale = 1 / math.sqrt(D)
    o1, l1 = attn(q, k, v, Hs, C, scale)
    o0, l0 = A.bruteforce_attention(q, k, v, Hs, C, scale)
    np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l0, rtol=0, atol=1e-12)


def check_causality(attn, C, N, Hs, H, D, seed):
    q, k, v = _round_inputs(C, N, Hs, H, D, seed)
    scale = 1 / math.sqrt(D)
    o, l = attn(q, k, v, Hs, C, scale)
    for j in range(N - 1):
        q2, k2, v2 = q.copy(), k.copy(), v.copy()
        lo_q, lo_k = (j + 1) * C, (Hs + j + 1) * C
        q2[lo_q:] = _rand(q2[lo_q:].shape, 99 + j, 3.0)
        k2[lo_k:] = _rand(k2[lo_k:].shape, 199 + j, 3.0)
        v2[lo_k:] = _rand(v2[lo_k:].shape, 299 + j, 3.0)
        o2, l2 = attn(q2, k2, v2, Hs, C, scale)
        assert np.array_equal(o2[:lo_q], o[:lo_q])
        assert np.array_equal(l2[:, :lo_q], l[:, :lo_q])
        # and the perturbation does reach the later chunks
        assert not np.allclose(o2[lo_q:], o[lo_q:])


def check_q_zero_closed_form(attn, C, N, Hs, H, D, seed):
    _, k, v = _round_inputs(C, N, Hs, H, D, seed)
    q = np.zeros((N * C, H, D))
    o, lse = attn(q, k, v, Hs, C, 0.3)
    for j in range(N):
        L = (Hs + j + 1) * C
        mean = v[:L].mean(axis=0)  # [H][D]
        for i in range(j * C, (j + 1) * C):
            np.testing.assert_allclose(o[i], mean, rtol=0, atol=1e-13)
            np.testing.assert_allclose(lse[:, i], math.log(L), rtol=0, atol=1e-13)


ATTN = A.chunk_causal_attention


# ---------------------------------------------------------------- attention pins

def test_hand_example():
    check_hand_example(ATTN)
    check_hand_example(A.dense_masked_attention)
    check_hand_example(A.bruteforce_attention)


def test_mask_fixture():
    check_mask_fixture(ATTN)
    check_mask_fixture(A.bruteforce_attention)


@pytest.mark.parametrize("C,N,Hs,H,D", [
    (1, 1, 0, 1, 2), (1, 4, 0, 2, 3), (3, 2, 1, 2, 4), (4, 3, 2, 1, 8),
    (5, 1, 3, 2, 2), (2, 3, 0, 2, 5), (7, 2, 2, 1, 3),
])
def test_bruteforce_agrees(C, N, Hs, H, D):
    check_bruteforce(ATTN, C, N, Hs, H, D, seed=C * 100 + N * 10 + Hs)


@pytest.mark.parametrize("C,N,Hs", [(3, 3, 2), (8, 4, 1), (16, 3, 0)])
def test_dense_form_agrees(C, N, Hs):
    q, k, v = _round_inputs(C, N, Hs, 2, 16, 11)
    o1, l1 = ATTN(q, k, v, Hs, C, 0.25, block=5)  # several row blocks per chunk
    o2, l2 = A.dense_masked_attention(q, k, v, Hs, C, 0.25)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)


def test_rows_subset_and_workers():
    q, k, v = _round_inputs(16, 3, 2, 2, 16, 21)
    o, l = ATTN(q, k, v, 2, 16, 0.25)
    rows = np.array([47, 0, 16, 31, 5])
    o2, l2 = ATTN(q, k, v, 2, 16, 0.25, rows=rows, workers=4)
    # BLAS may block a different row batch differently: equal up to rounding
    np.testing.assert_allclose(o2, o[rows], rtol=0, atol=1e-14)
    np.testing.assert_allclose(l2, l[:, rows], rtol=0, atol=1e-14)


def test_token_causal_reduction_matches_sdpa():
    """C = 1 and no history: chunk-wise causal attention is token-causal attention."""
    q, k, v = _round_inputs(1, 9, 0, 3, 8, 31)
    o, lse = ATTN(q, k, v, 0, 1, 1 / math.sqrt(8))
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x.transpose(1, 0, 2)))[None]
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True)
    np.testing.assert_allclose(o, ref[0].numpy().transpose(1, 0, 2), rtol=0, atol=1e-12)


def test_single_chunk_is_full_attention_over_history_and_chunk():
    """N = 1: the one chunk sees all history and itself, i.e. plain full attention."""
    C, Hs, H, D = 6, 3, 2, 8
    q, k, v = _round_inputs(C, 1, Hs, H, D, 41)
    o, _ = ATTN(q, k, v, Hs, C, 0.5)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x.transpose(1, 0, 2)))[None]
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), scale=0.5)
    np.testing.assert_allclose(o, ref[0].numpy().transpose(1, 0, 2), rtol=0, atol=1e-12)


def test_causality_invariant():
    check_causality(ATTN, 4, 4, 2, 2, 8, 51)


def test_q_zero_closed_form():
    check_q_zero_closed_form(ATTN, 3, 3, 1, 2, 4, 61)


def test_softmax_rows_sum_to_one():
    """With V the identity over keys (value of key k = unit vector e_k), a row of O
    is that row's softmax weights: they sum to 1, vanish exactly on invisible keys,
    and two visible keys' weights stand in the ratio exp(scale * score difference)."""
    C, N, Hs, H, scale = 5, 3, 2, 2, 0.4
    nk = (Hs + N) * C
    q, k, _ = _round_inputs(C, N, Hs, H, nk, 71)  # head_dim = key count, so V can be the identity
    v = np.broadcast_to(np.eye(nk)[:, None, :], (nk, H, nk)).copy()
    o, _ = ATTN(q, k, v, Hs, C, scale)
    for h in range(H):
        for i in range(N * C):
            w = o[i, h]
            L = (Hs + i // C + 1) * C
            assert abs(w.sum() - 1.0) <= 1e-14
            assert (w[:L] > 0).all() and not w[L:].any()
            a, b = 0, L - 1
            want = math.exp(scale * float(np.dot(q[i, h], k[a, h] - k[b, h])))
            assert abs(w[a] / w[b] / want - 1.0) <= 1e-12


def test_single_visible_key_returns_its_value():
    q, k, v = _round_inputs(1, 3, 0, 2, 4, 81)
    o, lse = ATTN(q, k, v, 0, 1, 0.5)
    assert np.array_equal(o[0], v[0])
    np.testing.assert_allclose(lse[:, 0], 0.5 * np.einsum("hd,hd->h", q[0], k[0]), atol=1e-15)


def test_large_logits_stay_finite():
    q, k, v = _round_inputs(4, 2, 1, 1, 4, 91)
    o, lse = ATTN(q * 300, k * 300, v, 1, 4, 1.0)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    o2, l2 = A.dense_masked_attention(q * 300, k * 300, v, 1, 4, 1.0)
    np.testing.assert_allclose(o, o2, atol=1e-12)


def test_shape_errors():
    q, k, v = _round_inputs(4, 2, 1, 1, 4, 1)
    with pytest.raises(ValueError):
        ATTN(q[:7], k, v, 1, 4, 1.0)
    with pytest.raises(ValueError):
        ATTN(q, k[:8], v, 1, 4, 1.0)


# ---------------------------------------------------------------- RoPE pins

def _rope_golden():
    out = []
    for l in open(os.path.join(GOLDEN, "rope_hand_example.txt")):
        if l.strip() and not l.startswith("#"):
            g, t, p, _, c, s = l.split()
            out.append((int(g), int(t), int(p), float(c), float(s)))
    return out


def check_rope_golden(rope):
    x = np.tile(np.array([1.0, 0.0] * 4), (16, 1, 1))
    for g, t, p, c, s in _rope_golden():
        y = rope(x, g, 16, 1, 2, 8, split=(4, 2, 2), theta=10000.0)
        np.testing.assert_allclose(y[t, 0, 2 * p:2 * p + 2], [c, s], rtol=0, atol=1e-14)


def test_rope_golden():
    check_rope_golden(R.rope3d)


def test_rope_preserves_pair_norms():
    x = _rand((2 * 60, 3, 12), 5)
    y = R.rope3d(x, 7, 60, 3, 4, 5, split=(4, 4, 4))
    n0 = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    n1 = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    np.testing.assert_allclose(n1, n0, rtol=1e-13)


def test_rope_zero_position_is_identity():
    x = _rand((60, 2, 12), 6)
    y = R.rope3d(x, 0, 60, 3, 4, 5, split=(4, 4, 4))
    np.testing.assert_array_equal(y[0], x[0])  # frame 0, row 0, col 0


def test_rope_relative_position_property():
    """Rotating q and k by positions shifted by a common frame offset leaves q.k unchanged."""
    C, H, D = 60, 2, 12
    q = _rand((2 * C, H, D), 7)
    k = _rand((2 * C, H, D), 8)
    s = []
    for g0 in (0, 5):
        qr = R.rope3d(q, g0, C, 3, 4, 5, split=(4, 4, 4))
        kr = R.rope3d(k, g0, C, 3, 4, 5, split=(4, 4, 4))
        s.append(np.einsum("ihd,jhd->hij", qr, kr))
    np.testing.assert_allclose(s[0], s[1], rtol=0, atol=1e-12)


def test_rope_positions_layout():
    pos = R.token_positions(2 * 4680, 3, 4680, 3, 30, 52)
    assert tuple(pos[0]) == (9, 0, 0)
    assert tuple(pos[52]) == (9, 1, 0)
    assert tuple(pos[1560]) == (10, 0, 0)
    assert tuple(pos[4679]) == (11, 29, 51)
    assert tuple(pos[4680]) == (12, 0, 0)


# ---------------------------------------------------------------- int8 pins

def _int8_golden():
    lines = [l.split() for l in open(os.path.join(GOLDEN, "int8_hand_example.txt"))
             if l.strip() and not l.startswith("#")]
    for i in range(0, len(lines), 3):
        yield (np.array(lines[i][1:], dtype=np.float32), float(lines[i + 1][1]),
               np.array(lines[i + 2][1:], dtype=np.int64))


def check_int8_golden(quantize):
    for vals, s, codes in _int8_golden():
        x = vals.reshape(-1, 1, 1)
        c, sc = quantize(x, len(vals))
        assert sc.shape == (1, 1) and sc[0, 0] == np.float32(s)
        np.testing.assert_array_equal(c[:, 0, 0].astype(np.int64), codes)


def test_int8_golden():
    check_int8_golden(Q.quantize_chunk_blocks)


def test_int8_block_boundaries_and_error_bound():
    x = (_rand((2 * 300, 2, 16), 9) * 3).astype(np.float32)
    codes, scales = Q.quantize_chunk_blocks(x, 300)
    assert scales.shape == (2, 2 * 3)  # blocks 128, 128, 44 per chunk
    xd = Q.dequantize(codes, scales, 300)
    t = np.arange(600)
    s = scales[:, (t // 300) * 3 + (t % 300) // 128].T[:, :, None]
    assert (np.abs(x - xd) <= s / 2 * (1 + 1e-6)).all()
    assert np.abs(codes).max() == 127


def test_int8_kmean_shift_keeps_attention_exact():
    """One per-(head, channel) key shift leaves every row's softmax unchanged."""
    C, N, Hs, H, D = 4, 3, 2, 2, 8
    q, k, v = _round_inputs(C, N, Hs, H, D, 13)
    mean = k.mean(axis=0)
    o1, l1 = ATTN(q, k, v, Hs, C, 0.35)
    o2, l2 = ATTN(q, k - mean[None], v, Hs, C, 0.35)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2 + 0.35 * np.einsum("ihd,hd->hi", q, mean), l1, atol=1e-12)


def _kmean_golden():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "int8_kmean_hand_example.txt"))
            if l.strip() and not l.startswith("#")]
    g = {"key": [], "block": []}
    for r in rows:
        if r[0] in ("key", "block"):
            g[r[0]].append([float(x) for x in r[1:]])
        else:
            g[r[0]] = [float(x) for x in r[1:]]
    return g


def check_kmean_golden(quantize_round):
    """The hand-derived key mean, K' block scales and codes (tests/golden)."""
    g = _kmean_golden()
    C, Hs = int(g["chunk_tokens"][0]), int(g["n_hist"][0])
    k = np.array(g["key"], dtype=np.float32)[:, None, :]  # [8][1 head][2 channels]
    n_chunks = k.shape[0] // C
    q = np.zeros(((n_chunks - Hs) * C, 1, 2), dtype=np.float32)
    r = quantize_round(q, k, Hs, C)
    np.testing.assert_array_equal(r["mean"], np.array([g["mean"]], dtype=np.float32))
    for c, blk in enumerate(g["block"]):
        assert r["k_scales"][0, c] == np.float32(blk[0]) / np.float32(127), f"chunk {c} scale"
        np.testing.assert_array_equal(r["k_codes"][c * C:(c + 1) * C, 0, :].ravel().astype(np.int64),
                                      np.array(blk[1:], dtype=np.int64), err_msg=f"chunk {c} codes")


def check_quantized_causality(quantize_round):
    """Quantized attention is chunk-wise causal too: Q, K and V of the chunks after
    in-flight chunk j perturbed, chunks 0..j keep bitwise equal O and LSE."""
    C, N, Hs, H, D = 6, 3, 2, 2, 8
    q, k, v = (a.astype(np.float32) for a in _round_inputs(C, N, Hs, H, D, 23))

    def run(q, k, v):
        return Q.quantized_attention(q, k, v, Hs, C, 0.3, quant=quantize_round(q, k, Hs, C))

    o, l = run(q, k, v)
    for j in range(N - 1):
        q2, k2, v2 = q.copy(), k.copy(), v.copy()
        lo_q, lo_k = (j + 1) * C, (Hs + j + 1) * C
        q2[lo_q:] = _rand(q2[lo_q:].shape, 77 + j, 3.0)
        k2[lo_k:] = _rand(k2[lo_k:].shape, 177 + j, 3.0)
        v2[lo_k:] = _rand(v2[lo_k:].shape, 277 + j, 3.0)
        o2, l2 = run(q2, k2, v2)
        assert np.array_equal(o2[:lo_q], o[:lo_q]), f"chunks 0..{j} changed"
        assert np.array_equal(l2[:, :lo_q], l[:, :lo_q])
        assert not np.allclose(o2[lo_q:], o[lo_q:])


def test_int8_key_mean_golden():
    check_kmean_golden(Q.quantize_round)


def test_quantized_attention_is_chunk_causal():
    check_quantized_causality(Q.quantize_round)


def test_key_mean_input_errors():
    with pytest.raises(ValueError):
        Q.key_channel_mean(np.zeros((5, 1, 2), np.float32), 2, 2)


def _with_key_mean(fn):
    """Q.quantize_round with a planted key mean (the mutation tests below)."""
    def quantize_round(q, k, Hs, C):
        saved = Q.key_channel_mean
        Q.key_channel_mean = fn
        try:
            return Q.quantize_round(q, k, Hs, C)
        finally:
            Q.key_channel_mean = saved
    return quantize_round


def _mean64(k, L):
    return (np.asarray(k[:L], np.float64).sum(axis=0) / L).astype(np.float32)


KMEAN_MUTANTS = {
    "divisor_off_by_7": lambda k, Hs, C: (np.asarray(k[:(Hs + 1) * C], np.float64).sum(axis=0)
                                          / ((Hs + 1) * C + 7)).astype(np.float32),
    "all_keys": lambda k, Hs, C: _mean64(k, k.shape[0]),
    "history_only": lambda k, Hs, C: _mean64(k, max(Hs, 1) * C),
    "no_shift": lambda k, Hs, C: np.zeros(k.shape[1:], np.float32),
    "refresh_chunk_only": lambda k, Hs, C: (np.asarray(k[Hs * C:(Hs + 1) * C], np.float64).mean(axis=0)
                                            ).astype(np.float32),
}


@pytest.mark.parametrize("name", sorted(KMEAN_MUTANTS))
def test_key_mean_mutants_are_caught(name):
    quantize_round = _with_key_mean(KMEAN_MUTANTS[name])
    caught = False
    for check in (check_kmean_golden, check_quantized_causality):
        try:
            check(quantize_round)
        except AssertionError:
            caught = True
    assert caught, name


def test_all_keys_mean_breaks_causality():
    """The reading that takes the mean over every key of the round leaks later
    chunks' keys into earlier chunks' codes: the causality pin itself sees it."""
    with pytest.raises(AssertionError):
        check_quantized_causality(_with_key_mean(KMEAN_MUTANTS["all_keys"]))


def test_unmutated_key_mean_passes_the_checks():
    quantize_round = _with_key_mean(Q.key_channel_mean)
    check_kmean_golden(quantize_round)
    check_quantized_causality(quantize_round)


def test_quantized_attention_close_to_exact():
    C, N, Hs, H, D = 128, 3, 2, 2, 64
    q, k, v = (a.astype(np.float32) for a in _round_inputs(C, N, Hs, H, D, 17))
    o, l = ATTN(q, k, v, Hs, C, 1 / 8)
    oq, lq = Q.quantized_attention(q, k, v, Hs, C, 1 / 8)
    rel = np.abs(oq - o).sum() / np.abs(o).sum()
    assert 1e-4 < rel < 3e-2
    np.testing.assert_allclose(lq, l, atol=2e-2)


# ---------------------------------------------------------------- ring model

def test_ring_model_matches_rebuild():
    rng = np.random.default_rng(3)
    ring = RingModel()
    ref = []
    mk = lambda: (rng.standard_normal((2, 1, 2)), rng.standard_normal((2, 1, 2)))
    for _ in range(5):
        kv = mk()
        ring.append(*kv)
        ref.append(kv)
    for step in range(12):
        kv = mk()
        ring.append(*kv)
        ref.append(kv)
        idx = int(rng.integers(0, len(ref)))
        kv = mk()
        ring.refresh(idx, *kv)
        ref[idx] = kv
        if step % 2:
            ring.evict(1)
            ref = ref[1:]
        K, V = ring.visible()
        np.testing.assert_array_equal(K, np.concatenate([e[0] for e in ref]))
        np.testing.assert_array_equal(V, np.concatenate([e[1] for e in ref]))
    with pytest.raises(IndexError):
        ring.refresh(len(ref), *mk())
    with pytest.raises(IndexError):
        ring.evict(len(ref) + 1)


# ---------------------------------------------------------------- mutation tests

def _attn_with_visible(fn):
    def attn(q, k, v, Hs, C, scale, **kw):
        saved = A.visible_key_count
        A.visible_key_count = fn
        try:
            return A.chunk_causal_attention(q, k, v, Hs, C, scale, **kw)
        finally:
            A.visible_key_count = saved
    return attn


def _attn_with_task(task):
    def attn(q, k, v, Hs, C, scale, **kw):
        saved = A._head_chunk_task
        A._head_chunk_task = task
        try:
            return A.chunk_causal_attention(q, k, v, Hs, C, scale, **kw)
        finally:
            A._head_chunk_task = saved
    return attn


def _task_no_scale(qh, kh, vh, L, scale):
    return A.__dict__["_orig_task"](qh, kh, vh, L, 1.0)


def _task_wrong_v_rows(qh, kh, vh, L, scale):
    return A.__dict__["_orig_task"](qh, kh, np.roll(vh, 1, axis=0), L, scale)


def _task_lse_without_max(qh, kh, vh, L, scale):
    o, lse = A.__dict__["_orig_task"](qh, kh, vh, L, scale)
    s = qh @ kh[:L].T * scale
    return o, lse - s.max(axis=1)


def _task_keys_as_values(qh, kh, vh, L, scale):
    return A.__dict__["_orig_task"](qh, kh, kh, L, scale)


A._orig_task = A._head_chunk_task

ATTN_MUTANTS = {
    "chunk_misses_itself": _attn_with_visible(lambda j, Hs, C: max(1, (Hs + j)) * C),
    "chunk_sees_next": _attn_with_visible(lambda j, Hs, C: (Hs + j + 2) * C),
    "history_ignored": _attn_with_visible(lambda j, Hs, C: (j + 1) * C),
    "no_scale": _attn_with_task(_task_no_scale),
    "wrong_value_rows": _attn_with_task(_task_wrong_v_rows),
    "lse_missing_max": _attn_with_task(_task_lse_without_max),
    "keys_as_values": _attn_with_task(_task_keys_as_values),
}


def _some_pin_fails(attn):
    checks = [
        lambda: check_hand_example(attn),
        lambda: check_mask_fixture(attn),
        lambda: check_bruteforce(attn, 3, 3, 2, 2, 4, 7),
        lambda: check_bruteforce(attn, 2, 2, 0, 2, 3, 8),
        lambda: check_q_zero_closed_form(attn, 3, 3, 1, 2, 4, 61),
    ]
    for c in checks:
        try:
            c()
        except (AssertionError, ValueError, IndexError):
            return True
    return False


@pytest.mark.parametrize("name", sorted(ATTN_MUTANTS))
def test_attention_mutants_are_caught(name):
    assert _some_pin_fails(ATTN_MUTANTS[name]), name


def test_unmutated_oracle_passes_all_mutation_checks():
    assert not _some_pin_fails(ATTN)


def _rope_mutant(kind):
    """The oracle's rotation rewritten with one planted mistake."""
    def rope(x, g0, C, fpc, gh, gw, split=(44, 42, 42), theta=10000.0):
        frame_mult = 2 * fpc if kind == "frame_stride" else fpc
        pos = R.token_positions(x.shape[0], g0, C, fpc, gh, gw).astype(np.float64)
        pos[:, 0] = pos[:, 0] / fpc * frame_mult
        y = np.array(x, dtype=np.float64, copy=True)
        off = 0
        for axis, d in enumerate(split):
            i = np.arange(d // 2)
            expo = -1.0 * i / d if kind == "half_exponent" else -2.0 * i / d
            phi = pos[:, axis][:, None] * theta ** expo
            c, s = np.cos(phi)[:, None, :], np.sin(phi)[:, None, :]
            if kind == "sin_sign":
                s = -s
            e, o = y[:, :, off:off + d:2].copy(), y[:, :, off + 1:off + d:2].copy()
            y[:, :, off:off + d:2] = e * c - o * s
            y[:, :, off + 1:off + d:2] = e * s + o * c
            off += d
        return y
    return rope


def test_rope_unmutated_rewrite_passes():
    check_rope_golden(_rope_mutant("none"))


@pytest.mark.parametrize("kind", ["sin_sign", "half_exponent", "frame_stride"])
def test_rope_mutants_are_caught(kind):
    with pytest.raises(AssertionError):
        check_rope_golden(_rope_mutant(kind))


def _quant_mutant(kind):
    def quantize(x, C, block=128):
        x = np.asarray(x, np.float32)
        a = np.abs(x).max(axis=(0, 2))
        if kind == "div128":
            s = np.where(a > 0, a / np.float32(128), 1).astype(np.float32)
        else:
            s = np.where(a > 0, a / np.float32(127), 1).astype(np.float32)
        y = x / s[None, :, None]
        if kind == "half_away":
            c = np.sign(y) * np.floor(np.abs(y) + 0.5)
        else:
            c = np.rint(y)
        return np.clip(c, -127, 127).astype(np.int8), s[:, None]
    return quantize


@pytest.mark.parametrize("kind", ["div128", "half_away"])
def test_quant_mutants_are_caught(kind):
    with pytest.raises(AssertionError):
        check_int8_golden(_quant_mutant(kind))


def test_rope_token_subset_equals_full():
    x = _rand((2 * 60, 2, 12), 10)
    full = R.rope3d(x, 3, 60, 3, 4, 5, split=(4, 4, 4))
    idx = np.array([119, 0, 61, 7])
    sub = R.rope3d(x[idx], 3, 60, 3, 4, 5, split=(4, 4, 4), tokens=idx)
    np.testing.assert_array_equal(sub, full[idx])
