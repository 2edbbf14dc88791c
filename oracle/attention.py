"""Chunk-wise causal attention, written out in numpy float64 (test oracle).

What is computed. Wave Forcing packs the in-flight chunks of one 1F1C round
(the cache-refresh chunk, then the denoising chunks from cleanest to noisiest)
into one query block. A chunk may read the history cache, every earlier (and
therefore cleaner) in-flight chunk and itself, but no later chunk
(Wave Forcing paper pages, Abstract: the chunk-wise causal attention lets a
chunk read earlier, cleaner chunks whose denoising is not finished yet;
airadar.tv summaries, first paragraph: later chunks read the cleaner context
of earlier chunks still being denoised).

Readings taken where the pages are silent:
  * inside a chunk attention is full (bidirectional): "chunk-wise" causality
    only orders chunks;
  * the keys are laid out in logical order: history oldest first, then the
    in-flight chunks j = 0..N-1, so query chunk j sees the first
    (n_hist + j + 1) * C keys;
  * softmax scale is given by the caller (1/sqrt(head_dim) in every workload);
  * outputs: O per query row and head, and LSE = ln sum_k exp(s_ik).

For every head h and query row i of in-flight chunk j
    s_ik   = scale * <q_ih, k_kh>                       for visible keys k
    O_ih   = sum_k exp(s_ik) v_kh / sum_k exp(s_ik)
    LSE_ih = ln sum_k exp(s_ik)
Array layout is token-major: q [N*C][H][D], keys/values [(n_hist+N)*C][H][D].
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "visible_key_count",
    "chunk_causal_attention",
    "dense_masked_attention",
    "bruteforce_attention",
]


def visible_key_count(j: int, n_hist: int, chunk_tokens: int) -> int:
    """Keys visible to in-flight chunk j: history plus in-flight chunks 0..j."""
    return (n_hist + j + 1) * chunk_tokens


def _head_chunk_task(qh, kh, vh, L, scale):
    """Attention of query rows qh [R][D] of one chunk and head over the first L
    keys of that head's keys kh and values vh ([keys][D], float64)."""
    s = (qh @ kh[:L].T) * scale
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    o = (p @ vh[:L]) / l
    lse = m[:, 0] + np.log(l[:, 0])
    return o, lse


def chunk_causal_attention(
    q: np.ndarray,
    k_vis: np.ndarray,
    v_vis: np.ndarray,
    n_hist: int,
    chunk_tokens: int,
    scale: float,
    rows: Optional[Sequence[int]] = None,
    block: int = 512,
    workers: int = 1,
) -> Tuple[np.ndarray, np.ndarray]:
    """Per-chunk-prefix form of the round's attention.

    q      [N*C][H][D] in-flight queries (refresh chunk first)
    k_vis  [(n_hist+N)*C][H][D] keys in logical order; v_vis likewise
    rows   optional subset of query rows (sorted or not); default all rows
    Returns O [R][H][D] float64 and LSE [H][R] float64 (natural log), R = len(rows).
    """
    C = chunk_tokens
    nq, H, D = q.shape
    if nq % C:
        raise ValueError("query block is not a whole number of chunks")
    N = nq // C
    if k_vis.shape[0] < (n_hist + N) * C or v_vis.shape[0] < (n_hist + N) * C:
        raise ValueError("fewer keys than history plus in-flight chunks")
    rows = np.arange(nq) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((len(rows), H, D), dtype=np.float64)
    lse = np.empty((H, len(rows)), dtype=np.float64)

    L_max = (n_hist + N) * C
    heads = list(range(H))

    def pool_map(fn, items):
        if workers <= 1:
            return [fn(x) for x in items]
        from threadpoolctl import threadpool_limits  # one BLAS thread per task
        with threadpool_limits(1), ThreadPoolExecutor(max_workers=workers) as ex:
            return list(ex.map(fn, items))

    # each head's visible keys and values in float64, made once and shared by its tasks
    kv64 = pool_map(lambda h: (np.asarray(k_vis[:L_max, h, :], dtype=np.float64),
                               np.asarray(v_vis[:L_max, h, :], dtype=np.float64)), heads)

    tasks = []
    chunk_of_row = rows // C
    for h in heads:
        for j in range(N):
            pos = np.nonzero(chunk_of_row == j)[0]
            L = visible_key_count(j, n_hist, C)
            for b in range(0, len(pos), block):
                sel = pos[b:b + block]
                tasks.append((h, sel, rows[sel], L))

    def run(t):
        h, sel, r, L = t
        qh = np.asarray(q[r, h, :], dtype=np.float64)
        o, ls = _head_chunk_task(qh, kv64[h][0], kv64[h][1], L, scale)
        out[sel, h, :] = o
        lse[h, sel] = ls

    pool_map(run, tasks)
    return out, lse


def _query_chunk(i: int, C: int) -> int:
    return i // C


def _key_chunk(k: int, C: int) -> int:
    return k // C


def dense_masked_attention(q, k_vis, v_vis, n_hist, chunk_tokens, scale):
    """Second vectorised form: one (Nq x Nkv) visibility matrix built from the rule
    "key chunk <= n_hist + query chunk", scores outside it excluded from the softmax.
    Returns O [Nq][H][D], LSE [H][Nq] (float64)."""
    C = chunk_tokens
    nq, H, D = q.shape
    nk = k_vis.shape[0]
    qc = np.arange(nq) // C
    kc = np.arange(nk) // C
    visible = kc[None, :] <= (n_hist + qc)[:, None]
    out = np.empty((nq, H, D))
    lse = np.empty((H, nq))
    for h in range(H):
        s = (q[:, h, :].astype(np.float64) @ k_vis[:, h, :].astype(np.float64).T) * scale
        s = np.where(visible, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        p = np.where(visible, np.exp(s - m), 0.0)
        l = p.sum(axis=1, keepdims=True)
        out[:, h, :] = (p @ v_vis[:, h, :].astype(np.float64)) / l
        lse[h] = m[:, 0] + np.log(l[:, 0])
    return out, lse


def bruteforce_attention(q, k_vis, v_vis, n_hist, chunk_tokens, scale):
    """Scalar loops for tiny inputs: visibility from the definition, math.exp,
    no vectorisation. Returns O [Nq][H][D], LSE [H][Nq] as float64 arrays."""
    C = chunk_tokens
    nq, H, D = q.shape
    nk = k_vis.shape[0]
    out = np.zeros((nq, H, D))
    lse = np.zeros((H, nq))
    for h in range(H):
        for i in range(nq):
            vis = [k for k in range(nk) if _key_chunk(k, C) <= n_hist + _query_chunk(i, C)]
            scores = []
            for k in vis:
                dot = 0.0
                for d in range(D):
                    dot += float(q[i, h, d]) * float(k_vis[k, h, d])
                scores.append(scale * dot)
            m = max(scores)
            w = [math.exp(s - m) for s in scores]
            tot = sum(w)
            for d in range(D):
                acc = 0.0
                for wk, k in zip(w, vis):
                    acc += wk * float(v_vis[k, h, d])
                out[i, h, d] = acc / tot
            lse[h, i] = m + math.log(tot)
    return out, lse
