"""The 1F1C round structure of Wave Forcing over a whole rollout (test oracle).

What the pages fix:
  * denoising stages and the cache-refresh stage are staggered and run
    concurrently, so that after the pipeline fills every forward round outputs
    one chunk (1F1C) (Wave Forcing paper pages, Abstract);
  * the run uses wp-size = steps + 1 concurrent stages, with the step lists
    1000,750,500,250 (4 steps) and 1000,800,600,400,200 (5 steps), and a chunk
    is 3 latent frames (airadar.tv summaries, usage section);
  * a chunk reads earlier, cleaner chunks before their denoising ends, and the
    history cache holds the finished chunks' K/V, written by the refresh pass
    (Abstract).

Reading taken here (the plainest one those passages support):
  * stage s of chunk c runs in round c + s: s = 0 .. S-1 are the denoising
    steps at timesteps steps[s], s = S is the refresh pass at t = 0;
  * so round r holds the chunks c with 0 <= r - c <= S (at most S + 1 = wp-size
    stages), listed cleanest first: ascending c, i.e. the refresh chunk, then
    stages S-1 .. 0;
  * the last denoising stage (s = S-1) yields the clean chunk: it is the
    round's output, so rounds 0 .. S-2 output nothing (the pipeline fill) and
    each later round outputs exactly one chunk;
  * the last chunk's refresh pass would feed no later chunk and is not run:
    F chunks take F + S - 1 rounds;
  * history in round r: the chunks whose refresh pass ran in an earlier round,
    the newest W of them (a rolling window).

Everything here is plain loops over chunks and rounds. Test infrastructure only:
the HIP library never calls this module.
"""
from __future__ import annotations

from typing import Callable, Dict, List, Optional, Sequence, Tuple

import numpy as np

from .attention import chunk_causal_attention
from .rope import rope3d

__all__ = ["timesteps", "n_rounds", "round_plan", "rollout_attention"]


def timesteps(n_steps: int) -> List[int]:
    """Denoising timesteps of stages 0 .. S-1: the pages' lists are 1000 (S - s) / S."""
    if n_steps < 1:
        raise ValueError("need at least one denoising step")
    return [1000 * (n_steps - s) // n_steps for s in range(n_steps)]


def n_rounds(n_steps: int, n_chunks: int) -> int:
    """Rounds for a rollout of n_chunks chunks: the last chunk's last stage runs in round F - 1 + S - 1."""
    return n_chunks + n_steps - 1


def round_plan(n_steps: int, n_chunks: int, hist_window: int, r: int) -> Dict:
    """What round r does.

    inflight  [(chunk, stage)] cleanest first; stage n_steps is the refresh pass
    hist      history chunks, oldest first
    output    chunk whose last denoising stage runs this round, or None
    new       chunk that enters at stage 0 this round, or None
    """
    S, F = n_steps, n_chunks
    if not 0 <= r < n_rounds(S, F):
        raise ValueError("round out of range")
    inflight = []
    for c in range(F):
        s = r - c
        if 0 <= s <= S and not (c == F - 1 and s == S):
            inflight.append((c, s))
    refreshed_before = [c for c in range(F) if c + S < r and c != F - 1]
    hist = refreshed_before[-hist_window:] if hist_window > 0 else []  # all of them when fewer than W
    output = None
    for c, s in inflight:
        if s == S - 1:
            output = c
    new = r if r < F else None
    return {"round": r, "inflight": inflight, "hist": hist, "output": output, "new": new}


def rollout_attention(n_steps: int, n_chunks: int, hist_window: int,
                      qkv: Callable[[int, int], Tuple[np.ndarray, np.ndarray, np.ndarray]],
                      scale: float, rounds: Optional[Sequence[int]] = None,
                      rows: Optional[Callable[[int], Optional[np.ndarray]]] = None,
                      workers: int = 1, rope: Optional[Dict] = None) -> Dict[int, Tuple[np.ndarray, np.ndarray, Dict]]:
    """Attention of every round of the rollout with a given per-(chunk, stage) model.

    qkv(c, s) returns the chunk's Q, K, V [C][H][D] at stage s (s = S: clean, the
    refresh pass). History entries hold the clean K/V, qkv(c, S). With rope
    (frames_per_chunk, grid_h, grid_w, optional split and theta), Q and K of chunk c
    are rotated at the positions of global chunk c (oracle.rope, the 3D convention
    of the round workloads), whatever the stage. Returns {round: (O, LSE, plan)} for
    the asked rounds (default all).
    """
    def rotate(x, c):
        if rope is None:
            return x
        return rope3d(x, c, x.shape[0], rope["frames_per_chunk"], rope["grid_h"], rope["grid_w"],
                      tuple(rope.get("split", (44, 42, 42))), rope.get("theta", 10000.0))

    out = {}
    for r in (range(n_rounds(n_steps, n_chunks)) if rounds is None else rounds):
        plan = round_plan(n_steps, n_chunks, hist_window, r)
        q_parts, k_parts, v_parts = [], [], []
        for c in plan["hist"]:
            _, k, v = qkv(c, n_steps)
            k_parts.append(rotate(k, c))
            v_parts.append(v)
        for c, s in plan["inflight"]:
            q, k, v = qkv(c, s)
            q_parts.append(rotate(q, c))
            k_parts.append(rotate(k, c))
            v_parts.append(v)
        C = q_parts[0].shape[0]
        o, lse = chunk_causal_attention(np.concatenate(q_parts), np.concatenate(k_parts),
                                        np.concatenate(v_parts), len(plan["hist"]), C, scale,
                                        rows=None if rows is None else rows(r), workers=workers)
        out[r] = (o, lse, plan)
    return out
