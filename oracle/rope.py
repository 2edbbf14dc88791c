"""3D rotary position embedding over (frame, height, width), numpy float64 (test oracle).

The pages do not mention rotary embeddings; the long-rollout workload applies
one to the in-flight queries and keys of each round. The convention below is a
reading chosen where the pages are silent, and the HIP kernel follows the same
one:
  * head_dim is split into three consecutive segments for frame, height and
    width (44/42/42 for head_dim 128);
  * inside a segment of width d_a, the pair (x[o+2i], x[o+2i+1]) is rotated by
    the angle pos_a * theta**(-2i/d_a), i = 0..d_a/2-1 (index restarts at 0 in
    every segment, theta = 10000);
  * a token at global chunk g, local latent frame f, latent row y and column x
    has positions (frames_per_chunk*g + f, y, x);
  * tokens inside a chunk are ordered frame, then row, then column.
Chunks are 3 latent frames of the 30x52 latent grid of an 832x480 video
(airadar.tv summaries, usage section: "--num-frames" counts latent frames and
must be divisible by 3; the released resolution is 832x480).
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np

__all__ = ["token_positions", "rope3d"]


def token_positions(n_tokens: int, first_global_chunk: int, chunk_tokens: int,
                    frames_per_chunk: int, grid_h: int, grid_w: int) -> np.ndarray:
    """Integer (frame, row, col) positions of each token of a block of whole chunks."""
    if chunk_tokens != frames_per_chunk * grid_h * grid_w:
        raise ValueError("chunk_tokens must equal frames_per_chunk * grid_h * grid_w")
    t = np.arange(n_tokens)
    g = first_global_chunk + t // chunk_tokens
    u = t % chunk_tokens
    f = u // (grid_h * grid_w)
    y = (u // grid_w) % grid_h
    x = u % grid_w
    return np.stack([frames_per_chunk * g + f, y, x], axis=1)


def rope3d(x: np.ndarray, first_global_chunk: int, chunk_tokens: int,
           frames_per_chunk: int, grid_h: int, grid_w: int,
           split: Sequence[int] = (44, 42, 42), theta: float = 10000.0,
           tokens=None) -> np.ndarray:
    """Rotate x [n_tokens][H][D] (whole chunks) and return a float64 copy.
    With ``tokens`` (indices into the block of whole chunks), x holds only
    those tokens' rows, in that order."""
    n, H, D = x.shape
    d_t, d_h, d_w = split
    if d_t + d_h + d_w != D or d_t % 2 or d_h % 2 or d_w % 2:
        raise ValueError("axis split must be even and sum to head_dim")
    if tokens is None:
        pos = token_positions(n, first_global_chunk, chunk_tokens, frames_per_chunk,
                              grid_h, grid_w).astype(np.float64)
    else:
        tokens = np.asarray(tokens)
        if len(tokens) != n:
            raise ValueError("one token index per row")
        every = token_positions(int(tokens.max()) // chunk_tokens * chunk_tokens + chunk_tokens,
                                first_global_chunk, chunk_tokens, frames_per_chunk, grid_h, grid_w)
        pos = every[tokens].astype(np.float64)
    y = np.array(x, dtype=np.float64, copy=True)
    offset = 0
    for axis, d_a in enumerate((d_t, d_h, d_w)):
        i = np.arange(d_a // 2, dtype=np.float64)
        omega = theta ** (-2.0 * i / d_a)  # [d_a/2]
        phi = pos[:, axis][:, None] * omega[None, :]  # [n][d_a/2]
        c = np.cos(phi)[:, None, :]
        s = np.sin(phi)[:, None, :]
        even = y[:, :, offset:offset + d_a:2].copy()
        odd = y[:, :, offset + 1:offset + d_a:2].copy()
        y[:, :, offset:offset + d_a:2] = even * c - odd * s
        y[:, :, offset + 1:offset + d_a:2] = even * s + odd * c
        offset += d_a
    return y


def rotation_angles(pos: Tuple[int, int, int], split=(44, 42, 42), theta=10000.0):
    """Angle applied to every pair of head_dim for one token position (for tests)."""
    out = []
    for p, d_a in zip(pos, split):
        for i in range(d_a // 2):
            out.append(p * theta ** (-2.0 * i / d_a))
    return np.array(out)
