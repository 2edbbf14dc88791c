"""int8 quantization of Q and K for the int8-QK round, numpy (test oracle).

The pages name a quantized-QK attention backend (SageAttention) for their
DiT-only throughput comparison (Wave Forcing paper pages, Abstract) and give
none of its internals. The scheme here is the one the 14B-shaped workload
fixes, with these readings where it is open:
  * per head, Q and K are cut into blocks of 128 tokens that start at every
    chunk start (the last block of a 4680-token chunk holds 72 tokens);
  * K is first shifted by one per-(head, channel) mean taken over the keys that
    every query chunk of the round sees: the history chunks and in-flight
    chunk 0 (the refresh chunk). One shift for every key keeps each query's
    softmax exact, because it adds the same constant <q_i, mean> to all of row
    i's logits; taking it over that common prefix keeps the round chunk-wise
    causal, since no later in-flight chunk's keys enter it (Abstract: a chunk
    reads only earlier chunks; airadar.tv summaries, first paragraph: K/V pass
    one way, from earlier chunks to later ones);
  * per block: a = max |x|, scale s = a / 127 (s = 1 when a = 0), code
    q = clip(round_half_even(x / s), -127, 127);
  * every decision that yields an integer (the shifted value, the scale, the
    division and the rounding) is taken in float32, as the kernel takes it;
    the mean is accumulated in float64 and rounded once to float32.
The "quantized" attention then runs the exact oracle on s*q for Q and for the
shifted K (V unchanged), with logits scale * <Q^_i, K^'_k + mean> so that LSE
refers to the unshifted keys.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from .attention import chunk_causal_attention

__all__ = ["BLOCK", "key_channel_mean", "quantize_chunk_blocks", "dequantize",
           "quantize_round", "quantized_attention"]

BLOCK = 128


def key_channel_mean(k_vis: np.ndarray, n_hist: int, chunk_tokens: int) -> np.ndarray:
    """Per-(head, channel) mean of the keys every query chunk sees, i.e. the
    first (n_hist + 1) * C keys of the logical order (history, then in-flight
    chunk 0): [H][D] float32, summed in float64 and rounded once."""
    L = (n_hist + 1) * chunk_tokens
    if k_vis.shape[0] < L:
        raise ValueError("fewer keys than history plus the refresh chunk")
    return (np.asarray(k_vis[:L], dtype=np.float64).sum(axis=0) / L).astype(np.float32)


def quantize_chunk_blocks(x: np.ndarray, chunk_tokens: int, block: int = BLOCK
                          ) -> Tuple[np.ndarray, np.ndarray]:
    """x [n_chunks*C][H][D] float32 -> codes int8 same shape, scales [H][n_blocks_total].

    Blocks restart at every chunk start; scales are listed chunk by chunk,
    ceil(C/block) per chunk."""
    x = np.asarray(x, dtype=np.float32)
    n, H, D = x.shape
    C = chunk_tokens
    nb = -(-C // block)
    n_chunks = n // C
    codes = np.zeros((n, H, D), dtype=np.int8)
    scales = np.zeros((H, n_chunks * nb), dtype=np.float32)
    for c in range(n_chunks):
        for b in range(nb):
            lo = c * C + b * block
            hi = min(c * C + C, lo + block)
            blk = x[lo:hi]  # [t][H][D]
            a = np.abs(blk).max(axis=(0, 2))  # [H] float32
            s = np.where(a > 0, a / np.float32(127.0), np.float32(1.0)).astype(np.float32)
            qv = np.rint(blk / s[None, :, None])  # float32 divide, ties to even
            codes[lo:hi] = np.clip(qv, -127, 127).astype(np.int8)
            scales[:, c * nb + b] = s
    return codes, scales


def dequantize(codes: np.ndarray, scales: np.ndarray, chunk_tokens: int,
               block: int = BLOCK) -> np.ndarray:
    """s * q in float64, [n][H][D]."""
    n, H, D = codes.shape
    C = chunk_tokens
    nb = -(-C // block)
    t = np.arange(n)
    bidx = (t // C) * nb + (t % C) // block  # [n]
    s = scales[:, bidx].T.astype(np.float64)  # [n][H]
    return codes.astype(np.float64) * s[:, :, None]


def quantize_round(q: np.ndarray, k_vis: np.ndarray, n_hist: int, chunk_tokens: int):
    """Quantize one round: returns dict with mean [H][D] f32, K' codes/scales, Q codes/scales."""
    mean = key_channel_mean(k_vis, n_hist, chunk_tokens)
    k_shift = (np.asarray(k_vis, np.float32) - mean[None, :, :]).astype(np.float32)
    kq, ks = quantize_chunk_blocks(k_shift, chunk_tokens)
    qq, qs = quantize_chunk_blocks(q, chunk_tokens)
    return {"mean": mean, "k_shift": k_shift, "k_codes": kq, "k_scales": ks,
            "q_codes": qq, "q_scales": qs}


def quantized_attention(q, k_vis, v_vis, n_hist, chunk_tokens, scale, rows=None,
                        workers=1, quant=None):
    """Exact attention on the dequantized operands (the int8 path's target)."""
    if quant is None:
        quant = quantize_round(q, k_vis, n_hist, chunk_tokens)
    q_hat = dequantize(quant["q_codes"], quant["q_scales"], chunk_tokens)
    k_hat = dequantize(quant["k_codes"], quant["k_scales"], chunk_tokens)
    k_hat = k_hat + quant["mean"].astype(np.float64)[None, :, :]
    return chunk_causal_attention(q_hat, k_hat, v_vis, n_hist, chunk_tokens, scale,
                                  rows=rows, workers=workers)
