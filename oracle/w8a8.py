"""W8A8 linear layer (int8 weights and activations), numpy (test oracle).

The pages name a W8A8 backend (8-bit weights and activations) for the DiT
linears around attention in their DiT-only tests (Wave Forcing paper pages,
Abstract) and give none of its internals. This is the reading used here:
  * activations X [M][K] are quantized per row (token): s_x = amax / 127
    (1 when amax = 0), code = clamp(round_half_even(x / s_x), -127, 127);
  * weights W [N][K] (output features x input features) are quantized the same
    way per output channel (row of W);
  * every decision that yields an integer (scale, division, rounding) is taken
    in float32, as the kernels take it;
  * the product accumulates exactly in integers: acc[m][n] = sum_k Xq[m,k] Wq[n,k];
  * y[m][n] = s_x[m] * s_w[n] * acc[m][n] + bias[n] (exact here, in float64).
Test infrastructure only: the HIP path never calls this module.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

__all__ = ["quantize_rows", "int8_matmul", "w8a8_linear"]


def quantize_rows(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """x [R][K] float32 -> codes int8 [R][K], scales float32 [R] (one per row)."""
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x).max(axis=1)
    s = np.where(a > 0, a / np.float32(127.0), np.float32(1.0)).astype(np.float32)
    q = np.rint(x / s[:, None])  # float32 divide, ties to even
    return np.clip(q, -127, 127).astype(np.int8), s


def int8_matmul(xq: np.ndarray, wq: np.ndarray) -> np.ndarray:
    """Exact integer product: acc[m][n] = sum_k xq[m,k] * wq[n,k], as int64."""
    return xq.astype(np.int64) @ wq.astype(np.int64).T


def w8a8_linear(xq: np.ndarray, sx: np.ndarray, wq: np.ndarray, sw: np.ndarray,
                bias: Optional[np.ndarray] = None) -> np.ndarray:
    """y = s_x[m] * s_w[n] * acc[m][n] + bias[n], float64."""
    acc = int8_matmul(xq, wq).astype(np.float64)
    y = acc * (sx.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :])
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    return y
