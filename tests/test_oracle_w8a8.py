"""Pins of the W8A8 oracle (oracle/w8a8.py) against things other than itself:
a hand-worked example, a scalar triple loop, the quantization error bound,
special rows, a float reference within the bound, and planted mistakes."""
import os

import numpy as np
import pytest

from oracle import w8a8 as W

GOLD = os.path.join(os.path.dirname(__file__), "golden", "w8a8_hand_example.txt")


def _gold():
    rows = {}
    for line in open(GOLD):
        if line.startswith("#") or not line.strip():
            continue
        key, *vals = line.split()
        rows.setdefault(key, []).append([float(v) for v in vals])
    return {k: np.array(v) for k, v in rows.items()}


X = np.array([[1, -2, 3, 0.5], [0, 0, 0, 0]], dtype=np.float32)
WT = np.array([[2, 0, -1, 5], [0.5, 0.5, 0.5, 0.5], [-3, 1, 0, 2]], dtype=np.float32)
BIAS = np.array([0.25, -1, 0], dtype=np.float32)


def _hand_check(linear):
    g = _gold()
    xq, sx = W.quantize_rows(X)
    wq, sw = W.quantize_rows(WT)
    assert np.array_equal(xq, g["xq"]) and np.array_equal(wq, g["wq"])
    assert np.array_equal(W.int8_matmul(xq, wq), g["acc"])
    np.testing.assert_allclose(linear(xq, sx, wq, sw, BIAS), g["y"], rtol=1e-6, atol=1e-7)


def test_hand_example():
    _hand_check(W.w8a8_linear)


def test_integer_product_matches_scalar_loops():
    rng = np.random.default_rng(1)
    xq = rng.integers(-127, 128, size=(5, 37)).astype(np.int8)
    wq = rng.integers(-127, 128, size=(7, 37)).astype(np.int8)
    ref = np.zeros((5, 7), dtype=np.int64)
    for m in range(5):
        for n in range(7):
            s = 0
            for k in range(37):
                s += int(xq[m, k]) * int(wq[n, k])
            ref[m, n] = s
    assert np.array_equal(W.int8_matmul(xq, wq), ref)


def test_quantization_bound_and_special_rows():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((64, 300)).astype(np.float32) * rng.uniform(0.01, 10, (64, 1)).astype(np.float32)
    x[3] = 0.0
    q, s = W.quantize_rows(x)
    assert s[3] == 1.0 and not q[3].any()
    err = np.abs(x.astype(np.float64) - q.astype(np.float64) * s[:, None])
    assert (err <= s[:, None] * (0.5 + 1e-6)).all()
    live = np.arange(64) != 3
    assert (np.abs(q[live]).max(axis=1) == 127).all()  # the row max maps to +-127


def test_close_to_float_linear():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((32, 256)).astype(np.float32)
    w = (rng.standard_normal((48, 256)) * 0.05).astype(np.float32)
    b = rng.standard_normal(48).astype(np.float32)
    xq, sx = W.quantize_rows(x)
    wq, sw = W.quantize_rows(w)
    y = W.w8a8_linear(xq, sx, wq, sw, b)
    ref = x.astype(np.float64) @ w.astype(np.float64).T + b
    # |x w - x^ w^| <= sum_k |x| e_w + |w^| e_x with e = s/2
    bound = (np.abs(x) @ np.broadcast_to(sw / 2, (256, 48)) + (sx[:, None] / 2) * np.abs(
        wq.astype(np.float64) * sw[:, None]).sum(axis=1)[None, :])
    assert (np.abs(y - ref) <= bound + 1e-9).all()
    assert np.abs(y - ref).mean() / np.abs(ref).mean() < 2e-2


@pytest.mark.parametrize("kind", ["transposed_scales", "no_bias", "weights_by_column"])
def test_planted_mistakes_are_caught(kind):
    def linear(xq, sx, wq, sw, bias):
        acc = W.int8_matmul(xq, wq).astype(np.float64)
        if kind == "transposed_scales":  # scale of row n used for row m
            sxx = np.resize(sw, sx.shape)
            return acc * (sxx[:, None] * sw[None, :]) + bias
        if kind == "no_bias":
            return acc * (sx[:, None] * sw[None, :])
        # quantize the weights per input column instead of per output row
        wf = wq.astype(np.float64) * sw[:, None]
        s2 = np.abs(wf).max(axis=0) / 127
        s2[s2 == 0] = 1
        wq2 = np.clip(np.rint(wf / s2), -127, 127)
        return (xq.astype(np.float64) @ (wq2 * s2).T) * sx[:, None] + bias
    with pytest.raises(AssertionError):
        _hand_check(linear)
