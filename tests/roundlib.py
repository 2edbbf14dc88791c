"""Helpers for the GPU tests: drive a round through the C ABI binding and compare
with the fp64 oracle on the same seeded inputs."""
from __future__ import annotations

import math
import os
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle.attention as OA  # noqa: E402

BF16_MAX_ABS = 2e-2
BF16_MEAN_REL = 5e-3
# per (query row, head): sum_d |o - ref| / sum_d |ref| over head_dim. Measured at most
# 3.4e-3 on every full-size round (p50 2.3e-3, from bf16 weights and the bf16 output);
# one dropped or doubled 64-key tile moves a row of a 32,760-key round by about 4 %.
BF16_ROW_REL = 6e-3
# rounds whose Q and K are rotated (3D RoPE) on the GPU and stored in bf16 before attention,
# while the oracle rotates in float64: one more bf16 rounding of every operand (measured at
# most 8.4e-3 per row over the 20 long-rollout rounds, mean rel 3.3e-3)
BF16_ROW_REL_ROPE = 1.2e-2
F32_MAX_ABS = 1e-4


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU in this environment")
    import chunk_causal_dit_amd as wf  # raises if the library is missing: no fallback
    wf.lib()
    return wf


def round_like(dtype: str):
    """Float32 -> values representable in dtype (bf16: nearest even), as float32 arrays."""
    from workloads import round_to_bf16
    if dtype == "bf16":
        return lambda a: round_to_bf16(np.asarray(a, dtype=np.float32))
    return lambda a: np.asarray(a, dtype=np.float32)


def torch_dtype(name: str):
    return torch.bfloat16 if name == "bf16" else torch.float32


def to_dev(a: np.ndarray, dtype) -> torch.Tensor:
    # inputs are already representable in dtype, so the conversion is exact
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda").to(dtype)


def chunks(a: torch.Tensor, C: int):
    return [a[i * C:(i + 1) * C] for i in range(a.shape[0] // C)]


def build_cache(wf, C, H, D, dtype, k_hist, v_hist, k_in, v_in, n_slots=None, table=None):
    """Fill a cache with history then in-flight chunks (logical order). With a
    table, the entries are placed in those physical slots via set_table+refresh."""
    kh, vh = chunks(k_hist, C), chunks(v_hist, C)
    ki, vi = chunks(k_in, C), chunks(v_in, C)
    n = len(kh) + len(ki)
    cache = wf.KVCache(n_slots or n, C, H, D, dtype)
    if table is None:
        for k, v in zip(kh + ki, vh + vi):
            cache.append(k, v)
    else:
        cache.set_table(table)
        for i, (k, v) in enumerate(zip(kh + ki, vh + vi)):
            cache.refresh(i, k, v)
    return cache


def split_workspace(wf, cache):
    """The key-split workspace of the cache, filled with NaN bytes so that a read of
    anything the kernels did not write shows in the result."""
    ws = wf.attn_fwd_workspace(cache)
    if ws is not None:
        ws.fill_(0xFF)
    return ws


def gpu_round(wf, inp, table=None, n_slots=None, with_lse=True, split=False):
    """One round through the C ABI; split=True calls the workspace entry (key split of chunk 0)."""
    cfg = inp.cfg
    dt = torch_dtype(cfg.dtype)
    C, H, D = cfg.chunk_tokens, cfg.n_heads, cfg.head_dim
    dev = {k: to_dev(getattr(inp, k), dt) for k in ("q", "k_hist", "v_hist", "k_in", "v_in")}
    cache = build_cache(wf, C, H, D, dt, dev["k_hist"], dev["v_hist"], dev["k_in"], dev["v_in"],
                        n_slots=n_slots, table=table)
    ws = split_workspace(wf, cache) if split else None
    out, lse = wf.chunk_causal_attn_fwd(dev["q"], cache, cfg.n_inflight, cfg.scale, with_lse=with_lse,
                                        workspace=ws)
    torch.cuda.synchronize()
    return out, lse, cache


def oracle_workers() -> int:
    return min(16, len(os.sched_getaffinity(0)))


def oracle_round(inp, rows=None, workers=None):
    cfg = inp.cfg
    k = np.concatenate([inp.k_hist, inp.k_in])
    v = np.concatenate([inp.v_hist, inp.v_in])
    workers = workers or oracle_workers()
    return OA.chunk_causal_attention(inp.q, k, v, cfg.n_hist, cfg.chunk_tokens, cfg.scale, rows=rows,
                                     workers=workers)


def error_stats(gpu: np.ndarray, ref: np.ndarray):
    d = np.abs(gpu.astype(np.float64) - ref)
    return float(d.max()), float(d.sum() / np.abs(ref).sum())


def row_rel_errors(gpu: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per (row, head) relative error over the last axis: sum |o - ref| / sum |ref|."""
    d = np.abs(gpu.astype(np.float64) - ref).sum(axis=-1)
    return d / np.maximum(np.abs(ref).sum(axis=-1), 1e-300)


def assert_close(gpu_out, ref_out, dtype: str, what: str = "O", row_rel: float = BF16_ROW_REL):
    """Aggregate bounds (max abs, mean relative error over all outputs) and, for
    bf16, the per-row bound row_rel on every (row, head) of a [rows][H][D]
    output, so that one wrong row cannot hide in the aggregate."""
    mx, rel = error_stats(gpu_out, ref_out)
    msg = f"[parity] {what}: max abs {mx:.3e}, mean rel {rel:.3e}"
    rows = None
    if dtype != "f32" and np.ndim(ref_out) == 3:
        rows = row_rel_errors(gpu_out, ref_out)
        msg += (f", per-row rel p50 {np.median(rows):.2e} p99.9 {np.quantile(rows, 0.999):.2e} "
                f"max {rows.max():.2e} over {rows.size} rows")
    print(msg, flush=True)
    assert np.isfinite(gpu_out).all(), f"{what}: non-finite values"
    if dtype == "f32":
        assert mx <= F32_MAX_ABS, f"{what}: max abs {mx} > {F32_MAX_ABS}"
    else:
        assert mx <= BF16_MAX_ABS, f"{what}: max abs {mx} > {BF16_MAX_ABS}"
        assert rel <= BF16_MEAN_REL, f"{what}: mean rel {rel} > {BF16_MEAN_REL}"
        if rows is not None:
            worst = np.unravel_index(np.argmax(rows), rows.shape)
            assert rows.max() <= row_rel, f"{what}: row {worst} rel {rows.max()} > {row_rel}"
    return mx, rel


def boundary_rows(C: int, N: int, n_sample: int, seed: int, tile: int = 256):
    """Sampled query rows: chunk edges, query-tile edges, the ragged tail, plus random rows."""
    rng = np.random.default_rng(seed)
    rows = set()
    for j in range(N):
        base = j * C
        for r in (0, 1, 31, 32, C - 1, C - 2):
            if 0 <= r < C:
                rows.add(base + r)
        for t in range(tile, C, tile):
            rows.update({base + t - 1, base + t})
        rows.update(int(base + x) for x in rng.integers(0, C, size=n_sample))
    return np.array(sorted(rows))
