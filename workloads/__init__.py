"""Seeded synthetic inputs for the chunk-wise causal attention round.

This module holds workload shapes and random-number generation only. It does
none of the method's arithmetic, and both the fp64 oracle (``oracle/``) and the
HIP path (``chunk_causal_dit_amd``) receive the exact same arrays from it.

Shapes follow the round the Wave Forcing pages describe: N in-flight chunks at
staggered noise levels (the step count plus one cache-refresh chunk; README
usage on the airadar.tv summary, "--wp-size 5 ... 1000,750,500,250") attend to
a history cache. Head count, head_dim and tokens per latent frame are those of
Wan2.1-T2V-1.3B (12 heads x 128, 1560 tokens per 30x52 latent frame) and of the
14B scale row (40 heads). Chunks are 3 latent frames ("--num-frames ... must be
divisible by 3", same README usage section).

Random draws: ``numpy.random.default_rng(seed).standard_normal(dtype=float32)``
in the fixed order documented on each generator; bf16 workloads are rounded to
bf16 with round-to-nearest-even on the host, so the oracle reads the very
values the GPU reads. Layout is token-major ``[tokens][heads][head_dim]``.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

__all__ = [
    "RoundConfig",
    "CONFIGS",
    "round_to_bf16",
    "bf16_bits",
    "RoundInputs",
    "make_round_inputs",
    "make_rollout_init",
    "make_rollout_round",
    "make_stale_refresh",
    "sample_rows",
    "slot_permutation",
    "make_linear_inputs",
    "NullModel",
]


@dataclass(frozen=True)
class RoundConfig:
    """One workload: the shape of a single 1F1C round (one layer)."""

    name: str
    n_heads: int
    head_dim: int
    chunk_tokens: int
    n_inflight: int  # in-flight chunks: refresh chunk first, noisiest last
    n_hist: int  # history chunks visible to every in-flight chunk
    dtype: str  # "f32" or "bf16"
    seed: int
    rope: bool = False
    int8_qk: bool = False
    n_slots: Optional[int] = None  # physical ring slots (default: n_hist + n_inflight)
    rounds: int = 1
    stale_refresh: bool = False  # refresh slot pre-filled with stale values
    frames_per_chunk: int = 3
    grid_h: int = 30
    grid_w: int = 52
    rope_split: Tuple[int, int, int] = (44, 42, 42)
    rope_theta: float = 10000.0
    description: str = ""

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))

    @property
    def nq(self) -> int:
        return self.n_inflight * self.chunk_tokens

    @property
    def nkv(self) -> int:
        return (self.n_hist + self.n_inflight) * self.chunk_tokens

    @property
    def slots(self) -> int:
        return self.n_slots if self.n_slots is not None else self.n_hist + self.n_inflight


CONFIGS: Dict[str, RoundConfig] = {
    c.name: c
    for c in [
        RoundConfig(
            "tiny_f32", 2, 64, 64, 3, 2, "f32", seed=1,
            description="tiny fp32: H2 D64, 3 in-flight chunks of 64 + 2 history chunks, no RoPE",
        ),
        RoundConfig(
            "wan13b_4step", 12, 128, 4680, 5, 2, "bf16", seed=2,
            description="Wan2.1-1.3B-shaped 4-step round: H12 D128, C=3x1560, 5 in-flight + 2 history",
        ),
        RoundConfig(
            "step5_refresh", 12, 128, 4680, 6, 3, "bf16", seed=3, stale_refresh=True,
            description="5-step round: 6 in-flight + 3 history; refresh chunk overwrites its slot first",
        ),
        RoundConfig(
            "long_rollout", 12, 128, 4680, 5, 6, "bf16", seed=4, rope=True, n_slots=12, rounds=20,
            description="long rollout: 6-chunk history window in 12 permuted slots, 3D RoPE, 20 rounds",
        ),
        RoundConfig(
            "i8qk_14b", 40, 128, 4680, 5, 2, "bf16", seed=5, int8_qk=True,
            description="14B-shaped round with int8 QK (per-128-token blocks, K mean-subtracted)",
        ),
    ]
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-representable."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _normal(rng: np.random.Generator, shape, dtype: str, mult: float = 1.0) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if mult != 1.0:
        a *= np.float32(mult)
    if dtype == "bf16":
        a = round_to_bf16(a)
    return a


@dataclass
class RoundInputs:
    """Host arrays (float32, bf16-representable for bf16 workloads) for one round.

    q:      [n_inflight*C][H][D] queries of the in-flight block, refresh chunk first
    k_hist: [n_hist*C][H][D]     history keys, oldest chunk first
    v_hist: [n_hist*C][H][D]
    k_in:   [n_inflight*C][H][D] this round's keys of the in-flight chunks
    v_in:   [n_inflight*C][H][D]
    """

    cfg: RoundConfig
    q: np.ndarray
    k_hist: np.ndarray
    v_hist: np.ndarray
    k_in: np.ndarray
    v_in: np.ndarray
    extra: Dict[str, np.ndarray] = field(default_factory=dict)


def make_round_inputs(cfg: RoundConfig, seed: Optional[int] = None) -> RoundInputs:
    """Draw one round. Order of draws: Q, K_hist, V_hist, K_in, V_in."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    H, D, C = cfg.n_heads, cfg.head_dim, cfg.chunk_tokens
    q = _normal(rng, (cfg.nq, H, D), cfg.dtype)
    k_hist = _normal(rng, (cfg.n_hist * C, H, D), cfg.dtype)
    v_hist = _normal(rng, (cfg.n_hist * C, H, D), cfg.dtype)
    k_in = _normal(rng, (cfg.nq, H, D), cfg.dtype)
    v_in = _normal(rng, (cfg.nq, H, D), cfg.dtype)
    return RoundInputs(cfg, q, k_hist, v_hist, k_in, v_in)


def make_stale_refresh(cfg: RoundConfig, seed: int = 33, mult: float = 8.0):
    """Stale K/V for the refresh chunk's slot, written before the refresh (finite, x8)."""
    rng = np.random.default_rng(seed)
    shape = (cfg.chunk_tokens, cfg.n_heads, cfg.head_dim)
    return _normal(rng, shape, cfg.dtype, mult), _normal(rng, shape, cfg.dtype, mult)


def make_rollout_init(cfg: RoundConfig):
    """Initial cache contents of the long rollout: n_hist history chunks plus the
    n_inflight-1 in-flight chunks that continue into round 0. Draw order: K then V,
    each [(n_hist + n_inflight - 1)*C][H][D], seed ``cfg.seed``."""
    rng = np.random.default_rng(cfg.seed)
    n = (cfg.n_hist + cfg.n_inflight - 1) * cfg.chunk_tokens
    shape = (n, cfg.n_heads, cfg.head_dim)
    return _normal(rng, shape, cfg.dtype), _normal(rng, shape, cfg.dtype)


def make_rollout_round(cfg: RoundConfig, r: int):
    """In-flight Q, K, V of rollout round ``r`` (seed 400 + r), each [N*C][H][D]."""
    rng = np.random.default_rng(400 + r)
    shape = (cfg.nq, cfg.n_heads, cfg.head_dim)
    return tuple(_normal(rng, shape, cfg.dtype) for _ in range(3))


def make_linear_inputs(M: int, N: int, K: int, seed: int, w_scale: float = 0.02):
    """Inputs of one linear layer (bf16-representable float32): X [M][K] ~ N(0,1),
    W [N][K] ~ N(0, w_scale^2), bias [N] ~ N(0, 0.1^2). Draw order: X, W, bias."""
    rng = np.random.default_rng(seed)
    x = _normal(rng, (M, K), "bf16")
    w = _normal(rng, (N, K), "bf16", w_scale)
    b = _normal(rng, (N,), "bf16", 0.1)
    return x, w, b


def slot_permutation(n_slots: int, seed: int) -> List[int]:
    """A seeded permutation of physical slot ids (for non-contiguous tables)."""
    return [int(s) for s in np.random.default_rng(seed).permutation(n_slots)]


def sample_rows(n_rows: int, n_sample: int, seed: int) -> np.ndarray:
    """Seeded sorted sample of row indices, always including the first and last row."""
    if n_sample >= n_rows:
        return np.arange(n_rows)
    rng = np.random.default_rng(seed)
    pick = rng.choice(np.arange(1, n_rows - 1), size=n_sample - 2, replace=False)
    return np.sort(np.concatenate([[0, n_rows - 1], pick]))


class NullModel:
    """Stand-in for the DiT in a multi-round rollout: the Q, K, V [C][H][D] that chunk c
    has at stage s (s = n_steps: the clean chunk of the refresh pass) are seeded draws,
    rng = default_rng([seed, c, s]), in the order Q, K, V, rounded to dtype as the round
    workloads are. Random numbers only; none of the method's arithmetic."""

    def __init__(self, seed: int, chunk_tokens: int, n_heads: int, head_dim: int, dtype: str = "bf16"):
        self.seed, self.shape, self.dtype = seed, (chunk_tokens, n_heads, head_dim), dtype
        self._memo: Dict[Tuple[int, int], Tuple[np.ndarray, np.ndarray, np.ndarray]] = {}

    def __call__(self, c: int, s: int):
        key = (c, s)
        if key not in self._memo:
            rng = np.random.default_rng([self.seed, c, s])
            self._memo[key] = tuple(_normal(rng, self.shape, self.dtype) for _ in range(3))
        return self._memo[key]
