"""Plain-list model of the history cache and the round structure (test oracle).

The pages describe a history cache that later chunks read and a cache-refresh
stage that re-runs a finished chunk so that its clean K/V replaces the noisy
one (Wave Forcing paper pages, Abstract: done one after the other, denoising
and the cache refresh cost two forward passes; WF runs the refresh stage
concurrently with the denoising stages). The model keeps the semantics only:
an ordered list of chunk entries, oldest first; no slots, no padding.

  append(k, v)   a new (noisiest) chunk joins at the end
  refresh(i, ..) entry i gets this round's K/V (in place)
  evict(n)       the n oldest entries leave
  attention      with n_inflight: the last n_inflight entries are the in-flight
                 chunks (refresh chunk first), the rest is history
"""
from __future__ import annotations

from typing import List, Tuple

import numpy as np

__all__ = ["RingModel"]


class RingModel:
    def __init__(self) -> None:
        self.entries: List[Tuple[np.ndarray, np.ndarray]] = []

    def append(self, k: np.ndarray, v: np.ndarray) -> None:
        self.entries.append((np.array(k, copy=True), np.array(v, copy=True)))

    def refresh(self, logical_idx: int, k: np.ndarray, v: np.ndarray) -> None:
        if not 0 <= logical_idx < len(self.entries):
            raise IndexError("refresh of an entry that does not exist")
        self.entries[logical_idx] = (np.array(k, copy=True), np.array(v, copy=True))

    def evict(self, n_oldest: int) -> None:
        if n_oldest > len(self.entries):
            raise IndexError("evict more entries than held")
        del self.entries[:n_oldest]

    def __len__(self) -> int:
        return len(self.entries)

    def visible(self) -> Tuple[np.ndarray, np.ndarray]:
        """All entries concatenated in logical order: K, V [(len)*C][H][D]."""
        return (np.concatenate([e[0] for e in self.entries], axis=0),
                np.concatenate([e[1] for e in self.entries], axis=0))

    def n_hist(self, n_inflight: int) -> int:
        return len(self.entries) - n_inflight
