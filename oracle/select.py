"""O3: retrieval-set selection by attention mass, top-p -- TEST INFRASTRUCTURE.

Retrieval heads keep the tokens that carry the attention (SegPagedAttention
runtime explainer, section 2: retrieval = the top-p important tokens, looked up
on demand; RedKnot summary). The selection, written out from its definition:

* mass of key j for unit (b, l, h): the decode row's (position N_b - 1)
  attention probability of key j over ALL N_b keys of the dense history, averaged
  over the G query heads of KV head h -- a distribution over j (sums to 1);
* top-p: order the keys by mass, larger first, equal masses by position; keep the
  shortest prefix of that order whose mass reaches p * (total mass) -- "reaches"
  up to fp64 summation rounding, a slack of 1e-12 of the total; return its
  positions sorted.

fp64 throughout. Only tests/ and bench.py's cpu leg may import this module.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np

from oracle.attention import bf16_bits_to_f64


def key_mass(q_bits: np.ndarray, k_bits: np.ndarray, scale: float) -> np.ndarray:
    """q_bits uint16 [G, D] (the G query heads of the group), k_bits uint16 [N, D].
    Mean over the G heads of softmax_j(scale * q_g . k_j); fp64 [N]."""
    q = bf16_bits_to_f64(q_bits)
    k = bf16_bits_to_f64(k_bits)
    s = scale * (q @ k.T)                      # [G, N]
    s = s - s.max(axis=1, keepdims=True)
    w = np.exp(s)
    w = w / w.sum(axis=1, keepdims=True)
    return w.mean(axis=0)


def top_p(mass: Sequence[float], p: float) -> np.ndarray:
    """Sorted positions of the shortest mass-ordered prefix (larger mass first,
    equal masses by position) whose mass reaches p * sum(mass)."""
    mass = np.asarray(mass, np.float64)
    n = len(mass)
    if n == 0:
        return np.zeros(0, np.int64)
    order = np.lexsort((np.arange(n), -mass))  # primary: -mass, then position
    cum = np.cumsum(mass[order])
    k = int(np.searchsorted(cum, p * cum[-1] - 1e-12 * cum[-1], side="left"))
    k = min(k, n - 1)
    return np.sort(order[:k + 1])


def threshold(mass: Sequence[float], p: float) -> float:
    """Mass of the last key the top-p set takes."""
    sel = top_p(mass, p)
    return float(np.min(np.asarray(mass, np.float64)[sel])) if len(sel) else 0.0
