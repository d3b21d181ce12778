"""O1: SegPaged attention as its plain definition, in fp64 -- TEST INFRASTRUCTURE.

What is computed (SegPagedAttention runtime explainer, section 4 -- the fused
kernel computes exactly the dense attention under each head's own visibility,
checked there against a dense+mask baseline; KV-cache guide section 10.2 --
softmax with a max shift):

    for query row at position i of sequence b, Q head hq, KV head h = hq // G:
        s_j   = scale * <q_i, k_j>            for j in vis(i)
        w_j   = exp(s_j - max s) / sum_j exp(s_j - max s)
        O_i   = sum_j w_j v_j
        LSE_i = max s + ln sum_j exp(s_j - max s)

GQA mapping (KV-cache guide section 5.3): query heads form contiguous groups of
G = Hq / Hkv that share one KV head.

vis(i) by head class (runtime explainer sections 1-2 and the summary's head
classes): every class is causal, j <= i, and
    GLOBAL / DENSE      all earlier tokens (full history)
    LOCAL(s, W)         the first s "sink" tokens and the W most recent tokens,
                        the current one included: j < s or i - W < j
    RETRIEVAL(R)        only the given token set: j in R
An empty visible set (only possible for RETRIEVAL) gives O = 0, LSE = -inf.
"""
from __future__ import annotations

import math
from typing import Sequence, Tuple

import numpy as np

from workloads import DENSE, GLOBAL, LOCAL, RETRIEVAL, Spec


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# visibility
# --------------------------------------------------------------------------

def visible(kind: int, sink: int, window: int, retr, i: int, j: int) -> bool:
    """Scalar visibility of key position j to the query at position i."""
    if j > i or j < 0:
        return False
    if kind in (GLOBAL, DENSE):
        return True
    if kind == LOCAL:
        return j < sink or j > i - window
    if kind == RETRIEVAL:
        return int(j) in set(int(x) for x in retr)
    raise ValueError(f"unknown head class {kind}")


def visibility_mask(kind: int, sink: int, window: int, retr, rows: np.ndarray,
                    n_keys: int) -> np.ndarray:
    """Boolean [len(rows), n_keys]: mask[r, j] = key j visible to query position rows[r]."""
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.arange(n_keys, dtype=np.int64)[None, :]
    causal = j <= i
    if kind in (GLOBAL, DENSE):
        return causal
    if kind == LOCAL:
        return causal & ((j < sink) | (j > i - window))
    if kind == RETRIEVAL:
        member = np.zeros(n_keys, dtype=bool)
        if retr is not None and len(retr):
            member[np.asarray(retr, dtype=np.int64)] = True
        return causal & member[None, :]
    raise ValueError(f"unknown head class {kind}")


# --------------------------------------------------------------------------
# the three ways of computing one head's rows
# --------------------------------------------------------------------------

def attend_masked(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray,
                  scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Dense scores, explicit mask, softmax. q [R, D], k/v [N, D] fp64, mask [R, N].
    Returns O [R, D] and LSE [R] (natural log)."""
    s = scale * (q @ k.T)
    s = np.where(mask, s, -np.inf)
    empty = ~mask.any(axis=1)
    m = np.where(empty, 0.0, s.max(axis=1, initial=-np.inf))
    w = np.exp(s - m[:, None])
    z = w.sum(axis=1)
    zs = np.where(empty, 1.0, z)
    o = (w @ v) / zs[:, None]
    o[empty] = 0.0
    lse = np.where(empty, -np.inf, m + np.log(zs))
    return o, lse


def attend_loops(q: np.ndarray, k: np.ndarray, v: np.ndarray, kind: int, sink: int,
                 window: int, retr, rows: Sequence[int], scale: float
                 ) -> Tuple[np.ndarray, np.ndarray]:
    """Scalar-loop variant for tiny inputs: visibility decided pair by pair with
    `visible`, scores and weights accumulated one key at a time."""
    d = q.shape[1]
    o = np.zeros((len(rows), d))
    lse = np.full(len(rows), -np.inf)
    for r, i in enumerate(rows):
        keys = [j for j in range(k.shape[0]) if visible(kind, sink, window, retr, i, j)]
        if not keys:
            continue
        scores = [scale * sum(q[r, t] * k[j, t] for t in range(d)) for j in keys]
        mx = max(scores)
        ws = [math.exp(sc - mx) for sc in scores]
        z = sum(ws)
        for wj, j in zip(ws, keys):
            o[r] += (wj / z) * v[j]
        lse[r] = mx + math.log(z)
    return o, lse


def attend_blocked(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray,
                   scale: float, block: int = 64) -> Tuple[np.ndarray, np.ndarray]:
    """Second algorithm: one pass over key blocks with the running (m, l, acc)
    update of the KV-cache guide section 10.2 -- the old accumulator and the old
    normaliser are both rescaled by exp(m_old - m_new). Blocks with no visible
    key for a row leave that row's state unchanged (no -inf - -inf)."""
    r_cnt, d = q.shape
    m = np.full(r_cnt, -np.inf)
    l = np.zeros(r_cnt)
    acc = np.zeros((r_cnt, d))
    for k0 in range(0, k.shape[0], block):
        k1 = min(k0 + block, k.shape[0])
        mb = mask[:, k0:k1]
        s = np.where(mb, scale * (q @ k[k0:k1].T), -np.inf)
        has = mb.any(axis=1)
        m_blk = np.where(has, s.max(axis=1, initial=-np.inf), -np.inf)
        m_new = np.maximum(m, m_blk)
        safe = np.where(np.isfinite(m_new), m_new, 0.0)
        a_old = np.where(np.isfinite(m), np.exp(m - safe), 0.0)
        p = np.exp(s - safe[:, None])
        l = a_old * l + p.sum(axis=1)
        acc = a_old[:, None] * acc + p @ v[k0:k1]
        m = m_new
    empty = l == 0.0
    o = acc / np.where(empty, 1.0, l)[:, None]
    lse = np.where(empty, -np.inf, m + np.log(np.where(empty, 1.0, l)))
    return o, lse


# --------------------------------------------------------------------------
# whole calls: every row q0_b .. N_b - 1 of every sequence, Q head and layer
# --------------------------------------------------------------------------

def default_scale(spec: Spec) -> float:
    return 1.0 / math.sqrt(spec.head_dim)


def attention(spec: Spec, layer: int, q_bits: np.ndarray, k_bits: np.ndarray,
              v_bits: np.ndarray, scale: float = None) -> Tuple[np.ndarray, np.ndarray]:
    """All rows of one layer. q_bits uint16 [T_q, Hq, D] (rows q0_b..N_b-1 of each
    sequence, packed in sequence order); k_bits/v_bits uint16 [T_total, Hkv, D].
    Returns O fp64 [T_q, Hq, D] and LSE fp64 [T_q, Hq]. A decode call is this
    with q0_b = N_b - 1 (one row per sequence)."""
    scale = default_scale(spec) if scale is None else scale
    g = spec.group
    q = bf16_bits_to_f64(q_bits)
    k = bf16_bits_to_f64(k_bits)
    v = bf16_bits_to_f64(v_bits)
    o = np.zeros(q.shape)
    lse = np.zeros(q.shape[:2])
    kvo, qo = spec.kv_row_offsets(), spec.q_row_offsets()
    for b, (nb, q0) in enumerate(zip(spec.seq_len, spec.first_query_pos)):
        rows = np.arange(q0, nb)
        if len(rows) == 0:
            continue
        qs = slice(qo[b], qo[b] + len(rows))
        for h in range(spec.num_kv_heads):
            kind, sink, window = spec.head_class(layer, h)
            retr = spec.retrieval.get((b, layer, h))
            mask = visibility_mask(kind, sink, window, retr, rows, nb)
            kh = k[kvo[b]:kvo[b] + nb, h]
            vh = v[kvo[b]:kvo[b] + nb, h]
            for hq in range(h * g, (h + 1) * g):
                o[qs, hq], lse[qs, hq] = attend_masked(q[qs, hq], kh, vh, mask, scale)
    return o, lse


def attention_rows(spec: Spec, layer: int, b: int, positions: Sequence[int],
                   q_rows_bits: np.ndarray, k_seq_bits: np.ndarray, v_seq_bits: np.ndarray,
                   scale: float = None) -> Tuple[np.ndarray, np.ndarray]:
    """Selected rows of one sequence: q_rows_bits uint16 [R, Hq, D] at the given
    positions, k/v_seq_bits uint16 [N_b, Hkv, D] of that sequence. Returns
    O [R, Hq, D], LSE [R, Hq]. Used for sampled-row checks on long inputs."""
    scale = default_scale(spec) if scale is None else scale
    g = spec.group
    q = bf16_bits_to_f64(q_rows_bits)
    rows = np.asarray(positions, dtype=np.int64)
    nb = spec.seq_len[b]
    o = np.zeros(q.shape)
    lse = np.zeros(q.shape[:2])
    for h in range(spec.num_kv_heads):
        kind, sink, window = spec.head_class(layer, h)
        retr = spec.retrieval.get((b, layer, h))
        mask = visibility_mask(kind, sink, window, retr, rows, nb)
        kh = bf16_bits_to_f64(k_seq_bits[:, h])
        vh = bf16_bits_to_f64(v_seq_bits[:, h])
        for hq in range(h * g, (h + 1) * g):
            o[:, hq], lse[:, hq] = attend_masked(q[:, hq], kh, vh, mask, scale)
    return o, lse


def visible_pairs(kind: int, sink: int, window: int, retr, n: int, q0: int = 0) -> int:
    """Number of visible (query, key) pairs over rows q0..n-1 of one head, by
    counting the mask row by row (no closed form used)."""
    total = 0
    for i0 in range(q0, n, 4096):
        rows = np.arange(i0, min(i0 + 4096, n))
        total += int(visibility_mask(kind, sink, window, retr, rows, n).sum())
    return total
