"""Seeded synthetic workloads for SegPagedAttention.

This is the one module that both the CPU oracle and the GPU path read. It holds
workload shapes, head classes, sequence lengths, retrieval index sets and the
bf16 bit patterns of Q/K/V. It holds none of the method's arithmetic: no
visibility rule, no page arithmetic, no attention.

Head classes follow the SegPagedAttention runtime explainer, section 2 (the
four per-(layer, KV head) policies: local, global, retrieval, dense) and the
released Llama-3.3-70B-style configuration quoted there (80 layers x 8 KV
heads, about 15% global, local window 8192, sink 4). Classes here are drawn by
seed, because the released files are not available.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional, Tuple

import numpy as np

GLOBAL, LOCAL, RETRIEVAL, DENSE = 0, 1, 2, 3
KIND_NAMES = {GLOBAL: "global", LOCAL: "local", RETRIEVAL: "retrieval", DENSE: "dense"}

# stream tags for numpy's seeded generators: rng([seed, TAG, ...])
_TAG_CLASS, _TAG_LEN, _TAG_RETR, _TAG_FREE = 0, 1, 2, 3
_TAG_Q, _TAG_K, _TAG_V = 10, 11, 12


@dataclass
class Spec:
    """Plain description of one SegPaged cache and the rows that will read it.

    seq_len[b]          N_b, tokens in sequence b's cache (including the current one)
    first_query_pos[b]  q0_b, lowest query position that will read the table
                        (0 = prefill form, N_b - 1 = decode form)
    kind/sink/window    per (layer, KV head), index l * num_kv_heads + h
    retrieval           {(b, l, h): sorted unique int32 positions} for RETRIEVAL heads
    free_list           page ids in allocation order (None = identity)
    capacity_pages      pool capacity in pages the caller provides (0 = exactly what is needed)
    doc_group[b]        document group of sequence b (-1 = none): sequences of one group
                        begin with the same doc_len[b] tokens (None = no groups)
    doc_len[b]          tokens of that shared document (equal within a group)
    """

    name: str
    num_layers: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    seq_len: List[int]
    first_query_pos: List[int]
    kind: List[int]
    sink: List[int]
    window: List[int]
    retrieval: Dict[Tuple[int, int, int], np.ndarray] = field(default_factory=dict)
    free_list: Optional[np.ndarray] = None
    capacity_pages: int = 0
    seed: int = 0
    doc_group: Optional[List[int]] = None
    doc_len: Optional[List[int]] = None

    @property
    def num_seqs(self) -> int:
        return len(self.seq_len)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seq_len))

    @property
    def total_q_rows(self) -> int:
        return int(sum(n - q for n, q in zip(self.seq_len, self.first_query_pos)))

    def kv_row_offsets(self) -> List[int]:
        out, acc = [], 0
        for n in self.seq_len:
            out.append(acc)
            acc += n
        return out

    def q_row_offsets(self) -> List[int]:
        out, acc = [], 0
        for n, q in zip(self.seq_len, self.first_query_pos):
            out.append(acc)
            acc += n - q
        return out

    def head_class(self, layer: int, kv_head: int) -> Tuple[int, int, int]:
        i = layer * self.num_kv_heads + kv_head
        return self.kind[i], self.sink[i], self.window[i]


# ----------------------------------------------------------------------------
# forms: the same cache read by prefill rows (q0 = 0) or by the decode row (q0 = N-1)
# ----------------------------------------------------------------------------

def prefill_form(spec: Spec) -> Spec:
    return replace(spec, first_query_pos=[0] * spec.num_seqs)


def decode_form(spec: Spec) -> Spec:
    return replace(spec, first_query_pos=[max(n - 1, 0) for n in spec.seq_len])


# ----------------------------------------------------------------------------
# head classes and lengths
# ----------------------------------------------------------------------------

def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng([int(k) for k in key])


def seeded_classes(num_layers: int, num_kv_heads: int, seed: int,
                   frac_global: float, frac_retrieval: float = 0.0) -> List[int]:
    """Per-(layer, KV head) classes: round(f * count) heads of each non-local
    class (Python rounding), chosen by a seeded permutation; the rest LOCAL."""
    n = num_layers * num_kv_heads
    n_glob = int(round(frac_global * n))
    n_retr = int(round(frac_retrieval * n))
    perm = _rng(seed, _TAG_CLASS).permutation(n)
    kind = [LOCAL] * n
    for i in perm[:n_glob]:
        kind[int(i)] = GLOBAL
    for i in perm[n_glob:n_glob + n_retr]:
        kind[int(i)] = RETRIEVAL
    return kind


def seeded_retrieval_sets(spec_seq_len: List[int], kind: List[int], num_layers: int,
                          num_kv_heads: int, seed: int, frac: float
                          ) -> Dict[Tuple[int, int, int], np.ndarray]:
    """For every sequence b and every RETRIEVAL (l, h): round(frac * N_b)
    positions sampled without replacement from [0, N_b), sorted."""
    out = {}
    for b, nb in enumerate(spec_seq_len):
        for l in range(num_layers):
            for h in range(num_kv_heads):
                if kind[l * num_kv_heads + h] != RETRIEVAL:
                    continue
                cnt = int(round(frac * nb))
                r = _rng(seed, _TAG_RETR, b, l, h)
                pos = np.sort(r.choice(nb, size=cnt, replace=False)).astype(np.int32)
                out[(b, l, h)] = pos
    return out


def seeded_free_list(capacity: int, seed: int) -> np.ndarray:
    return _rng(seed, _TAG_FREE).permutation(capacity).astype(np.int32)


# ----------------------------------------------------------------------------
# the five workloads (tiny, Mistral-7B-shaped layer, Llama-3.3-70B-shaped decode,
# long prefill, mixed-length decode) plus knobs that shrink them for parity tests
# ----------------------------------------------------------------------------

def tiny(form: str = "prefill", n: int = 512) -> Spec:
    """1 layer, 1 sequence, 8 Q / 4 KV heads, D 64, page 16. KV head 0 global,
    heads 1-3 local (sink 4, window 64). Prefill over n tokens; the decode step
    reads a cache of n + 1 tokens at position n."""
    nb = n if form == "prefill" else n + 1
    s = Spec(name="tiny", num_layers=1, num_q_heads=8, num_kv_heads=4, head_dim=64,
             page_size=16, seq_len=[nb], first_query_pos=[0],
             kind=[GLOBAL, LOCAL, LOCAL, LOCAL], sink=[4] * 4, window=[64] * 4, seed=1)
    return prefill_form(s) if form == "prefill" else decode_form(s)


def mistral_layer(form: str = "prefill", seqs: int = 4, n: int = 8192,
                  window: int = 1024) -> Spec:
    """Mistral-7B-shaped single layer: 32 Q / 8 KV heads, D 128, page 64. KV head 0
    global, heads 1-7 local (sink 4, window 1024)."""
    nb = n if form == "prefill" else n + 1
    kind = [GLOBAL] + [LOCAL] * 7
    s = Spec(name="mistral7b-layer", num_layers=1, num_q_heads=32, num_kv_heads=8,
             head_dim=128, page_size=64, seq_len=[nb] * seqs, first_query_pos=[0] * seqs,
             kind=kind, sink=[4] * 8, window=[window] * 8, seed=2)
    return prefill_form(s) if form == "prefill" else decode_form(s)


def llama70b_decode(num_layers: int = 80, seqs: int = 8, n: int = 32768,
                    window: int = 8192, seed: int = 3) -> Spec:
    """Llama-3.3-70B-shaped decode: 8 KV heads / 64 Q heads per layer, D 128, page 64,
    15% of the (layer, head) pairs global by seed, the rest local (sink 4, window 8192).
    One query token per sequence at position n - 1."""
    kind = seeded_classes(num_layers, 8, seed, 0.15)
    s = Spec(name="llama70b-decode", num_layers=num_layers, num_q_heads=64, num_kv_heads=8,
             head_dim=128, page_size=64, seq_len=[n] * seqs, first_query_pos=[0] * seqs,
             kind=kind, sink=[4] * len(kind), window=[window] * len(kind), seed=seed)
    return decode_form(s)


def long_prefill(num_layers: int = 64, n: int = 131072, window: int = 8192,
                 seed: int = 4) -> Spec:
    """One long sequence, 64 Q / 8 KV heads, D 128, page 64, 15% global by seed,
    local (sink 4, window 8192). Causal prefill of all n tokens."""
    kind = seeded_classes(num_layers, 8, seed, 0.15)
    s = Spec(name="long-prefill", num_layers=num_layers, num_q_heads=64, num_kv_heads=8,
             head_dim=128, page_size=64, seq_len=[n], first_query_pos=[0],
             kind=kind, sink=[4] * len(kind), window=[window] * len(kind), seed=seed)
    return prefill_form(s)


def mixed_lengths(seqs: int, lo: int, hi: int, seed: int) -> List[int]:
    """N_b = round(exp(U[ln lo, ln hi])) by seed."""
    u = _rng(seed, _TAG_LEN).uniform(math.log(lo), math.log(hi), size=seqs)
    return [int(round(math.exp(x))) for x in u]


def mixed_varlen_decode(seqs: int = 32, num_layers: int = 48, lo: int = 2048,
                        hi: int = 131072, window: int = 4096, seed: int = 5,
                        retrieval_frac: float = 0.05) -> Spec:
    """Mixed-length decode: log-uniform lengths, 64 Q / 8 KV heads, D 128, page 64;
    12% global, 8% retrieval (each attends a seeded sorted 5% index set, stored
    gathered), the rest local (sink 4, window 4096)."""
    kind = seeded_classes(num_layers, 8, seed, 0.12, 0.08)
    lens = mixed_lengths(seqs, lo, hi, seed)
    retr = seeded_retrieval_sets(lens, kind, num_layers, 8, seed, retrieval_frac)
    s = Spec(name="mixed-varlen-decode", num_layers=num_layers, num_q_heads=64,
             num_kv_heads=8, head_dim=128, page_size=64, seq_len=lens,
             first_query_pos=[0] * seqs, kind=kind, sink=[4] * len(kind),
             window=[window] * len(kind), retrieval=retr, seed=seed)
    return decode_form(s)


# ----------------------------------------------------------------------------
# Q/K/V bit patterns: N(0,1) in fp32, rounded to nearest even bf16
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to the nearest bf16 (ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def _normal_bits(shape, *key: int) -> np.ndarray:
    return f32_to_bf16_bits(_rng(*key).standard_normal(size=shape, dtype=np.float32))


def kv_bits(spec: Spec, layer: int, seed: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Dense K and V of one layer, uint16 bf16 bits [T_total, Hkv, D]. Each
    sequence draws its rows from its own stream, so the first n rows of a
    sequence do not depend on its length."""
    seed = spec.seed if seed is None else seed
    hk, d = spec.num_kv_heads, spec.head_dim
    ks, vs = [], []
    for b, nb in enumerate(spec.seq_len):
        ks.append(_normal_bits((nb, hk, d), seed, _TAG_K, layer, b))
        vs.append(_normal_bits((nb, hk, d), seed, _TAG_V, layer, b))
    if spec.doc_group is not None:
        # a shared document: every member's first doc_len rows are the first
        # member's (the same tokens at the same positions)
        first = {}
        for b, g in enumerate(spec.doc_group):
            if g < 0:
                continue
            if g not in first:
                first[g] = b
                continue
            c, b0 = spec.doc_len[b], first[g]
            ks[b][:c] = ks[b0][:c]
            vs[b][:c] = vs[b0][:c]
    return np.concatenate(ks, axis=0), np.concatenate(vs, axis=0)


def q_bits(spec: Spec, layer: int, seed: Optional[int] = None) -> np.ndarray:
    """Q rows of one layer for positions q0_b .. N_b - 1 of each sequence, packed in
    sequence order: uint16 bf16 bits [T_q, Hq, D]."""
    seed = spec.seed if seed is None else seed
    out = []
    for b, (nb, q0) in enumerate(zip(spec.seq_len, spec.first_query_pos)):
        out.append(_normal_bits((nb - q0, spec.num_q_heads, spec.head_dim),
                                seed, _TAG_Q, layer, b, q0))
    return np.concatenate(out, axis=0)


def randn_bf16_device(shape, seed: int, tag: int, layer: int, device="cuda"):
    """Large inputs drawn on the GPU: torch's seeded device generator, N(0,1) fp32
    rounded to bf16. The oracle receives the same bits by a device-to-host copy."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + tag * 10_007 + layer) & 0x7FFFFFFFFFFFFFFF)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


TAG_Q, TAG_K, TAG_V = _TAG_Q, _TAG_K, _TAG_V
