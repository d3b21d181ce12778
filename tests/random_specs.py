"""Seeded random specs shared by the CPU planner tests and the GPU parity tests:
classes, lengths (including 0 and 1), sinks, windows, retrieval sets, page sizes,
head dims, group sizes, first query rows and free lists, all drawn from a seed."""
from dataclasses import replace

import numpy as np

import workloads as W
from oracle import layout as OL


def random_spec(seed):
    r = np.random.default_rng([seed, 0x5E6])
    P = int(r.choice([16, 32, 64, 128]))
    D = int(r.choice([64, 128]))
    Hkv = int(r.integers(1, 4))
    G = int(r.choice([1, 2, 3, 4, 8]))
    L = int(r.integers(1, 3))
    B = int(r.integers(1, 4))
    lens = [int(x) for x in r.choice([0, 1, 2, 17, 63, 64, 65, 200, 511, 700, 1300], size=B)]
    if max(lens) == 0:
        lens[0] = 33
    kind = [int(x) for x in r.choice([W.GLOBAL, W.LOCAL, W.LOCAL, W.RETRIEVAL, W.DENSE],
                                     size=L * Hkv)]
    sink = [int(x) for x in r.choice([0, 1, 4, 40], size=L * Hkv)]
    window = [int(x) for x in r.choice([1, 2, 31, 64, 100, 900], size=L * Hkv)]
    retr = {}
    for b, n in enumerate(lens):
        for l in range(L):
            for h in range(Hkv):
                if kind[l * Hkv + h] == W.RETRIEVAL:
                    cnt = int(r.integers(0, n + 1)) if n else 0
                    retr[(b, l, h)] = np.sort(r.choice(n, size=cnt, replace=False)).astype(np.int32) \
                        if cnt else np.array([], np.int32)
    form = r.choice(["prefill", "decode", "mid"])
    if form == "prefill":
        q0 = [0] * B
    elif form == "decode":
        q0 = [max(n - 1, 0) for n in lens]
    else:
        q0 = [int(r.integers(0, max(n, 1))) for n in lens]
    spec = W.Spec(name=f"rand{seed}", num_layers=L, num_q_heads=G * Hkv, num_kv_heads=Hkv,
                  head_dim=D, page_size=P, seq_len=lens, first_query_pos=q0, kind=kind,
                  sink=sink, window=window, retrieval=retr, seed=seed)
    npg = OL.num_pages(spec)
    if r.random() < 0.5:  # a permuted free list over a larger pool
        cap = npg + int(r.integers(0, 50))
        spec = replace(spec, free_list=W.seeded_free_list(max(cap, 1), seed),
                       capacity_pages=max(cap, 1))
    return spec
