"""GPU parity on seeded random specs: classes, lengths (including 0 and 1), sinks,
windows, retrieval sets, page sizes, head dims, group sizes, first query rows and
free lists all drawn from a fixed seed list, so every run checks the same cases.
Prefill and decode of every layer against the oracle, and the table against the
oracle's table."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as OA
from oracle import layout as OL
from tests.gpu_util import lse_parity, parity, to_dev, to_f64

sp = pytest.importorskip("sparse_attention_segmentpagetable_amd")
pytestmark = pytest.mark.gpu

DEV = "cuda"
SEEDS = list(range(100, 164))


def _random_spec(seed):
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


@pytest.mark.parametrize("seed", SEEDS)
def test_random_spec(seed):
    spec = _random_spec(seed)
    plan = sp.Plan(spec)
    bufs = plan.allocate(DEV)
    assert np.array_equal(plan.table_host()[:plan.sizes.table_len], OL.table(spec))
    scale = 1 / np.sqrt(spec.head_dim)
    for l in range(spec.num_layers):
        kb, vb = W.kv_bits(spec, l)
        if kb.shape[0] == 0:
            continue
        sp.build(plan, l, to_dev(kb), to_dev(vb), bufs["table"], bufs["k_pool"], bufs["v_pool"])
        qb = W.q_bits(spec, l)
        if qb.shape[0] > 0:
            q = to_dev(qb)
            o = torch.full_like(q, float("nan"))
            lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device=DEV)
            sp.prefill(plan, l, q, bufs["table"], bufs["k_pool"], bufs["v_pool"], scale, o, lse)
            torch.cuda.synchronize()
            ref, ref_lse = OA.attention(spec, l, qb, kb, vb, scale=scale)
            parity(to_f64(o), ref, f"seed {seed} prefill L{l}")
            lse_parity(lse.cpu().numpy(), ref_lse, f"seed {seed} prefill L{l}")
        # the decode row of every sequence (position N_b - 1), on the same table
        dspec = W.decode_form(spec)
        qd_bits = W.q_bits(dspec, l)
        if qd_bits.shape[0] == spec.num_seqs:
            qd = to_dev(qd_bits)
            od = torch.full_like(qd, float("nan"))
            lsed = torch.full(qd.shape[:2], float("nan"), dtype=torch.float32, device=DEV)
            sp.decode(plan, l, qd, bufs["table"], bufs["k_pool"], bufs["v_pool"], scale, od, lsed,
                      workspace=bufs["workspace"])
            torch.cuda.synchronize()
            ref, ref_lse = OA.attention(dspec, l, qd_bits, kb, vb, scale=scale)
            parity(to_f64(od), ref, f"seed {seed} decode L{l}")
            lse_parity(lsed.cpu().numpy(), ref_lse, f"seed {seed} decode L{l}")
