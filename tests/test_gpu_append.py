"""Decode loop with append on the GPU: a cache planned once in decode form grows
step by step (segpaged_plan_append + segpaged_append, then segpaged_decode);
every step's O and LSE against the oracle on the grown dense history, the pool
bit-exact at every position the decode row sees (the oracle's ring model), and
the device table equal to the plan's image."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as OA
from oracle import layout as OL
from tests.gpu_util import assert_image_equal, lse_parity, parity, to_bits, to_dev, to_f64

sp = pytest.importorskip("sparse_attention_segmentpagetable_amd")
pytestmark = pytest.mark.gpu
DEV = "cuda"


def _spec(hd, ps, n0):
    kind = [W.GLOBAL, W.LOCAL, W.LOCAL, W.RETRIEVAL, W.DENSE, W.LOCAL]
    retr = {(0, 1, 0): np.array([1, 2, 30, 31, 32], np.int32),
            (2, 1, 0): np.array([0], np.int32)}
    s = W.Spec(name="append", num_layers=2, num_q_heads=6, num_kv_heads=3, head_dim=hd,
               page_size=ps, seq_len=list(n0), first_query_pos=[0] * len(n0), kind=kind,
               sink=[0, 3, 0, 0, 0, 20], window=[1, 37, 20, 1, 1, 5], retrieval=retr, seed=21)
    return W.decode_form(s)


def _pack(per_seq, n):
    return np.concatenate([a[:m] for a, m in zip(per_seq, n)], axis=0)


CASES = [
    ("d64-p16-per-layer", 64, 16, (50, 17, 1, 0), 60, False),
    ("d128-p64-all-layers", 128, 64, (130, 3, 70, 1), 150, True),
    ("d128-p32-all-layers", 128, 32, (40, 0, 9, 100), 90, True),
]


@pytest.mark.parametrize("name,hd,ps,n0,cap,all_layers", CASES, ids=[c[0] for c in CASES])
def test_decode_loop_with_append(name, hd, ps, n0, cap, all_layers):
    spec = _spec(hd, ps, n0)
    L, B, Hkv = spec.num_layers, spec.num_seqs, spec.num_kv_heads
    full = replace(spec, seq_len=[n + cap for n in n0],
                   first_query_pos=[n + cap - 1 for n in n0])
    kvo = full.kv_row_offsets()
    hist = []  # per layer: per sequence K and V bits [N_max, Hkv, D]
    for l in range(L):
        kb, vb = W.kv_bits(full, l)
        hist.append(([kb[kvo[b]:kvo[b] + full.seq_len[b]] for b in range(B)],
                     [vb[kvo[b]:kvo[b] + full.seq_len[b]] for b in range(B)]))
    plan = sp.Plan(spec, append_capacity=cap, decode_split_tokens=64, append_chunk=13)
    bufs = plan.allocate(DEV)
    n = list(n0)
    for l in range(L):
        sp.build(plan, l, to_dev(_pack(hist[l][0], n)), to_dev(_pack(hist[l][1], n)),
                 bufs["table"], bufs["k_pool"], bufs["v_pool"])
    rng = np.random.default_rng(hd + ps)
    scale = 1.0 / np.sqrt(hd)
    steps = 0
    while steps < 24 and any(x < y for x, y in zip(n, full.seq_len)):
        add = [int(x) for x in rng.choice([0, 1, 2, 5, 13], size=B)]
        add = [min(a, full.seq_len[b] - n[b]) for b, a in enumerate(add)]
        plan.append(add)
        new_k = [np.concatenate([hist[l][0][b][n[b]:n[b] + add[b]] for b in range(B)])
                 for l in range(L)]
        new_v = [np.concatenate([hist[l][1][b][n[b]:n[b] + add[b]] for b in range(B)])
                 for l in range(L)]
        n = [a + x for a, x in zip(n, add)]
        if all_layers:
            sp.append(plan, -1, to_dev(np.stack(new_k)), to_dev(np.stack(new_v)), bufs["table"],
                      bufs["k_pool"], bufs["v_pool"])
        else:
            for l in range(L):
                sp.append(plan, l, to_dev(new_k[l]), to_dev(new_v[l]), bufs["table"],
                          bufs["k_pool"], bufs["v_pool"])
        cur = replace(spec, seq_len=list(n), first_query_pos=[max(x - 1, 0) for x in n])
        rows = [b for b in range(B) if n[b] > 0]  # an empty sequence has no decode row
        for l in range(L):
            qb = W.q_bits(cur, l, seed=100 + steps)
            qfull = np.zeros((B, spec.num_q_heads, hd), np.uint16)
            qfull[rows] = qb
            q = to_dev(qfull)
            o = torch.full_like(q, float("nan"))
            lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device=DEV)
            sp.decode(plan, l, q, bufs["table"], bufs["k_pool"], bufs["v_pool"], scale, o, lse,
                      workspace=bufs["workspace"])
            torch.cuda.synchronize()
            ref, ref_lse = OA.attention(cur, l, qb, _pack(hist[l][0], n), _pack(hist[l][1], n),
                                        scale)
            of, lf = to_f64(o), lse.cpu().numpy()
            parity(of[rows], ref, f"{name} step {steps} L{l} n={n}")
            lse_parity(lf[rows], ref_lse, f"{name} step {steps} L{l}")
            empty = [b for b in range(B) if n[b] == 0]
            assert np.all(of[empty] == 0) and np.all(lf[empty] == -np.inf)
        steps += 1
    # pool: every key the decode row sees, at the slot the ring model gives
    t = plan.table_host()
    assert_image_equal(bufs["table"].cpu().numpy(), plan)
    moved = 0  # local windows that recycled at least one ring page
    for (u, b, l, h) in OL.units(spec):
        kind, s, w = spec.head_class(l, h)
        if kind == W.LOCAL:
            moved += int(t[int(t[12]) + 16 * u + 12]) - max(s, n0[b] - w) >= ps
    assert moved > 0
    pages = OL.append_unit_pages(spec, cap, 13)
    P, D = ps, hd
    kp = to_bits(bufs["k_pool"]).reshape(-1, D // 8, P, 8)
    vp = to_bits(bufs["v_pool"]).reshape(-1, P // 8, D, 8)
    for (u, b, l, h) in OL.units(spec):
        kind, s, w = spec.head_class(l, h)
        if kind == W.RETRIEVAL or n[b] == 0:
            continue
        vis = np.nonzero(OA.visibility_mask(kind, s, w, None, np.array([n[b] - 1]), n[b])[0])[0]
        for p in vis:
            pg, slot = OL.append_slot(spec, b, l, h, int(p), 13)
            pid = pages[(b, l, h)][pg]
            kref = hist[l][0][b][p, h]
            vref = hist[l][1][b][p, h]
            assert np.array_equal(kp[pid, :, slot, :].reshape(-1), kref), (name, u, p)
            assert np.array_equal(vp[pid, slot // 8, :, slot % 8], vref), (name, u, p)


CHUNK_CASES = [
    ("d128-p64-chunk128", 128, 64, 16, 128),
    ("d64-p16-chunk100", 64, 16, 4, 100),
]


@pytest.mark.parametrize("name,hd,ps,hq,chunk", CHUNK_CASES, ids=[c[0] for c in CHUNK_CASES])
def test_chunked_prefill(name, hd, ps, hq, chunk):
    """A long prefill taken a chunk at a time over a cache whose local heads hold
    only sink + a ring: each chunk's rows equal the oracle's full prefill rows."""
    final = [700, 333, 1029]
    kind = [W.GLOBAL, W.LOCAL, W.LOCAL, W.DENSE]
    s0 = W.Spec(name="chunked", num_layers=1, num_q_heads=hq, num_kv_heads=4, head_dim=hd,
                page_size=ps, seq_len=final, first_query_pos=[0, 0, 0], kind=kind,
                sink=[0, 4, 0, 0], window=[1, 130, 64, 1], seed=33)
    kb, vb = W.kv_bits(s0, 0)
    kvo = s0.kv_row_offsets()
    K = [kb[kvo[b]:kvo[b] + final[b]] for b in range(3)]
    V = [vb[kvo[b]:kvo[b] + final[b]] for b in range(3)]
    n = [min(chunk, f) for f in final]
    spec = replace(s0, seq_len=list(n), first_query_pos=[0, 0, 0])
    plan = sp.Plan(spec, append_capacity=max(final) - chunk, append_chunk=chunk)
    assert plan.sizes.num_pages < sp.Plan(s0).sizes.num_pages  # local heads: sink + ring only
    bufs = plan.allocate(DEV)
    sp.build(plan, 0, to_dev(_pack(K, n)), to_dev(_pack(V, n)), bufs["table"], bufs["k_pool"],
             bufs["v_pool"])
    q0 = [0, 0, 0]
    scale = 1.0 / np.sqrt(hd)
    step = 0
    while True:
        cur = replace(s0, seq_len=list(n), first_query_pos=list(q0))
        qb = W.q_bits(cur, 0, seed=200 + step)
        q = to_dev(qb)
        o = torch.full_like(q, float("nan"))
        lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device=DEV)
        sp.prefill(plan, 0, q, bufs["table"], bufs["k_pool"], bufs["v_pool"], scale, o, lse)
        torch.cuda.synchronize()
        ref, ref_lse = OA.attention(cur, 0, qb, _pack(K, n), _pack(V, n), scale)
        parity(to_f64(o), ref, f"{name} chunk {step} n={n} q0={q0}")
        lse_parity(lse.cpu().numpy(), ref_lse, f"{name} chunk {step}")
        add = [min(chunk, f - x) for f, x in zip(final, n)]
        if not any(add):
            break
        plan.append(add)
        nk = np.concatenate([K[b][n[b]:n[b] + add[b]] for b in range(3)])
        nv = np.concatenate([V[b][n[b]:n[b] + add[b]] for b in range(3)])
        sp.append(plan, 0, to_dev(nk), to_dev(nv), bufs["table"], bufs["k_pool"], bufs["v_pool"])
        n = [x + a for x, a in zip(n, add)]
        q0 = [x - max(a, 1) for x, a in zip(n, add)]
        step += 1
    assert n == final and step >= 7
