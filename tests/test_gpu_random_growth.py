"""GPU parity of growth plans on seeded random specs: a cache planned with an append
capacity and chunk grows by random counts per sequence (segpaged_plan_append +
segpaged_append, per layer or all layers at once); after every append the newest
rows (prefill) and the last row (decode) of every layer against the oracle on the
grown dense history."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as OA
from tests.gpu_util import assert_image_equal, lse_parity, parity, to_dev, to_f64

sp = pytest.importorskip("sparse_attention_segmentpagetable_amd")
pytestmark = pytest.mark.gpu

DEV = "cuda"
SEEDS = list(range(300, 332))


def _case(seed):
    r = np.random.default_rng([seed, 0x6A0])
    P = int(r.choice([16, 32, 64, 128]))
    D = int(r.choice([64, 128]))
    Hkv = int(r.integers(1, 4))
    G = int(r.choice([1, 2, 4, 8]))
    L = int(r.integers(1, 3))
    B = int(r.integers(1, 4))
    chunk = int(r.choice([1, 3, 16, 64]))
    cap = int(r.integers(1, 300))
    n0 = [int(x) for x in r.integers(0, 400, size=B)]
    if seed % 4 == 0:
        n0[0] = 0  # a sequence that starts empty
    kind = [int(x) for x in r.choice([W.GLOBAL, W.LOCAL, W.LOCAL, W.RETRIEVAL, W.DENSE],
                                     size=L * Hkv)]
    sink = [int(x) for x in r.choice([0, 1, 4, 40], size=L * Hkv)]
    window = [int(x) for x in r.choice([1, 2, 31, 64, 100], size=L * Hkv)]
    retr = {}
    for b, n in enumerate(n0):
        for l in range(L):
            for h in range(Hkv):
                if kind[l * Hkv + h] == W.RETRIEVAL:
                    cnt = int(r.integers(0, n + 1)) if n else 0
                    retr[(b, l, h)] = (np.sort(r.choice(n, size=cnt, replace=False)).astype(np.int32)
                                       if cnt else np.array([], np.int32))
    q0 = [max(n - int(r.integers(1, chunk + 1)), 0) for n in n0]  # at most one chunk of rows
    spec = W.Spec(name=f"grow{seed}", num_layers=L, num_q_heads=G * Hkv, num_kv_heads=Hkv,
                  head_dim=D, page_size=P, seq_len=n0, first_query_pos=q0, kind=kind,
                  sink=sink, window=window, retrieval=retr, seed=seed)
    return spec, cap, chunk, bool(r.random() < 0.5), r


def _pack(per_seq, n):
    return np.concatenate([a[:m] for a, m in zip(per_seq, n)], axis=0)


@pytest.mark.parametrize("seed", SEEDS)
def test_random_growth(seed):
    spec, cap, chunk, all_layers, r = _case(seed)
    L, B, Hkv, D = spec.num_layers, spec.num_seqs, spec.num_kv_heads, spec.head_dim
    full = replace(spec, seq_len=[n + cap for n in spec.seq_len],
                   first_query_pos=[n + cap - 1 for n in spec.seq_len])
    kvo = full.kv_row_offsets()
    hist = []
    for l in range(L):
        kb, vb = W.kv_bits(full, l)
        hist.append(([kb[kvo[b]:kvo[b] + full.seq_len[b]] for b in range(B)],
                     [vb[kvo[b]:kvo[b] + full.seq_len[b]] for b in range(B)]))
    plan = sp.Plan(spec, append_capacity=cap, append_chunk=chunk)
    bufs = plan.allocate(DEV)
    n = list(spec.seq_len)
    for l in range(L):
        if sum(n):
            sp.build(plan, l, to_dev(_pack(hist[l][0], n)), to_dev(_pack(hist[l][1], n)),
                     bufs["table"], bufs["k_pool"], bufs["v_pool"])
        else:
            sp.build(plan, l, to_dev(np.zeros((1, Hkv, D), np.uint16)),
                     to_dev(np.zeros((1, Hkv, D), np.uint16)), bufs["table"], bufs["k_pool"],
                     bufs["v_pool"])
    scale = 1.0 / np.sqrt(D)
    for step in range(10):
        add = [int(min(r.integers(0, chunk + 1), full.seq_len[b] - n[b])) for b in range(B)]
        plan.append(add)
        nk = [np.concatenate([hist[l][0][b][n[b]:n[b] + add[b]] for b in range(B)]) for l in range(L)]
        nv = [np.concatenate([hist[l][1][b][n[b]:n[b] + add[b]] for b in range(B)]) for l in range(L)]
        n = [x + a for x, a in zip(n, add)]
        if sum(add):
            if all_layers:
                sp.append(plan, -1, to_dev(np.stack(nk)), to_dev(np.stack(nv)), bufs["table"],
                          bufs["k_pool"], bufs["v_pool"])
            else:
                for l in range(L):
                    sp.append(plan, l, to_dev(nk[l]), to_dev(nv[l]), bufs["table"],
                              bufs["k_pool"], bufs["v_pool"])
        else:  # nothing new: the call still uploads the updated image
            sp.append(plan, -1, None, None, bufs["table"], bufs["k_pool"], bufs["v_pool"])
        q0 = [max(x - max(a, 1), 0) for x, a in zip(n, add)]
        cur = replace(spec, seq_len=list(n), first_query_pos=q0)
        for l in range(L):
            K, V = _pack(hist[l][0], n), _pack(hist[l][1], n)
            # the rows of the newest chunk
            qb = W.q_bits(cur, l, seed=1000 + step)
            if qb.shape[0]:
                q = to_dev(qb)
                o = torch.full_like(q, float("nan"))
                lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device=DEV)
                sp.prefill(plan, l, q, bufs["table"], bufs["k_pool"], bufs["v_pool"], scale, o, lse)
                torch.cuda.synchronize()
                ref, ref_lse = OA.attention(cur, l, qb, K, V, scale)
                parity(to_f64(o), ref, f"seed {seed} step {step} prefill L{l} n={n}")
                lse_parity(lse.cpu().numpy(), ref_lse, f"seed {seed} step {step} prefill L{l}")
            # the last row
            rows = [b for b in range(B) if n[b] > 0]
            dec = replace(spec, seq_len=list(n), first_query_pos=[max(x - 1, 0) for x in n])
            qd = W.q_bits(dec, l, seed=2000 + step)
            qfull = np.zeros((B, spec.num_q_heads, D), np.uint16)
            qfull[rows] = qd
            qt = to_dev(qfull)
            od = torch.full_like(qt, float("nan"))
            lsed = torch.full(qt.shape[:2], float("nan"), dtype=torch.float32, device=DEV)
            sp.decode(plan, l, qt, bufs["table"], bufs["k_pool"], bufs["v_pool"], scale, od, lsed,
                      workspace=bufs["workspace"])
            torch.cuda.synchronize()
            if rows:
                ref, ref_lse = OA.attention(dec, l, qd, K, V, scale)
                of, lf = to_f64(od), lsed.cpu().numpy()
                parity(of[rows], ref, f"seed {seed} step {step} decode L{l} n={n}")
                lse_parity(lf[rows], ref_lse, f"seed {seed} step {step} decode L{l}")
    assert_image_equal(bufs["table"].cpu().numpy(), plan)
