"""Retrieval-set selection on seeded random specs: group sizes 1-16, head dims 64
and 128, lengths at the edges of the 2048-key chunks and of the register-resident
path (32768 keys), empty and one-key sequences, mixed head classes, random p;
every set against the oracle with the checks of test_gpu_select."""
import numpy as np
import pytest

import workloads as W
from tests.test_gpu_select import _run, _scaled_q, check_sets

pytest.importorskip("sparse_attention_segmentpagetable_amd")
pytestmark = pytest.mark.gpu

SEEDS = list(range(500, 524))
LENS = [0, 1, 2, 63, 700, 2047, 2048, 2049, 4097, 9000, 32767, 32768, 32769, 70000]


def _case(seed):
    r = np.random.default_rng([seed, 0x5E1])
    hd = int(r.choice([64, 128]))
    G = int(r.choice([1, 2, 3, 4, 5, 8, 16]))
    Hkv = int(r.integers(1, 4))
    L = int(r.integers(1, 3))
    B = int(r.integers(1, 4))
    n = [int(x) for x in r.choice(LENS, size=B)]
    if max(n) == 0:
        n[0] = 2049
    kind = [int(x) for x in r.choice([W.RETRIEVAL, W.RETRIEVAL, W.LOCAL, W.GLOBAL], size=L * Hkv)]
    kind[int(r.integers(0, L * Hkv))] = W.RETRIEVAL
    retr = {(b, l, h): np.zeros(0, np.int32) for b in range(B) for l in range(L)
            for h in range(Hkv) if kind[l * Hkv + h] == W.RETRIEVAL}
    s = W.Spec(name=f"selrand{seed}", num_layers=L, num_q_heads=G * Hkv, num_kv_heads=Hkv,
               head_dim=hd, page_size=64, seq_len=n, first_query_pos=[0] * B, kind=kind,
               sink=[4] * (L * Hkv), window=[64] * (L * Hkv), retrieval=retr, seed=seed)
    p = float(r.choice([0.3, 0.8, 0.95, 0.999, 1.0]))
    return W.decode_form(s), p, float(r.choice([1.0, 4.0, 8.0]))


@pytest.mark.parametrize("seed", SEEDS)
def test_select_random_spec(seed):
    spec, p, qscale = _case(seed)
    rows = [b for b, n in enumerate(spec.seq_len) if n > 0]
    for layer in range(spec.num_layers):
        qb = np.zeros((spec.num_seqs, spec.num_q_heads, spec.head_dim), np.uint16)
        qb[rows] = _scaled_q(spec, layer, qscale)  # empty sequences have no decode row
        kb, _ = W.kv_bits(spec, layer)
        pos, cnt = _run(spec, layer, qb, kb, p)
        check_sets(spec, layer, qb, kb, pos, cnt, p, f"seed {seed}")
