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
from tests.random_specs import random_spec as _random_spec

sp = pytest.importorskip("sparse_attention_segmentpagetable_amd")
pytestmark = pytest.mark.gpu

DEV = "cuda"
SEEDS = list(range(100, 164))


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
