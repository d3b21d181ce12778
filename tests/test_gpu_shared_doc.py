"""Document chunks shared by several sequences (doc_group / doc_len): the pages
inside a group's shared document are stored once per (layer, KV head) and listed in
every member's page list. On the GPU: the pool is bit-exact against the oracle's
(each distinct page written once), prefill and decode of every member match the
oracle, and a page stream carries each distinct page once and imports into a plan
of the same spec with other page ids."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as OA
from oracle import layout as OL
from tests.gpu_util import assert_image_equal, lse_parity, parity, to_bits, to_dev, to_f64
from tests.test_planner import _doc_specs

sp = pytest.importorskip("sparse_attention_segmentpagetable_amd")
pytestmark = pytest.mark.gpu

DEV = "cuda"


def _mistral_doc(form):
    s = W.mistral_layer("prefill", seqs=3, n=3000, window=512)
    s = replace(s, name=f"mistral-doc-{form}", seq_len=[3000, 2600, 3000],
                first_query_pos=[0, 0, 0], doc_group=[0, 0, 0], doc_len=[2000] * 3)
    return s if form == "prefill" else W.decode_form(s)


SPECS = [(s.name, s) for s in _doc_specs()] + [
    ("mistral-doc-prefill", _mistral_doc("prefill")), ("mistral-doc-decode", _mistral_doc("decode"))]


@pytest.mark.parametrize("name,spec", SPECS, ids=[n for n, _ in SPECS])
def test_shared_document_pool_and_attention(name, spec):
    plan = sp.Plan(spec)
    assert plan.sizes.num_pages == OL.distinct_pages(spec) < OL.num_pages(spec)
    bufs = plan.allocate(DEV)
    P, D = spec.page_size, spec.head_dim
    scale = 1 / np.sqrt(D)
    decode = all(q0 == max(n - 1, 0) for n, q0 in zip(spec.seq_len, spec.first_query_pos))
    for l in range(spec.num_layers):
        kb, vb = W.kv_bits(spec, l)
        sp.build(plan, l, to_dev(kb), to_dev(vb), bufs["table"], bufs["k_pool"], bufs["v_pool"])
        torch.cuda.synchronize()
        kp_ref, vp_ref, written = OL.pool(spec, l, kb, vb, plan.sizes.pool_pages)
        kp = to_bits(bufs["k_pool"]).reshape(-1, D // 8, P, 8)
        vp = to_bits(bufs["v_pool"]).reshape(-1, P // 8, D, 8)
        assert np.array_equal(kp[written], kp_ref[written]), (name, l)
        assert np.array_equal(vp[written], vp_ref[written]), (name, l)
        qb = W.q_bits(spec, l)
        q = to_dev(qb)
        o = torch.full_like(q, float("nan"))
        lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device=DEV)
        if decode:
            sp.decode(plan, l, q, bufs["table"], bufs["k_pool"], bufs["v_pool"], scale, o, lse,
                      workspace=bufs["workspace"])
        else:
            sp.prefill(plan, l, q, bufs["table"], bufs["k_pool"], bufs["v_pool"], scale, o, lse)
        torch.cuda.synchronize()
        ref, ref_lse = OA.attention(spec, l, qb, kb, vb, scale)
        parity(to_f64(o), ref, f"{name} {'decode' if decode else 'prefill'} L{l}")
        lse_parity(lse.cpu().numpy(), ref_lse, f"{name} L{l}")
    assert_image_equal(bufs["table"].cpu().numpy(), plan)


def test_shared_document_page_stream():
    spec = _mistral_doc("decode")
    src = sp.Plan(spec)
    sb = src.allocate(DEV)
    kb, vb = W.kv_bits(spec, 0)
    sp.build(src, 0, to_dev(kb), to_dev(vb), sb["table"], sb["k_pool"], sb["v_pool"])
    n = sp.stream_elems(src, 0)
    assert n == OL.distinct_pages(spec) * spec.page_size * spec.head_dim
    ko = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    vo = torch.empty_like(ko)
    sp.export_pages(src, 0, sb["table"], sb["k_pool"], sb["v_pool"], ko, vo)
    torch.cuda.synchronize()
    ks_ref, vs_ref = OL.transfer_stream(spec, 0, kb, vb)
    assert np.array_equal(to_bits(ko), ks_ref.reshape(-1))
    assert np.array_equal(to_bits(vo), vs_ref.reshape(-1))
    cap = OL.distinct_pages(spec) + 37
    recv_spec = replace(spec, free_list=W.seeded_free_list(cap, 5), capacity_pages=cap)
    recv = sp.Plan(recv_spec)
    rb = recv.allocate(DEV)
    sp.import_pages(recv, 0, ko, vo, rb["table"], rb["k_pool"], rb["v_pool"])
    qb = W.q_bits(spec, 0)
    q = to_dev(qb)
    o = torch.empty_like(q)
    sp.decode(recv, 0, q, rb["table"], rb["k_pool"], rb["v_pool"], 1 / np.sqrt(128), o,
              workspace=rb["workspace"])
    torch.cuda.synchronize()
    ref, _ = OA.attention(spec, 0, qb, kb, vb)
    parity(to_f64(o), ref, "decode after importing a shared-document stream")
