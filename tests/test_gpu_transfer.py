"""GPU: a cache moved as a page stream (segpaged_export_pages / segpaged_import_pages)
against the oracle's stream and pool, bit for bit, and the moved cache read by a
decode on the receiving plan."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as OA
from oracle import layout as OL
from tests.gpu_util import lse_parity, parity, to_bits, to_dev, to_f64

sp = pytest.importorskip("sparse_attention_segmentpagetable_amd")
pytestmark = pytest.mark.gpu

DEV = "cuda"


def _spec(ps, free=None, cap=0, hd=128):
    """Three layers of mixed classes in decode form: sink pages with zero tails,
    two-segment local heads, gathered retrieval sets, ragged lengths."""
    kind = [W.GLOBAL, W.LOCAL, W.RETRIEVAL, W.LOCAL, W.LOCAL, W.GLOBAL]
    lens = [1500, 333, 2100]
    retr = W.seeded_retrieval_sets(lens, kind, 3, 2, 17, 0.1)
    s = W.Spec(name="moved", num_layers=3, num_q_heads=8, num_kv_heads=2, head_dim=hd,
               page_size=ps, seq_len=lens, first_query_pos=[0, 0, 0], kind=kind,
               sink=[0, 4, 0, 7, 0, 0], window=[1, 200, 1, 90, 1000, 1], retrieval=retr,
               free_list=free, capacity_pages=cap, seed=31)
    return W.decode_form(s)


@pytest.mark.parametrize("ps,hd", [(16, 128), (64, 128), (128, 64)])
def test_export_then_import_into_another_plan(ps, hd):
    sender = _spec(ps, hd=hd)
    send = sp.Plan(sender)
    sb = send.allocate(DEV)
    kvs = [W.kv_bits(sender, l) for l in range(3)]
    sp.build(send, -1, to_dev(np.stack([k for k, _ in kvs])), to_dev(np.stack([v for _, v in kvs])),
             sb["table"], sb["k_pool"], sb["v_pool"])
    P, D = ps, hd

    # the stream of each layer, and of all layers in one call
    streams = []
    for l in range(3):
        n = sp.stream_elems(send, l)
        ko = torch.full((n,), float("nan"), dtype=torch.bfloat16, device=DEV)
        vo = torch.full((n,), float("nan"), dtype=torch.bfloat16, device=DEV)
        sp.export_pages(send, l, sb["table"], sb["k_pool"], sb["v_pool"], ko, vo)
        torch.cuda.synchronize()
        ks_ref, vs_ref = OL.transfer_stream(sender, l, *kvs[l])
        assert np.array_equal(to_bits(ko).reshape(ks_ref.shape), ks_ref), f"K stream L{l}"
        assert np.array_equal(to_bits(vo).reshape(vs_ref.shape), vs_ref), f"V stream L{l}"
        streams.append((ko, vo))
    n_all = sp.stream_elems(send, -1)
    assert n_all == sum(k.numel() for k, _ in streams)
    ka = torch.empty(n_all, dtype=torch.bfloat16, device=DEV)
    va = torch.empty(n_all, dtype=torch.bfloat16, device=DEV)
    sp.export_pages(send, -1, sb["table"], sb["k_pool"], sb["v_pool"], ka, va)
    torch.cuda.synchronize()
    assert torch.equal(ka.view(torch.int16), torch.cat([k for k, _ in streams]).view(torch.int16))
    assert torch.equal(va.view(torch.int16), torch.cat([v for _, v in streams]).view(torch.int16))

    # the receiver: same spec, other page ids (seeded permutation of a larger pool)
    npg = send.sizes.num_pages
    cap = npg + 37
    receiver = replace(sender, free_list=W.seeded_free_list(cap, seed=8), capacity_pages=cap)
    recv = sp.Plan(receiver)
    rb = recv.allocate(DEV)
    rb["k_pool"].zero_()
    rb["v_pool"].zero_()
    for l in (2, 0, 1):  # any order; each call uploads its layer's table slice
        sp.import_pages(recv, l, *streams[l], rb["table"], rb["k_pool"], rb["v_pool"])
    torch.cuda.synchronize()
    kp = to_bits(rb["k_pool"]).reshape(-1, D // 8, P, 8)
    vp = to_bits(rb["v_pool"]).reshape(-1, P // 8, D, 8)
    written = np.zeros(len(kp), bool)
    for l in range(3):
        kp_ref, vp_ref, w = OL.pool(receiver, l, *kvs[l], len(kp))
        assert np.array_equal(kp[w], kp_ref[w]) and np.array_equal(vp[w], vp_ref[w]), f"pool L{l}"
        written |= w
    assert not kp[~written].any() and not vp[~written].any()  # no other page touched

    # the moved cache serves a decode on the receiver
    scale = 1 / np.sqrt(hd)
    for l in range(3):
        qb = W.q_bits(receiver, l)
        q = to_dev(qb)
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=DEV)
        sp.decode(recv, l, q, rb["table"], rb["k_pool"], rb["v_pool"], scale, o, lse,
                  workspace=rb["workspace"])
        torch.cuda.synchronize()
        ref, ref_lse = OA.attention(receiver, l, qb, *kvs[l], scale=scale)
        parity(to_f64(o), ref, f"decode after import L{l}")
        lse_parity(lse.cpu().numpy(), ref_lse, f"decode after import L{l}")


def test_import_all_layers_in_one_call():
    sender = _spec(32)
    send = sp.Plan(sender)
    sb = send.allocate(DEV)
    kvs = [W.kv_bits(sender, l) for l in range(3)]
    sp.build(send, -1, to_dev(np.stack([k for k, _ in kvs])), to_dev(np.stack([v for _, v in kvs])),
             sb["table"], sb["k_pool"], sb["v_pool"])
    n = sp.stream_elems(send, -1)
    ko = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    vo = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    sp.export_pages(send, -1, sb["table"], sb["k_pool"], sb["v_pool"], ko, vo)
    cap = send.sizes.num_pages + 5
    receiver = replace(sender, free_list=W.seeded_free_list(cap, seed=4), capacity_pages=cap)
    recv = sp.Plan(receiver)
    rb = recv.allocate(DEV)
    sp.import_pages(recv, -1, ko, vo, rb["table"], rb["k_pool"], rb["v_pool"])
    torch.cuda.synchronize()
    kp = to_bits(rb["k_pool"]).reshape(-1, 128 // 8, 32, 8)
    for l in range(3):
        kp_ref, _, w = OL.pool(receiver, l, *kvs[l], len(kp))
        assert np.array_equal(kp[w], kp_ref[w]), f"pool L{l}"
    # the whole table image was uploaded: it equals the receiver's host copy
    t_host = recv.table_host()
    assert np.array_equal(rb["table"].cpu().numpy()[:len(t_host)], t_host)


def test_transfer_argument_errors():
    spec = _spec(16)
    plan = sp.Plan(spec)
    bufs = plan.allocate(DEV)
    n = sp.stream_elems(plan, 0)
    small = torch.empty(n - 1, dtype=torch.bfloat16, device=DEV)
    ok = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        sp.export_pages(plan, 0, bufs["table"], bufs["k_pool"], bufs["v_pool"], small, ok)
    with pytest.raises(sp.SegPagedError):
        sp.export_pages(plan, 3, bufs["table"], bufs["k_pool"], bufs["v_pool"], ok, ok)
    with pytest.raises(sp.SegPagedError):
        sp.import_pages(plan, -2, ok, ok, bufs["table"], bufs["k_pool"], bufs["v_pool"])
