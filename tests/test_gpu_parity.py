"""GPU parity: the HIP path (through the C-ABI) against the CPU oracle, element by
element, on seeded inputs. Sizes span several tiles and ragged tails; the
full-size workloads are covered on sampled rows in test_gpu_fullsize.py."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as OA
from oracle import layout as OL
from tests.gpu_util import assert_image_equal, counter_lines, lse_parity, parity, to_bits, to_dev, to_f64

sp = pytest.importorskip("sparse_attention_segmentpagetable_amd")
pytestmark = pytest.mark.gpu

DEV = "cuda"


def _mixed(q0=(0, 30), free=None, cap=0, n=(37, 45), hd=64, ps=16):
    kind = [W.GLOBAL, W.LOCAL, W.RETRIEVAL, W.LOCAL, W.DENSE, W.RETRIEVAL]
    retr = {(0, 1, 0): np.array([1, 2, 30, 31, 32], np.int32),
            (1, 1, 0): np.array([], np.int32),
            (0, 2, 1): np.array([3, 17], np.int32),
            (1, 2, 1): np.array([0, 1, 2, 3, 4, 5, 6, 7, 8, 40, 41], np.int32)}
    return W.Spec(name="mixed", num_layers=3, num_q_heads=4, num_kv_heads=2, head_dim=hd,
                  page_size=ps, seq_len=list(n), first_query_pos=list(q0), kind=kind,
                  sink=[2, 3, 0, 4, 0, 0], window=[1, 9, 1, 5, 1, 1], retrieval=retr,
                  free_list=free, capacity_pages=cap, seed=11)


def _long_mixed(form, hd=128, ps=64, g=8):
    """Several tiles, ragged tails, two-segment local heads, page boundaries; g Q heads
    per KV head (a tile holds 256 // g positions, so g = 3 leaves a row of it unused)."""
    kind = [W.GLOBAL, W.LOCAL, W.LOCAL, W.RETRIEVAL]
    lens = [700, 333, 1029]
    retr = W.seeded_retrieval_sets(lens, kind, 1, 4, 7, 0.1)
    s = W.Spec(name="long-mixed", num_layers=1, num_q_heads=4 * g, num_kv_heads=4, head_dim=hd,
               page_size=ps, seq_len=lens, first_query_pos=[0, 0, 0], kind=kind,
               sink=[4, 4, 0, 0], window=[1, 130, 64, 1], retrieval=retr, seed=12)
    if form == "decode":
        return W.decode_form(s)
    if form == "mid":
        return replace(s, first_query_pos=[350, 0, 900])
    return s


def _run_layer(spec, layer, form, split=0, plan=None, bufs=None):
    plan = plan or sp.Plan(spec, decode_split_tokens=split)
    bufs = bufs or plan.allocate(DEV)
    kb, vb = W.kv_bits(spec, layer)
    qb = W.q_bits(spec, layer)
    sp.build(plan, layer, to_dev(kb), to_dev(vb), bufs["table"], bufs["k_pool"], bufs["v_pool"])
    q = to_dev(qb)
    o = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device=DEV)
    scale = 1.0 / np.sqrt(spec.head_dim)
    if form == "prefill":
        sp.prefill(plan, layer, q, bufs["table"], bufs["k_pool"], bufs["v_pool"], scale, o, lse)
    else:
        sp.decode(plan, layer, q, bufs["table"], bufs["k_pool"], bufs["v_pool"], scale, o, lse,
                  workspace=bufs["workspace"])
    torch.cuda.synchronize()
    return plan, bufs, (qb, kb, vb), to_f64(o), lse.cpu().numpy()


POOL_SPECS = [
    ("tiny-prefill", lambda: W.tiny("prefill")),
    ("tiny-decode", lambda: W.tiny("decode")),
    ("mixed-free", lambda: _mixed(free=W.seeded_free_list(300, 4), cap=300)),
    ("mixed-q0", lambda: _mixed(q0=(10, 44), hd=128, ps=32)),
    ("long-mixed-p128", lambda: _long_mixed("decode", ps=128)),
    ("mistral-small-decode", lambda: W.mistral_layer("decode", seqs=2, n=900, window=200)),
]


@pytest.mark.parametrize("name,mk", POOL_SPECS, ids=[p[0] for p in POOL_SPECS])
def test_build_table_and_pool_bit_exact(name, mk):
    spec = mk()
    plan = sp.Plan(spec)
    bufs = plan.allocate(DEV)
    P, D = spec.page_size, spec.head_dim
    for layer in range(spec.num_layers):
        kb, vb = W.kv_bits(spec, layer)
        sp.build(plan, layer, to_dev(kb), to_dev(vb), bufs["table"], bufs["k_pool"], bufs["v_pool"])
        torch.cuda.synchronize()
        kp_ref, vp_ref, written = OL.pool(spec, layer, kb, vb, plan.sizes.pool_pages)
        kp = to_bits(bufs["k_pool"]).reshape(-1, D // 8, P, 8)
        vp = to_bits(bufs["v_pool"]).reshape(-1, P // 8, D, 8)
        assert np.array_equal(kp[written], kp_ref[written]), (name, layer)
        assert np.array_equal(vp[written], vp_ref[written]), (name, layer)
    dev_table = bufs["table"].cpu().numpy()
    assert_image_equal(dev_table, plan)
    assert np.array_equal(dev_table[:plan.sizes.table_len], OL.table(spec))


def test_build_all_layers_in_one_call():
    spec = _mixed(free=W.seeded_free_list(200, 9), cap=200)
    plan = sp.Plan(spec)
    bufs = plan.allocate(DEV)
    ks, vs = zip(*[W.kv_bits(spec, l) for l in range(spec.num_layers)])
    sp.build(plan, -1, to_dev(np.stack(ks)), to_dev(np.stack(vs)), bufs["table"], bufs["k_pool"],
             bufs["v_pool"])
    torch.cuda.synchronize()
    P, D = spec.page_size, spec.head_dim
    kp = to_bits(bufs["k_pool"]).reshape(-1, D // 8, P, 8)
    for l in range(spec.num_layers):
        kp_ref, _, written = OL.pool(spec, l, ks[l], vs[l], plan.sizes.pool_pages)
        assert np.array_equal(kp[written], kp_ref[written])


PREFILL_SPECS = [
    ("tiny-512", lambda: W.tiny("prefill")),
    ("tiny-n1", lambda: W.tiny("prefill", n=1)),
    ("tiny-n70", lambda: W.tiny("prefill", n=70)),
    ("mixed", lambda: _mixed()),
    ("mixed-d128-p32", lambda: _mixed(q0=(5, 40), hd=128, ps=32)),
    ("long-mixed", lambda: _long_mixed("prefill")),
    ("long-mixed-mid", lambda: _long_mixed("mid")),
    ("long-mixed-p16", lambda: _long_mixed("prefill", ps=16)),
    ("long-mixed-p128", lambda: _long_mixed("prefill", ps=128)),
    ("long-mixed-g1", lambda: _long_mixed("prefill", g=1)),
    ("long-mixed-g3-d64", lambda: _long_mixed("prefill", hd=64, g=3)),
    ("long-mixed-g16", lambda: _long_mixed("prefill", g=16)),
    ("mistral-small", lambda: W.mistral_layer("prefill", seqs=2, n=777, window=128)),
    ("llama-g8-small", lambda: replace(W.long_prefill(num_layers=2, n=1500, window=256),
                                       seq_len=[1500, 260], first_query_pos=[0, 0])),
]


@pytest.mark.parametrize("name,mk", PREFILL_SPECS, ids=[p[0] for p in PREFILL_SPECS])
def test_prefill_parity(name, mk):
    spec = mk()
    plan = bufs = None
    for layer in range(spec.num_layers):
        plan, bufs, (qb, kb, vb), o, lse = _run_layer(spec, layer, "prefill", plan=plan, bufs=bufs)
        ref, ref_lse = OA.attention(spec, layer, qb, kb, vb)
        parity(o, ref, f"{name} prefill L{layer}")
        lse_parity(lse, ref_lse, f"{name} prefill L{layer}")


DECODE_SPECS = [
    ("tiny-513", lambda: W.tiny("decode")),
    ("mixed", lambda: _mixed(q0=(36, 44))),
    ("mixed-free", lambda: replace(_mixed(q0=(36, 44), free=W.seeded_free_list(64, 2), cap=64))),
    ("long-mixed", lambda: _long_mixed("decode")),
    ("long-mixed-p16", lambda: _long_mixed("decode", ps=16)),
    ("long-mixed-p128", lambda: _long_mixed("decode", ps=128)),
    ("long-mixed-g1", lambda: _long_mixed("decode", g=1)),
    ("long-mixed-g3-d64", lambda: _long_mixed("decode", hd=64, g=3)),
    ("long-mixed-g16", lambda: _long_mixed("decode", g=16)),
    ("mistral-small", lambda: W.mistral_layer("decode", seqs=3, n=2000, window=300)),
    ("llama70b-small", lambda: W.llama70b_decode(num_layers=3, seqs=2, n=3000, window=512)),
    ("varlen-small", lambda: W.mixed_varlen_decode(seqs=5, num_layers=2, lo=100, hi=6000,
                                                   window=256)),
]


@pytest.mark.parametrize("name,mk", DECODE_SPECS, ids=[p[0] for p in DECODE_SPECS])
@pytest.mark.parametrize("split", [0, 64, 512])
def test_decode_parity(name, mk, split):
    spec = mk()
    plan = bufs = None
    for layer in range(spec.num_layers):
        plan, bufs, (qb, kb, vb), o, lse = _run_layer(spec, layer, "decode", split=split,
                                                      plan=plan, bufs=bufs)
        ref, ref_lse = OA.attention(spec, layer, qb, kb, vb)
        parity(o, ref, f"{name} decode L{layer} split {split}")
        lse_parity(lse, ref_lse, f"{name} decode L{layer}")


def test_decode_on_prefill_form_uses_all_layers_call():
    """A prefill-form table read by the decode row (window predicate ranges not
    page aligned), all layers in one call."""
    spec = replace(W.llama70b_decode(num_layers=2, seqs=2, n=1500, window=300),
                   first_query_pos=[0, 0])
    dspec = W.decode_form(spec)
    plan = sp.Plan(spec)
    bufs = plan.allocate(DEV)
    kvs = [W.kv_bits(spec, l) for l in range(2)]
    sp.build(plan, -1, to_dev(np.stack([k for k, _ in kvs])), to_dev(np.stack([v for _, v in kvs])),
             bufs["table"], bufs["k_pool"], bufs["v_pool"])
    qs = [W.q_bits(dspec, l) for l in range(2)]
    q = to_dev(np.stack(qs))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    sp.decode(plan, -1, q, bufs["table"], bufs["k_pool"], bufs["v_pool"], 1 / np.sqrt(128), o, lse,
              workspace=bufs["workspace"])
    torch.cuda.synchronize()
    of = to_f64(o)
    for l in range(2):
        ref, ref_lse = OA.attention(dspec, l, qs[l], *kvs[l])
        parity(of[l], ref, f"decode prefill-form L{l}")
        lse_parity(lse[l].cpu().numpy(), ref_lse, f"decode prefill-form L{l}")


def test_prefill_all_layers_in_one_call():
    spec = _mixed(hd=128, ps=32)
    plan = sp.Plan(spec)
    bufs = plan.allocate(DEV)
    kvs = [W.kv_bits(spec, l) for l in range(3)]
    sp.build(plan, -1, to_dev(np.stack([k for k, _ in kvs])), to_dev(np.stack([v for _, v in kvs])),
             bufs["table"], bufs["k_pool"], bufs["v_pool"])
    qs = [W.q_bits(spec, l) for l in range(3)]
    q = to_dev(np.stack(qs))
    o = torch.empty_like(q)
    sp.prefill(plan, -1, q, bufs["table"], bufs["k_pool"], bufs["v_pool"], 0.125, o)
    torch.cuda.synchronize()
    of = to_f64(o)
    for l in range(3):
        ref, _ = OA.attention(spec, l, qs[l], *kvs[l], scale=0.125)
        parity(of[l], ref, f"prefill all-layers L{l}")


def test_split_count_invariance():
    spec = W.llama70b_decode(num_layers=1, seqs=2, n=5000, window=700)
    outs = []
    for split in (64, 256, 2048):
        _, _, _, o, lse = _run_layer(spec, 0, "decode", split=split)
        outs.append((o, lse))
    for o, lse in outs[1:]:
        assert np.max(np.abs(o - outs[0][0])) <= 2 ** -7  # fp32 merge order only
        assert np.max(np.abs(lse - outs[0][1])) <= 1e-4


def test_decode_row_matches_last_prefill_row():
    pre = _long_mixed("prefill")
    _, _, (qb, kb, vb), o_pre, lse_pre = _run_layer(pre, 0, "prefill")
    dec = W.decode_form(pre)
    plan = sp.Plan(dec)
    bufs = plan.allocate(DEV)
    sp.build(plan, 0, to_dev(kb), to_dev(vb), bufs["table"], bufs["k_pool"], bufs["v_pool"])
    last = np.cumsum(pre.seq_len) - 1
    q = to_dev(qb[last])
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=DEV)
    sp.decode(plan, 0, q, bufs["table"], bufs["k_pool"], bufs["v_pool"], 1 / np.sqrt(128), o, lse,
              workspace=bufs["workspace"])
    torch.cuda.synchronize()
    parity(to_f64(o), o_pre[last], "decode vs last prefill row")
    assert np.max(np.abs(lse.cpu().numpy() - lse_pre[last])) <= 1e-3


def _run_kv(spec, form, kb, vb, qb, scale=0.09):
    plan = sp.Plan(spec)
    bufs = plan.allocate(DEV)
    sp.build(plan, 0, to_dev(kb), to_dev(vb), bufs["table"], bufs["k_pool"], bufs["v_pool"])
    q = to_dev(qb)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=DEV)
    if form == "prefill":
        sp.prefill(plan, 0, q, bufs["table"], bufs["k_pool"], bufs["v_pool"], scale, o, lse)
    else:
        sp.decode(plan, 0, q, bufs["table"], bufs["k_pool"], bufs["v_pool"], scale, o, lse,
                  workspace=bufs["workspace"])
    torch.cuda.synchronize()
    return to_bits(o), lse.cpu().numpy()


def test_invisible_keys_do_not_change_output_bitwise():
    """Perturbing K/V at keys no query row sees leaves O and LSE bit-identical:
    those keys are never stored (decode form) or never read unmasked (prefill)."""
    base = W.Spec(name="perturb", num_layers=1, num_q_heads=16, num_kv_heads=2, head_dim=128,
                  page_size=64, seq_len=[3000], first_query_pos=[0], kind=[W.LOCAL, W.LOCAL],
                  sink=[4, 0], window=[257, 64], seed=21)
    for form in ("prefill", "decode"):
        s = base if form == "prefill" else W.decode_form(base)
        kb, vb = W.kv_bits(s, 0)
        qb = W.q_bits(s, 0)
        n = s.seq_len[0]
        rows = np.arange(s.first_query_pos[0], n)
        kb2, vb2 = kb.copy(), vb.copy()
        changed = 0
        for h in range(2):
            kind, sk, w = s.head_class(0, h)
            inv = ~OA.visibility_mask(kind, sk, w, None, rows, n).any(axis=0)
            kb2[inv, h] ^= 0x1234
            vb2[inv, h] ^= 0x0F0F
            changed += int(inv.sum())
        if form == "decode":
            assert changed > 5000
        o1, l1 = _run_kv(s, form, kb, vb, qb)
        o2, l2 = _run_kv(s, form, kb2, vb2, qb)
        assert np.array_equal(o1, o2), form
        assert np.array_equal(l1, l2), form
    # prefill: keys outside every row's window exist only relative to a row
    # range; perturb keys invisible to rows >= 2000 and run the table planned
    # for those rows (q0 = 2000)
    s = replace(base, first_query_pos=[2000])
    kb, vb = W.kv_bits(s, 0)
    qb = W.q_bits(s, 0)
    rows = np.arange(2000, 3000)
    kb2, vb2 = kb.copy(), vb.copy()
    for h in range(2):
        kind, sk, w = s.head_class(0, h)
        inv = ~OA.visibility_mask(kind, sk, w, None, rows, 3000).any(axis=0)
        assert inv.sum() > 1000
        kb2[inv, h] ^= 0x1234
        vb2[inv, h] ^= 0x0F0F
    o1, l1 = _run_kv(s, "prefill", kb, vb, qb)
    o2, l2 = _run_kv(s, "prefill", kb2, vb2, qb)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_empty_and_degenerate_rows():
    """Empty sequence, empty retrieval set, rows before the first retrieved key."""
    kind = [W.RETRIEVAL, W.GLOBAL]
    spec = W.Spec(name="degen", num_layers=1, num_q_heads=4, num_kv_heads=2, head_dim=64,
                  page_size=16, seq_len=[40, 0, 25], first_query_pos=[0, 0, 0], kind=kind,
                  sink=[0, 0], window=[1, 1],
                  retrieval={(0, 0, 0): np.array([7, 8, 30], np.int32),
                             (1, 0, 0): np.array([], np.int32),
                             (2, 0, 0): np.array([], np.int32)}, seed=5)
    _, _, (qb, kb, vb), o, lse = _run_layer(spec, 0, "prefill")
    ref, ref_lse = OA.attention(spec, 0, qb, kb, vb)
    parity(o, ref, "degenerate prefill")
    lse_parity(lse, ref_lse, "degenerate prefill")
    assert np.all(o[:7, :2] == 0) and np.all(np.isneginf(lse[:7, :2]))
    # decode: Q/O have one row per sequence; the empty sequence's row is O = 0, LSE = -inf
    dspec = W.decode_form(spec)
    qb = W.q_bits(replace(dspec, seq_len=[40, 1, 25], first_query_pos=[39, 0, 24]), 0)
    ob, lse = _run_kv(dspec, "decode", kb, vb, qb, scale=0.125)
    o = OA.bf16_bits_to_f64(ob)
    ref, ref_lse = OA.attention(dspec, 0, qb[[0, 2]], kb, vb, scale=0.125)
    parity(o[[0, 2]], ref, "degenerate decode")
    lse_parity(lse[[0, 2]], ref_lse, "degenerate decode")
    assert np.all(o[1] == 0) and np.all(np.isneginf(lse[1]))


@pytest.mark.parametrize("slope", [0.05, 2.0])
def test_prefill_growing_scores(slope):
    """Scores that rise along the sequence. A gentle slope keeps the hot loop's
    fixed reference max (p up to ~2^30); a steep one exceeds its 2^64 margin
    and sends the tiles to the per-block rescaling path. Both must match."""
    n, D = 300, 64
    spec = W.Spec(name="growth", num_layers=1, num_q_heads=8, num_kv_heads=1, head_dim=D,
                  page_size=16, seq_len=[n], first_query_pos=[0], kind=[W.GLOBAL], sink=[0],
                  window=[1], seed=31)
    rng = np.random.default_rng(31)
    q = rng.standard_normal((n, 8, D)).astype(np.float32) * 0.1
    k = rng.standard_normal((n, 1, D)).astype(np.float32) * 0.1
    v = rng.standard_normal((n, 1, D)).astype(np.float32)
    q[:, :, 0] = 16.0
    k[:, 0, 0] = slope * np.arange(n) / 2.0
    qb, kb, vb = (W.f32_to_bf16_bits(x) for x in (q, k, v))
    ob, lse = _run_kv(spec, "prefill", kb, vb, qb, scale=0.125)
    ref, ref_lse = OA.attention(spec, 0, qb, kb, vb, scale=0.125)
    parity(OA.bf16_bits_to_f64(ob), ref, f"growing scores slope {slope}")
    assert np.max(np.abs(lse - ref_lse) / np.maximum(1.0, np.abs(ref_lse))) <= 1e-5


def test_decode_long_items_small_pages():
    """Items spanning more than 64 pages (P = 16, 4096-key items): the kernel's
    per-lane page-id window has to move along the item."""
    spec = W.Spec(name="longitems", num_layers=1, num_q_heads=16, num_kv_heads=2, head_dim=128,
                  page_size=16, seq_len=[5000, 2600], first_query_pos=[0, 0],
                  kind=[W.GLOBAL, W.LOCAL], sink=[0, 5], window=[1, 2500], seed=41)
    dspec = W.decode_form(spec)
    _, _, (qb, kb, vb), o, lse = _run_layer(dspec, 0, "decode", split=4096)
    ref, ref_lse = OA.attention(dspec, 0, qb, kb, vb)
    parity(o, ref, "decode long items P=16")
    lse_parity(lse, ref_lse, "decode long items P=16")


def _parts(nitems, keys, recs, resident=2048):
    """Waves per decode item the library picks for a launch (a copy of its rule, so
    the test can check that it runs the path it means to): at most 16, no more
    waves than the chip holds at once (2048 decode waves on MI355X; the launches
    here are far below that), >= 256 keys a wave, partials within the workspace."""
    return max(1, min(16, resident // nitems, recs // nitems, keys // (nitems * 256)))


@pytest.mark.parametrize("ps,hd", [(16, 128), (64, 128), (32, 64)])
def test_decode_item_parts(ps, hd):
    """One layer of a two-layer plan with 4096-key items, launched alone with room
    for more partials: each item is dealt to several waves (parts). Layer 0's local
    head keeps sink 4 + window 60, one short item over the sink page and two window
    pages; with 7 parts some parts get no step at all, and (page 64) one part's only
    step lies in the sink page's zero tail, so it holds no key. Layer 1 deals its
    items to 8 parts. The same layers from the all-layer call with the minimal
    workspace run one wave per item."""
    kind = [W.GLOBAL, W.LOCAL, W.LOCAL, W.RETRIEVAL]
    lens = [9000, 4400]
    retr = W.seeded_retrieval_sets(lens, kind, 2, 2, 5, 0.2)
    spec = W.decode_form(W.Spec(name="parts", num_layers=2, num_q_heads=8, num_kv_heads=2,
                                head_dim=hd, page_size=ps, seq_len=lens,
                                first_query_pos=[0, 0], kind=kind, sink=[0, 4, 7, 0],
                                window=[1, 60, 3000, 1], retrieval=retr, seed=21))
    plan = sp.Plan(spec, decode_split_tokens=4096)
    bufs = plan.allocate(DEV)
    kvs = [W.kv_bits(spec, l) for l in range(2)]
    sp.build(plan, -1, to_dev(np.stack([k for k, _ in kvs])), to_dev(np.stack([v for _, v in kvs])),
             bufs["table"], bufs["k_pool"], bufs["v_pool"])
    qs = [W.q_bits(spec, l) for l in range(2)]
    scale = 1 / np.sqrt(hd)
    q_all = to_dev(np.stack(qs))
    o_all = torch.empty_like(q_all)
    lse_all = torch.empty(q_all.shape[:3], dtype=torch.float32, device=DEV)
    sp.decode(plan, -1, q_all, bufs["table"], bufs["k_pool"], bufs["v_pool"], scale, o_all,
              lse_all, workspace=bufs["workspace"])
    big_ws = torch.empty(16 * bufs["workspace"].numel() + 4096, dtype=bufs["workspace"].dtype,
                         device=DEV)
    rec = spec.num_q_heads // spec.num_kv_heads * (hd + 4) * 4
    for l in range(2):
        st = plan.stats(l)
        assert _parts(st["decode_items"], st["decode_tokens"],
                      big_ws.numel() * big_ws.element_size() // rec) == (7 if l == 0 else 8)
        q = to_dev(qs[l])
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=DEV)
        sp.decode(plan, l, q, bufs["table"], bufs["k_pool"], bufs["v_pool"], scale, o, lse,
                  workspace=big_ws)
        torch.cuda.synchronize()
        ref, ref_lse = OA.attention(spec, l, qs[l], *kvs[l], scale=scale)
        parity(to_f64(o), ref, f"decode parts L{l}")
        lse_parity(lse.cpu().numpy(), ref_lse, f"decode parts L{l}")
        parity(to_f64(o_all[l]), ref, f"decode one wave per item L{l}")
        assert np.max(np.abs(to_f64(o) - to_f64(o_all[l]))) <= 2 ** -7  # fp32 merge order only


def test_prefill_work_counter_left_raised():
    """A work counter that an earlier launch left raised (one that never reached its
    end, or a launch of another generation) skips no tile: each call claims the
    counter line with a generation of its own, and leaves (generation, 0)."""
    spec = _long_mixed("prefill")
    plan = sp.Plan(spec)
    bufs = plan.allocate(DEV)
    kb, vb = W.kv_bits(spec, 0)
    qb = W.q_bits(spec, 0)
    sp.build(plan, 0, to_dev(kb), to_dev(vb), bufs["table"], bufs["k_pool"], bufs["v_pool"])
    ref, ref_lse = OA.attention(spec, 0, qb, kb, vb)
    q = to_dev(qb)
    # no growth capacity: the L + 1 counter lines of 16 ints end the image
    off_ctr = counter_lines(plan)[0]
    table = bufs["table"]
    gens = []
    # (next item, generation) words as a stalled or foreign launch could leave them
    for lo, hi in [(0, 0), (5, 0), (123456, 7), (0x7FFFFFFF, 1), (3, 0x7FFFFFFF), (0, 0)]:
        table[off_ctr:off_ctr + 2] = torch.tensor([lo, hi], dtype=torch.int32, device=DEV)
        o = torch.full_like(q, float("nan"))
        lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device=DEV)
        sp.prefill(plan, 0, q, table, bufs["k_pool"], bufs["v_pool"], 1 / np.sqrt(128), o, lse)
        torch.cuda.synchronize()
        parity(to_f64(o), ref, f"prefill after counter ({lo}, {hi})")
        lse_parity(lse.cpu().numpy(), ref_lse, f"prefill after counter ({lo}, {hi})")
        word = table[off_ctr:off_ctr + 2].cpu().numpy()
        assert word[0] == 0 and word[1] not in (0, hi), word
        gens.append(int(word[1]))
    # back to back, no reset in between: a new generation each call
    for _ in range(3):
        o = torch.full_like(q, float("nan"))
        sp.prefill(plan, 0, q, table, bufs["k_pool"], bufs["v_pool"], 1 / np.sqrt(128), o)
        torch.cuda.synchronize()
        parity(to_f64(o), ref, "prefill back to back")
        gens.append(int(table[off_ctr + 1].item()))
    assert len(set(gens)) == len(gens)


def test_graph_replay_of_prefill_and_decode():
    """HIP graphs captured from segpaged_prefill and segpaged_decode replay the
    captured calls exactly. The captured prefill launch keeps the generation it was
    given at capture; its last work-counter fetch leaves (generation, 0) for the next
    replay, and an eager call on the same counter line in between (another
    generation) is claimed over. Every replay is compared bit for bit with the eager
    result, with eager work and synchronisations between the replays."""
    scale = 1 / np.sqrt(128)
    spec = _long_mixed("prefill")
    plan = sp.Plan(spec)
    bufs = plan.allocate(DEV)
    kb, vb = W.kv_bits(spec, 0)
    qb = W.q_bits(spec, 0)
    table, kpool, vpool = bufs["table"], bufs["k_pool"], bufs["v_pool"]
    sp.build(plan, 0, to_dev(kb), to_dev(vb), table, kpool, vpool)
    q = to_dev(qb)
    o_ref = torch.empty_like(q)
    lse_ref = torch.empty(q.shape[:2], dtype=torch.float32, device=DEV)
    sp.prefill(plan, 0, q, table, kpool, vpool, scale, o_ref, lse_ref)
    torch.cuda.synchronize()
    ref, ref_lse = OA.attention(spec, 0, qb, kb, vb)
    parity(to_f64(o_ref), ref, "prefill eager before graph")
    lse_parity(lse_ref.cpu().numpy(), ref_lse, "prefill eager before graph")

    o_g = torch.empty_like(q)
    lse_g = torch.empty_like(lse_ref)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sp.prefill(plan, 0, q, table, kpool, vpool, scale, o_g, lse_g)
    torch.cuda.synchronize()
    off_ctr = counter_lines(plan)[0]
    for step, eager_between in enumerate([False, True, False, True]):
        o_g.fill_(float("nan"))
        lse_g.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(o_g), to_bits(o_ref)), f"prefill replay {step}"
        assert np.array_equal(lse_g.cpu().numpy().view(np.int32), lse_ref.cpu().numpy().view(np.int32)), step
        assert int(table[off_ctr].item()) == 0  # (generation, 0) after the replay
        if eager_between:
            o_e = torch.full_like(q, float("nan"))
            sp.prefill(plan, 0, q, table, kpool, vpool, scale, o_e)
            torch.cuda.synchronize()
            assert np.array_equal(to_bits(o_e), to_bits(o_ref)), f"prefill eager after replay {step}"
    del graph

    dspec = W.decode_form(spec)
    dplan = sp.Plan(dspec)
    dbufs = dplan.allocate(DEV)
    sp.build(dplan, 0, to_dev(kb), to_dev(vb), dbufs["table"], dbufs["k_pool"], dbufs["v_pool"])
    dq = to_dev(W.q_bits(dspec, 0))
    args = (dbufs["table"], dbufs["k_pool"], dbufs["v_pool"], scale)
    od_ref = torch.empty_like(dq)
    sp.decode(dplan, 0, dq, *args, od_ref, workspace=dbufs["workspace"])
    torch.cuda.synchronize()
    od_g = torch.empty_like(dq)
    dgraph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(dgraph):
        sp.decode(dplan, 0, dq, *args, od_g, workspace=dbufs["workspace"])
    torch.cuda.synchronize()
    for step in range(3):
        od_g.fill_(float("nan"))
        torch.cuda.synchronize()
        dgraph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(od_g), to_bits(od_ref)), f"decode replay {step}"
        o_e = torch.empty_like(dq)
        sp.decode(dplan, 0, dq, *args, o_e, workspace=dbufs["workspace"])
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(o_e), to_bits(od_ref)), f"decode eager after replay {step}"


@pytest.mark.parametrize("D,P,G", [(128, 64, 2), (64, 16, 4)])
def test_decode_last_items_in_four_parts(D, P, G):
    """An all-layer decode launch of 4096 items of 1024 keys (16 layers x 2 sequences x
    8 global KV heads x 16K keys; one K/V shared by the layers, Q per layer): more
    items than the chip holds decode waves at once (2048 at head dim 128, 3072 at 64),
    so the launch deals its last items (up to 512, the last layers') to 4 waves each
    and merges 4 partials for each of them. Layer 0 and the last four layers (whose
    items hold the split ones) against the oracle; every layer against the same
    layers launched one at a time (one round, items dealt evenly)."""
    L, B, Hkv, N = 16, 2, 8, 16384
    spec = W.decode_form(W.Spec(name="tail", num_layers=L, num_q_heads=G * Hkv, num_kv_heads=Hkv,
                                head_dim=D, page_size=P, seq_len=[N] * B, first_query_pos=[0] * B,
                                kind=[W.GLOBAL] * (L * Hkv), sink=[0] * (L * Hkv),
                                window=[1] * (L * Hkv), seed=31))
    plan = sp.Plan(spec)
    st = plan.stats(-1)
    assert st["decode_items"] == 4096 and st["decode_tokens"] == 4096 * 1024
    bufs = plan.allocate(DEV)
    kb, vb = W.kv_bits(spec, 0)
    kd, vd = to_dev(kb), to_dev(vb)
    for l in range(L):
        sp.build(plan, l, kd, vd, bufs["table"], bufs["k_pool"], bufs["v_pool"])
    qs = [W.q_bits(spec, l) for l in range(L)]
    q = to_dev(np.stack(qs))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    scale = 1 / np.sqrt(D)
    args = (bufs["table"], bufs["k_pool"], bufs["v_pool"], scale)
    sp.decode(plan, -1, q, *args, o, lse, workspace=bufs["workspace"])
    o1 = torch.empty_like(q)
    for l in range(L):
        sp.decode(plan, l, q[l], *args, o1[l], workspace=bufs["workspace"])
    torch.cuda.synchronize()
    for l in range(L):
        if l == 0 or l >= L - 4:
            ref, ref_lse = OA.attention(spec, l, qs[l], kb, vb, scale=scale)
            parity(to_f64(o[l]), ref, f"decode last items in 4 parts D{D} P{P} L{l}")
            lse_parity(lse[l].cpu().numpy(), ref_lse, f"decode last items in 4 parts D{D} L{l}")
        assert np.max(np.abs(to_f64(o[l]) - to_f64(o1[l]))) <= 2 ** -7  # fp32 merge order only
