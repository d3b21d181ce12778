"""Pins for the table and pool oracle (O2). CPU only."""
import json
import os

import numpy as np
import pytest

import workloads as W
from oracle import attention as A
from oracle import layout as L

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_block_table_golden_example():
    g = json.load(open(os.path.join(GOLDEN, "block_table_example.json")))
    n, p = g["tokens"], g["block_size"]
    phys = g["physical_blocks"]
    free = np.array(phys + [i for i in range(16) if i not in phys], dtype=np.int32)
    spec = W.Spec(name="blk", num_layers=1, num_q_heads=1, num_kv_heads=1, head_dim=8,
                  page_size=p, seq_len=[n], first_query_pos=[0], kind=[W.GLOBAL],
                  sink=[0], window=[1], free_list=free, capacity_pages=16)
    t = L.table(spec)
    assert int(t[9]) == len(phys)
    assert list(t[int(t[13]):int(t[13]) + int(t[9])]) == phys
    kb, vb = W.kv_bits(spec, 0)
    kp, vp, written = L.pool(spec, 0, kb, vb, 16)
    assert set(np.nonzero(written)[0]) == set(phys)
    for pid, toks in zip(phys, g["tokens_per_block"]):
        for slot in range(p):
            krow = kp[pid, :, slot, :].reshape(-1)
            vrow = vp[pid, slot // 8, :, slot % 8]
            if slot < len(toks):
                assert np.array_equal(krow, kb[toks[slot], 0])
                assert np.array_equal(vrow, vb[toks[slot], 0])
            else:
                assert not krow.any() and not vrow.any()
    assert p - len(g["tokens_per_block"][-1]) == g["empty_slots_last_block"]


def test_kv_size_golden_example():
    g = json.load(open(os.path.join(GOLDEN, "kv_size_example.json")))
    b = L.dense_kv_bytes(g["layers"], g["kv_heads"], g["head_dim"], g["tokens"],
                         g["bytes_per_element"])
    assert b == 2 ** 31 and round(b / 1e9, 1) == g["approx_gb"]
    # an all-GLOBAL cache retains exactly the dense bytes
    spec = W.Spec(name="dense", num_layers=2, num_q_heads=4, num_kv_heads=2, head_dim=16,
                  page_size=16, seq_len=[40, 7], first_query_pos=[0, 3],
                  kind=[W.GLOBAL, W.DENSE] * 2, sink=[0] * 4, window=[1] * 4)
    assert L.retained_kv_bytes(spec) == L.dense_kv_bytes(2, 2, 16, 47)


RET_CASES = [(W.GLOBAL, 0, 0), (W.DENSE, 4, 8), (W.LOCAL, 4, 8), (W.LOCAL, 0, 5),
             (W.LOCAL, 10, 1), (W.LOCAL, 3, 100), (W.LOCAL, 20, 6)]


@pytest.mark.parametrize("kind,s,w", RET_CASES)
@pytest.mark.parametrize("n", [1, 2, 9, 25, 64])
def test_retention_is_union_of_visible_keys(kind, s, w, n):
    for q0 in sorted({0, n // 2, n - 1}):
        rows = np.arange(q0, n)
        brute = np.nonzero(A.visibility_mask(kind, s, w, None, rows, n).any(axis=0))[0]
        segs = L.retained_segments(kind, s, w, n, q0, None)
        kept = np.concatenate([L.segment_positions(sg) for sg in segs]) if segs else np.array([], int)
        assert np.array_equal(kept, brute), (kind, s, w, n, q0, segs)
        assert len(segs) <= 2
        if len(segs) == 2:  # two segments only when there is a gap between them
            assert segs[0][0] + segs[0][1] < segs[1][0]


def test_retention_retrieval():
    r = np.array([0, 5, 6, 19], dtype=np.int32)
    for q0 in (0, 10, 19):
        segs = L.retained_segments(W.RETRIEVAL, 0, 0, 20, q0, r)
        assert len(segs) == 1 and np.array_equal(segs[0][1], r)
    assert L.retained_segments(W.RETRIEVAL, 0, 0, 20, 0, np.array([], np.int32)) == []


def test_page_counts_closed_forms():
    # tiny decode form: N = 513, P = 16; global ceil(513/16) = 33 pages, local
    # ceil(4/16) + ceil(64/16) = 5 pages; 33 + 3*5 = 48
    t = L.table(W.tiny("decode"))
    assert int(t[9]) == 48
    t = L.table(W.tiny("prefill"))
    assert int(t[9]) == 4 * 32
    # mistral layer decode form, N = 8193, P = 64: 4 * (129 + 7 * (1 + 16))
    assert L.num_pages(W.mistral_layer("decode")) == 4 * (129 + 7 * 17)


def test_llama70b_decode_page_count_and_classes():
    g = json.load(open(os.path.join(GOLDEN, "head_class_config.json")))
    spec = W.llama70b_decode()
    n_glob = sum(1 for k in spec.kind if k == W.GLOBAL)
    assert len(spec.kind) == g["layers"] * g["kv_heads"]
    assert n_glob == round(g["global_fraction"] * len(spec.kind)) == 96
    assert set(spec.window) == {g["local_window"]} and set(spec.sink) == {g["local_sink"]}
    assert spec.page_size == g["page_size"]
    # global: ceil(32768/64) = 512 pages; local: 1 sink page + 8192/64 window pages
    per_seq = n_glob * 512 + (640 - n_glob) * 129
    seqs = spec.num_seqs
    # count straight from the oracle's retention (not from its table) for one layer
    l0 = [L.unit_segments(spec, 0, 0, h) for h in range(8)]
    for h, segs in enumerate(l0):
        npg = sum(L.ceil_div(len(L.segment_positions(s)), 64) for s in segs)
        assert npg == (512 if spec.kind[h] == W.GLOBAL else 129)
    assert per_seq * seqs == 954_624


def _spec_mixed(free=None, cap=0):
    kind = [W.GLOBAL, W.LOCAL, W.RETRIEVAL, W.LOCAL, W.DENSE, W.RETRIEVAL]
    retr = {(0, 1, 0): np.array([1, 2, 30, 31, 32], np.int32),
            (1, 1, 0): np.array([], np.int32),
            (0, 2, 1): np.array([3, 17], np.int32),
            (1, 2, 1): np.array([0, 1, 2, 3, 4, 5, 6, 7, 8, 40, 41], np.int32)}
    return W.Spec(name="mixed", num_layers=3, num_q_heads=4, num_kv_heads=2, head_dim=16,
                  page_size=8, seq_len=[37, 45], first_query_pos=[0, 30],
                  kind=kind, sink=[2, 3, 0, 4, 0, 0], window=[1, 9, 1, 5, 1, 1],
                  retrieval=retr, free_list=free, capacity_pages=cap)


def test_table_structure_and_free_list():
    free = W.seeded_free_list(200, seed=9)
    spec = _spec_mixed(free, 200)
    t = L.table(spec)
    assert int(t[0]) == L.MAGIC and int(t[15]) == len(t)
    npg = int(t[9])
    pages = t[int(t[13]):int(t[13]) + npg]
    assert np.array_equal(pages, free[:npg])  # ids taken from the free list, in order
    recs = t[int(t[12]):int(t[13])].reshape(-1, L.UNIT_INTS)
    assert len(recs) == 3 * 2 * 2
    # page_off increases by each unit's page count; kv_len = sum of segment lengths
    off = 0
    for r in recs:
        assert r[14] == off
        segs = [(r[10], r[11]), (r[12], r[13])][:r[9]]
        assert r[8] == sum(s[1] for s in segs)
        off += sum(L.ceil_div(int(s[1]), 8) for s in segs)
    assert off == npg
    # retrieval positions land in the retr region in unit order
    retr = t[int(t[14]):]
    assert list(retr) == [1, 2, 30, 31, 32, 3, 17, 0, 1, 2, 3, 4, 5, 6, 7, 8, 40, 41]


def test_transfer_stream_elements_and_pool_pages():
    """The transfer stream, element by element from the page-layout formulas of the
    pool (K (slot, d) at [d // 8][slot][d % 8], V at [slot // 8][d][slot % 8]), and
    page by page equal to the pool pages its table lists for the layer, in order."""
    free = W.seeded_free_list(120, seed=5)
    spec = _spec_mixed(free, 120)
    t = L.table(spec)
    P, D = spec.page_size, spec.head_dim
    kvo = spec.kv_row_offsets()
    page_b = 0
    for layer in range(3):
        kb, vb = W.kv_bits(spec, layer)
        ks, vs = L.transfer_stream(spec, layer, kb, vb)
        # expected pages from the retained positions of each unit, in table order
        j = 0
        for b in range(spec.num_seqs):
            for h in range(spec.num_kv_heads):
                c = layer * spec.num_kv_heads + h
                retr = spec.retrieval.get((b, layer, h)) if spec.retrieval else None
                for seg in L.retained_segments(spec.kind[c], spec.sink[c], spec.window[c],
                                               spec.seq_len[b], spec.first_query_pos[b], retr):
                    pos = (list(range(seg[0], seg[0] + seg[1])) if seg[0] != "gathered"
                           else [int(x) for x in seg[1]])
                    npg = -(-len(pos) // P)
                    for slot in range(npg * P):
                        for d in range(D):
                            if slot < len(pos):
                                ek = kb[kvo[b] + pos[slot], h, d]
                                ev = vb[kvo[b] + pos[slot], h, d]
                            else:
                                ek = ev = 0
                            jj, sl = j + slot // P, slot % P
                            assert ks[jj, d // 8, sl, d % 8] == ek
                            assert vs[jj, sl // 8, d, sl % 8] == ev
                    j += npg
        assert j == len(ks) == len(vs)
        # the same pages, found through the table's page ids
        kp, vp, _ = L.pool(spec, layer, kb, vb, 120)
        ids = t[int(t[13]) + page_b:int(t[13]) + page_b + j]
        assert np.array_equal(ks, kp[ids]) and np.array_equal(vs, vp[ids])
        page_b += j
    assert page_b == int(t[9])


def test_pool_round_trip_and_loops_agree():
    free = W.seeded_free_list(120, seed=3)
    spec = _spec_mixed(free, 120)
    for layer in range(3):
        kb, vb = W.kv_bits(spec, layer)
        kp, vp, written = L.pool(spec, layer, kb, vb, 120)
        kp2, vp2, w2 = L.pool_loops(spec, layer, kb, vb, 120)
        assert np.array_equal(kp, kp2) and np.array_equal(vp, vp2) and np.array_equal(written, w2)
        # gather back through the oracle's own table
        kvo = spec.kv_row_offsets()
        for b in range(2):
            for h in range(2):
                for pos, pids in L.unit_page_ids(spec, b, layer, h):
                    for t_idx, p in enumerate(pos):
                        pid, slot = pids[t_idx // 8], t_idx % 8
                        kg = kp[pid, :, slot, :].reshape(-1)
                        vg = vp[pid, slot // 8, :, slot % 8]
                        assert np.array_equal(kg, kb[kvo[b] + p, h])
                        assert np.array_equal(vg, vb[kvo[b] + p, h])
                    tail = len(pids) * 8 - len(pos)
                    for slot in range(8 - tail, 8) if tail else []:
                        assert not kp[pids[-1], :, slot, :].any()
                        assert not vp[pids[-1], slot // 8, :, slot % 8].any()


def _doc_spec(form="prefill", P=64, n=(700, 900, 400), c=500):
    """Sequences 0 and 1 share a 500-token document; sequence 2 has none. KV heads:
    global, local (sink 4, window 100), retrieval."""
    kind = [W.GLOBAL, W.LOCAL, W.RETRIEVAL]
    retr = {(b, 0, 2): np.arange(0, nb, 7, dtype=np.int32) for b, nb in enumerate(n)}
    s = W.Spec(name=f"doc-{form}", num_layers=1, num_q_heads=6, num_kv_heads=3, head_dim=64,
               page_size=P, seq_len=list(n), first_query_pos=[0] * len(n), kind=kind,
               sink=[0, 4, 0], window=[1, 100, 1], retrieval=retr, seed=44,
               doc_group=[0, 0, -1], doc_len=[c, c, 0])
    return s if form == "prefill" else W.decode_form(s)


def test_shared_document_pages_closed_forms():
    """Two sequences with one 500-token document, page 64: a global head (and a local
    head whose prefill-form segment is the whole context) stores the 7 full pages
    inside the document once, so 11 + 15 - 7 pages; the page holding positions
    448..511 crosses the document's end and stays private. Retrieval pages are never
    shared. In decode form the local head's sink page (positions 0..3) is shared and
    its windows (600..699, 800..899) are not."""
    spec = _doc_spec("prefill")
    third = L.ceil_div(400, 64)
    for h in (0, 1):
        pages = {}
        for slot, (u, b, l, hh, seg, pos, key) in enumerate(L.unit_pages(spec)):
            if hh == h:
                pages.setdefault(key if key is not None else ("own", slot), 0)
        assert len(pages) == 11 + 15 - 7 + third, h
    retr_keys = [k for (_, _, _, hh, _, _, k) in L.unit_pages(spec) if hh == 2]
    assert all(k is None for k in retr_keys)
    per_seq_retr = sum(L.ceil_div(len(range(0, nb, 7)), 64) for nb in spec.seq_len)
    assert L.distinct_pages(spec) == 2 * (11 + 15 - 7 + third) + per_seq_retr
    # the table lists every unit's pages, ids repeating where shared
    assert L.num_pages(spec) == 2 * (11 + 15 + third) + per_seq_retr
    dspec = _doc_spec("decode")
    local = [k for (_, _, _, hh, _, _, k) in L.unit_pages(dspec) if hh == 1]
    # sequences 0, 1, 2: sink page + 2 window pages each; the first two sinks are one page
    assert len(local) == 9 and sum(k is not None for k in local) == 2
    assert L.distinct_pages(dspec) == L.num_pages(dspec) - 1 - 7


def test_shared_document_pool_round_trip():
    """Gathering each unit's pages through the table gives back that sequence's own
    dense K/V at every retained position (so a page is shared only where the
    members' rows are identical), and the pool holds each shared page once."""
    for form in ("prefill", "decode"):
        spec = _doc_spec(form, P=32)
        kb, vb = W.kv_bits(spec, 0)
        kvo = spec.kv_row_offsets()
        assert np.array_equal(kb[kvo[0]:kvo[0] + 500], kb[kvo[1]:kvo[1] + 500])
        assert not np.array_equal(kb[kvo[0] + 500:kvo[0] + 600], kb[kvo[1] + 500:kvo[1] + 600])
        tab = L.table(spec)
        n_pool = L.distinct_pages(spec)
        kp, vp, written = L.pool(spec, 0, kb, vb, n_pool)
        assert written.sum() == n_pool
        kl, vl, wl = L.pool_loops(spec, 0, kb, vb, n_pool)
        assert np.array_equal(kp, kl) and np.array_equal(vp, vl) and np.array_equal(written, wl)
        for b in range(spec.num_seqs):
            for h in range(spec.num_kv_heads):
                for pos, pids in L.unit_page_ids(spec, b, 0, h, tab):
                    for i, p in enumerate(pos):
                        pid, slot = pids[i // 32], i % 32
                        k_el = kp[pid, :, slot, :].reshape(-1)
                        v_el = vp[pid, slot // 8, :, slot % 8]
                        assert np.array_equal(k_el, kb[kvo[b] + p, h])
                        assert np.array_equal(v_el, vb[kvo[b] + p, h])
        # the stream moves every distinct page once
        ks, vs = L.transfer_stream(spec, 0, kb, vb)
        assert len(ks) == n_pool
