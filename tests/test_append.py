"""Append mode on the host: the oracle's ring model (pinned by the invariant a
ring buffer must keep: no newer key overwrites a key the decode row still sees),
the planner's image after appends against that model position by position, the
decode work lists after appends, and the error paths."""
import ctypes
from dataclasses import replace

import numpy as np
import pytest

import workloads as W
from oracle import attention as OA
from oracle import layout as OL
from tests.table_image import work_lists

sp = pytest.importorskip("sparse_attention_segmentpagetable_amd")


def _spec(n0=(50, 17, 1, 0), ps=16, hd=64):
    kind = [W.GLOBAL, W.LOCAL, W.LOCAL, W.RETRIEVAL, W.DENSE, W.LOCAL]
    retr = {(0, 1, 0): np.array([1, 2, 30, 31, 32], np.int32),
            (2, 1, 0): np.array([0], np.int32)}
    s = W.Spec(name="append", num_layers=2, num_q_heads=6, num_kv_heads=3, head_dim=hd,
               page_size=ps, seq_len=list(n0), first_query_pos=[0] * len(n0), kind=kind,
               sink=[0, 3, 0, 0, 0, 20], window=[1, 37, 20, 1, 1, 5], retrieval=retr, seed=21)
    return W.decode_form(s)


def _visible(spec, b, l, h, n):
    kind, s, w = spec.head_class(l, h)
    if n == 0:
        return []
    r = spec.retrieval.get((b, l, h))
    return list(np.nonzero(OA.visibility_mask(kind, s, w, r, np.array([n - 1]), n)[0])[0])


@pytest.mark.parametrize("s,w,P,n0,chunk", [(0, 1, 16, 0, 1), (3, 37, 16, 50, 1),
                                            (20, 5, 16, 3, 1), (4, 64, 64, 200, 1),
                                            (0, 63, 32, 1, 1), (5, 16, 16, 21, 1),
                                            (3, 37, 16, 50, 9), (4, 64, 64, 200, 100),
                                            (0, 20, 16, 7, 7), (2, 5, 32, 40, 40)])
def test_ring_model_keeps_every_visible_key(s, w, P, n0, chunk):
    q0 = max(n0 - chunk, 0)
    spec = W.Spec(name="r", num_layers=1, num_q_heads=1, num_kv_heads=1, head_dim=64,
                  page_size=P, seq_len=[n0], first_query_pos=[q0], kind=[W.LOCAL],
                  sink=[s], window=[w], seed=1)
    res = OL.append_reserved_pages(spec, 0, 0, 0, 0, chunk)
    w0 = max(s, q0 - w + 1)
    for n in range(n0, n0 + 5 * (w + P + chunk) + 3):
        cells = {}
        for p in range(n):  # replay writes in position order; the last writer owns a cell
            if p < n0 and not (p < s or p >= w0):
                continue  # never stored: dropped before planning
            cells[OL.append_slot(spec, 0, 0, 0, p, chunk)] = p
        # every key any row of the newest chunk (rows n - chunk .. n - 1) sees
        rows = np.arange(max(n - chunk, q0 if n == n0 else 0), n)
        rows = rows[rows >= 0]
        need = set()
        for i in rows:
            need |= set(np.nonzero(OA.visibility_mask(W.LOCAL, s, w, None, np.array([i]), n)[0])[0])
        for p in sorted(need):
            pg, slot = OL.append_slot(spec, 0, 0, 0, int(p), chunk)
            assert 0 <= pg < res and 0 <= slot < P
            assert cells[(pg, slot)] == p, (n, p)


def _slot_from_table(t, u, p, P):
    """(page id, slot) of position p read through the table as the kernels do."""
    off_units, off_pages = int(t[12]), int(t[13])
    r = t[off_units + 16 * u: off_units + 16 * (u + 1)]
    nseg = int(r[9])
    segs = [(int(r[10 + 2 * k]), int(r[11 + 2 * k])) for k in range(nseg)]
    base = 0
    for pos0, ln in segs:
        if pos0 >= 0 and pos0 <= p < pos0 + ln:
            slot = base + p - pos0
            return int(t[off_pages + int(r[14]) + slot // P]), slot % P
        base += -(-ln // P) * P
    return None


@pytest.mark.parametrize("free", [False, True])
def test_planner_image_follows_the_ring_model(free):
    spec = _spec()
    cap = 120
    if free:
        spec = replace(spec, free_list=W.seeded_free_list(400, 5), capacity_pages=400)
    plan = sp.Plan(spec, append_capacity=cap, append_chunk=3)
    pages = OL.append_unit_pages(spec, cap, 3)
    rng = np.random.default_rng(3)
    n = list(spec.seq_len)
    for step in range(40):
        add = [int(x) for x in rng.integers(0, 4, size=len(n))]
        add = [min(a, spec.seq_len[b] + cap - n[b]) for b, a in enumerate(add)]
        plan.append(add)
        n = [a + x for a, x in zip(n, add)]
        t = plan.table_host()
        for b in range(len(n)):
            assert t[16 + 4 * b] == n[b] and t[16 + 4 * b + 1] == max(n[b] - max(add[b], 1), 0)
        for (u, b, l, h) in OL.units(spec):
            kind, _, _ = spec.head_class(l, h)
            if kind == W.RETRIEVAL:
                continue
            for p in _visible(spec, b, l, h, n[b]):
                pg, slot = OL.append_slot(spec, b, l, h, p, 3)
                assert _slot_from_table(t, u, p, spec.page_size) == (pages[(b, l, h)][pg], slot)


def test_decode_items_cover_visible_keys_after_appends():
    spec = _spec(ps=16)
    cap = 200
    plan = sp.Plan(spec, append_capacity=cap, decode_split_tokens=64, append_chunk=70)
    n = list(spec.seq_len)
    for add in ([1, 1, 1, 1], [3, 0, 2, 5], [64, 1, 0, 40], [0, 0, 0, 0], [17, 33, 70, 2]):
        plan.append(add)
        n = [a + x for a, x in zip(n, add)]
        t = plan.table_host()
        z = plan.sizes
        du, items, _, _ = work_lists(t, z, spec.group, spec.num_q_heads)
        P = spec.page_size
        for (u, b, l, h) in OL.units(spec):
            kind, _, _ = spec.head_class(l, h)
            if kind == W.RETRIEVAL:
                continue
            pos_of = {}
            for p in range(n[b]):
                x = _slot_from_table(t, u, p, P)
                if x is not None:
                    pos_of.setdefault(x, p)
            # slot index within the unit -> position
            off_pages = int(t[13]); r0 = int(t[int(t[12]) + 16 * u + 14])
            unit_ids = list(t[off_pages + r0: off_pages + r0 + 64])
            seen = []
            for it in range(*du[u]):
                uu, lo, hi, gap = items[it]
                gap_hi = -(-gap // P) * P if gap else 0
                for x in range(lo, hi):
                    if gap and gap <= x < gap_hi:
                        continue
                    seen.append(pos_of[(int(unit_ids[x // P]), x % P)])
            assert sorted(seen) == _visible(spec, b, l, h, n[b]), (u, n[b])
        assert plan.sizes.decode_items <= plan.sizes.decode_workspace_bytes // (4 * 2 * (64 + 4))


def test_append_errors():
    spec = _spec()
    plan = sp.Plan(spec, append_capacity=5, append_chunk=5)
    with pytest.raises(sp.SegPagedError) as e:
        plan.append([6, 0, 0, 0])
    assert e.value.status == -1  # more than one chunk
    plan.append([3, 0, 0, 0])
    with pytest.raises(sp.SegPagedError) as e:
        plan.append([3, 0, 0, 0])
    assert e.value.status == -3  # past the capacity
    plan = sp.Plan(spec, append_capacity=5, append_chunk=5)
    with pytest.raises(sp.SegPagedError) as e:
        plan.append([-1, 0, 0, 0])
    assert e.value.status == -1
    plan.append([5, 5, 5, 5])
    with pytest.raises(sp.SegPagedError):
        plan.append([1, 0, 0, 0])
    with pytest.raises(sp.SegPagedError) as e:
        sp.Plan(spec).append([1, 0, 0, 0])
    assert e.value.status == -5
    # growth: at most one chunk of rows per sequence
    with pytest.raises(sp.SegPagedError) as e:
        sp.Plan(replace(spec, first_query_pos=[0, 0, 0, 0]), append_capacity=4)
    assert e.value.status == -1
    sp.Plan(replace(spec, first_query_pos=[0, 0, 0, 0]), append_capacity=4, append_chunk=50)
    lib = sp.library()
    assert lib.segpaged_append(None, 0, None, None, None, None, None, None) == -1
    assert lib.segpaged_plan_append(None, None) == -1


def test_sizes_do_not_change_with_appends():
    spec = _spec()
    plan = sp.Plan(spec, append_capacity=64, append_chunk=64)
    z0 = plan.sizes.as_dict()
    plan.append([64, 10, 0, 3])
    z1 = plan.sizes.as_dict()
    for k in ("table_int32s", "pool_pages", "pool_bytes", "decode_workspace_bytes", "num_pages"):
        assert z0[k] == z1[k], k
    assert plan.sizes.kv_rows == sum(spec.seq_len) + 77


def test_failed_append_leaves_the_plan_unchanged():
    """An append that fails (a count above the chunk, below zero, or past the planned
    capacity) changes nothing: image, sizes and work counts are those from before."""
    spec = _spec()
    plan = sp.Plan(spec, append_capacity=9, append_chunk=4)
    plan.append([4, 1, 0, 2])
    before = (plan.table_host().copy(), plan.sizes.as_dict(), plan.stats(-1))
    for bad, status in (([5, 0, 0, 0], -1), ([0, -1, 0, 0], -1)):
        with pytest.raises(sp.SegPagedError) as e:
            plan.append(bad)
        assert e.value.status == status
        assert np.array_equal(plan.table_host(), before[0])
        assert plan.sizes.as_dict() == before[1] and plan.stats(-1) == before[2]
    plan.append([4, 4, 4, 4])
    mid = plan.table_host().copy()
    with pytest.raises(sp.SegPagedError) as e:
        plan.append([2, 0, 0, 0])  # 50 + 8 + 2 > 50 + 9
    assert e.value.status == -3
    assert np.array_equal(plan.table_host(), mid)
