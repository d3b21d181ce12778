"""Host planner (C++) against the oracle, on the CPU: the SegmentPageTable must
match bit for bit; work counts must match brute-force counts; work lists must
cover exactly what each row sees; invalid specs must fail before any launch."""
import ctypes
import os
import re
import subprocess
from dataclasses import replace

import numpy as np
import pytest

import workloads as W
from oracle import attention as OA
from oracle import layout as OL
from tests.table_image import DI_INTS, DU_INTS, PI_INTS, work_lists
from tests.random_specs import random_spec

sp = pytest.importorskip("sparse_attention_segmentpagetable_amd")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _mixed(q0=(0, 30), free=None, cap=0):
    kind = [W.GLOBAL, W.LOCAL, W.RETRIEVAL, W.LOCAL, W.DENSE, W.RETRIEVAL]
    retr = {(0, 1, 0): np.array([1, 2, 30, 31, 32], np.int32),
            (1, 1, 0): np.array([], np.int32),
            (0, 2, 1): np.array([3, 17], np.int32),
            (1, 2, 1): np.array([0, 1, 2, 3, 4, 5, 6, 7, 8, 40, 41], np.int32)}
    return W.Spec(name="mixed", num_layers=3, num_q_heads=4, num_kv_heads=2, head_dim=64,
                  page_size=16, seq_len=[37, 45], first_query_pos=list(q0), kind=kind,
                  sink=[2, 3, 0, 4, 0, 0], window=[1, 9, 1, 5, 1, 1], retrieval=retr,
                  free_list=free, capacity_pages=cap)


def _specs():
    yield W.tiny("prefill")
    yield W.tiny("decode")
    yield W.tiny("prefill", n=1)
    yield W.mistral_layer("decode", seqs=2, n=1000, window=100)
    yield W.mistral_layer("prefill", seqs=3, n=700, window=64)
    yield _mixed()
    yield _mixed(q0=(36, 44))
    yield _mixed(q0=(10, 0), free=W.seeded_free_list(300, 4), cap=300)
    yield W.llama70b_decode(num_layers=3, seqs=2, n=3000, window=512)
    yield W.mixed_varlen_decode(seqs=4, num_layers=2, lo=64, hi=5000, window=256)
    s = W.tiny("prefill", n=50)
    yield replace(s, seq_len=[50, 0, 7], first_query_pos=[0, 0, 6])  # empty + ragged sequences
    for seed in range(100, 132):  # the first half of the GPU tests' random specs
        yield random_spec(seed)
    yield from _doc_specs()


def _doc_specs():
    """Document groups: sequences 0 and 2 share 300 tokens, 1 and 3 share 64, 4 none."""
    kind = [W.GLOBAL, W.LOCAL, W.RETRIEVAL, W.LOCAL, W.DENSE, W.GLOBAL]
    n = [700, 333, 301, 64, 90]
    retr = {(b, 1, 0): np.arange(1, nb, 5, dtype=np.int32) for b, nb in enumerate(n)}
    base = W.Spec(name="doc", num_layers=3, num_q_heads=8, num_kv_heads=2, head_dim=64,
                  page_size=32, seq_len=n, first_query_pos=[0] * 5, kind=kind,
                  sink=[0, 4, 0, 33, 0, 0], window=[1, 60, 1, 8, 1, 1], retrieval=retr, seed=7,
                  doc_group=[0, 1, 0, 1, -1], doc_len=[300, 64, 300, 64, 0])
    yield base
    yield replace(W.decode_form(base), name="doc-decode")
    yield replace(base, name="doc-p16-free", page_size=16,
                  free_list=W.seeded_free_list(400, 3), capacity_pages=400)


@pytest.mark.parametrize("spec", list(_specs()), ids=lambda s: f"{s.name}")
def test_table_bit_exact_vs_oracle(spec):
    plan = sp.Plan(spec)
    got = plan.table_host()
    ref = OL.table(spec)
    assert plan.sizes.table_len == len(ref)
    assert np.array_equal(got[:len(ref)], ref)
    assert plan.sizes.num_pages == OL.distinct_pages(spec)  # the table lists ref[9] slots
    assert plan.sizes.q_rows == spec.total_q_rows and plan.sizes.kv_rows == spec.total_tokens


@pytest.mark.parametrize("spec", list(_specs()), ids=lambda s: f"{s.name}")
def test_stats_vs_bruteforce(spec):
    plan = sp.Plan(spec)
    for layer in range(spec.num_layers):
        st = plan.stats(layer)
        pairs = dec = rows = 0
        for b, n in enumerate(spec.seq_len):
            q0 = spec.first_query_pos[b]
            for h in range(spec.num_kv_heads):
                kind, s, w = spec.head_class(layer, h)
                r = spec.retrieval.get((b, layer, h))
                pairs += OA.visible_pairs(kind, s, w, r, n, q0)
                if n > 0:
                    dec += int(OA.visibility_mask(kind, s, w, r, np.array([n - 1]), n).sum())
                rows += n - q0
        assert st["prefill_pairs"] == pairs
        assert st["decode_tokens"] == dec
        assert st["q_rows"] == rows
        assert st["retained_tokens"] == OL.kv_len_total(spec, layers={layer})
    tot = plan.stats(-1)
    assert tot["retained_tokens"] == OL.kv_len_total(spec)


def _decode_items(plan, spec):
    t = plan.table_host()
    z = plan.sizes
    du, items, pre, end = work_lists(t, z, spec.group, spec.num_q_heads)
    assert np.all(t[end:] == 0)  # work counters start at zero
    return t, du, items, pre


@pytest.mark.parametrize("spec", list(_specs()), ids=lambda s: f"{s.name}")
@pytest.mark.parametrize("split", [0, 64, 192])
def test_decode_items_cover_visible_keys_once(spec, split):
    plan = sp.Plan(spec, decode_split_tokens=split)
    t, du, items, _ = _decode_items(plan, spec)
    P = spec.page_size
    for (u, b, l, h) in OL.units(spec):
        n = spec.seq_len[b]
        kind, s, w = spec.head_class(l, h)
        r = spec.retrieval.get((b, l, h))
        seen = []
        ib, ie = du[u]
        slot_base = 0
        pos_of_slot = {}
        for seg in OL.unit_segments(spec, b, l, h):
            for k, p in enumerate(OL.segment_positions(seg)):
                pos_of_slot[slot_base + k] = int(p)
            slot_base += OL.ceil_div(len(OL.segment_positions(seg)), P) * P
        for it in range(ib, ie):
            uu, lo, hi, gap = items[it]
            assert uu == u and hi > lo
            gap_hi = OL.ceil_div(gap, P) * P if gap else 0
            if split:  # at most `split` keys, plus a sink of at most `split` before a gap
                assert hi - lo - (gap_hi - gap) <= 2 * split
            seen += [pos_of_slot[x] for x in range(lo, hi) if not gap <= x < gap_hi]
        want = [] if n == 0 else list(np.nonzero(
            OA.visibility_mask(kind, s, w, r, np.array([n - 1]), n)[0])[0])
        assert sorted(seen) == want and len(seen) == len(set(seen))


@pytest.mark.parametrize("spec", list(_specs()), ids=lambda s: f"{s.name}")
def test_prefill_items_tile_every_row_once(spec):
    plan = sp.Plan(spec)
    _, _, _, pre = _decode_items(plan, spec)
    G = spec.group
    bq = 256 // G
    got = {}
    for u, r0 in pre:
        got.setdefault(int(u), []).append(int(r0) & 0x7FFFFFFF)
    precise = {(int(u), int(r0) & 0x7FFFFFFF): int(r0) < 0 for u, r0 in pre}
    for (u, b, l, h) in OL.units(spec):
        n, q0 = spec.seq_len[b], spec.first_query_pos[b]
        assert sorted(got.get(u, [])) == list(range(q0, n, bq))
        # bit 31 marks the tiles whose first row sees fewer than 128 keys
        kind, s, w = spec.head_class(l, h)
        r = spec.retrieval.get((b, l, h))
        for r0 in range(q0, n, bq):
            keys = int(OA.visibility_mask(kind, s, w, r, np.array([r0]), n).sum())
            assert precise[(u, r0)] == (keys < 128), (u, r0, keys)
    assert len(pre) == plan.sizes.prefill_items


def test_split_and_workspace_sizes():
    spec = W.tiny("decode")
    plan = sp.Plan(spec, decode_split_tokens=64)
    z = plan.sizes
    # one partial per item, plus the 1536 extra partials of the items a launch of
    # several rounds deals to 4 waves each (512 items)
    assert z.decode_workspace_bytes == (z.decode_items + 1536) * spec.group * (spec.head_dim + 4) * 4
    # global unit: 513 keys -> 9 items of <= 64; local: sink 4 + window 64 in one item
    # (the sink page's zero tail is a gap inside it)
    assert z.decode_items == 9 + 3 * 1


def _rc(spec_kwargs, **plan_kwargs):
    s = replace(W.tiny("prefill", n=40), **spec_kwargs)
    try:
        sp.Plan(s, **plan_kwargs)
        return 0
    except sp.SegPagedError as e:
        return e.status


def test_validation_errors():
    assert _rc({}) == 0
    assert _rc({"head_dim": 96}) == -2
    assert _rc({"page_size": 48}) == -2
    assert _rc({"page_size": 0}) == -1
    assert _rc({"num_q_heads": 6}) == -1          # not a multiple of Hkv
    assert _rc({"num_q_heads": 4 * 32}) == -2     # group of 32 unsupported
    assert _rc({"window": [64, 0, 64, 64]}) == -1  # LOCAL window < 1
    assert _rc({"sink": [4, -1, 4, 4]}) == -1
    assert _rc({"kind": [0, 1, 9, 1]}) == -1
    assert _rc({"first_query_pos": [40]}) == -1   # q0 beyond N-1
    assert _rc({"seq_len": [-1]}) == -1
    assert _rc({"kind": [0, 2, 1, 1]}) == -1      # retrieval head without positions
    assert _rc({"kind": [0, 2, 1, 1], "retrieval": {(0, 0, 1): np.array([3, 3], np.int32)}}) == -1
    assert _rc({"kind": [0, 2, 1, 1], "retrieval": {(0, 0, 1): np.array([5, 40], np.int32)}}) == -1
    assert _rc({"kind": [0, 2, 1, 1], "retrieval": {(0, 0, 1): np.array([5, 39], np.int32)}}) == 0
    assert _rc({"retrieval": {(0, 0, 1): np.array([5], np.int32)}}) == -1  # set on a LOCAL head
    assert _rc({"capacity_pages": 5}) == -3       # needs 3 + 3*3 = 12 pages
    assert _rc({"free_list": np.arange(5, dtype=np.int32)}) == -3
    assert _rc({"free_list": np.array([0] * 12, np.int32), "capacity_pages": 20}) == -1
    assert _rc({"free_list": np.arange(12, dtype=np.int32) + 10, "capacity_pages": 20}) == -1
    assert _rc({"free_list": np.arange(12, dtype=np.int32) + 8, "capacity_pages": 20}) == 0
    assert _rc({}, decode_split_tokens=100) == -1
    assert _rc({}, decode_split_tokens=64 * 64) == 0


def test_call_validation_without_gpu():
    """Entry points reject bad arguments before touching the GPU."""
    lib = sp.library()
    plan = sp.Plan(W.tiny("prefill", n=40))
    vp = ctypes.c_void_p
    fake = vp(1 << 20)  # aligned, never dereferenced: validation fails first
    assert lib.segpaged_build(plan.handle, 0, None, fake, fake, fake, fake, None) == -1
    assert lib.segpaged_build(plan.handle, 1, fake, fake, fake, fake, fake, None) == -5
    assert lib.segpaged_build(plan.handle, 0, vp((1 << 20) + 2), fake, fake, fake, fake, None) == -1
    assert lib.segpaged_prefill(plan.handle, -2, fake, fake, fake, fake, ctypes.c_float(0.1),
                                fake, None, None, 0, None) == -5
    assert lib.segpaged_prefill(plan.handle, 0, fake, fake, fake, fake, ctypes.c_float(-1.0),
                                fake, None, None, 0, None) == -1
    dspec = W.tiny("decode")
    dplan = sp.Plan(dspec)
    need = dplan.stats(0)["decode_items"] * dspec.group * (dspec.head_dim + 4) * 4  # the call's items
    assert need < dplan.sizes.decode_workspace_bytes
    assert lib.segpaged_decode(dplan.handle, 0, fake, fake, fake, fake, ctypes.c_float(0.1),
                               fake, None, fake, need - 1, None) == -3
    assert lib.segpaged_decode(dplan.handle, 0, fake, fake, fake, fake, ctypes.c_float(0.1),
                               fake, None, None, need, None) == -1
    assert lib.segpaged_plan_stats(plan.handle, 3, ctypes.byref(sp.Stats())) == -5


def test_library_exports_every_header_symbol():
    hdr = open(os.path.join(ROOT, "include", "segpaged.h")).read()
    names = re.findall(r"SEGPAGED_API\s+[\w\s\*]+?\b(segpaged_\w+)\s*\(", hdr)
    assert len(names) >= 9
    lib = sp.library()
    for nm in names:
        assert hasattr(lib, nm), nm
    out = subprocess.run(["nm", "-D", "--defined-only", sp.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r" T (segpaged_\w+)", out))
    assert set(names) == exported
    assert lib.segpaged_version() >= 100


def test_probe_library_exports_its_header_symbols():
    from sparse_attention_segmentpagetable_amd import probe
    hdr = open(os.path.join(ROOT, "include", "segpaged_probe.h")).read()
    names = re.findall(r"SEGPAGED_API\s+[\w\s\*]+?\b(segpaged_\w+)\s*\(", hdr)
    assert sorted(names) == ["segpaged_probe_hbm_read", "segpaged_probe_mfma_bf16"]
    lib = probe.library()
    out = subprocess.run(["nm", "-D", "--defined-only", probe.PROBE_LIB_PATH],
                         capture_output=True, text=True).stdout
    assert set(re.findall(r" T (segpaged_\w+)", out)) == set(names)
    # argument checks happen before any launch (no GPU needed)
    fake = ctypes.c_void_p(4096)
    assert lib.segpaged_probe_mfma_bf16(None, 1, 1, fake, None) == -1
    assert lib.segpaged_probe_mfma_bf16(fake, 0, 1, fake, None) == -1
    assert lib.segpaged_probe_hbm_read(fake, 24, 1, 8, fake, None) == -1
    assert lib.segpaged_probe_hbm_read(fake, 16, 0, 8, fake, None) == -1
    assert lib.segpaged_probe_hbm_read(fake, 16, 1, 5, fake, None) == -1


def test_select_and_transfer_validation_without_gpu():
    """segpaged_select_topp and the page-stream calls reject bad arguments before
    touching the GPU: null or misaligned buffers (EINVAL), scale or p out of range
    (EINVAL), a layer out of range (ESTATE), a workspace one byte short (ENOSPACE)."""
    lib = sp.library()
    vp, f32 = ctypes.c_void_p, ctypes.c_float
    fake = vp(1 << 20)
    kind = [W.RETRIEVAL, W.LOCAL, W.GLOBAL, W.RETRIEVAL]
    spec = W.Spec(name="sel", num_layers=2, num_q_heads=8, num_kv_heads=2, head_dim=128,
                  page_size=64, seq_len=[300, 70], first_query_pos=[0, 0], kind=kind,
                  sink=[0, 4, 0, 0], window=[1, 20, 1, 1],
                  retrieval={(b, l, h): np.zeros(0, np.int32) for b in range(2) for l in range(2)
                             for h in range(2) if kind[l * 2 + h] == W.RETRIEVAL}, seed=3)
    plan = sp.Plan(W.decode_form(spec))
    need = plan.sizes.select_workspace_bytes

    def sel(layer=0, q=fake, scale=0.1, p=0.9, ws=fake, nbytes=need):
        return lib.segpaged_select_topp(plan.handle, layer, q, fake, fake, f32(scale), f32(p),
                                        fake, fake, ws, nbytes, None)

    assert sel(q=None) == -1
    assert sel(q=vp((1 << 20) + 8)) == -1        # Q not 16-byte aligned
    assert sel(ws=None) == -1
    for p in (0.0, -0.5, 1.01, float("nan")):
        assert sel(p=p) == -1, p
    for scale in (0.0, -1.0, float("inf"), float("nan")):
        assert sel(scale=scale) == -1, scale
    assert sel(layer=2) == -5 and sel(layer=-1) == -5
    assert sel(nbytes=need - 1) == -3
    for fn in (lib.segpaged_export_pages, lib.segpaged_import_pages):
        assert fn(plan.handle, 0, None, fake, fake, fake, fake, fake, None) == -1
        assert fn(plan.handle, 0, fake, vp((1 << 20) + 4), fake, fake, fake, fake, None) == -1
        assert fn(plan.handle, 2, fake, fake, fake, fake, fake, fake, None) == -5
        assert fn(plan.handle, -2, fake, fake, fake, fake, fake, fake, None) == -5


def test_decode_without_items_returns_a_status():
    """A decode-form layer where no unit holds a key (retrieval heads with empty
    sets) has no decode items: choosing the parts per item must not divide by the
    item count. Without a GPU the call ends in a HIP status, not a crash."""
    lib = sp.library()
    kind = [W.RETRIEVAL, W.RETRIEVAL]
    spec = W.Spec(name="noitems", num_layers=1, num_q_heads=4, num_kv_heads=2, head_dim=128,
                  page_size=64, seq_len=[300, 5], first_query_pos=[0, 0], kind=kind,
                  sink=[0, 0], window=[1, 1],
                  retrieval={(b, 0, h): np.zeros(0, np.int32) for b in range(2) for h in range(2)},
                  seed=9)
    plan = sp.Plan(W.decode_form(spec))
    assert plan.sizes.decode_items == 0 and plan.sizes.pool_bytes == 0
    fake, f32 = ctypes.c_void_p(1 << 20), ctypes.c_float
    rc = lib.segpaged_decode(plan.handle, 0, fake, fake, None, None, f32(0.1), fake, None,
                             None, 0, None)
    assert rc in (0, -4), rc


@pytest.mark.parametrize("spec", list(_specs()), ids=lambda s: f"{s.name}")
@pytest.mark.parametrize("cap", [0, 7])
def test_counter_lines_aligned_and_zero(spec, cap):
    """The L + 1 prefill work-counter lines (16 ints each, the first 8 bytes a 64-bit
    counter) start 16-byte aligned in the image and are uploaded as zeros: the state
    a prefill call's generation claim starts from."""
    if cap:  # growth plans reserve more pages than the spec's own free list holds,
        # and share no document pages
        spec = replace(spec, free_list=None, capacity_pages=0, doc_group=None, doc_len=None)
        if any(n - q0 > 1 for n, q0 in zip(spec.seq_len, spec.first_query_pos)):
            spec = W.decode_form(spec)
    plan = sp.Plan(spec, append_capacity=cap)
    t = plan.table_host()
    tail = 2 * spec.num_seqs + 1 if cap else 0
    c1 = len(t) - tail
    c0 = c1 - 16 * (spec.num_layers + 1)
    assert c0 % 4 == 0 and np.all(t[c0:c1] == 0)
    z = plan.sizes
    assert c0 >= (z.table_len + DU_INTS * z.num_units + DI_INTS * z.decode_items
                  + PI_INTS * z.prefill_items)


@pytest.mark.parametrize("spec", list(_doc_specs()), ids=lambda s: s.name)
def test_shared_document_pages_and_build_list(spec):
    """Shared document pages: distinct pages and the build list (the table page
    slots that own a page, first use in table order) as the oracle assigns them."""
    plan = sp.Plan(spec)
    z = plan.sizes
    _, first = OL.page_assignment(spec)
    assert z.num_pages == OL.distinct_pages(spec) == len(first)
    assert z.num_pages < OL.num_pages(spec)  # some pages are shared
    t = plan.table_host()
    assert list(t[z.table_len:z.table_len + z.num_pages]) == first
    for l in range(spec.num_layers):
        assert plan.stats(l)["pages"] == OL.distinct_pages(spec, l)


def test_shared_document_validation():
    spec = next(_doc_specs())
    def rc(**kw):
        try:
            sp.Plan(replace(spec, **kw))
            return 0
        except sp.SegPagedError as e:
            return e.status
    assert rc() == 0
    assert rc(doc_len=[300, 64, 299, 64, 0]) == -1      # members disagree on the length
    assert rc(doc_len=[300, 64, 300, 65, 0]) == -1      # longer than a member's sequence
    assert rc(doc_len=[300, 64, 300, 64, 3]) == -1      # a length without a group
    assert rc(doc_group=[0, 1, 0, 1, 5]) == -1          # group id out of range
    assert rc(doc_len=None) == -1                        # groups without lengths
    d = replace(W.decode_form(spec), name="g")
    with pytest.raises(sp.SegPagedError) as e:
        sp.Plan(d, append_capacity=4)
    assert e.value.status == -2                          # growth plans share nothing
