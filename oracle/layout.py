"""O2: the SegmentPageTable and the page pool, written out from the rules --
TEST INFRASTRUCTURE.

Rules (SegPagedAttention runtime explainer, section 3: a three-level table
(layer, head, segment) -> contiguous virtual pages; local heads get pages for
sink + recent tokens only, global heads for the whole context; local heads keep
only visible tokens; retrieval heads fetch pages on demand):

* Retention, for the rows q0..N-1 that will read the table: a key is kept iff
  it is visible to at least one of those rows.
    GLOBAL / DENSE   one segment [0, N)
    LOCAL(s, W)      [0, min(s, N))  and  [max(min(s, N), q0 - W + 1), N),
                     one merged segment when the two touch
    RETRIEVAL(R)     one gathered segment holding R in order
* Packing (KV-cache guide section 4.3, block tables): token t of a segment sits
  in the segment's page t // P at slot t % P; every segment starts on a fresh
  page; unused tail slots hold zeros.
* Page ids: units in order u = (l * B + b) * Hkv + h, segments in order, pages
  in order, each taking the next id of the free list (identity by default).
* Shared documents (RedKnot summary: identical document chunks reuse their
  KV; runtime explainer section 1: storage per layer x head x segment):
  sequences of one document group begin with the same doc_len tokens. A page of
  a member whose positions all lie in [0, doc_len) is the same page for every
  member of the group whose page, in the same layer and KV head, holds exactly
  the same positions: it takes an id once, at its first use in table order, and
  the pool holds it once (written from that first use). Gathered (retrieval)
  pages are never shared.

Table format, version 1 (all int32):
    header  16 ints  magic 0x53475054, version 1, num_seqs, num_layers, Hq, Hkv,
                     D, P, num_units, num_pages, num_retr, off_seqs, off_units,
                     off_pages, off_retr, table_len
    seqs     4 ints per sequence  N_b, q0_b, dense K/V row offset, Q row offset
    units   16 ints per unit      class (DENSE stored as GLOBAL), b, l, h, N_b, q0_b,
                                  sink, window, kv_len, nseg, seg0_pos, seg0_len,
                                  seg1_pos, seg1_len, page_off, retr_off
                                  (gathered segment: seg0_pos = -1;
                                  retr_off = -1 for non-RETRIEVAL units)
    pages   page id of each table page
    retr    retrieval positions, units in order

Pool layout (bf16 bits):
    K page  [D/8][P][8]   K_pool[p, d // 8, slot, d % 8]
    V page  [P/8][D][8]   V_pool[p, slot // 8, d, slot % 8]
"""
from __future__ import annotations

from typing import Dict, List, Tuple

import numpy as np

from workloads import DENSE, GLOBAL, LOCAL, RETRIEVAL, Spec

MAGIC = 0x53475054
VERSION = 1
HEADER_INTS, SEQ_INTS, UNIT_INTS = 16, 4, 16


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def retained_segments(kind: int, sink: int, window: int, n: int, q0: int, retr) -> List:
    """List of segments; a contiguous segment is (pos0, length), a gathered one is
    ('gathered', positions)."""
    if kind in (GLOBAL, DENSE):
        return [(0, n)] if n > 0 else []
    if kind == LOCAL:
        a = min(sink, n)
        w0 = max(a, q0 - window + 1)
        segs = []
        if a > 0:
            segs.append((0, a))
        if n > w0:
            if segs and w0 == a:
                segs = [(0, n)]
            else:
                segs.append((w0, n - w0))
        return segs
    if kind == RETRIEVAL:
        r = np.asarray(retr if retr is not None else [], dtype=np.int32)
        return [("gathered", r)] if len(r) else []
    raise ValueError(kind)


def segment_positions(seg) -> np.ndarray:
    if seg[0] == "gathered":
        return np.asarray(seg[1], dtype=np.int64)
    return np.arange(seg[0], seg[0] + seg[1], dtype=np.int64)


def units(spec: Spec):
    """(u, b, l, h) in table order."""
    out = []
    B, H = spec.num_seqs, spec.num_kv_heads
    for l in range(spec.num_layers):
        for b in range(B):
            for h in range(H):
                out.append(((l * B + b) * H + h, b, l, h))
    return out


def unit_segments(spec: Spec, b: int, l: int, h: int) -> List:
    kind, sink, window = spec.head_class(l, h)
    return retained_segments(kind, sink, window, spec.seq_len[b], spec.first_query_pos[b],
                             spec.retrieval.get((b, l, h)))


def page_share_key(spec: Spec, b: int, l: int, h: int, seg, positions: np.ndarray):
    """The identity of a page that sequences of a document group share, or None when
    the page is the unit's own: (layer, KV head, group, its positions)."""
    groups = spec.doc_group
    if groups is None or groups[b] < 0 or seg[0] == "gathered":
        return None
    if len(positions) == 0 or int(positions[-1]) >= spec.doc_len[b]:
        return None
    return (l, h, groups[b], tuple(int(x) for x in positions))


def unit_pages(spec: Spec):
    """Every page slot of the table in order: (u, b, l, h, segment, positions, key)."""
    P = spec.page_size
    out = []
    for (u, b, l, h) in units(spec):
        for seg in unit_segments(spec, b, l, h):
            pos = segment_positions(seg)
            for p0 in range(0, len(pos), P):
                pp = pos[p0:p0 + P]
                out.append((u, b, l, h, seg, pp, page_share_key(spec, b, l, h, seg, pp)))
    return out


def page_assignment(spec: Spec) -> Tuple[List[int], List[int]]:
    """(distinct page index of every page slot, the slots where a distinct page is
    first used): a shared page takes its index at its first slot."""
    index, first, seen = [], [], {}
    for slot, (_, _, _, _, _, _, key) in enumerate(unit_pages(spec)):
        if key is not None and key in seen:
            index.append(seen[key])
            continue
        d = len(first)
        if key is not None:
            seen[key] = d
        first.append(slot)
        index.append(d)
    return index, first


def distinct_pages(spec: Spec, layer: int = None) -> int:
    """Pages the pool holds (of one layer, or all)."""
    if layer is None:
        return len(page_assignment(spec)[1])
    slots = unit_pages(spec)
    return sum(1 for s in page_assignment(spec)[1] if slots[s][2] == layer)


def table(spec: Spec) -> np.ndarray:
    """The expected table ints (int32)."""
    P = spec.page_size
    B = spec.num_seqs
    recs, page_ids, retr = [], [], []
    free = spec.free_list
    index, _ = page_assignment(spec)
    nxt = 0
    for (u, b, l, h) in units(spec):
        kind, sink, window = spec.head_class(l, h)
        segs = unit_segments(spec, b, l, h)
        rec = [GLOBAL if kind == DENSE else kind, b, l, h, spec.seq_len[b],
               spec.first_query_pos[b], sink, window, 0, len(segs), 0, 0, 0, 0,
               len(page_ids), -1]
        if kind == RETRIEVAL:
            rec[15] = len(retr)
        kv_len = 0
        for si, seg in enumerate(segs):
            if seg[0] == "gathered":
                pos0, ln = -1, len(seg[1])
                retr.extend(int(x) for x in seg[1])
            else:
                pos0, ln = seg
            rec[10 + 2 * si] = pos0
            rec[11 + 2 * si] = ln
            kv_len += ln
            for _ in range(ceil_div(ln, P)):
                d = index[nxt]
                page_ids.append(d if free is None else int(free[d]))
                nxt += 1
        rec[8] = kv_len
        recs.append(rec)
    off_seqs = HEADER_INTS
    off_units = off_seqs + SEQ_INTS * B
    off_pages = off_units + UNIT_INTS * len(recs)
    off_retr = off_pages + len(page_ids)
    total = off_retr + len(retr)
    hdr = [MAGIC, VERSION, B, spec.num_layers, spec.num_q_heads, spec.num_kv_heads,
           spec.head_dim, P, len(recs), len(page_ids), len(retr), off_seqs, off_units,
           off_pages, off_retr, total]
    seqs = []
    kvo, qo = spec.kv_row_offsets(), spec.q_row_offsets()
    for b in range(B):
        seqs += [spec.seq_len[b], spec.first_query_pos[b], kvo[b], qo[b]]
    flat = hdr + seqs + [x for r in recs for x in r] + page_ids + retr
    return np.asarray(flat, dtype=np.int64).astype(np.int32)


def num_pages(spec: Spec) -> int:
    return int(table(spec)[9])


def unit_page_ids(spec: Spec, b: int, l: int, h: int, t: np.ndarray = None
                  ) -> List[Tuple[np.ndarray, List[int]]]:
    """[(segment positions, [page ids])] for one unit, from the oracle's own table
    (pass `t = table(spec)` to avoid rebuilding it)."""
    t = table(spec) if t is None else t
    off_units, off_pages = int(t[12]), int(t[13])
    u = (l * spec.num_seqs + b) * spec.num_kv_heads + h
    rec = t[off_units + UNIT_INTS * u: off_units + UNIT_INTS * (u + 1)]
    segs = unit_segments(spec, b, l, h)
    out, p = [], int(rec[14])
    for seg in segs:
        pos = segment_positions(seg)
        npg = ceil_div(len(pos), spec.page_size)
        out.append((pos, [int(x) for x in t[off_pages + p: off_pages + p + npg]]))
        p += npg
    return out


def pool_loops(spec: Spec, layer: int, k_bits: np.ndarray, v_bits: np.ndarray,
               pool_pages: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Expected pool contents after building `layer`, element by element: (K_pool
    uint16 [pool_pages, D/8, P, 8], V_pool uint16 [pool_pages, P/8, D, 8],
    written bool [pool_pages]). Pages of other layers are not written (zeros)."""
    P, D = spec.page_size, spec.head_dim
    kp = np.zeros((pool_pages, D // 8, P, 8), dtype=np.uint16)
    vp = np.zeros((pool_pages, P // 8, D, 8), dtype=np.uint16)
    written = np.zeros(pool_pages, dtype=bool)
    kvo = spec.kv_row_offsets()
    tab = table(spec)
    for b in range(spec.num_seqs):
        for h in range(spec.num_kv_heads):
            for pos, pids in unit_page_ids(spec, b, layer, h, tab):
                for pi, pid in enumerate(pids):
                    if written[pid]:
                        continue  # a shared page, written by its first use
                    written[pid] = True
                    for slot in range(P):
                        t = pi * P + slot
                        if t >= len(pos):
                            break  # tail slots stay zero
                        row = kvo[b] + int(pos[t])
                        for d in range(D):
                            kp[pid, d // 8, slot, d % 8] = k_bits[row, h, d]
                            vp[pid, slot // 8, d, slot % 8] = v_bits[row, h, d]
    return kp, vp, written


def pool(spec: Spec, layer: int, k_bits: np.ndarray, v_bits: np.ndarray,
         pool_pages: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Same result as pool_loops, one page at a time: the page's token rows
    [P, D] (zero rows past the segment's end) are regrouped into the K
    [D/8][P][8] and V [P/8][D][8] layouts."""
    P, D = spec.page_size, spec.head_dim
    kp = np.zeros((pool_pages, D // 8, P, 8), dtype=np.uint16)
    vp = np.zeros((pool_pages, P // 8, D, 8), dtype=np.uint16)
    written = np.zeros(pool_pages, dtype=bool)
    kvo = spec.kv_row_offsets()
    tab = table(spec)
    for b in range(spec.num_seqs):
        for h in range(spec.num_kv_heads):
            for pos, pids in unit_page_ids(spec, b, layer, h, tab):
                for pi, pid in enumerate(pids):
                    if written[pid]:
                        continue  # a shared page, written by its first use
                    written[pid] = True
                    rows = kvo[b] + pos[pi * P:(pi + 1) * P]
                    kt = np.zeros((P, D), dtype=np.uint16)
                    vt = np.zeros((P, D), dtype=np.uint16)
                    kt[:len(rows)] = k_bits[rows, h]
                    vt[:len(rows)] = v_bits[rows, h]
                    # K: element (slot, d) -> [d // 8][slot][d % 8]
                    kp[pid] = kt.reshape(P, D // 8, 8).transpose(1, 0, 2)
                    # V: element (slot, d) -> [slot // 8][d][slot % 8]
                    vp[pid] = vt.reshape(P // 8, 8, D).transpose(0, 2, 1)
    return kp, vp, written


def transfer_stream(spec: Spec, layer: int, k_bits: np.ndarray, v_bits: np.ndarray
                    ) -> Tuple[np.ndarray, np.ndarray]:
    """The pages of one layer as a transfer stream (K uint16 [pages, D/8, P, 8],
    V uint16 [pages, P/8, D, 8]): units in table order, their segments in order,
    each segment's pages in order, every page in the pool layout with zero tail
    slots; a page that sequences of a document group share comes once, at its
    first use. Only what each head keeps is moved (RedKnot summary, system gains:
    KV bytes moved between prefill and decode machines); the stream does not depend
    on page ids. k_bits/v_bits: that layer's dense K/V [T_total, Hkv, D]."""
    P, D = spec.page_size, spec.head_dim
    kvo = spec.kv_row_offsets()
    ks, vs, sent = [], [], set()
    for (u, b, l, h, seg, pos, key) in unit_pages(spec):
        if l != layer:
            continue
        if key is not None:
            if key in sent:
                continue
            sent.add(key)
        rows = kvo[b] + pos
        kt = np.zeros((P, D), dtype=np.uint16)
        vt = np.zeros((P, D), dtype=np.uint16)
        kt[:len(rows)] = k_bits[rows, h]
        vt[:len(rows)] = v_bits[rows, h]
        ks.append(kt.reshape(P, D // 8, 8).transpose(1, 0, 2))
        vs.append(vt.reshape(P // 8, 8, D).transpose(0, 2, 1))
    if not ks:
        return (np.zeros((0, D // 8, P, 8), np.uint16), np.zeros((0, P // 8, D, 8), np.uint16))
    return np.stack(ks), np.stack(vs)


def kv_len_total(spec: Spec, layers=None) -> int:
    """Retained tokens summed over all units (of the given layers)."""
    tot = 0
    for (u, b, l, h) in units(spec):
        if layers is not None and l not in layers:
            continue
        for seg in unit_segments(spec, b, l, h):
            tot += len(segment_positions(seg))
    return tot


def dense_kv_bytes(num_layers: int, num_kv_heads: int, head_dim: int, tokens: int,
                   bytes_per_elem: int = 2) -> int:
    """KV-cache size of a dense cache (KV-guide section 3.2):
    2 (K and V) x layers x KV heads x head dim x tokens x bytes per element."""
    return 2 * num_layers * num_kv_heads * head_dim * tokens * bytes_per_elem


def retained_kv_bytes(spec: Spec, bytes_per_elem: int = 2) -> int:
    """K and V bytes the SegPaged cache keeps (tail padding excluded)."""
    return 2 * spec.head_dim * bytes_per_elem * kv_len_total(spec)


# ----------------------------------------------------------------------------
# Growth (append mode: a decode loop, or a prefill taken in chunks). The layout
# is written once, when K/V is written, and afterwards only extended (runtime
# explainer, section 5); local heads keep only sink + recent tokens (section 3).
# The rules, for a plan made at lengths N0_b with first rows q0_b
# (N0_b - q0_b <= chunk), an append capacity `cap` and at most `chunk` tokens
# per append:
#   * reserved pages per unit (ids taken from the free list in unit order):
#       GLOBAL / DENSE  ceil((N0 + cap) / P)
#       LOCAL(s, W)     ceil(s / P) sink pages, then a ring of
#                       R = ceil((W + chunk - 1) / P) + 1
#       RETRIEVAL(R)    ceil(|R| / P)
#   * GLOBAL position p: unit page p // P, slot p % P.
#   * LOCAL position p < s: unit page p // P, slot p % P (the sink).
#   * LOCAL position p >= w0 = max(s, q0 - W + 1): ring offset o = (p - w0) mod
#     (R P), unit page ceil(s / P) + o // P, slot o % P -- a ring buffer holding
#     more than W + chunk - 1 recent positions, so every key a row of the
#     newest chunk sees is still held.
# ----------------------------------------------------------------------------

def append_reserved_pages(spec: Spec, cap: int, b: int, l: int, h: int, chunk: int = 1) -> int:
    kind, s, w = spec.head_class(l, h)
    P = spec.page_size
    if kind == LOCAL:
        return ceil_div(s, P) + ceil_div(w + chunk - 1, P) + 1
    if kind == RETRIEVAL:
        return ceil_div(len(spec.retrieval.get((b, l, h), [])), P)
    return ceil_div(spec.seq_len[b] + cap, P)


def append_unit_pages(spec: Spec, cap: int, chunk: int = 1
                      ) -> Dict[Tuple[int, int, int], List[int]]:
    """Reserved page ids of every unit (b, l, h), in allocation order."""
    out, cursor = {}, 0
    fl = spec.free_list
    for (u, b, l, h) in units(spec):
        n = append_reserved_pages(spec, cap, b, l, h, chunk)
        out[(b, l, h)] = [int(fl[cursor + i]) if fl is not None else cursor + i
                          for i in range(n)]
        cursor += n
    return out


def append_slot(spec: Spec, b: int, l: int, h: int, p: int, chunk: int = 1) -> Tuple[int, int]:
    """(unit page index, slot) of position p of unit (b, l, h) in append mode
    (positions a local head no longer keeps map onto the slot that replaced them);
    `spec` is the spec the plan was made from."""
    kind, s, w = spec.head_class(l, h)
    P = spec.page_size
    if kind == LOCAL and p >= s:
        w0 = max(s, spec.first_query_pos[b] - w + 1)
        ring = (ceil_div(w + chunk - 1, P) + 1) * P
        o = (p - w0) % ring
        return ceil_div(s, P) + o // P, o % P
    return p // P, p % P
