// Host planner: spec validation, SegmentPageTable construction, page allocation
// and the per-head varlen work lists. Host code only -- no HIP call, so it runs
// (and is tested) without a GPU.
//
// Retention and table rules: SegPagedAttention runtime explainer, section 3
// (per-(layer, head, segment) pages; local heads keep sink + recent pages,
// global heads the whole context; local heads are cut to visible tokens) and
// section 5 (the layout is built once, when KV is written, and reused).
#include <algorithm>
#include <cstring>
#include <limits>
#include <map>
#include <new>
#include <numeric>
#include <tuple>
#include <vector>

#include "plan.hpp"

using namespace segpaged;

namespace {

struct Seg {
  int64_t pos0;  // first logical position, -1 for a gathered (retrieval) segment
  int64_t len;
};

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Keys visible to at least one query row in [q0, n): see segpaged_plan_create.
int retained(int kind, int64_t sink, int64_t window, int64_t n, int64_t q0, int64_t retr_len,
             Seg out[2]) {
  if (kind == SEGPAGED_GLOBAL || kind == SEGPAGED_DENSE) {
    if (n <= 0) return 0;
    out[0] = {0, n};
    return 1;
  }
  if (kind == SEGPAGED_RETRIEVAL) {
    if (retr_len <= 0) return 0;
    out[0] = {-1, retr_len};
    return 1;
  }
  // LOCAL: sink [0, a) and window [w0, n), w0 = max(a, q0 - window + 1)
  const int64_t a = std::min(sink, n);
  const int64_t w0 = std::max(a, q0 - window + 1);
  int cnt = 0;
  if (a > 0) out[cnt++] = {0, a};
  if (n > w0) {
    if (cnt == 1 && w0 == a) {
      out[0] = {0, n};
    } else {
      out[cnt++] = {w0, n - w0};
    }
  }
  return cnt;
}

// Visible (row, key) pairs over rows q0..n-1 of one head.
int64_t pairs_global(int64_t n, int64_t q0) { return (n * (n + 1) - q0 * (q0 + 1)) / 2; }

int64_t pairs_local(int64_t n, int64_t q0, int64_t s, int64_t w) {
  // row i sees min(i + 1, s + w) keys
  const int64_t a = s + w;
  int64_t tot = 0;
  const int64_t lo_end = std::min(n, a);  // rows i < lo_end see i + 1 keys
  if (lo_end > q0) tot += (lo_end * (lo_end + 1) - q0 * (q0 + 1)) / 2;
  const int64_t hi_begin = std::max(q0, a);
  if (n > hi_begin) tot += (n - hi_begin) * a;
  return tot;
}

int64_t pairs_retrieval(int64_t n, int64_t q0, const int32_t* r, int64_t cnt) {
  int64_t tot = 0;
  for (int64_t k = 0; k < cnt; ++k) tot += n - std::max<int64_t>(r[k], q0);
  return tot;
}

// Keys the decode row n - 1 sees: count and slot ranges (at most 3).
struct SlotRange { int64_t lo, hi; };

int decode_ranges(int kind, int64_t sink, int64_t window, int64_t n, const Seg* segs, int nseg,
                  int64_t P, SlotRange out[4]) {
  int cnt = 0;
  int64_t slot_base = 0;
  for (int s = 0; s < nseg; ++s) {
    const Seg& sg = segs[s];
    if (sg.pos0 < 0 || kind == SEGPAGED_GLOBAL || kind == SEGPAGED_DENSE) {
      out[cnt++] = {slot_base, slot_base + sg.len};
    } else {
      // LOCAL: positions [pos0, pos0+len) intersected with [0, sink) U [n - window, n)
      int64_t alo = std::max<int64_t>(sg.pos0, 0), ahi = std::min(sg.pos0 + sg.len, sink);
      int64_t blo = std::max(sg.pos0, n - window), bhi = sg.pos0 + sg.len;
      const bool a_ok = ahi > alo, b_ok = bhi > blo;
      if (a_ok && b_ok && blo <= ahi) {
        alo = std::min(alo, blo);
        ahi = std::max(ahi, bhi);
        out[cnt++] = {slot_base + alo - sg.pos0, slot_base + ahi - sg.pos0};
      } else {
        if (a_ok) out[cnt++] = {slot_base + alo - sg.pos0, slot_base + ahi - sg.pos0};
        if (b_ok) out[cnt++] = {slot_base + blo - sg.pos0, slot_base + bhi - sg.pos0};
      }
    }
    slot_base += ceil_div(sg.len, P) * P;
  }
  return cnt;
}

// Keys query row i of a unit sees (the fewest of a tile's rows: its first).
int64_t row_keys(int kind, int64_t sink, int64_t window, int64_t i, const int32_t* retr,
                 int64_t retr_len) {
  if (kind == SEGPAGED_GLOBAL) return i + 1;
  if (kind == SEGPAGED_LOCAL) return std::min(i + 1, sink + window);
  return std::upper_bound(retr, retr + retr_len, (int32_t)i) - retr;
}

// KV blocks a prefill tile visits (cost model for heaviest-first ordering).
int64_t tile_cost(int kind, int64_t sink, int64_t window, int64_t r0, int64_t r1,
                  const Seg* segs, int nseg, const int32_t* retr) {
  int64_t blocks = 0;
  for (int s = 0; s < nseg; ++s) {
    const Seg& sg = segs[s];
    if (sg.pos0 < 0) {  // gathered
      const int64_t c = std::upper_bound(retr, retr + sg.len, (int32_t)(r1 - 1)) - retr;
      blocks += ceil_div(c, kBlockN);
      continue;
    }
    const int64_t end = std::min(sg.pos0 + sg.len, r1);
    if (kind == SEGPAGED_LOCAL) {
      const int64_t a_hi = std::min(end, sink);
      if (a_hi > sg.pos0) blocks += ceil_div(a_hi - sg.pos0, kBlockN);
      const int64_t b_lo = std::max(sg.pos0, std::max(sink, r0 - window + 1));
      if (end > b_lo) blocks += ceil_div(end - b_lo, kBlockN) + 1;
    } else if (end > sg.pos0) {
      blocks += ceil_div(end - sg.pos0, kBlockN);
    }
  }
  return blocks;
}

// Sequence rows from lengths and first query positions (dense K/V rows and Q
// rows are packed in sequence order).
void write_seq_rows(segpaged_plan* pl, const int32_t* n, const int32_t* q0) {
  int64_t kvo = 0, qo = 0;
  for (int64_t b = 0; b < pl->B; ++b) {
    int32_t* r = &pl->buf[pl->off_seqs + kSeqInts * b];
    r[S_N] = n[b]; r[S_Q0] = q0[b];
    r[S_KVOFF] = (int32_t)kvo; r[S_QOFF] = (int32_t)qo;
    kvo += n[b];
    qo += n[b] - q0[b];
  }
  pl->kv_rows = kvo;
  pl->q_rows = qo;
}

// The per-head varlen work lists of the kernels [runtime explainer, section 4],
// derived from the unit records of the image alone: per layer, the decode items
// (slot ranges of the keys row N-1 sees, cut into <= split keys) with each unit's
// item range, and the prefill tiles heaviest-first; plus the per-layer work
// counts (pages excepted).
struct WorkLists {
  std::vector<int32_t> decunits, dec, pre;
  std::vector<LayerRange> ranges;
  std::vector<segpaged_stats> stats;
  int64_t n_dec() const { return (int64_t)dec.size() / kDecItemInts; }
  int64_t n_pre() const { return (int64_t)pre.size() / kPreItemInts; }
};

void make_work_lists(const segpaged_plan* pl, const int32_t* unit_recs, WorkLists& wl) {
  const int32_t* t = pl->buf.data();
  const int64_t B = pl->B, L = pl->L, Hkv = pl->Hkv, P = pl->P, U = pl->num_units;
  const int64_t split = pl->split, BQ = kPrefillRows / pl->G;
  wl.decunits.assign(kDecUnitInts * U, 0);
  wl.dec.clear();
  wl.pre.clear();
  wl.ranges.assign(L, LayerRange{});
  wl.stats.assign(L, segpaged_stats{});
  for (int64_t l = 0; l < L; ++l) {
    LayerRange& lr = wl.ranges[l];
    segpaged_stats& st = wl.stats[l];
    lr.dec_b = wl.n_dec();
    lr.pre_b = wl.n_pre();
    lr.max_unit_items = 0;
    struct PreTile { int64_t cost, unit, r0; bool precise; };
    std::vector<PreTile> tiles;
    for (int64_t u = l * B * Hkv; u < (l + 1) * B * Hkv; ++u) {
      const int32_t* r = unit_recs + kUnitInts * u;
      const int eff = r[U_KIND];
      const int64_t n = r[U_N], q0 = r[U_Q0], sink = r[U_SINK], win = r[U_WIN];
      const int ns = r[U_NSEG];
      Seg sg[2] = {{0, 0}, {0, 0}};
      for (int k = 0; k < ns; ++k) sg[k] = {r[U_S0POS + 2 * k], r[U_S0LEN + 2 * k]};
      const int32_t* rpos = r[U_RETROFF] >= 0 ? t + pl->off_retr + r[U_RETROFF] : nullptr;
      const int64_t rl = rpos && ns > 0 ? sg[0].len : 0;

      st.units += 1;
      st.retained_tokens += r[U_KVLEN];
      st.q_rows += n - q0;
      if (eff == SEGPAGED_GLOBAL) {
        st.prefill_pairs += pairs_global(n, q0);
      } else if (eff == SEGPAGED_LOCAL) {
        st.prefill_pairs += pairs_local(n, q0, sink, win);
      } else {
        st.prefill_pairs += pairs_retrieval(n, q0, rpos, rl);
      }

      // decode items: visible slot ranges of row n - 1, cut into <= split keys
      int32_t* du = &wl.decunits[kDecUnitInts * u];
      du[0] = (int32_t)wl.n_dec();
      du[2] = r[U_B] * (int32_t)pl->Hq + r[U_H] * (int32_t)pl->G;
      du[3] = r[U_L];
      auto push_item = [&](int64_t unit, int64_t lo, int64_t hi, int64_t gap) {
        const int32_t rec[kDecItemInts] = {(int32_t)unit, (int32_t)lo, (int32_t)hi, (int32_t)gap,
                                           r[U_B], r[U_L], r[U_H], r[U_PAGEOFF]};
        wl.dec.insert(wl.dec.end(), rec, rec + kDecItemInts);
      };
      SlotRange rr[4];
      const int nr = decode_ranges(eff, sink, win, n, sg, ns, P, rr);
      for (int k = 0; k < nr; ++k) st.decode_tokens += rr[k].hi - rr[k].lo;
      int k0 = 0;
      if (nr == 2 && rr[1].lo == ceil_div(rr[0].hi, P) * P && rr[0].hi < rr[1].lo &&
          rr[0].hi - rr[0].lo <= split) {
        // a short first range (a sink) and a range starting on the next page: one
        // item covers both, the zero tail of the first range's last page is a gap
        const int64_t hi0 = std::min(rr[1].lo + split, rr[1].hi);
        push_item(u, rr[0].lo, hi0, rr[0].hi);
        rr[1].lo = hi0;
        k0 = 1;
      }
      for (int k = k0; k < nr; ++k) {
        for (int64_t lo = rr[k].lo; lo < rr[k].hi; lo += split) {
          push_item(u, lo, std::min(lo + split, rr[k].hi), 0);
        }
      }
      du[1] = (int32_t)wl.n_dec();
      lr.max_unit_items = std::max<int64_t>(lr.max_unit_items, du[1] - du[0]);

      // prefill tiles
      for (int64_t r0 = q0; r0 < n; r0 += BQ) {
        const int64_t r1 = std::min(n, r0 + BQ);
        // a row with few keys carries the rounding of each softmax weight into O
        // almost undiluted: such tiles run the precise path
        const bool precise = row_keys(eff, sink, win, r0, rpos, rl) < kPreciseKeys;
        tiles.push_back({tile_cost(eff, sink, win, r0, r1, sg, ns, rpos), u, r0, precise});
      }
    }
    std::stable_sort(tiles.begin(), tiles.end(),
                     [](const PreTile& a, const PreTile& b) { return a.cost > b.cost; });
    for (const PreTile& tl : tiles) {
      wl.pre.push_back((int32_t)tl.unit);
      wl.pre.push_back((int32_t)tl.r0 | (tl.precise ? kPrecise : 0));
    }
    lr.dec_e = wl.n_dec();
    lr.pre_e = wl.n_pre();
    st.decode_items = lr.dec_e - lr.dec_b;
    st.prefill_items = lr.pre_e - lr.pre_b;
  }
}

// Work lists into the image (unused capacity zeroed) and the plan's ranges and counts.
void store_work_lists(segpaged_plan* pl, const WorkLists& wl) {
  std::vector<int32_t>& t = pl->buf;
  std::copy(wl.decunits.begin(), wl.decunits.end(), t.begin() + pl->off_decunits);
  std::copy(wl.dec.begin(), wl.dec.end(), t.begin() + pl->off_dec);
  std::fill(t.begin() + pl->off_dec + wl.dec.size(),
            t.begin() + pl->off_dec + kDecItemInts * pl->dec_cap, 0);
  std::copy(wl.pre.begin(), wl.pre.end(), t.begin() + pl->off_pre);
  std::fill(t.begin() + pl->off_pre + wl.pre.size(),
            t.begin() + pl->off_pre + kPreItemInts * pl->pre_cap, 0);
  pl->n_dec = wl.n_dec();
  pl->n_pre = wl.n_pre();
  pl->max_unit_items = 0;
  segpaged_stats& tot = pl->total;
  tot = segpaged_stats{};
  for (int64_t l = 0; l < pl->L; ++l) {
    LayerRange& lr = pl->layers[l];
    lr.dec_b = wl.ranges[l].dec_b; lr.dec_e = wl.ranges[l].dec_e;
    lr.pre_b = wl.ranges[l].pre_b; lr.pre_e = wl.ranges[l].pre_e;
    lr.max_unit_items = wl.ranges[l].max_unit_items;
    pl->max_unit_items = std::max(pl->max_unit_items, lr.max_unit_items);
    const int64_t pages = pl->stats[l].pages;
    segpaged_stats& st = pl->stats[l];
    st = wl.stats[l];
    st.pages = pages;
    tot.units += st.units; tot.pages += st.pages; tot.retained_tokens += st.retained_tokens;
    tot.decode_tokens += st.decode_tokens; tot.prefill_pairs += st.prefill_pairs;
    tot.q_rows += st.q_rows; tot.decode_items += st.decode_items;
    tot.prefill_items += st.prefill_items;
  }
}

}  // namespace

extern "C" {

SEGPAGED_API int segpaged_plan_create(const segpaged_spec* spec, segpaged_plan** plan_out,
                                      segpaged_sizes* sizes) {
  if (plan_out) *plan_out = nullptr;
  if (!spec || !plan_out) return SEGPAGED_EINVAL;
  const segpaged_spec& s = *spec;
  if (s.num_seqs < 1 || s.num_layers < 1 || s.num_kv_heads < 1 || s.num_q_heads < 1)
    return SEGPAGED_EINVAL;
  if (s.num_q_heads % s.num_kv_heads != 0) return SEGPAGED_EINVAL;
  if (s.head_dim <= 0 || s.page_size <= 0) return SEGPAGED_EINVAL;
  if (s.head_dim != 64 && s.head_dim != 128) return SEGPAGED_EUNSUPPORTED;
  if (s.page_size != 16 && s.page_size != 32 && s.page_size != 64 && s.page_size != 128)
    return SEGPAGED_EUNSUPPORTED;
  const int32_t G = s.num_q_heads / s.num_kv_heads;
  if (G > kMaxGroup) return SEGPAGED_EUNSUPPORTED;
  if (!s.seq_len || !s.first_query_pos || !s.kind || !s.sink || !s.window) return SEGPAGED_EINVAL;
  if (s.decode_split_tokens < 0 || s.decode_split_tokens % 64 != 0) return SEGPAGED_EINVAL;
  if (s.capacity_pages < 0 || s.free_list_len < 0) return SEGPAGED_EINVAL;
  if (s.append_capacity < 0 || s.append_chunk < 0) return SEGPAGED_EINVAL;
  const int64_t chunk = std::max<int64_t>(s.append_chunk, 1);

  const int64_t B = s.num_seqs, L = s.num_layers, Hkv = s.num_kv_heads, P = s.page_size;
  const int64_t U = L * B * Hkv;
  const int64_t kI32Max = std::numeric_limits<int32_t>::max();
  if (U > kI32Max / kUnitInts) return SEGPAGED_EINVAL;

  int64_t kv_rows = 0, q_rows = 0;
  for (int64_t b = 0; b < B; ++b) {
    const int64_t n = s.seq_len[b], q0 = s.first_query_pos[b];
    if (n < 0 || q0 < 0 || q0 > std::max<int64_t>(n - 1, 0)) return SEGPAGED_EINVAL;
    kv_rows += n;
    q_rows += n - q0;
  }
  if (kv_rows > kI32Max || q_rows > kI32Max) return SEGPAGED_EINVAL;
  if (s.append_capacity > 0) {
    // growth: every sequence holds the rows of at most one chunk
    if (kv_rows + (int64_t)s.append_capacity * B > kI32Max) return SEGPAGED_EINVAL;
    for (int64_t b = 0; b < B; ++b)
      if ((int64_t)s.seq_len[b] - s.first_query_pos[b] > chunk) return SEGPAGED_EINVAL;
  }

  bool any_retr = false;
  for (int64_t i = 0; i < L * Hkv; ++i) {
    const int k = s.kind[i];
    if (k < SEGPAGED_GLOBAL || k > SEGPAGED_DENSE) return SEGPAGED_EINVAL;
    if (k == SEGPAGED_LOCAL && (s.sink[i] < 0 || s.window[i] < 1)) return SEGPAGED_EINVAL;
    if (k == SEGPAGED_RETRIEVAL) any_retr = true;
  }
  if (any_retr && (!s.retr_offsets || !s.retr_pos)) return SEGPAGED_EINVAL;
  if (s.retr_offsets) {
    if (s.retr_offsets[0] != 0) return SEGPAGED_EINVAL;
    for (int64_t l = 0; l < L; ++l)
      for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < Hkv; ++h) {
          const int64_t u = (l * B + b) * Hkv + h;
          const int64_t o0 = s.retr_offsets[u], o1 = s.retr_offsets[u + 1];
          if (o1 < o0) return SEGPAGED_EINVAL;
          if (s.kind[l * Hkv + h] != SEGPAGED_RETRIEVAL) {
            if (o1 != o0) return SEGPAGED_EINVAL;
            continue;
          }
          if (o1 - o0 > kI32Max) return SEGPAGED_EINVAL;
          for (int64_t k = o0; k < o1; ++k) {
            const int32_t p = s.retr_pos[k];
            if (p < 0 || p >= s.seq_len[b]) return SEGPAGED_EINVAL;
            if (k > o0 && p <= s.retr_pos[k - 1]) return SEGPAGED_EINVAL;
          }
        }
  }

  // document groups: members share doc_len leading tokens (same for all members)
  const bool share = s.doc_group != nullptr;
  if (share != (s.doc_len != nullptr)) return SEGPAGED_EINVAL;
  std::vector<int64_t> group_len;  // per group id: its doc_len, -1 = not seen
  if (share) {
    if (s.append_capacity > 0) return SEGPAGED_EUNSUPPORTED;  // appends could write shared pages
    for (int64_t b = 0; b < B; ++b) {
      const int64_t g = s.doc_group[b], c = s.doc_len[b];
      if (g < -1 || g >= B || c < 0 || c > s.seq_len[b]) return SEGPAGED_EINVAL;
      if (g < 0) {
        if (c != 0) return SEGPAGED_EINVAL;
        continue;
      }
      if ((int64_t)group_len.size() <= g) group_len.resize(g + 1, -1);
      if (group_len[g] >= 0 && group_len[g] != c) return SEGPAGED_EINVAL;
      group_len[g] = c;
    }
  }

  segpaged_plan* pl = new (std::nothrow) segpaged_plan();
  if (!pl) return SEGPAGED_ENOSPACE;
  pl->B = (int32_t)B; pl->L = (int32_t)L; pl->Hq = s.num_q_heads; pl->Hkv = (int32_t)Hkv;
  pl->D = s.head_dim; pl->P = (int32_t)P; pl->G = G;
  pl->log2P = 0;
  while ((1 << pl->log2P) < P) ++pl->log2P;
  pl->num_units = U; pl->q_rows = q_rows; pl->kv_rows = kv_rows;
  pl->append_cap = s.append_capacity;
  pl->append_chunk = chunk;
  if (pl->append_cap > 0) {
    pl->n_max.resize(B);
    for (int64_t b = 0; b < B; ++b) pl->n_max[b] = (int64_t)s.seq_len[b] + pl->append_cap;
  }

  // ---- pass 1: segments per unit, reserved pages, retrieval totals
  // Append mode keeps room to grow: a global head reserves the pages of its
  // length limit; a local head always has two segments, the sink (its pages
  // reserved) and the window, whose pages form a ring of
  // ceil((W + chunk - 1)/P) + 1, enough for the windows of a chunk's rows.
  const bool grow = pl->append_cap > 0;
  std::vector<Seg> segs(U * 2);
  std::vector<int> nseg(U);
  std::vector<int64_t> res_pages(U);
  int64_t num_pages = 0, num_retr = 0;
  for (int64_t l = 0; l < L; ++l)
    for (int64_t b = 0; b < B; ++b)
      for (int64_t h = 0; h < Hkv; ++h) {
        const int64_t u = (l * B + b) * Hkv + h, c = l * Hkv + h;
        const int64_t rl = s.retr_offsets ? s.retr_offsets[u + 1] - s.retr_offsets[u] : 0;
        const int64_t n = s.seq_len[b];
        const int kind = s.kind[c];
        if (grow && kind == SEGPAGED_LOCAL) {
          const int64_t a = std::min<int64_t>(s.sink[c], n);
          const int64_t w0 = std::max<int64_t>(s.sink[c], s.first_query_pos[b] - s.window[c] + 1);
          segs[2 * u] = {0, a};
          segs[2 * u + 1] = {w0, std::max<int64_t>(n - w0, 0)};
          nseg[u] = 2;
          res_pages[u] = ceil_div(s.sink[c], P) + ceil_div(s.window[c] + chunk - 1, P) + 1;
        } else if (grow && kind != SEGPAGED_RETRIEVAL) {
          segs[2 * u] = {0, n};
          nseg[u] = 1;
          res_pages[u] = ceil_div(n + pl->append_cap, P);
        } else {
          nseg[u] = retained(kind, s.sink[c], s.window[c], n, s.first_query_pos[b], rl,
                             &segs[2 * u]);
          res_pages[u] = 0;
          for (int k = 0; k < nseg[u]; ++k) res_pages[u] += ceil_div(segs[2 * u + k].len, P);
        }
        for (int k = 0; k < nseg[u]; ++k)
          if (segs[2 * u + k].len > kI32Max / 2) { delete pl; return SEGPAGED_EINVAL; }
        num_pages += res_pages[u];
        if (kind == SEGPAGED_RETRIEVAL) num_retr += rl;
      }
  if (num_pages > kI32Max || num_retr > kI32Max) { delete pl; return SEGPAGED_EINVAL; }

  // Distinct pages: every page slot owns a page of its own, except that a page of a
  // document group member whose positions all lie in the group's shared prefix is
  // the same page for every member holding the same positions (same first position
  // and occupancy) in the same layer and KV head. slot_page: slot -> distinct page
  // index (ids in order of first use); build: the slots that own their page.
  const int64_t num_slots = num_pages;
  std::vector<int32_t> slot_page(num_slots);
  std::vector<int32_t> build;
  build.reserve(num_slots);
  {
    std::map<std::tuple<int64_t, int64_t, int64_t, int64_t, int64_t>, int32_t> shared;
    int64_t slot = 0, distinct = 0;
    for (int64_t u = 0; u < U; ++u) {
      const int64_t l = u / (B * Hkv), b = (u / Hkv) % B, h = u % Hkv;
      const int64_t g = share ? s.doc_group[b] : -1;
      const int64_t c = g >= 0 ? s.doc_len[b] : 0;
      int64_t left = res_pages[u];
      for (int k = 0; k < nseg[u]; ++k) {
        const Seg& sg = segs[2 * u + k];
        for (int64_t t = 0; t < ceil_div(sg.len, P) && left > 0; ++t, --left, ++slot) {
          const int64_t first = sg.pos0 + t * P, occ = std::min(P, sg.len - t * P);
          if (g >= 0 && sg.pos0 >= 0 && first + occ <= c) {
            auto key = std::make_tuple(l, h, g, first, occ);
            auto it = shared.find(key);
            if (it != shared.end()) {
              slot_page[slot] = it->second;
              continue;
            }
            shared.emplace(key, (int32_t)distinct);
          }
          slot_page[slot] = (int32_t)distinct++;
          build.push_back((int32_t)slot);
        }
      }
      for (; left > 0; --left, ++slot) {  // reserved pages past the segments (growth)
        slot_page[slot] = (int32_t)distinct++;
        build.push_back((int32_t)slot);
      }
    }
    num_pages = distinct;
  }

  int64_t capacity = s.capacity_pages ? s.capacity_pages : num_pages;
  if (capacity < num_pages) { delete pl; return SEGPAGED_ENOSPACE; }
  if (capacity > kI32Max) { delete pl; return SEGPAGED_EINVAL; }
  if (s.free_list) {
    if (s.free_list_len < num_pages) { delete pl; return SEGPAGED_ENOSPACE; }
    std::vector<uint8_t> seen(capacity, 0);
    for (int64_t i = 0; i < num_pages; ++i) {
      const int32_t id = s.free_list[i];
      if (id < 0 || id >= capacity || seen[id]) { delete pl; return SEGPAGED_EINVAL; }
      seen[id] = 1;
    }
  }
  pl->num_pages = num_pages;
  pl->num_slots = num_slots;
  pl->pool_pages = capacity;
  pl->num_retr = num_retr;

  // ---- table layout
  pl->off_seqs = kHeaderInts;
  pl->off_units = pl->off_seqs + kSeqInts * B;
  pl->off_pages = pl->off_units + kUnitInts * U;
  pl->off_retr = pl->off_pages + num_slots;
  pl->table_len = pl->off_retr + num_retr;

  // decode split: automatic = enough items to fill the GPU several times over
  int64_t dec_tokens_all = 0;
  for (int64_t u = 0; u < U; ++u) {
    const int64_t l = u / (B * Hkv), b = (u / Hkv) % B, h = u % Hkv, c = l * Hkv + h;
    SlotRange rr[4];
    const int nr = decode_ranges(s.kind[c], s.sink[c], s.window[c], s.seq_len[b], &segs[2 * u],
                                 nseg[u], P, rr);
    for (int k = 0; k < nr; ++k) dec_tokens_all += rr[k].hi - rr[k].lo;
  }
  int64_t split = s.decode_split_tokens;
  if (split == 0) {  // long items amortise each item's set-up; keep enough of them
    split = 4096;
    while (split > 64 && dec_tokens_all / split < 4096) split /= 2;
  }
  pl->split = (int32_t)split;

  std::vector<int32_t>& t = pl->buf;
  pl->off_bld = pl->table_len;
  t.assign(pl->off_bld + num_pages, 0);
  std::copy(build.begin(), build.end(), t.begin() + pl->off_bld);
  pl->off_decunits = pl->off_bld + num_pages;

  // header and sequences
  const int32_t hdr[kHeaderInts] = {kMagic, kVersion, (int32_t)B, (int32_t)L, s.num_q_heads,
                                    (int32_t)Hkv, s.head_dim, (int32_t)P, (int32_t)U,
                                    (int32_t)num_slots, (int32_t)num_retr, (int32_t)pl->off_seqs,
                                    (int32_t)pl->off_units, (int32_t)pl->off_pages,
                                    (int32_t)pl->off_retr, (int32_t)pl->table_len};
  std::memcpy(t.data(), hdr, sizeof(hdr));
  write_seq_rows(pl, s.seq_len, s.first_query_pos);

  // ---- pass 2: unit records, page ids, retrieval positions
  pl->layers.resize(L);
  pl->stats.assign(L, segpaged_stats{});
  int64_t page_cursor = 0, retr_cursor = 0;
  int64_t dec_cap = 0;
  for (int64_t l = 0; l < L; ++l) {
    LayerRange& lr = pl->layers[l];
    lr.unit_b = l * B * Hkv; lr.unit_e = (l + 1) * B * Hkv;
    lr.page_b = page_cursor; lr.retr_b = retr_cursor;
    for (int64_t b = 0; b < B; ++b)
      for (int64_t h = 0; h < Hkv; ++h) {
        const int64_t u = (l * B + b) * Hkv + h, c = l * Hkv + h;
        const int kind = s.kind[c];
        const int eff = kind == SEGPAGED_DENSE ? SEGPAGED_GLOBAL : kind;
        int32_t* r = &t[pl->off_units + kUnitInts * u];
        r[U_KIND] = eff; r[U_B] = (int32_t)b; r[U_L] = (int32_t)l; r[U_H] = (int32_t)h;
        r[U_N] = s.seq_len[b]; r[U_Q0] = s.first_query_pos[b];
        r[U_SINK] = s.sink[c]; r[U_WIN] = s.window[c];
        r[U_NSEG] = nseg[u];
        r[U_PAGEOFF] = (int32_t)page_cursor;
        r[U_RETROFF] = -1;
        if (kind == SEGPAGED_RETRIEVAL) {
          r[U_RETROFF] = (int32_t)retr_cursor;
          const int64_t rl = s.retr_offsets[u + 1] - s.retr_offsets[u];
          const int32_t* rpos = s.retr_pos + s.retr_offsets[u];
          std::copy(rpos, rpos + rl, t.begin() + pl->off_retr + retr_cursor);
          retr_cursor += rl;
        }
        int64_t kv_len = 0;
        for (int k = 0; k < nseg[u]; ++k) {
          const Seg& sg = segs[2 * u + k];
          r[U_S0POS + 2 * k] = (int32_t)sg.pos0;
          r[U_S0LEN + 2 * k] = (int32_t)sg.len;
          kv_len += sg.len;
        }
        r[U_KVLEN] = (int32_t)kv_len;
        for (int64_t p = 0; p < res_pages[u]; ++p, ++page_cursor) {
          const int32_t d = slot_page[page_cursor];
          t[pl->off_pages + page_cursor] = s.free_list ? s.free_list[d] : d;
        }
        if (grow) {  // most decode items this unit can ever need
          if (eff == SEGPAGED_LOCAL)
            dec_cap += ceil_div(s.sink[c], split) + ceil_div(s.window[c], split) + 2;
          else
            dec_cap += ceil_div(segs[2 * u].len + pl->append_cap, split) + 1;
        }
      }
    lr.page_e = page_cursor; lr.retr_e = retr_cursor;
    // the build list is in slot order, so a layer's owners are contiguous
    lr.bld_b = std::lower_bound(build.begin(), build.end(), (int32_t)lr.page_b) - build.begin();
    lr.bld_e = std::lower_bound(build.begin(), build.end(), (int32_t)lr.page_e) - build.begin();
    pl->stats[l].pages = lr.bld_e - lr.bld_b;
  }

  // ---- work lists after the table: decode units, decode items, prefill items,
  // then the prefill work counters (and, in append mode, the append list)
  WorkLists wl;
  make_work_lists(pl, t.data() + pl->off_units, wl);
  pl->dec_cap = grow ? std::max<int64_t>(dec_cap, wl.n_dec()) : wl.n_dec();
  pl->pre_cap = grow ? std::max<int64_t>(U * ceil_div(chunk, kPrefillRows / G), wl.n_pre())
                     : wl.n_pre();
  pl->off_dec = pl->off_decunits + kDecUnitInts * U;
  pl->off_pre = pl->off_dec + kDecItemInts * pl->dec_cap;
  // counter lines 16-byte aligned in the image (64-bit atomics)
  pl->off_ctr = (pl->off_pre + kPreItemInts * pl->pre_cap + 3) / 4 * 4;
  pl->off_app = pl->off_ctr + (int64_t)kCtrInts * (L + 1);
  pl->total_ints = pl->off_app + (grow ? 2 * B + 1 : 0);
  if (pl->total_ints > kI32Max) { delete pl; return SEGPAGED_EINVAL; }
  t.resize(pl->total_ints, 0);  // work counters and append list start at zero
  store_work_lists(pl, wl);
  pl->pages_dirty.assign(L, 0);
  pl->pre_gen.reset(new (std::nothrow) std::atomic<uint32_t>[L + 1]);
  if (!pl->pre_gen) { delete pl; return SEGPAGED_ENOSPACE; }
  for (int64_t i = 0; i <= L; ++i) pl->pre_gen[i].store(0);
  *plan_out = pl;
  if (sizes) segpaged_plan_sizes(pl, sizes);
  return SEGPAGED_OK;
}

SEGPAGED_API void segpaged_plan_destroy(segpaged_plan* plan) { delete plan; }

SEGPAGED_API int segpaged_plan_sizes(const segpaged_plan* pl, segpaged_sizes* z) {
  if (!pl || !z) return SEGPAGED_EINVAL;
  z->num_pages = pl->num_pages;
  z->pool_pages = pl->pool_pages;
  z->pool_bytes = pl->pool_pages * (int64_t)pl->P * pl->D * 2;
  z->table_int32s = pl->total_ints;
  z->table_len = pl->table_len;
  z->num_units = pl->num_units;
  z->q_rows = pl->q_rows;
  z->kv_rows = pl->kv_rows;
  z->decode_items = pl->n_dec;
  z->prefill_items = pl->n_pre;
  z->decode_workspace_bytes = (pl->dec_cap + kDecTailRecords) * (int64_t)pl->G * (pl->D + 4) * 4;
  z->prefill_workspace_bytes = 0;
  {  // scores, masses and block partials of segpaged_select_topp at the largest lengths
    int64_t t_max = 0, n_max = 0;
    for (int64_t b = 0; b < pl->B; ++b) {
      const int64_t n = pl->append_cap > 0 ? pl->n_max[b]
                                           : pl->buf[pl->off_seqs + kSeqInts * b + S_N];
      t_max += n;
      n_max = std::max(n_max, n);
    }
    const int64_t nblk = std::max<int64_t>(1, (n_max + 255) / 256);
    const int64_t nchunk = std::max<int64_t>(1, (n_max + kSelChunk - 1) / kSelChunk);
    const int64_t floats = pl->Hkv * t_max * (pl->G + 1) + pl->Hkv * (int64_t)pl->B * nblk * pl->G * 2;
    // then, 16-byte aligned, the per-chunk histograms: 64-bit mass sums (256 bins and
    // the chunk total) and 32-bit counts
    z->select_workspace_bytes = (4 * floats + 15) / 16 * 16 +
                                pl->Hkv * (int64_t)pl->B * nchunk * (257 * 8 + 256 * 4);
  }
  return SEGPAGED_OK;
}

SEGPAGED_API int segpaged_plan_append(segpaged_plan* pl, const int32_t* n_new) {
  if (!pl || !n_new) return SEGPAGED_EINVAL;
  if (pl->append_cap <= 0) return SEGPAGED_ESTATE;
  std::vector<int32_t>& t = pl->buf;
  const int64_t B = pl->B, P = pl->P;
  std::vector<int32_t> n_old(B), n_now(B), q0(B);
  for (int64_t b = 0; b < B; ++b) {
    n_old[b] = t[pl->off_seqs + kSeqInts * b + S_N];
    if (n_new[b] < 0 || n_new[b] > pl->append_chunk) return SEGPAGED_EINVAL;
    if (n_old[b] + (int64_t)n_new[b] > pl->n_max[b]) return SEGPAGED_ENOSPACE;
    n_now[b] = n_old[b] + n_new[b];
    q0[b] = std::max(n_now[b] - std::max(n_new[b], 1), 0);
  }
  // New unit records and ring moves in temporaries: the plan changes only once the
  // work lists are known to fit. A local head's window keeps positions [p0, N):
  // when that outgrows its ring of pages, p0 moves on by a page and the page that
  // held the oldest positions becomes the last one.
  const int64_t U = pl->num_units;
  std::vector<int32_t> units(t.begin() + pl->off_units, t.begin() + pl->off_units + kUnitInts * U);
  std::vector<int64_t> moves(U, 0);
  for (int64_t u = 0; u < U; ++u) {
    int32_t* r = &units[kUnitInts * u];
    const int32_t n = n_now[r[U_B]];
    r[U_N] = n;
    r[U_Q0] = q0[r[U_B]];
    if (r[U_KIND] == SEGPAGED_GLOBAL) {
      r[U_S0LEN] = n;
      r[U_KVLEN] = n;
    } else if (r[U_KIND] == SEGPAGED_LOCAL) {
      const int64_t sink = r[U_SINK], win = r[U_WIN];
      const int64_t len0 = std::min<int64_t>(sink, n);
      const int64_t ring_pages = ceil_div(win + pl->append_chunk - 1, P) + 1;
      int64_t p0 = r[U_S1POS];
      int64_t len1 = std::max<int64_t>(n - p0, 0);
      if (len1 > ring_pages * P) {
        const int64_t k = ceil_div(len1 - ring_pages * P, P);
        p0 += k * P;
        len1 -= k * P;
        moves[u] = k;
      }
      r[U_S0LEN] = (int32_t)len0;
      r[U_S1POS] = (int32_t)p0;
      r[U_S1LEN] = (int32_t)len1;
      r[U_KVLEN] = (int32_t)(len0 + len1);
    }
  }
  WorkLists wl;
  make_work_lists(pl, units.data(), wl);
  if (wl.n_dec() > pl->dec_cap || wl.n_pre() > pl->pre_cap) return SEGPAGED_ENOSPACE;

  // commit: sequence rows, the append list (where each sequence's new K/V rows
  // start, and their positions), unit records, rotated rings, work lists
  write_seq_rows(pl, n_now.data(), q0.data());
  int32_t* app = &t[pl->off_app];
  int64_t row = 0;
  for (int64_t b = 0; b < B; ++b) {
    app[b] = (int32_t)row;
    app[B + 1 + b] = n_old[b];
    row += n_new[b];
  }
  app[B] = (int32_t)row;
  std::copy(units.begin(), units.end(), t.begin() + pl->off_units);
  for (int64_t u = 0; u < U; ++u) {
    if (moves[u] == 0) continue;
    const int32_t* r = &units[kUnitInts * u];
    const int64_t ring_pages = ceil_div(r[U_WIN] + pl->append_chunk - 1, P) + 1;
    int32_t* ring = &t[pl->off_pages + r[U_PAGEOFF] + ceil_div(r[U_SINK], P)];
    std::rotate(ring, ring + moves[u] % ring_pages, ring + ring_pages);
    pl->pages_dirty[r[U_L]] = 1;
  }
  store_work_lists(pl, wl);
  pl->app_upload = true;
  return SEGPAGED_OK;
}

SEGPAGED_API int segpaged_plan_table_host(const segpaged_plan* pl, int32_t* out, int64_t n) {
  if (!pl || !out) return SEGPAGED_EINVAL;
  if (n < pl->total_ints) return SEGPAGED_ENOSPACE;
  std::memcpy(out, pl->buf.data(), sizeof(int32_t) * pl->total_ints);
  return SEGPAGED_OK;
}

SEGPAGED_API int segpaged_plan_stats(const segpaged_plan* pl, int32_t layer, segpaged_stats* st) {
  if (!pl || !st) return SEGPAGED_EINVAL;
  if (layer < -1 || layer >= pl->L) return SEGPAGED_ESTATE;
  *st = layer < 0 ? pl->total : pl->stats[layer];
  return SEGPAGED_OK;
}

SEGPAGED_API const char* segpaged_status_str(int status) {
  switch (status) {
    case SEGPAGED_OK: return "ok";
    case SEGPAGED_EINVAL: return "invalid argument";
    case SEGPAGED_EUNSUPPORTED: return "unsupported shape";
    case SEGPAGED_ENOSPACE: return "insufficient space";
    case SEGPAGED_EHIP: return "HIP runtime error";
    case SEGPAGED_ESTATE: return "call does not fit the plan";
    default: return "unknown status";
  }
}

SEGPAGED_API int segpaged_version(void) { return 100; }

}  // extern "C"
