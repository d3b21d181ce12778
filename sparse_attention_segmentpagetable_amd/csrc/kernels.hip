// SegPagedAttention kernels for MI355X (gfx950, wave64, bf16 MFMA) and the C-ABI
// entry points that launch them.
//
//   build_kernel           build_segpaged_cache: dense K/V rows -> per-head pages
//   append_kernel          new tokens' K/V into their slots (growth plans)
//   decode_partial_kernel  split-K decode: one wave per (unit, key range) item part
//   decode_combine_kernel  log-sum-exp merge of the partials of each unit
//   prefill_kernel         GQA flash-style prefill over each head's own pages
//   page_copy_kernel       a layer's pages as one contiguous stream and back (moving
//                          a cache between devices or processes)
//
// Method: SegPagedAttention runtime explainer, section 3 (per-(layer, head,
// segment) page table and pool; local heads keep only sink + recent tokens) and
// section 4 (one fused varlen pass, each head at its own length, no mask).
// Online softmax recurrence: KV-cache guide, section 10.2.
//
// Pool layout (bf16): K page [D/8][P][8] and V page [P/8][D][8]. Every MFMA
// operand a lane needs is then one 16-byte load: 8 consecutive head dims of a
// key (K) or 8 consecutive keys of one head dim (V).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "plan.hpp"

using namespace segpaged;

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// decode partial per (item, query column): D floats of unnormalised output, then
// the running max (log2 units) and the normaliser; padded to keep float4 stores aligned
template <int D>
constexpr int kWsStride = D + 4;

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(uint16_t* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// two fp32 -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// the two bf16 of a packed word as fp32 (exact)
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) {
  return __builtin_bit_cast(float, w & 0xFFFF0000u);
}
// Precise softmax weights: p ~ hi + lo with both terms bf16 (hi = p rounded to
// nearest even, lo = the remainder rounded), so a product with V that takes both
// carries p to ~2^-16 relative instead of bf16's 2^-8.
// Eight weights p[0..7] as packed hi and lo words (element order as pack_bf16x2).
__device__ __forceinline__ void split_bf16x8(const float* p, u32x4& hi, u32x4& lo) {
  hi.x = pack_bf16x2(p[0], p[1]);
  hi.y = pack_bf16x2(p[2], p[3]);
  hi.z = pack_bf16x2(p[4], p[5]);
  hi.w = pack_bf16x2(p[6], p[7]);
  lo.x = pack_bf16x2(p[0] - bf16_lo(hi.x), p[1] - bf16_hi(hi.x));
  lo.y = pack_bf16x2(p[2] - bf16_lo(hi.y), p[3] - bf16_hi(hi.y));
  lo.z = pack_bf16x2(p[4] - bf16_lo(hi.z), p[5] - bf16_hi(hi.z));
  lo.w = pack_bf16x2(p[6] - bf16_lo(hi.w), p[7] - bf16_hi(hi.w));
}

__device__ __forceinline__ float wave_max_xor(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, 64));
}

// ---------------------------------------------------------------------------
// build: one workgroup per distinct page (the table slots of the build list; a
// page that sequences of a document group share is written once, from the slot
// that owns it). Rows are read coalesced into LDS, then written out in the K
// [D/8][P][8] and V [P/8][D][8] page layouts. Tail slots are zero.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void build_kernel(
    const int32_t* __restrict__ tab, int32_t off_seqs, int32_t off_units, int32_t off_pages,
    int32_t off_retr, int32_t off_bld, int32_t unit_b, int32_t unit_e, int32_t bld_b,
    int32_t Hkv, int32_t P, int32_t log2P, const uint16_t* __restrict__ kd,
    const uint16_t* __restrict__ vd, int64_t dense_layer_stride, uint16_t* __restrict__ kp,
    uint16_t* __restrict__ vp) {
  constexpr int KCH = D / 8;        // 16-byte chunks per row
  constexpr int PITCH = D + 8;      // LDS row pitch (elements), breaks bank aliasing
  __shared__ __attribute__((aligned(16))) uint16_t rows[128 * PITCH];

  const int32_t pg = tab[off_bld + bld_b + (int32_t)blockIdx.x];  // page slot in the table
  // owning unit: last unit in [unit_b, unit_e) whose page_off <= pg
  int32_t lo = unit_b, hi = unit_e - 1;
  while (lo < hi) {
    const int32_t mid = (lo + hi + 1) >> 1;
    if (tab[off_units + kUnitInts * mid + U_PAGEOFF] <= pg) lo = mid; else hi = mid - 1;
  }
  const int32_t* ur = tab + off_units + kUnitInts * lo;
  const int32_t b = ur[U_B], l = ur[U_L], h = ur[U_H];
  const int32_t pr = pg - ur[U_PAGEOFF];
  const int32_t np0 = (ur[U_S0LEN] + P - 1) >> log2P;
  const int sg = pr < np0 ? 0 : 1;
  const int32_t t0 = (sg == 0 ? pr : pr - np0) << log2P;  // first segment token of this page
  const int32_t pos0 = ur[U_S0POS + 2 * sg], len = ur[U_S0LEN + 2 * sg];
  const int32_t count = min(P, len - t0);
  const bool gathered = pos0 < 0;
  const int32_t* rpos = tab + off_retr + ur[U_RETROFF] + t0;
  const int64_t kvrow0 = tab[off_seqs + kSeqInts * b + S_KVOFF];
  const int64_t lstride = (int64_t)l * dense_layer_stride;
  const int32_t pid = tab[off_pages + pg];
  uint16_t* kpage = kp + (int64_t)pid * P * D;
  uint16_t* vpage = vp + (int64_t)pid * P * D;
  const int nchunk = P * KCH;

  for (int pass = 0; pass < 2; ++pass) {
    const uint16_t* src = pass == 0 ? kd : vd;
    for (int c = threadIdx.x; c < nchunk; c += 256) {
      const int slot = c / KCH, dc = c % KCH;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (slot < count) {
        const int64_t pos = gathered ? rpos[slot] : pos0 + t0 + slot;
        v = ld16(src + lstride + ((kvrow0 + pos) * Hkv + h) * D + dc * 8);
      }
      st16(&rows[slot * PITCH + dc * 8], v);
    }
    __syncthreads();
    if (pass == 0) {
      for (int c = threadIdx.x; c < nchunk; c += 256) {  // K: chunk (dc, slot)
        const int dc = c >> log2P, slot = c & (P - 1);
        st16(kpage + ((int64_t)dc * P + slot) * 8, ld16(&rows[slot * PITCH + dc * 8]));
      }
    } else {
      for (int c = threadIdx.x; c < nchunk; c += 256) {  // V: chunk (tc, d)
        const int tc = c / D, d = c % D;
        u32x4 v;
        v.x = rows[(8 * tc + 0) * PITCH + d] | ((uint32_t)rows[(8 * tc + 1) * PITCH + d] << 16);
        v.y = rows[(8 * tc + 2) * PITCH + d] | ((uint32_t)rows[(8 * tc + 3) * PITCH + d] << 16);
        v.z = rows[(8 * tc + 4) * PITCH + d] | ((uint32_t)rows[(8 * tc + 5) * PITCH + d] << 16);
        v.w = rows[(8 * tc + 6) * PITCH + d] | ((uint32_t)rows[(8 * tc + 7) * PITCH + d] << 16);
        st16(vpage + ((int64_t)tc * D + d) * 8, v);
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// append: the K/V of tokens added to the sequences since planning go to their
// slots, the layout fixed when K/V is written [runtime explainer, section 5].
// One wave per (layer, new row, KV head). A global head's token at position p
// sits at slot p; a local head's at slot p in the sink, or in the window
// segment, whose positions [p0, N) the plan keeps in a ring of pages; tokens
// already outside it, and retrieval heads (a given index set), store nothing.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void append_kernel(
    const int32_t* __restrict__ tab, int32_t off_units, int32_t off_pages, int32_t off_app,
    int32_t B, int32_t Hkv, int32_t layer0, int32_t nl, int32_t t_new,
    const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vn, int64_t new_layer_stride,
    uint16_t* __restrict__ kp, uint16_t* __restrict__ vp, int32_t P, int32_t log2P) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t idx = (int64_t)blockIdx.x * 4 + wave;
  const int64_t per_layer = (int64_t)t_new * Hkv;
  if (idx >= per_layer * nl) return;
  const int32_t li = (int32_t)(idx / per_layer);
  const int32_t t = (int32_t)((idx % per_layer) / Hkv), h = (int32_t)(idx % Hkv);
  const int32_t l = layer0 + li;
  // sequence b owns new rows [app[b], app[b+1]); its first new position is app[B+1+b]
  const int32_t* app = tab + off_app;
  int32_t b = 0;
  while (b + 1 < B && app[b + 1] <= t) ++b;
  const int32_t p = app[B + 1 + b] + (t - app[b]);
  const int32_t* ur = tab + off_units + kUnitInts * ((l * B + b) * Hkv + h);
  int32_t slot = -1;
  if (ur[U_KIND] == SEGPAGED_GLOBAL) {
    slot = p;
  } else if (ur[U_KIND] == SEGPAGED_LOCAL) {
    if (p < ur[U_SINK]) {
      slot = p;
    } else if (p >= ur[U_S1POS]) {
      slot = (((ur[U_S0LEN] + P - 1) >> log2P) << log2P) + (p - ur[U_S1POS]);
    }
  }
  if (slot < 0) return;
  const int32_t pid = tab[off_pages + ur[U_PAGEOFF] + (slot >> log2P)];
  const int32_t ts = slot & (P - 1);
  const int64_t src = (int64_t)li * new_layer_stride + ((int64_t)t * Hkv + h) * D;
  uint16_t* kpage = kp + (int64_t)pid * P * D;
  uint16_t* vpage = vp + (int64_t)pid * P * D;
  // K page [D/8][P][8]: the token's 16-byte chunks; V page [P/8][D][8]: one
  // element of each dim's 8-slot brick
  if (lane < D / 8) st16(kpage + ((int64_t)lane * P + ts) * 8, ld16(kn + src + lane * 8));
  for (int d = lane; d < D; d += 64)
    vpage[((int64_t)(ts >> 3) * D + d) * 8 + (ts & 7)] = vn[src + d];
}

// How a decode launch deals its items to waves: the first `head` items to `nh`
// consecutive waves each, the others to `nt` each. Partial records follow the
// wave order, so record = wave index.
struct DecParts {
  int32_t head, nh, nt;
  // waves (and records) of the launch's items [0, i)
  __host__ __device__ int32_t waves_before(int32_t i) const {
    return i <= head ? i * nh : head * nh + (i - head) * nt;
  }
};

// ---------------------------------------------------------------------------
// decode, split-K. One wave per part of a work item (unit, slots [lo, hi)), all
// of which the decode row sees: an item's 32-slot steps are dealt to its parts
// (one part unless a launch has too few items to fill the chip, or the item is
// among the last of a launch of several rounds, see DecParts), each writing its
// own partial. Per 32-key step, with
// v_mfma_f32_16x16x32_bf16:
//   S^T[16 keys][16 cols] = K[keys][D] . Q^T[D][cols]   (cols = the G query heads)
//   O^T[16 dims][16 cols] += V^T[dims][32 keys] . P^T[32 keys][cols]
// The key order inside an S^T tile is permuted so that the 8 keys a lane holds
// after the softmax are 8 consecutive slots: exactly one V brick.
// Writes (unnormalised O^T, running max in log2 units, normaliser) per column.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void decode_partial_kernel(
    const int32_t* __restrict__ tab, int32_t off_pages, int32_t off_dec,
    int32_t item_b, int32_t item_e, DecParts dp, const uint16_t* __restrict__ q,
    int64_t q_layer_stride, const uint16_t* __restrict__ kp, const uint16_t* __restrict__ vp,
    float* __restrict__ ws, int32_t G, int32_t Hq, int32_t P, int32_t log2P, float c) {
  constexpr int KS = D / 32;  // k-steps of the QK^T contraction
  constexpr int DT = D / 16;  // 16-row tiles of O^T
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int32_t wid = (int32_t)blockIdx.x * 4 + wave;
  int32_t rel, part, np;  // item within the launch, its part, its parts
  {
    const int32_t hw = dp.head * dp.nh;
    if (wid < hw) {
      rel = wid / dp.nh; part = wid % dp.nh; np = dp.nh;
    } else {
      rel = dp.head + (wid - hw) / dp.nt; part = (wid - hw) % dp.nt; np = dp.nt;
    }
  }
  const int32_t it = item_b + rel;
  if (it >= item_e) return;
  // the item record through the constant address space (scalar loads; the table
  // is not written while a kernel runs): it carries the unit's fields, so the
  // page ids are the next read
  typedef const __attribute__((address_space(4))) int32_t* cint_ptr;
  const cint_ptr item = (cint_ptr)(tab + off_dec + (int64_t)kDecItemInts * it);
  // slots [lo, hi) minus the gap [gap_lo, gap_hi): the zero tail of a sink page
  // between a local head's sink segment and its window segment
  const int32_t gap_lo = item[3];
  int32_t lo = item[1], hi = item[2];
  const int32_t b = item[4], l = item[5], h = item[6];
  const int32_t* pages = tab + off_pages + item[7];
  const int n = lane & 15, g = lane >> 4;
  const int64_t PD = (int64_t)P * D;
  const int32_t gap_hi = gap_lo > 0 ? ((gap_lo + P - 1) >> log2P) << log2P : 0;
  // this part's steps: the item's steps of 32 slots from lo & ~7, dealt in runs
  // whose lengths differ by at most one
  int32_t s_first = lo & ~7;
  {
    const int32_t nst = (hi - s_first + 31) >> 5;
    const int32_t st0 = part * nst / np, st1 = (part + 1) * nst / np;
    hi = min(hi, s_first + 32 * st1);
    s_first += 32 * st0;
    lo = max(lo, s_first);
    while (s_first >= gap_lo && s_first + 32 <= gap_hi) s_first += 32;  // whole step in the gap
  }
  const int32_t lo8 = s_first;

  // a window of the item's page ids, one per lane; each step reads the ids it
  // needs with readlane into scalar registers, and the window moves on when a
  // step would leave it
  const int32_t pg_last = (hi - 1) >> log2P;
  int32_t pg_first = lo8 >> log2P;
  int32_t pid_lane = lo8 < hi && pg_first + lane <= pg_last ? pages[pg_first + lane] : 0;

  bf16x8 qf[KS];
  {
    const uint16_t* qrow = q + (int64_t)l * q_layer_stride + ((int64_t)b * Hq + h * G + n) * D + g * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (n < G) v = ld16(qrow + ks * 32);
      qf[ks] = as_bf16x8(v);
    }
  }

  float m = -INFINITY, lsum = 0.f;
  f32x4 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int r = lane & 15;
  const int koff = 8 * (r >> 2) + (r & 3);  // key of S^T row r in tile t: koff + 4t

  // operand loads of the 32-key step at s0: K row r of tile t <- key s0 + koff + 4t,
  // dims (4ks + g)*8 .. +7; V row (dim) 16dt + r <- keys s0 + 8g .. +7 (one brick)
  u32x4 kbuf[2][2][KS], vbuf[2][DT];
  auto load_step = [&](int32_t s0, u32x4 (&kr)[2][KS], u32x4 (&vr)[DT]) {
    const int32_t p0 = s0 >> log2P;
    const int32_t p2 = min((s0 + 31) >> log2P, pg_last);
    if (p2 - pg_first >= 64) {  // uniform: move the page-id window
      pg_first = p0;
      pid_lane = pg_first + lane <= pg_last ? pages[pg_first + lane] : 0;
    }
    const int32_t pidA = __builtin_amdgcn_readlane(pid_lane, p0 - pg_first);
    const int32_t pidB = __builtin_amdgcn_readlane(pid_lane, p2 - pg_first);
    const int32_t pidC = __builtin_amdgcn_readlane(pid_lane, min((s0 + 16) >> log2P, pg_last) - pg_first);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int32_t key = s0 + koff + 4 * t;
      const bool ok = key < hi;
      const int32_t pk = key >> log2P;
      const int32_t pid = pk == p0 ? pidA : (pk == ((s0 + 31) >> log2P) ? pidB : pidC);
      const uint16_t* base = kp + pid * PD + (int64_t)(key & (P - 1)) * 8 + (int64_t)g * P * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (ok) v = ld16(base + (int64_t)ks * 4 * P * 8);
        kr[t][ks] = v;
      }
    }
    {
      const int32_t key = s0 + 8 * g;
      const bool ok = key < hi;
      const int32_t pk = key >> log2P;
      const int32_t pid = pk == p0 ? pidA : (pk == ((s0 + 31) >> log2P) ? pidB : pidC);
      const uint16_t* base = vp + pid * PD + ((int64_t)((key & (P - 1)) >> 3) * D + r) * 8;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (ok) v = ld16(base + dt * 16 * 8);
        vr[dt] = v;
      }
    }
  };

  auto compute_step = [&](int32_t s0, const u32x4 (&kr)[2][KS], const u32x4 (&vr)[DT]) {
    f32x4 st[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      st[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        st[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[t][ks]), qf[ks], st[t], 0, 0, 0);
    }
    // lane (n, g) reg i of tile t holds key s0 + 8g + 4t + i
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int32_t key = s0 + 8 * g + 4 * t + i;
        if (key < lo || key >= hi || (key >= gap_lo && key < gap_hi)) st[t][i] = -INFINITY;
        mx = fmaxf(mx, st[t][i]);
      }
    mx = wave_max_xor(mx, 16);
    mx = wave_max_xor(mx, 32);
    const float m_new = fmaxf(m, mx * c);
    // a part's step can hold no key of the part: then every p and alpha are 0
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    float p[8];
    float ps = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[4 * t + i] = fast_exp2(fmaf(st[t][i], c, -m_use));
        ps += p[4 * t + i];
      }
    lsum = lsum * alpha + ps;
    m = m_new;
    // the weights as hi + lo bf16 terms, both multiplied into O: O then carries each
    // weight to ~2^-16 relative, as the fp32 normaliser does (the matrix cores
    // have time to spare here: the kernel waits on HBM)
    u32x4 ph, pl;
    split_bf16x8(p, ph, pl);
    const bf16x8 pfh = as_bf16x8(ph), pfl = as_bf16x8(pl);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      acc[dt] *= alpha;
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vr[dt]), pfh, acc[dt], 0, 0, 0);
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vr[dt]), pfl, acc[dt], 0, 0, 0);
    }
  };

  // steps of 32 slots from lo8; a step lying entirely in the gap is skipped
  auto next_step = [&](int32_t s) {
    s += 32;
    while (s >= gap_lo && s + 32 <= gap_hi) s += 32;
    return s;
  };
  // two-deep register pipeline: the next step's operands are in flight while a step computes
  // (a part without keys runs one step that loads nothing and leaves m, l, O as they are)
  int32_t s0 = lo8;
  load_step(s0, kbuf[0], vbuf[0]);
  for (;;) {
    const int32_t s1 = next_step(s0);
    if (s1 < hi) load_step(s1, kbuf[1], vbuf[1]);
    compute_step(s0, kbuf[0], vbuf[0]);
    if (s1 >= hi) break;
    const int32_t s2 = next_step(s1);
    if (s2 < hi) load_step(s2, kbuf[0], vbuf[0]);
    compute_step(s1, kbuf[1], vbuf[1]);
    if (s2 >= hi) break;
    s0 = s2;
  }

  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  if (n < G) {  // a part without keys writes m = -inf, l = 0, O = 0
    float* w = ws + ((int64_t)wid * G + n) * kWsStride<D>;  // record = wave
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<f32x4*>(w + 16 * dt + 4 * g) = acc[dt];  // dims 16dt + 4g + i
    if (g == 0) {
      w[D] = m;
      w[D + 1] = lsum;
    }
  }
}

// Merge the item partials of each (unit, query head of its group) pair by their
// log-sum-exp weights. WPP waves work on one pair (WPP = 1: four pairs per
// workgroup; WPP = 4: one). Inside a wave, groups of D/4 lanes each take one
// record (a float4 of O per lane, plus m and l) and fold it into a running max,
// normaliser and O, so every record load is issued in one pass (four unrolled);
// the partials are L2-resident and the merge is bound by load latency, not bytes.
// The groups, then the waves of a pair, meet at their common max.
template <int D, int WPP>
__global__ __launch_bounds__(256) void decode_combine_kernel(
    const int32_t* __restrict__ tab, int32_t off_decunits, int32_t unit_b, int32_t unit_e,
    int32_t item_b, DecParts dp, const float* __restrict__ ws, int32_t G, int32_t Hq,
    int32_t B, uint16_t* __restrict__ o, float* __restrict__ lse, int32_t all_layers) {
  constexpr int LPI = D / 4;        // lanes per record
  constexpr int IPW = 64 / LPI;     // records per wave at a time
  constexpr int NS = IPW * WPP;     // records per pair at a time
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wp = wave % WPP;        // wave within its pair
  const int64_t idx = (int64_t)blockIdx.x * (4 / WPP) + wave / WPP;
  const int64_t u = unit_b + idx / G;
  const int j = (int)(idx % G);
  if (u >= unit_e) return;          // uniform over the waves of a pair
  // the unit's record: item range, first output row within its layer, layer
  const int32_t* du = tab + off_decunits + (int64_t)kDecUnitInts * u;
  const int32_t ib = dp.waves_before(du[0] - item_b), ie = dp.waves_before(du[1] - item_b);
  const int64_t row = (all_layers ? (int64_t)du[3] * B * Hq : 0) + du[2] + j;
  // record of (item part t, query column j): D floats of O, then m (log2 units) and l
  const float* rec0 = ws + ((int64_t)ib * G + j) * kWsStride<D>;
  const int64_t rstride = (int64_t)G * kWsStride<D>;
  float m = -INFINITY, lsum = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  {
    const int slot = wp * IPW + lane / LPI, d0 = 4 * (lane % LPI);
#pragma unroll 4
    for (int32_t t = slot; t < ie - ib; t += NS) {
      const float* w = rec0 + t * rstride;
      const f32x4 v = *reinterpret_cast<const f32x4*>(w + d0);
      const float2 ml = *reinterpret_cast<const float2*>(w + D);
      // a part without keys (m = -inf, l = 0, O = 0) adds nothing
      const float m_new = fmaxf(m, ml.x);
      const float s_old = m_new == m ? 1.f : fast_exp2(m - m_new);  // m = -inf: 0
      const float s_new = ml.x == -INFINITY ? 0.f : fast_exp2(ml.x - m_new);
      acc = acc * s_old + v * s_new;
      lsum = lsum * s_old + ml.y * s_new;
      m = m_new;
    }
  }
  // the wave's record groups at their common max
  {
    float mw = m;
#pragma unroll
    for (int off = LPI; off < 64; off <<= 1) mw = fmaxf(mw, __shfl_xor(mw, off, 64));
    const float f = m == -INFINITY ? 0.f : fast_exp2(m - mw);
    acc *= f;
    lsum *= f;
    m = mw;
  }
#pragma unroll
  for (int off = LPI; off < 64; off <<= 1) {
    lsum += __shfl_xor(lsum, off, 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += __shfl_xor(acc[i], off, 64);
  }
  if constexpr (WPP > 1) {
    __shared__ f32x4 sAcc[WPP][LPI];
    __shared__ float sL[WPP], sM[WPP];
    if (lane < LPI) sAcc[wp][lane] = acc;
    if (lane == 0) { sL[wp] = lsum; sM[wp] = m; }
    __syncthreads();
    if (wp != 0) return;
    float mp = sM[0];
#pragma unroll
    for (int w2 = 1; w2 < WPP; ++w2) mp = fmaxf(mp, sM[w2]);
    acc = f32x4{0.f, 0.f, 0.f, 0.f};
    lsum = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < WPP; ++w2) {
      const float f = sM[w2] == -INFINITY ? 0.f : fast_exp2(sM[w2] - mp);
      if (lane < LPI) acc += sAcc[w2][lane] * f;
      lsum += sL[w2] * f;
    }
    m = mp;
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  if (lane < LPI) {
    uint16_t r4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) r4[i] = __builtin_bit_cast(uint16_t, (__bf16)(acc[i] * inv));
    *reinterpret_cast<uint2*>(o + row * D + 4 * lane) =
        make_uint2(r4[0] | ((uint32_t)r4[1] << 16), r4[2] | ((uint32_t)r4[3] << 16));
  }
  if (lse && lane == 0) lse[row] = lsum > 0.f ? (m + __builtin_amdgcn_logf(lsum)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// prefill. One workgroup (8 waves, two per SIMD) per tile of 256 query rows =
// the G query heads of one KV head x (256 / G) consecutive positions, so every
// K/V block read serves all G heads. Keys stream in blocks of 32 slots straight
// into LDS (global_load_lds_dwordx4, an 8-buffer ring, one barrier per block);
// the LDS tiles have the page layouts. Per block, each wave (32 query rows)
// runs v_mfma_f32_32x32x16_bf16:
//   S^T[32 keys][32 rows] = K . Q^T
//   O^T[32 dims][32 rows] += V^T . P^T   (D/32 dim tiles)
// While one wave of a SIMD does its softmax the other's MFMAs run. Only blocks
// some row of the tile can see are visited; blocks every row sees entirely skip
// the per-element predicate. Each row's reference max is fixed by its first
// block with a visible key, so the hot loop never rescales O (exp2 of scores up
// to 2^64 above it stays finite in fp32 and bf16, with unchanged relative
// precision); a tile whose scores outgrow that margin is recomputed on a path
// that rescales per block.
// ---------------------------------------------------------------------------
// The key blocks a tile visits: per segment at most two runs of consecutive
// blocks (A: sink / prefix, B: window), in four fixed scalar slots 0A, 0B, 1A,
// 1B; empty runs have zero length.
struct TileRuns {
  int32_t a0, n0, a1, n1, a2, n2, a3, n3;  // first block and block count per slot
  __device__ __forceinline__ int32_t total() const { return n0 + n1 + n2 + n3; }
  // block k of the sequence -> (segment, block index within the segment)
  __device__ __forceinline__ void at(int32_t k, int& seg, int32_t& kb) const {
    if (k < n0) { seg = 0; kb = a0 + k; return; }
    k -= n0;
    if (k < n1) { seg = 0; kb = a1 + k; return; }
    k -= n1;
    if (k < n2) { seg = 1; kb = a2 + k; return; }
    k -= n2;
    seg = 1;
    kb = a3 + k;
  }
};

// Wave-uniform int32 read through the scalar data cache (a read only); it waits
// on lgkmcnt, so unlike a vector load it never forces a vmcnt wait that would
// drain the in-flight LDS-DMA transfers.
__device__ __forceinline__ int32_t scalar_load_i32(const int32_t* p) {
  // the address is uniform; readfirstlane states it for the SGPR operand
  const uint64_t a = (uint64_t)p;
  const uint64_t sa = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(a >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)a);
  int32_t v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)"
               : "=s"(v)
               : "s"((const int32_t*)sa));
  return v;
}

// LDS-DMA: each lane's 4 bytes at gsrc land at lds_wave_base + lane * 4 (the
// 16-byte forms below: + lane * 16). Issued as inline asm so the compiler's
// wait-count pass does not see an LDS write it cannot place in the ring and
// drain every transfer in flight before each LDS read; the kernel waits on
// vmcnt for exactly the block it needs, then passes a barrier. M0 carries the wave's LDS base (the kernel uses
// M0 for nothing else).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ void lds_dma4(const int32_t* gsrc, int32_t* lds_wave_base) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr(lds_wave_base));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(gsrc), "s"(m0v)
               : "memory");
}
// The 16-byte transfer with the LDS destination as a wave-uniform byte address,
// and a variant whose source is a wave-uniform 64-bit base in SGPRs plus a
// per-lane 32-bit byte offset (no per-lane address arithmetic).
__device__ __forceinline__ void lds_dma16_a(const uint16_t* gsrc, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gsrc), "s"(lds_base)
               : "memory");
}
__device__ __forceinline__ void lds_dma16_s(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds_base)
               : "memory");
}
// Empty asm that takes a value in registers: the value is computed before this
// point, so the compiler cannot sink its computation below a later barrier.
__device__ __forceinline__ void pin_vgpr(const f32x16& x) { asm volatile("" ::"v"(x)); }
// Workgroup barrier without the release/acquire fence of __syncthreads (which
// would wait for every LDS-DMA in flight); the memory clobber keeps LDS reads
// below it. Callers first wait on vmcnt for the data the barrier publishes.
__device__ __forceinline__ void ring_barrier() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt with only vmcnt constrained (expcnt / lgkmcnt left at their maxima)
#define WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt((0x0F70) | ((n) & 15) | (((n) >> 4) << 14))
// s_waitcnt vmcnt(n) lgkmcnt(0): also every LDS read and scalar load issued so far
#define WAIT_VM_LGKM0(n) __builtin_amdgcn_s_waitcnt((0x0070) | ((n) & 15) | (((n) >> 4) << 14))


// Nonempty block runs of a tile in visiting order: first block within its
// segment, block count, segment.
struct RunList {
  int32_t k0 = 0, k1 = 0, k2 = 0, k3 = 0, n0 = 0, n1 = 0, n2 = 0, n3 = 0;
  int32_t s0 = 0, s1 = 0, s2 = 0, s3 = 0, nr = 0;
};
__device__ __forceinline__ void run_push(RunList& rl, int32_t kb, int32_t cnt, int32_t seg) {
  if (cnt <= 0) return;
  rl.k0 = rl.nr == 0 ? kb : rl.k0;
  rl.k1 = rl.nr == 1 ? kb : rl.k1;
  rl.k2 = rl.nr == 2 ? kb : rl.k2;
  rl.k3 = rl.nr == 3 ? kb : rl.k3;
  rl.n0 = rl.nr == 0 ? cnt : rl.n0;
  rl.n1 = rl.nr == 1 ? cnt : rl.n1;
  rl.n2 = rl.nr == 2 ? cnt : rl.n2;
  rl.n3 = rl.nr == 3 ? cnt : rl.n3;
  rl.s0 = rl.nr == 0 ? seg : rl.s0;
  rl.s1 = rl.nr == 1 ? seg : rl.s1;
  rl.s2 = rl.nr == 2 ? seg : rl.s2;
  rl.s3 = rl.nr == 3 ? seg : rl.s3;
  ++rl.nr;
}
// Runs of one segment for query rows [r0, rmax]: A = blocks [0, an), B = [b0, b0 + bn).
__device__ __forceinline__ void segment_runs(int kind, int32_t pos0, int32_t len, int32_t sink,
                                             int32_t win, int32_t r0, int32_t rmax,
                                             const int32_t* rpos, int32_t& an, int32_t& b0,
                                             int32_t& bn) {
  constexpr int BK = kBlockN;
  an = 0; b0 = 0; bn = 0;
  if (len <= 0) return;
  if (pos0 < 0) {  // gathered: keys with position <= rmax form a prefix
    int32_t a = 0, z = len;
    while (a < z) {
      const int32_t mid = (a + z) >> 1;
      if (rpos[mid] <= rmax) a = mid + 1; else z = mid;
    }
    an = (a + BK - 1) / BK;
  } else if (kind == SEGPAGED_LOCAL) {
    const int32_t ahi = min(len, min(sink, rmax + 1) - pos0);
    const int32_t blo = max(0, r0 - win + 1 - pos0);
    const int32_t bhi = min(len, rmax + 1 - pos0);
    const int32_t A1 = ahi > 0 ? (ahi + BK - 1) / BK : 0;
    const int32_t B0 = blo / BK, B1 = bhi > blo ? (bhi + BK - 1) / BK : B0;
    if (A1 > 0 && B1 > B0 && B0 <= A1) {
      an = max(A1, B1);
    } else {
      an = A1;
      b0 = B0;
      bn = B1 - B0;
    }
  } else {
    const int32_t hi = min(len, rmax + 1 - pos0);
    an = hi > 0 ? (hi + BK - 1) / BK : 0;
  }
}

// Prefill work counter: one 64-bit word, (launch generation << 32) | next item.
// Every workgroup fetches items until it gets one past the list, so a launch makes
// exactly items + workgroups fetches; the last fetch sets the word to (gen, 0),
// ready for a launch of the same generation (a replayed graph). A word left by a
// launch of another generation (in any state) is claimed by one workgroup's
// compare-and-swap, which takes item 0; the other workgroups then count on.
__device__ __forceinline__ uint32_t prefill_fetch(unsigned long long* ctr, uint32_t gen,
                                                  uint32_t last) {
  const uint32_t v = (uint32_t)atomicAdd(ctr, 1ull);
  if (v == last) atomicExch(ctr, (unsigned long long)gen << 32);
  return v;
}
__device__ __forceinline__ uint32_t prefill_claim(unsigned long long* ctr, uint32_t gen,
                                                  uint32_t last) {
  unsigned long long old = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // two rounds suffice unless launches on one counter overlap (not allowed)
  for (int round = 0; round < 64; ++round) {
    if ((uint32_t)(old >> 32) == gen) return prefill_fetch(ctr, gen, last);
    const unsigned long long prev = atomicCAS(ctr, old, ((unsigned long long)gen << 32) | 1ull);
    if (prev == old) return 0;
    old = prev;
  }
  return 0x7FFFFFFFu;  // past any list: this workgroup takes no item
}

template <int D, bool SMALLP>
__global__ __launch_bounds__(512) void prefill_kernel(
    const int32_t* __restrict__ tab, int32_t off_seqs, int32_t off_units, int32_t off_pages,
    int32_t off_retr, int32_t off_pre, int32_t item_b, int32_t item_e,
    unsigned long long* __restrict__ ctr, uint32_t gen,
    const uint16_t* __restrict__ q, uint16_t* __restrict__ o, float* __restrict__ lse,
    int64_t q_layer_stride, int64_t lse_layer_stride, const uint16_t* __restrict__ kp,
    const uint16_t* __restrict__ vp, int32_t G, int32_t Hq, int32_t P, int32_t log2P, float c) {
  constexpr int BK = kBlockN;          // keys per block (32)
  constexpr int KCH = D / 8;           // 16 B chunks per key row
  constexpr int KSTEP = D / 16;        // k-steps of QK^T
  constexpr int MD = D / 32;           // O^T dim tiles
  constexpr int NT = 512;              // threads per workgroup
  constexpr int TILE = KCH * BK * 8;   // elements of one K (or V) block tile
  constexpr int CH = TILE / 8;         // 16 B chunks per tile
  constexpr int NBUF = 8;              // LDS ring of K/V block tiles
  constexpr int PER_BLOCK = 2;         // LDS-DMA instructions per block and lane (K and V)
  // a wave's own blocks still in flight when a phase ends (see the phase loop)
  constexpr int INFLIGHT = (NBUF - 4) * PER_BLOCK;
  static_assert(CH % 64 == 0 && CH <= NT, "one 16 B chunk per lane and tile, whole waves");
  static_assert(BK == 32, "block index arithmetic below shifts by 5");
  static_assert(KSTEP == 2 * MD && KSTEP % 4 == 0, "QK and PV steps pair up in the MFMA phase");
  __shared__ __attribute__((aligned(16))) uint16_t sK[NBUF][TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sV[NBUF][TILE];
  __shared__ __attribute__((aligned(16))) int32_t sPos[NBUF][64];
  __shared__ int32_t sRun[4][4];
  __shared__ int32_t sOverflow;
  __shared__ int32_t sItem[2];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, g = lane >> 5;
  // this wave's 32 query rows: lane column n is row 32 * wave + n
  const int row = 32 * wave + n;
  const int32_t pq = row / G, jh = row % G;

  // O accumulators and row statistics; they outlive a tile, whose O is written
  // once the next tile's Q and first K/V blocks are in flight
  f32x16 oacc[MD];
  float m_run = -INFINITY, l_run = 0.f;
  bool e_valid = false, e_row_ok = false;
  int64_t e_obase = 0, e_lidx = 0;
#define SEGPAGED_EPILOGUE_PREV()                                                              \
  do {                                                                                        \
    if (e_valid) {                                                                            \
      /* O^T lane (n, g) reg i of dim tile md -> dim 32md + 8(i/4) + 4g + (i%4) */            \
      const float l_tot_ = l_run + __shfl_xor(l_run, 32, 64);                                 \
      if (e_row_ok) {                                                                         \
        const float inv_ = l_tot_ > 0.f ? 1.f / l_tot_ : 0.f;                                 \
        uint16_t* op_ = o + e_obase;                                                          \
        _Pragma("unroll") for (int md = 0; md < MD; ++md)                                     \
            _Pragma("unroll") for (int qd = 0; qd < 4; ++qd) {                                \
          u32x2 w_;                                                                           \
          w_.x = pack_bf16x2(oacc[md][4 * qd + 0] * inv_, oacc[md][4 * qd + 1] * inv_);       \
          w_.y = pack_bf16x2(oacc[md][4 * qd + 2] * inv_, oacc[md][4 * qd + 3] * inv_);       \
          *reinterpret_cast<u32x2*>(op_ + 32 * md + 8 * qd + 4 * g) = w_;                     \
        }                                                                                     \
        if (lse && g == 0)                                                                    \
          lse[e_lidx] = l_tot_ > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot_)) * kLn2         \
                                     : -INFINITY;                                             \
      }                                                                                       \
    }                                                                                         \
    _Pragma("unroll") for (int md = 0; md < MD; ++md)                                         \
        _Pragma("unroll") for (int i = 0; i < 16; ++i) oacc[md][i] = 0.f;                     \
    m_run = -INFINITY;                                                                        \
    l_run = 0.f;                                                                              \
  } while (0)

  // Persistent workgroups take items of the heaviest-first list from the work
  // counter, so faster compute units take more: the next item is fetched while
  // the current one runs.
  const uint32_t nitems = (uint32_t)(item_e - item_b);
  const uint32_t last_fetch = nitems + gridDim.x - 1;
  if (tid == 0) sItem[0] = (int32_t)prefill_claim(ctr, gen, last_fetch);
  __syncthreads();
  for (int32_t round = 0;; ++round) {
  const uint32_t it_idx = (uint32_t)__builtin_amdgcn_readfirstlane(sItem[round & 1]);
  if (it_idx >= nitems) break;
  const int32_t it = item_b + (int32_t)it_idx;
  int32_t it_next = 0;  // the item after this one (wave 0, lane 0)
  // tile metadata through the constant address space: scalar loads (the table
  // is not written while a kernel runs)
  typedef const __attribute__((address_space(4))) int32_t* cint_ptr;
  const cint_ptr ctab = (cint_ptr)tab;
  const int32_t u = ctab[off_pre + kPreItemInts * it];
  const int32_t r0_flag = ctab[off_pre + kPreItemInts * it + 1];
  // tiles whose rows see few keys: weights carried as hi + lo bf16 terms
  const bool precise = r0_flag < 0;
  const int32_t r0 = r0_flag & 0x7FFFFFFF;
  const cint_ptr ur = ctab + off_units + kUnitInts * u;
  const int32_t kind = ur[U_KIND], b = ur[U_B], l = ur[U_L], h = ur[U_H], N = ur[U_N];
  const int32_t q0 = ur[U_Q0], sink = ur[U_SINK], win = ur[U_WIN], nseg = ur[U_NSEG];
  const int32_t* pages = tab + off_pages + ur[U_PAGEOFF];
  const int32_t* rpos = tab + off_retr + ur[U_RETROFF];
  const int32_t qrow0 = ctab[off_seqs + kSeqInts * b + S_QOFF];
  const int32_t BQ = kPrefillRows / G;
  const int32_t r1 = min(N, r0 + BQ), rmax = r1 - 1;
  const int64_t PD = (int64_t)P * D;
  const int32_t log2PD = log2P + __builtin_ctz(D);  // page elements P * D, a power of two
  const bool gathered = ur[U_S0POS] < 0;
  const bool local = kind == SEGPAGED_LOCAL;
  // page table through the constant address space: compiler-tracked scalar loads
  const cint_ptr cpages = (cint_ptr)pages;

  if (tid == 0) sOverflow = 0;
  const int32_t qpos = r0 + pq;
  const bool row_ok = pq < r1 - r0;
  const int64_t orow = (int64_t)qrow0 + (qpos - q0);
  const int hq = h * G + jh;
  bf16x8 qf[KSTEP];
  {
    // rows past the tile read row q0 of the sequence (valid memory) and are never stored
    const int64_t qrow = row_ok ? orow : (int64_t)qrow0;
    const uint16_t* qp = q + (int64_t)l * q_layer_stride + (qrow * Hq + hq) * D + g * 8;
#pragma unroll
    for (int ks = 0; ks < KSTEP; ++ks) qf[ks] = as_bf16x8(ld16(qp + ks * 16));
  }

  // ---- block runs this tile visits (uniform across the workgroup)
  const int32_t sp0 = ur[U_S0POS], sl0 = ur[U_S0LEN];
  const int32_t sp1 = ur[U_S1POS], sl1 = ur[U_S1LEN];
  const int32_t sb1 = ((sl0 + P - 1) >> log2P) << log2P;  // slot base of segment 1
  TileRuns runs;
  {
    int32_t an, b0, bn;
    segment_runs(kind, sp0, nseg > 0 ? sl0 : 0, sink, win, r0, rmax, rpos, an, b0, bn);
    runs.a0 = 0; runs.n0 = an; runs.a1 = b0; runs.n1 = bn;
    segment_runs(kind, sp1, nseg > 1 ? sl1 : 0, sink, win, r0, rmax, rpos, an, b0, bn);
    runs.a2 = 0; runs.n2 = an; runs.a3 = b0; runs.n3 = bn;
  }
  const int32_t nblocks = runs.total();

  float neg_m = 0.f;

  // Lane chunk of a block tile: K chunk (head-dim group cidx / BK, key cidx % BK),
  // V chunk cidx (key group cidx / D, head dim cidx % D); both land at LDS chunk
  // cidx. With P >= BK a block lies inside one page, so its source is the page's
  // block base (scalar) plus a per-lane byte offset fixed for the whole tile.
  const int cidx = 64 * wave + lane;
  const bool dma_wave = 64 * wave < CH;
  const uint32_t k_off = (uint32_t)((((cidx / BK) << log2P) + (cidx % BK)) * 16);
  const uint32_t v_off = (uint32_t)(cidx * 16);
  const uint32_t lds_k = lds_addr(&sK[0][0]) + 64 * 16 * wave;  // this wave's chunks
  const uint32_t lds_v = lds_addr(&sV[0][0]) + 64 * 16 * wave;

  // K/V block BLK -> LDS buffer BLK % NBUF (general form: any page size). Indexes
  // past the last block re-read the last block (the ring's wait counts stay
  // uniform; nothing reads those buffers). With P < BK a block spans two pages
  // and slots past the segment's end re-read its last key.
#define SEGPAGED_ISSUE(BLK)                                                                   \
  do {                                                                                        \
    int s_;                                                                                   \
    int32_t kb_;                                                                              \
    runs.at(min((BLK), nblocks - 1), s_, kb_);                                                \
    const int buf_ = (BLK) % NBUF;                                                            \
    const int32_t len_ = s_ ? sl1 : sl0, base_ = s_ ? sb1 : 0;                                \
    const int32_t first_ = base_ + kb_ * BK;                                                  \
    const int32_t pi0_ = first_ >> log2P;                                                     \
    const int64_t pg0_ = (int64_t)scalar_load_i32(pages + pi0_) * PD;                         \
    if (!SMALLP) {                                                                            \
      const int32_t in_ = first_ & (P - 1);                                                   \
      if (dma_wave) {                                                                         \
        lds_dma16_s(kp + pg0_ + in_ * 8, k_off, lds_k + buf_ * (TILE * 2));                   \
        lds_dma16_s(vp + pg0_ + (in_ >> 3) * (D * 8), v_off, lds_v + buf_ * (TILE * 2));      \
      }                                                                                       \
    } else {                                                                                  \
      const int64_t pg1_ = kb_ * BK + P < len_                                                \
                               ? (int64_t)scalar_load_i32(pages + pi0_ + 1) * PD              \
                               : pg0_;                                                        \
      if (dma_wave) {                                                                         \
        {                                                                                     \
          const int dc = cidx / BK, t = cidx % BK;                                            \
          const int32_t slot = base_ + min(kb_ * BK + t, len_ - 1);                           \
          const int64_t pg = (slot >> log2P) == pi0_ ? pg0_ : pg1_;                           \
          lds_dma16_a(kp + pg + ((int64_t)dc * P + (slot & (P - 1))) * 8,                     \
                      lds_k + buf_ * (TILE * 2));                                             \
        }                                                                                     \
        {                                                                                     \
          const int tc = cidx / D, d = cidx % D;                                              \
          int32_t off8 = kb_ * BK + 8 * tc;                                                   \
          if (off8 >= len_) off8 = (len_ - 1) & ~7;                                           \
          const int32_t slot = base_ + off8;                                                  \
          const int64_t pg = (slot >> log2P) == pi0_ ? pg0_ : pg1_;                           \
          lds_dma16_a(vp + pg + ((int64_t)((slot & (P - 1)) >> 3) * D + d) * 8,               \
                      lds_v + buf_ * (TILE * 2));                                             \
        }                                                                                     \
      }                                                                                       \
    }                                                                                         \
    if (gathered && wave == 0)                                                                \
      lds_dma4(rpos + min(kb_ * BK + lane, len_ - 1), &sPos[buf_][0]);                        \
  } while (0)

  // S^T row rho of the 32-key tile <- key 16(q'/2) + 8gg + 4(q'%2) + e', rho = 8q' + 4gg + e';
  // then lane (n, g) reg i holds key 16(i/8) + 8g + (i%8): for PV k-step kk it owns the
  // 8 consecutive keys 16kk + 8g .. +7, one V brick.
  const int rq = n >> 3, rgg = (n >> 2) & 1, re = n & 3;
  const int tokA = 16 * (rq >> 1) + 8 * rgg + 4 * (rq & 1) + re;

  // MFMA operands of a block, read from LDS into registers
#define SEGPAGED_LOAD_K(BUF, KF)                                                              \
  _Pragma("unroll") for (int ks = 0; ks < KSTEP; ++ks)                                        \
      KF[ks] = as_bf16x8(ld16(&sK[(BUF)][((2 * ks + g) * BK + tokA) * 8]))
#define SEGPAGED_LOAD_V(BUF, VF)                                                              \
  _Pragma("unroll") for (int md = 0; md < MD; ++md)                                           \
      _Pragma("unroll") for (int kk = 0; kk < 2; ++kk)                                        \
          VF[2 * md + kk] = as_bf16x8(ld16(&sV[(BUF)][((2 * kk + g) * D + 32 * md + n) * 8]))
  // S^T = K . Q^T of one block
#define SEGPAGED_QK(KF, SC)                                                                   \
  do {                                                                                        \
    const f32x16 zero_ = {};                                                                  \
    SC = __builtin_amdgcn_mfma_f32_32x32x16_bf16(KF[0], qf[0], zero_, 0, 0, 0);               \
    _Pragma("unroll") for (int ks = 1; ks < KSTEP; ++ks)                                      \
        SC = __builtin_amdgcn_mfma_f32_32x32x16_bf16(KF[ks], qf[ks], SC, 0, 0, 0);            \
  } while (0)
  // O^T += V^T . P^T of one block
#define SEGPAGED_PV(VF, PF)                                                                   \
  _Pragma("unroll") for (int md = 0; md < MD; ++md)                                           \
      _Pragma("unroll") for (int kk = 0; kk < 2; ++kk)                                        \
          oacc[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(VF[2 * md + kk], PF[kk], oacc[md], 0, 0, 0)
  // k-step KS of QK^T (the dependent chain) paired with PV step KS (independent)
#define SEGPAGED_QK_PV_STEP(KS, KF, SC, VF, PF)                                               \
  do {                                                                                        \
    const f32x16 zero_ = {};                                                                  \
    SC = __builtin_amdgcn_mfma_f32_32x32x16_bf16(KF[KS], qf[KS], (KS) ? SC : zero_, 0, 0, 0); \
    oacc[(KS) >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(VF[KS], PF[(KS) & 1],           \
                                                              oacc[(KS) >> 1], 0, 0, 0);      \
  } while (0)

  // Predicate of a block's scores from its mask parameters: first key position
  // POS (non-gathered), keys left in the segment REM, LDS buffer BUF (gathered
  // positions). Lane (n, g) reg i holds key tk = 16(i/8) + 8g + (i%8) of the block;
  // a key past the segment's end is never visible.
#define SEGPAGED_MASK(GATH, POS, REM, BUF, SC)                                                \
  do {                                                                                        \
    if (!(GATH)) {                                                                            \
      /* key e = tk - 8g of the lane's two 8-key groups is at position kb0 + e */             \
      const int32_t kb0 = (POS) + 8 * g;                                                      \
      const int32_t hi = min(qpos - kb0, (REM) - 8 * g - 1); /* e <= hi */                    \
      const int32_t sk = sink - kb0;          /* e < sk: sink key */                          \
      const int32_t wl = qpos - win - kb0;    /* e > wl: inside the window */                 \
      if (local) {                                                                            \
        _Pragma("unroll") for (int i = 0; i < 16; ++i) {                                      \
          const int e = 16 * (i >> 3) + (i & 7);                                              \
          SC[i] = (e <= hi) & ((e < sk) | (e > wl)) ? SC[i] : -INFINITY;                      \
        }                                                                                     \
      } else {                                                                                \
        _Pragma("unroll") for (int i = 0; i < 16; ++i) {                                      \
          const int e = 16 * (i >> 3) + (i & 7);                                              \
          SC[i] = e <= hi ? SC[i] : -INFINITY;                                                \
        }                                                                                     \
      }                                                                                       \
    } else {                                                                                  \
      _Pragma("unroll") for (int i = 0; i < 16; ++i) {                                        \
        const int tk = 16 * (i >> 3) + 8 * g + (i & 7);                                       \
        const int32_t gp_ = sPos[(BUF)][tk];                                                  \
        const int32_t kpos = tk < (REM) ? gp_ : 0x7FFFFFFF;                                   \
        SC[i] = kpos <= qpos ? SC[i] : -INFINITY;                                             \
      }                                                                                       \
    }                                                                                         \
  } while (0)

  // mask parameters of block BLK (general form, for the prologue and the safe path)
#define SEGPAGED_MASK_BLOCK(BLK, SC)                                                          \
  do {                                                                                        \
    int s_;                                                                                   \
    int32_t kb_;                                                                              \
    runs.at((BLK), s_, kb_);                                                                  \
    const int32_t pos0_ = s_ ? sp1 : sp0;                                                     \
    const int32_t rem_ = (s_ ? sl1 : sl0) - kb_ * BK;                                         \
    const int32_t pos_ = pos0_ + kb_ * BK;                                                    \
    if (!block_interior(pos0_ < 0, pos_, rem_)) SEGPAGED_MASK(pos0_ < 0, pos_, rem_, (BLK) % NBUF, SC); \
  } while (0)

  // every row of the tile sees every key of a (non-gathered) block
  auto block_interior = [&](bool gath, int32_t pos, int32_t rem) -> bool {
    const int32_t last = pos + BK - 1;
    bool in = !gath & (rem >= BK) & (last <= r0);
    if (local) in = in & ((last < sink) | (pos > rmax - win));
    return in;
  };

  // exp2 of the scaled scores against the reference, packed to bf16 for PV
#define SEGPAGED_EXP(SC, PF)                                                                  \
  do {                                                                                        \
    float p_[16];                                                                             \
    _Pragma("unroll") for (int i = 0; i < 16; ++i) p_[i] = fast_exp2(fmaf(SC[i], c, neg_m));  \
    _Pragma("unroll") for (int i = 0; i < 16; ++i) l_run += p_[i];                            \
    _Pragma("unroll") for (int kk = 0; kk < 2; ++kk) {                                        \
      u32x4 w_;                                                                               \
      w_.x = pack_bf16x2(p_[8 * kk + 0], p_[8 * kk + 1]);                                     \
      w_.y = pack_bf16x2(p_[8 * kk + 2], p_[8 * kk + 3]);                                     \
      w_.z = pack_bf16x2(p_[8 * kk + 4], p_[8 * kk + 5]);                                     \
      w_.w = pack_bf16x2(p_[8 * kk + 6], p_[8 * kk + 7]);                                     \
      PF[kk] = as_bf16x8(w_);                                                                 \
    }                                                                                         \
  } while (0)

  // the same with the weights as hi + lo bf16 terms (PF, PL), whose products with V
  // carry them to ~2^-16 relative, like the fp32 normaliser l_run
#define SEGPAGED_EXP_PRECISE(SC, PF, PL)                                                      \
  do {                                                                                        \
    float p_[16];                                                                             \
    _Pragma("unroll") for (int i = 0; i < 16; ++i) p_[i] = fast_exp2(fmaf(SC[i], c, neg_m));  \
    _Pragma("unroll") for (int i = 0; i < 16; ++i) l_run += p_[i];                            \
    _Pragma("unroll") for (int kk = 0; kk < 2; ++kk) {                                        \
      u32x4 h_, l_;                                                                           \
      split_bf16x8(&p_[8 * kk], h_, l_);                                                      \
      PF[kk] = as_bf16x8(h_);                                                                 \
      PL[kk] = as_bf16x8(l_);                                                                 \
    }                                                                                         \
  } while (0)

  // Reference of rows that have none yet (scaled log2 units): the max of the
  // first block with a visible key; afterwards no max is taken. Scores far above
  // the reference show up as a row sum above 2^64 at the end of the tile.
#define SEGPAGED_REFERENCE(SC)                                                                \
  do {                                                                                        \
    if (__builtin_amdgcn_ballot_w64(m_run == -INFINITY)) {                                    \
      float mx_ = SC[0];                                                                      \
      _Pragma("unroll") for (int i = 1; i < 16; ++i) mx_ = fmaxf(mx_, SC[i]);                 \
      mx_ = wave_max_xor(mx_, 32);                                                            \
      if (m_run == -INFINITY) m_run = mx_ * c;                                                \
      neg_m = m_run == -INFINITY ? 0.f : -m_run;                                              \
    }                                                                                         \
  } while (0)

  // softmax with per-block rescaling and precise weights (tiles whose rows see few
  // keys, and tiles that overflowed)
#define SEGPAGED_SOFTMAX_SAFE(BLK, SC, PF, PL)                                                \
  do {                                                                                        \
    SEGPAGED_MASK_BLOCK(BLK, SC);                                                             \
    float mx_ = SC[0];                                                                        \
    _Pragma("unroll") for (int i = 1; i < 16; ++i) mx_ = fmaxf(mx_, SC[i]);                   \
    mx_ = wave_max_xor(mx_, 32);                                                              \
    const float mc_ = mx_ * c;                                                                \
    const bool need_ = mc_ > m_run + 8.f;                                                     \
    if (__builtin_amdgcn_ballot_w64(need_)) {                                                 \
      const float alpha = need_ ? fast_exp2(m_run - mc_) : 1.f;                               \
      if (need_) m_run = mc_;                                                                 \
      l_run *= alpha;                                                                         \
      _Pragma("unroll") for (int md = 0; md < MD; ++md) oacc[md] *= alpha;                    \
      neg_m = m_run == -INFINITY ? 0.f : -m_run;                                              \
    }                                                                                         \
    SEGPAGED_EXP_PRECISE(SC, PF, PL);                                                         \
  } while (0)

  // End of a phase: this wave's share of the block the next phase may read has
  // landed; after the barrier, every wave's share has.
#define SEGPAGED_PHASE_END()                                                                  \
  do {                                                                                        \
    __builtin_amdgcn_sched_barrier(0);                                                        \
    WAIT_VMCNT(INFLIGHT);                                                                     \
    ring_barrier();                                                                           \
    __builtin_amdgcn_sched_barrier(0);                                                        \
  } while (0)

  if (nblocks > 0) {
    bf16x8 kf[KSTEP], vf[2 * MD], pf[2];
    f32x16 s;

    // Compacted list of the nonempty runs (first block within its segment, block
    // count, segment), kept in LDS: the cursors below read it only when a run ends.
    RunList rl;
    run_push(rl, runs.a0, runs.n0, 0);
    run_push(rl, runs.a1, runs.n1, 0);
    run_push(rl, runs.a2, runs.n2, 1);
    run_push(rl, runs.a3, runs.n3, 1);
    // Every wave writes its own copy (the same values): the issue cursor reads the
    // list in the prologue, before any barrier, so a wave must not depend on
    // another wave's write.
    if (lane == 0) {
      sRun[0][0] = rl.k0; sRun[0][1] = rl.n0; sRun[0][2] = rl.s0;
      sRun[1][0] = rl.k1; sRun[1][1] = rl.n1; sRun[1][2] = rl.s1;
      sRun[2][0] = rl.k2; sRun[2][1] = rl.n2; sRun[2][2] = rl.s2;
      sRun[3][0] = rl.k3; sRun[3][1] = rl.n3; sRun[3][2] = rl.s3;
    }
    const int32_t nr = rl.nr;
#define SEGPAGED_RUNF(R, F) __builtin_amdgcn_readfirstlane(sRun[(R)][(F)])

    // Issue cursor: block to fetch next. Per block: its slot, blocks left in its
    // run, its first retrieval entry (kb * BK) and segment length; past the last
    // block it stays there.
    int32_t ic_run = 0, ic_left = rl.n0, ic_slot = (rl.s0 ? sb1 : 0) + rl.k0 * BK;
    int32_t ic_kb32 = rl.k0 * BK, ic_len = rl.s0 ? sl1 : sl0;
#define SEGPAGED_IC_NEXT()                                                                    \
  do {                                                                                        \
    if (__builtin_expect(--ic_left > 0, 1)) {                                                 \
      ic_slot += BK;                                                                          \
      ic_kb32 += BK;                                                                          \
    } else if (ic_run + 1 < nr) {                                                             \
      ++ic_run;                                                                               \
      const int32_t kb0_ = SEGPAGED_RUNF(ic_run, 0), seg_ = SEGPAGED_RUNF(ic_run, 2);         \
      ic_left = SEGPAGED_RUNF(ic_run, 1);                                                     \
      ic_slot = (seg_ ? sb1 : 0) + kb0_ * BK;                                                 \
      ic_kb32 = kb0_ * BK;                                                                    \
      ic_len = seg_ ? sl1 : sl0;                                                              \
    } else {                                                                                  \
      ic_left = 1;                                                                            \
    }                                                                                         \
  } while (0)

    // Mask cursor: block whose scores the next softmax phase predicates. Its mask
    // parameters (first key position, keys left in the segment, flags 1: gathered,
    // 2: every row sees every key) hold for m_span more blocks; they are recomputed
    // in closed form at run ends and where the block starts or stops being interior.
    int32_t mk_run = 0, mk_kb = rl.k0, mk_end = rl.k0 + rl.n0, mk_seg = rl.s0;
    int32_t m_pos = 0, m_rem = 0, m_flags = 0, m_span = 1;
    auto blocks_lt = [](int32_t x) { return x > 0 ? (x + BK - 1) >> 5 : 0; };  // #{kb >= 0: kb*BK < x}
#define SEGPAGED_MASK_STATE()                                                                 \
  do {                                                                                        \
    const int32_t pos0_ = mk_seg ? sp1 : sp0, len_ = mk_seg ? sl1 : sl0;                      \
    m_pos = pos0_ + mk_kb * BK;                                                               \
    m_rem = len_ - mk_kb * BK;                                                                \
    if (pos0_ < 0) {                                                                          \
      m_flags = 1;                                                                            \
      m_span = mk_end - mk_kb;                                                                \
    } else {                                                                                  \
      /* interior blocks of the segment: kb in [0, a1) or [u, a) */                           \
      const int32_t a_ = min(blocks_lt(len_ - BK + 1), blocks_lt(r0 - pos0_ - BK + 2));       \
      int32_t a1_ = a_, u_ = a_;                                                              \
      if (local) {                                                                            \
        a1_ = min(a_, blocks_lt(sink - pos0_ - BK + 1));                                      \
        u_ = max(a1_, ((rmax - win - pos0_) >> 5) + 1);                                       \
      }                                                                                       \
      int32_t nxt_;                                                                           \
      if (mk_kb < a1_) { m_flags = 2; nxt_ = a1_; }                                           \
      else if (mk_kb < u_) { m_flags = 0; nxt_ = u_; }                                        \
      else if (mk_kb < a_) { m_flags = 2; nxt_ = a_; }                                        \
      else { m_flags = 0; nxt_ = mk_end; }                                                    \
      m_span = min(nxt_, mk_end) - mk_kb;                                                     \
    }                                                                                         \
  } while (0)
#define SEGPAGED_MC_NEXT()                                                                    \
  do {                                                                                        \
    m_pos += BK;                                                                              \
    m_rem -= BK;                                                                              \
    ++mk_kb;                                                                                  \
    if (__builtin_expect(--m_span == 0, 0)) {                                                 \
      if (mk_kb >= mk_end) {                                                                  \
        if (mk_run + 1 < nr) {                                                                \
          ++mk_run;                                                                           \
          mk_kb = SEGPAGED_RUNF(mk_run, 0);                                                   \
          mk_end = mk_kb + SEGPAGED_RUNF(mk_run, 1);                                          \
          mk_seg = SEGPAGED_RUNF(mk_run, 2);                                                  \
        } else {                                                                              \
          mk_kb = mk_end - 1; /* past the last block: stay on it */                           \
        }                                                                                     \
      }                                                                                       \
      SEGPAGED_MASK_STATE();                                                                  \
    }                                                                                         \
  } while (0)

    // ---- prologue: blocks 0 .. NBUF - 2 in flight; blocks 0 and 1 landed; block
    // 0's scores and probabilities; operands of the first MFMA phase
    if (!SMALLP) {
      // the page ids of those blocks in one round trip, then their transfers
      int32_t pid_[NBUF - 1], in_[NBUF - 1], kb32_[NBUF - 1], len_[NBUF - 1];
#pragma unroll
      for (int k = 0; k < NBUF - 1; ++k) {
        int s_;
        int32_t kb_;
        runs.at(min(k, nblocks - 1), s_, kb_);
        const int32_t first_ = (s_ ? sb1 : 0) + kb_ * BK;
        pid_[k] = cpages[first_ >> log2P];
        in_[k] = first_ & (P - 1);
        kb32_[k] = kb_ * BK;
        len_[k] = s_ ? sl1 : sl0;
      }
#pragma unroll
      for (int k = 0; k < NBUF - 1; ++k) {
        const int64_t pg0_ = (int64_t)pid_[k] * PD;
        if (dma_wave) {
          lds_dma16_s(kp + pg0_ + in_[k] * 8, k_off, lds_k + k * (TILE * 2));
          lds_dma16_s(vp + pg0_ + (in_[k] >> 3) * (D * 8), v_off, lds_v + k * (TILE * 2));
        }
        if (gathered && wave == 0) lds_dma4(rpos + min(kb32_[k] + lane, len_[k] - 1), &sPos[k][0]);
      }
    } else {
      for (int32_t k = 0; k < NBUF - 1; ++k) SEGPAGED_ISSUE(k);
    }
    // issue sources of block NBUF - 1 (page base, byte offset within the page,
    // retrieval entries); the cursor then stays one block ahead, its page id
    // prefetched a phase before use
    const char* i_kbase = (const char*)kp;
    const char* i_vbase = (const char*)vp;
    int32_t i_in = 0, i_rk = 0, i_rlen = 1, ic_pid = 0;
    const int log2PDB = log2PD + 1;  // bytes per page, log2
#define SEGPAGED_BLOCK_SOURCES(PID)                                                           \
  do {                                                                                        \
    const uint64_t pg_ = (uint64_t)(uint32_t)(PID) << log2PDB;                                \
    i_kbase = (const char*)kp + pg_;                                                          \
    i_vbase = (const char*)vp + pg_;                                                          \
    i_in = ic_slot & (P - 1);                                                                 \
    i_rk = ic_kb32;                                                                           \
    i_rlen = ic_len;                                                                          \
  } while (0)
    if (!SMALLP) {
      for (int32_t k = 0; k < NBUF - 1; ++k) SEGPAGED_IC_NEXT();
      SEGPAGED_BLOCK_SOURCES(cpages[ic_slot >> log2P]);
      SEGPAGED_IC_NEXT();
      ic_pid = cpages[ic_slot >> log2P];
    }
    SEGPAGED_MASK_STATE();
    // the previous tile's O while this tile's Q and first blocks are in flight
    SEGPAGED_EPILOGUE_PREV();
    // the next item; its return is waited for with the blocks below
    if (tid == 0) it_next = (int32_t)(uint32_t)atomicAdd(ctr, 1ull);
    // Q and blocks 0 and 1 landed: vector loads complete in issue order and the
    // O stores can only lower the count
    WAIT_VM_LGKM0((NBUF - 3) * PER_BLOCK);
    ring_barrier();
    __builtin_amdgcn_sched_barrier(0);
    SEGPAGED_LOAD_K(0, kf);
    SEGPAGED_QK(kf, s);
    if (!(m_flags & 2)) SEGPAGED_MASK(m_flags & 1, m_pos, m_rem, 0, s);
    SEGPAGED_REFERENCE(s);
    // rows without a reference yet (no visible key so far) keep the check per block
    bool need_ref = __builtin_amdgcn_ballot_w64(m_run == -INFINITY) != 0;
    SEGPAGED_EXP(s, pf);
    SEGPAGED_MC_NEXT();
    SEGPAGED_LOAD_K(1, kf);
    SEGPAGED_LOAD_V(0, vf);
    uint32_t i_lds = lds_k + (NBUF - 1) * (TILE * 2);  // LDS destination of the next issue

    // Ping-pong: phases alternate between the two waves of each SIMD (w and
    // w + 4): while one runs its MFMA phase the other runs its softmax phase.
    //   MFMA phase j:    S = K(j+1) . Q^T;  O^T += V(j)^T . P(j)^T; in the MFMAs'
    //                    shadow, issue block j + NBUF - 1 and advance both cursors
    //   softmax phase j: P(j+1) from S; operands of K(j+2) and V(j+1)
    // Waves 4-7 run one phase behind waves 0-3 (an idle first phase); waves 0-3
    // idle in the last. After phase t every wave has block t/2 + 2 (so at most
    // NBUF - 4 blocks of its own in flight).
    // (a precise tile only runs the prologue, for the previous tile's O and the
    // next item, and leaves its blocks to the loop further below)
    const bool late = wave >= 4;
    const int32_t nfast = precise ? 0 : nblocks;
    if (late) SEGPAGED_PHASE_END();
    for (int32_t j = 0; j < nfast; ++j) {
      // ---- MFMA phase (its operands were read before the barrier; waiting for
      // them here keeps the scalar loads below from being waited on mid-phase)
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      SEGPAGED_QK_PV_STEP(0, kf, s, vf, pf);
      __builtin_amdgcn_sched_barrier(0);
      const int32_t ibuf = (j + NBUF - 1) % NBUF;
      const int32_t s_rk = i_rk, s_rlen = i_rlen;  // retrieval entries of block j + NBUF - 1
      if (!SMALLP) {
        if (CH == NT || dma_wave) {
          lds_dma16_s(i_kbase, k_off + i_in * 16, i_lds);
          lds_dma16_s(i_vbase, v_off + (i_in >> 3) * (D * 16), i_lds + (lds_v - lds_k));
        }
        i_lds = i_lds == lds_k + (NBUF - 1) * (TILE * 2) ? lds_k : i_lds + TILE * 2;
      } else {
        SEGPAGED_ISSUE(j + NBUF - 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      // the other step pairs, with the cursors' scalar work in the MFMAs' shadow;
      // each pair in issue order, so no two dependent QK MFMAs follow each other
#pragma unroll
      for (int ks = 1; ks < KSTEP / 2; ++ks) {
        SEGPAGED_QK_PV_STEP(ks, kf, s, vf, pf);
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (!SMALLP) {
        SEGPAGED_BLOCK_SOURCES(ic_pid);
        SEGPAGED_IC_NEXT();
        ic_pid = cpages[ic_slot >> log2P];
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = KSTEP / 2; ks < 3 * KSTEP / 4; ++ks) {
        SEGPAGED_QK_PV_STEP(ks, kf, s, vf, pf);
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_sched_barrier(0);
      // mask parameters of block j + 1 for the softmax phase, then block j + 2's
      const int32_t c_pos = m_pos, c_rem = m_rem, c_flags = m_flags;
      SEGPAGED_MC_NEXT();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 3 * KSTEP / 4; ks < KSTEP; ++ks) {
        SEGPAGED_QK_PV_STEP(ks, kf, s, vf, pf);
        __builtin_amdgcn_sched_barrier(0);
      }
      // computed here, not sunk below the barrier; every MFMA issued before it
      pin_vgpr(s);
#pragma unroll
      for (int md = 0; md < MD; ++md) pin_vgpr(oacc[md]);
      SEGPAGED_PHASE_END();
      // ---- softmax phase: operand reads first, their latency under the exps. It
      // is the longer phase, so its wave issues first (raised priority; measured
      // +1.6% on the 128K layers over raising the MFMA phase's)
      __builtin_amdgcn_s_setprio(1);
      SEGPAGED_LOAD_K((j + 2) % NBUF, kf);
      SEGPAGED_LOAD_V((j + 1) % NBUF, vf);
      if (!SMALLP && __builtin_expect(gathered, 0) && wave == 0)
        lds_dma4(rpos + min(s_rk + lane, s_rlen - 1), &sPos[ibuf][0]);
      if (__builtin_expect(j + 1 < nblocks, 1)) {
        if (__builtin_expect(!(c_flags & 2), 0))
          SEGPAGED_MASK(c_flags & 1, c_pos, c_rem, (j + 1) % NBUF, s);
        if (__builtin_expect(need_ref, 0)) {
          SEGPAGED_REFERENCE(s);
          need_ref = __builtin_amdgcn_ballot_w64(m_run == -INFINITY) != 0;
        }
        SEGPAGED_EXP(s, pf);
      }
      __builtin_amdgcn_s_setprio(0);
      SEGPAGED_PHASE_END();
    }
    if (!late) SEGPAGED_PHASE_END();
    WAIT_VM_LGKM0(0);
    {
      // a row sum above 2^64 means scores outgrew the reference: redo with rescaling
      const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
      if (__builtin_amdgcn_ballot_w64(!(l_tot <= 0x1p64f))) sOverflow = 1;
    }
    __syncthreads();
    if (precise || sOverflow) {  // uniform
      bf16x8 plo[2];
#pragma unroll
      for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[md][i] = 0.f;
      m_run = -INFINITY;
      l_run = 0.f;
      neg_m = 0.f;
      // one barrier per block, every wave in the same order
      for (int32_t k = 0; k < NBUF - 1; ++k) SEGPAGED_ISSUE(k);
      WAIT_VM_LGKM0((NBUF - 3) * PER_BLOCK);
      ring_barrier();
      SEGPAGED_LOAD_K(0, kf);
      SEGPAGED_QK(kf, s);
      for (int32_t j = 0; j < nblocks; ++j) {
        f32x16 sn;
        SEGPAGED_LOAD_K((j + 1) % NBUF, kf);
        SEGPAGED_LOAD_V(j % NBUF, vf);
        SEGPAGED_QK(kf, sn);
        SEGPAGED_SOFTMAX_SAFE(j, s, pf, plo);
        SEGPAGED_PV(vf, pf);
        SEGPAGED_PV(vf, plo);
        s = sn;
        // block j + 2 landed and block j's buffer free before it is refilled
        WAIT_VM_LGKM0((NBUF - 4) * PER_BLOCK);
        ring_barrier();
        SEGPAGED_ISSUE(j + NBUF - 1);
      }
      WAIT_VM_LGKM0(0);
    }
  } else {
    SEGPAGED_EPILOGUE_PREV();
    if (tid == 0) it_next = (int32_t)(uint32_t)atomicAdd(ctr, 1ull);
  }
#undef SEGPAGED_PHASE_END
#undef SEGPAGED_BLOCK_SOURCES
#undef SEGPAGED_MC_NEXT
#undef SEGPAGED_MASK_STATE
#undef SEGPAGED_IC_NEXT
#undef SEGPAGED_RUNF
#undef SEGPAGED_SOFTMAX_SAFE
#undef SEGPAGED_REFERENCE
#undef SEGPAGED_EXP
#undef SEGPAGED_MASK_BLOCK
#undef SEGPAGED_MASK
#undef SEGPAGED_QK_PV_STEP
#undef SEGPAGED_PV
#undef SEGPAGED_QK
#undef SEGPAGED_LOAD_V
#undef SEGPAGED_LOAD_K
#undef SEGPAGED_ISSUE
  if (tid == 0) {
    // the last fetch of the launch leaves the counter at (generation, 0)
    if ((uint32_t)it_next == last_fetch) atomicExch(ctr, (unsigned long long)gen << 32);
    sItem[(round + 1) & 1] = it_next;
  }
  // every wave is done with the ring and sOverflow before the next tile's set-up
  __syncthreads();
  e_valid = true;
  e_row_ok = row_ok;
  e_obase = (int64_t)l * q_layer_stride + (orow * Hq + hq) * D;
  e_lidx = (int64_t)l * lse_layer_stride + orow * Hq + hq;
  }  // tile loop
  SEGPAGED_EPILOGUE_PREV();
#undef SEGPAGED_EPILOGUE_PREV
}

// ---------------------------------------------------------------------------
// page transfer: the pages of a range of table slots as one contiguous stream
// (table order, each page in the pool layout), or back into a pool under the page
// ids of a table. Grid-stride over 16-byte chunks; blockIdx.y picks K or V.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void page_copy_kernel(
    const int32_t* __restrict__ tab, int32_t off_pages, int32_t off_bld, int32_t bld_b,
    int64_t npages,
    int32_t log2c, const uint16_t* __restrict__ k_src, const uint16_t* __restrict__ v_src,
    uint16_t* __restrict__ k_dst, uint16_t* __restrict__ v_dst, int32_t to_stream) {
  const uint16_t* src = blockIdx.y ? v_src : k_src;
  uint16_t* dst = blockIdx.y ? v_dst : k_dst;
  const int64_t nchunks = npages << log2c, cmask = ((int64_t)1 << log2c) - 1;
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < nchunks;
       c += (int64_t)gridDim.x * 256) {
    const int64_t pid = tab[off_pages + tab[off_bld + bld_b + (c >> log2c)]];
    const int64_t pc = (pid << log2c) + (c & cmask);  // the chunk in the pool
    if (to_stream)
      st16(dst + c * 8, ld16(src + pc * 8));
    else
      st16(dst + pc * 8, ld16(src + c * 8));
  }
}

// ---------------------------------------------------------------------------
// host helpers
// ---------------------------------------------------------------------------
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }
inline bool aligned8(const void* p) { return ((uintptr_t)p & 7u) == 0; }

// Compute units of the current device (cached per device id; 0 on error). The
// caches are atomics: host threads may call on one device at once.
int device_cus() {
  static std::atomic<int> cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Waves of decode_partial_kernel<D> the current device holds at once (its
// resident workgroups per compute unit x 4 waves x compute units; cached per
// device id; at least 4).
int64_t decode_resident_waves(int D) {
  static std::atomic<int> cached[64][2] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 4;
  std::atomic<int>& slot = cached[dev][D == 128 ? 1 : 0];
  int c = slot.load(std::memory_order_relaxed);
  if (c == 0) {
    int per_cu = 0;
    const hipError_t e =
        D == 128 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(
                       &per_cu, reinterpret_cast<const void*>(&decode_partial_kernel<128>), 256, 0)
                 : hipOccupancyMaxActiveBlocksPerMultiprocessor(
                       &per_cu, reinterpret_cast<const void*>(&decode_partial_kernel<64>), 256, 0);
    c = std::max(1, e == hipSuccess ? per_cu : 1) * 4 * std::max(device_cus(), 1);
    slot.store(c, std::memory_order_relaxed);
  }
  return c;
}

int check_launch() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? SEGPAGED_OK : SEGPAGED_EHIP;
}

struct Span {
  int64_t unit_b, unit_e, page_b, page_e, retr_b, retr_e, dec_b, dec_e, pre_b, pre_e;
  int64_t max_unit_items, bld_b, bld_e;
};

// The pools may be NULL when the plan has no pages (no head keeps a token).
bool pools_ok(const segpaged_plan* pl, const void* k_pool, const void* v_pool) {
  return (k_pool && v_pool) || pl->pool_pages == 0;
}

Span span_of(const segpaged_plan* pl, int32_t layer) {
  if (layer >= 0) {
    const LayerRange& r = pl->layers[layer];
    return {r.unit_b, r.unit_e, r.page_b, r.page_e, r.retr_b, r.retr_e,
            r.dec_b, r.dec_e, r.pre_b, r.pre_e, r.max_unit_items, r.bld_b, r.bld_e};
  }
  return {0, pl->num_units, 0, pl->num_slots, 0, pl->num_retr, 0, pl->n_dec, 0, pl->n_pre,
          pl->max_unit_items, 0, pl->num_pages};
}

int upload(const segpaged_plan* pl, int32_t* d_table, int64_t off, int64_t count,
           hipStream_t st) {
  if (count <= 0) return SEGPAGED_OK;
  const hipError_t e = hipMemcpyAsync(d_table + off, pl->buf.data() + off, count * sizeof(int32_t),
                                      hipMemcpyHostToDevice, st);
  return e == hipSuccess ? SEGPAGED_OK : SEGPAGED_EHIP;
}

// The table slice of `layer` into d_table (everything when layer = -1): what
// segpaged_build and segpaged_import_pages upload before writing pages.
int upload_layer_table(const segpaged_plan* pl, int32_t layer, int32_t* d_table,
                       hipStream_t st) {
  if (layer < 0) return upload(pl, d_table, 0, pl->total_ints, st);
  const Span sp = span_of(pl, layer);
  const int64_t U = kUnitInts;
  int rc;
  if ((rc = upload(pl, d_table, 0, pl->off_units, st))) return rc;
  if ((rc = upload(pl, d_table, pl->off_units + U * sp.unit_b, U * (sp.unit_e - sp.unit_b), st)))
    return rc;
  if ((rc = upload(pl, d_table, pl->off_pages + sp.page_b, sp.page_e - sp.page_b, st))) return rc;
  if ((rc = upload(pl, d_table, pl->off_retr + sp.retr_b, sp.retr_e - sp.retr_b, st))) return rc;
  if ((rc = upload(pl, d_table, pl->off_bld + sp.bld_b, sp.bld_e - sp.bld_b, st))) return rc;
  if ((rc = upload(pl, d_table, pl->off_decunits + kDecUnitInts * sp.unit_b,
                   kDecUnitInts * (sp.unit_e - sp.unit_b), st)))
    return rc;
  if ((rc = upload(pl, d_table, pl->off_dec + kDecItemInts * sp.dec_b,
                   kDecItemInts * (sp.dec_e - sp.dec_b), st)))
    return rc;
  if ((rc = upload(pl, d_table, pl->off_pre + kPreItemInts * sp.pre_b,
                   kPreItemInts * (sp.pre_e - sp.pre_b), st)))
    return rc;
  // the padding before the counter lines, then the zeroed prefill work counters of
  // this layer and of all-layer calls
  const int64_t pad_b = pl->off_pre + kPreItemInts * pl->pre_cap;
  if ((rc = upload(pl, d_table, pad_b, pl->off_ctr - pad_b, st))) return rc;
  if ((rc = upload(pl, d_table, pl->off_ctr + kCtrInts * layer, kCtrInts, st))) return rc;
  return upload(pl, d_table, pl->off_ctr + kCtrInts * pl->L, kCtrInts, st);
}

// The distinct pages of a layer range (build list order) between a pool and a
// contiguous stream.
int launch_page_copy(const segpaged_plan* pl, const Span& sp, const int32_t* d_table,
                     const void* k_src, const void* v_src, void* k_dst, void* v_dst,
                     int32_t to_stream, hipStream_t st) {
  const int64_t npages = sp.bld_e - sp.bld_b;
  if (npages == 0) return SEGPAGED_OK;  // empty streams may be NULL
  if (!k_src || !v_src || !k_dst || !v_dst) return SEGPAGED_EINVAL;
  const int32_t log2c = pl->log2P + __builtin_ctz((unsigned)pl->D) - 3;  // 16-byte chunks per page
  const int64_t nchunks = npages << log2c;
  const int64_t cus = std::max(device_cus(), 1);
  const dim3 grid((unsigned)std::min<int64_t>((nchunks + 255) / 256, cus * 64), 2), block(256);
  hipLaunchKernelGGL(page_copy_kernel, grid, block, 0, st, d_table, (int32_t)pl->off_pages,
                     (int32_t)pl->off_bld, (int32_t)sp.bld_b, npages, log2c, (const uint16_t*)k_src,
                     (const uint16_t*)v_src, (uint16_t*)k_dst, (uint16_t*)v_dst, to_stream);
  return check_launch();
}

// Decode workspace of segpaged_decode_noalloc: a file-scope device array, one copy
// per GPU, held until the process ends. Host code reaches it only through the
// address hipGetSymbolAddress returns on each device (the array's name is a host
// stand-in, not a device address).
__device__ __attribute__((aligned(256))) float scratch[kNoAllocScratchBytes / 4];

// The device address of `scratch` on the current device (looked up once per device).
int scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return SEGPAGED_EHIP;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SEGPAGED_EHIP;
    addr[dev] = p;
  }
  *out = addr[dev];
  return SEGPAGED_OK;
}

}  // namespace

extern "C" {

SEGPAGED_API int segpaged_build(const segpaged_plan* pl, int32_t layer, const void* k_dense,
                                const void* v_dense, int32_t* d_table, void* k_pool,
                                void* v_pool, void* stream) {
  if (!pl || !k_dense || !v_dense || !d_table || !pools_ok(pl, k_pool, v_pool))
    return SEGPAGED_EINVAL;
  if (!aligned16(k_dense) || !aligned16(v_dense) || !aligned16(k_pool) || !aligned16(v_pool) ||
      !aligned4(d_table))
    return SEGPAGED_EINVAL;
  if (layer < -1 || layer >= pl->L) return SEGPAGED_ESTATE;
  hipStream_t st = (hipStream_t)stream;
  const Span sp = span_of(pl, layer);
  const int rc = upload_layer_table(pl, layer, d_table, st);
  if (rc) return rc;
  const int64_t npages = sp.bld_e - sp.bld_b;
  if (npages == 0) return SEGPAGED_OK;
  const int64_t dstride = layer < 0 ? pl->kv_rows * pl->Hkv * pl->D : 0;
  auto* kd = (const uint16_t*)k_dense;
  auto* vd = (const uint16_t*)v_dense;
  auto* kpp = (uint16_t*)k_pool;
  auto* vpp = (uint16_t*)v_pool;
  const dim3 grid((unsigned)npages), block(256);
  if (pl->D == 128)
    hipLaunchKernelGGL(build_kernel<128>, grid, block, 0, st, d_table, (int32_t)pl->off_seqs,
                       (int32_t)pl->off_units, (int32_t)pl->off_pages, (int32_t)pl->off_retr,
                       (int32_t)pl->off_bld, (int32_t)sp.unit_b, (int32_t)sp.unit_e,
                       (int32_t)sp.bld_b, pl->Hkv, pl->P, pl->log2P, kd, vd, dstride, kpp, vpp);
  else
    hipLaunchKernelGGL(build_kernel<64>, grid, block, 0, st, d_table, (int32_t)pl->off_seqs,
                       (int32_t)pl->off_units, (int32_t)pl->off_pages, (int32_t)pl->off_retr,
                       (int32_t)pl->off_bld, (int32_t)sp.unit_b, (int32_t)sp.unit_e,
                       (int32_t)sp.bld_b, pl->Hkv, pl->P, pl->log2P, kd, vd, dstride, kpp, vpp);
  return check_launch();
}

SEGPAGED_API int segpaged_export_pages(const segpaged_plan* pl, int32_t layer,
                                       const int32_t* d_table, const void* k_pool,
                                       const void* v_pool, void* k_out, void* v_out,
                                       void* stream) {
  if (!pl || !d_table || !pools_ok(pl, k_pool, v_pool)) return SEGPAGED_EINVAL;
  if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(k_out) || !aligned16(v_out) ||
      !aligned4(d_table))
    return SEGPAGED_EINVAL;
  if (layer < -1 || layer >= pl->L) return SEGPAGED_ESTATE;
  const Span sp = span_of(pl, layer);
  if (sp.bld_e > sp.bld_b && (!k_out || !v_out)) return SEGPAGED_EINVAL;
  return launch_page_copy(pl, sp, d_table, k_pool, v_pool, k_out, v_out, 1, (hipStream_t)stream);
}

SEGPAGED_API int segpaged_import_pages(const segpaged_plan* pl, int32_t layer, const void* k_in,
                                       const void* v_in, int32_t* d_table, void* k_pool,
                                       void* v_pool, void* stream) {
  if (!pl || !d_table || !pools_ok(pl, k_pool, v_pool)) return SEGPAGED_EINVAL;
  if (!aligned16(k_in) || !aligned16(v_in) || !aligned16(k_pool) || !aligned16(v_pool) ||
      !aligned4(d_table))
    return SEGPAGED_EINVAL;
  if (layer < -1 || layer >= pl->L) return SEGPAGED_ESTATE;
  const Span sp = span_of(pl, layer);
  if (sp.bld_e > sp.bld_b && (!k_in || !v_in)) return SEGPAGED_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  const int rc = upload_layer_table(pl, layer, d_table, st);
  if (rc) return rc;
  return launch_page_copy(pl, sp, d_table, k_in, v_in, k_pool, v_pool, 0, st);
}

SEGPAGED_API int segpaged_append(segpaged_plan* pl, int32_t layer, const void* k_new,
                                 const void* v_new, int32_t* d_table, void* k_pool, void* v_pool,
                                 void* stream) {
  if (!pl || !d_table || !pools_ok(pl, k_pool, v_pool)) return SEGPAGED_EINVAL;
  if (pl->append_cap <= 0) return SEGPAGED_ESTATE;
  if (layer < -1 || layer >= pl->L) return SEGPAGED_ESTATE;
  const int64_t B = pl->B, Hkv = pl->Hkv;
  const int32_t t_new = pl->buf[pl->off_app + B];
  if (t_new > 0 && (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new)))
    return SEGPAGED_EINVAL;
  if (!aligned4(d_table) || !aligned16(k_pool) || !aligned16(v_pool)) return SEGPAGED_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  int rc;
  if (pl->app_upload) {  // what the last segpaged_plan_append changed, all layers
    if ((rc = upload(pl, d_table, pl->off_seqs, kSeqInts * B, st))) return rc;
    if ((rc = upload(pl, d_table, pl->off_units, kUnitInts * pl->num_units, st))) return rc;
    for (int32_t l = 0; l < pl->L; ++l) {
      if (!pl->pages_dirty[l]) continue;
      const LayerRange& r = pl->layers[l];
      if ((rc = upload(pl, d_table, pl->off_pages + r.page_b, r.page_e - r.page_b, st))) return rc;
      pl->pages_dirty[l] = 0;
    }
    if ((rc = upload(pl, d_table, pl->off_decunits,
                     pl->off_pre + kPreItemInts * pl->pre_cap - pl->off_decunits, st)))
      return rc;
    if ((rc = upload(pl, d_table, pl->off_app, 2 * B + 1, st))) return rc;
    pl->app_upload = false;
  }
  if (t_new == 0) return SEGPAGED_OK;
  const int32_t nl = layer < 0 ? pl->L : 1;
  const int64_t waves = (int64_t)nl * t_new * Hkv;
  const int64_t lstride = layer < 0 ? (int64_t)t_new * Hkv * pl->D : 0;
  const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
  auto* kn = (const uint16_t*)k_new;
  auto* vn = (const uint16_t*)v_new;
  auto* kpp = (uint16_t*)k_pool;
  auto* vpp = (uint16_t*)v_pool;
  const int32_t l0 = layer < 0 ? 0 : layer;
  if (pl->D == 128)
    hipLaunchKernelGGL(append_kernel<128>, grid, block, 0, st, d_table, (int32_t)pl->off_units,
                       (int32_t)pl->off_pages, (int32_t)pl->off_app, (int32_t)B, (int32_t)Hkv, l0,
                       nl, t_new, kn, vn, lstride, kpp, vpp, pl->P, pl->log2P);
  else
    hipLaunchKernelGGL(append_kernel<64>, grid, block, 0, st, d_table, (int32_t)pl->off_units,
                       (int32_t)pl->off_pages, (int32_t)pl->off_app, (int32_t)B, (int32_t)Hkv, l0,
                       nl, t_new, kn, vn, lstride, kpp, vpp, pl->P, pl->log2P);
  return check_launch();
}

SEGPAGED_API int segpaged_prefill(const segpaged_plan* pl, int32_t layer, const void* q,
                                  int32_t* d_table, const void* k_pool, const void* v_pool,
                                  float scale, void* o, float* lse, void* workspace,
                                  int64_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (!pl || !q || !d_table || !pools_ok(pl, k_pool, v_pool) || !o) return SEGPAGED_EINVAL;
  if (!aligned16(q) || !aligned16(o) || !aligned16(k_pool) || !aligned16(v_pool) ||
      !aligned8(d_table) || (lse && !aligned4(lse)))
    return SEGPAGED_EINVAL;
  if (!(scale > 0.f) || !std::isfinite(scale)) return SEGPAGED_EINVAL;
  if (layer < -1 || layer >= pl->L) return SEGPAGED_ESTATE;
  const Span sp = span_of(pl, layer);
  const int64_t nitems = sp.pre_e - sp.pre_b;
  if (nitems == 0) return SEGPAGED_OK;
  hipStream_t st = (hipStream_t)stream;
  const int64_t qstride = layer < 0 ? pl->q_rows * pl->Hq * pl->D : 0;
  const int64_t lstride = layer < 0 ? pl->q_rows * pl->Hq : 0;
  const float c = scale * kLog2e;
  // persistent workgroups, one per compute unit (a workgroup fills a CU's
  // registers), each walking its share of the items
  const int cus = device_cus();
  if (cus <= 0) return SEGPAGED_EHIP;
  const dim3 grid((unsigned)std::min<int64_t>(nitems, cus)), block(512);
  // the work counter of this call's line and a generation no earlier launch on it
  // used (0 is the uploaded state)
  const int32_t line = layer < 0 ? pl->L : layer;
  auto* ctr = reinterpret_cast<unsigned long long*>(d_table + pl->off_ctr + kCtrInts * line);
  uint32_t gen = pl->pre_gen[line].fetch_add(1) + 1;
  if (gen == 0) gen = pl->pre_gen[line].fetch_add(1) + 1;
  auto* qq = (const uint16_t*)q;
  auto* oo = (uint16_t*)o;
  auto* kpp = (const uint16_t*)k_pool;
  auto* vpp = (const uint16_t*)v_pool;
#define SEGPAGED_LAUNCH_PREFILL(DD, SP)                                                         \
  hipLaunchKernelGGL((prefill_kernel<DD, SP>), grid, block, 0, st, d_table,                     \
                     (int32_t)pl->off_seqs, (int32_t)pl->off_units, (int32_t)pl->off_pages,     \
                     (int32_t)pl->off_retr, (int32_t)pl->off_pre, (int32_t)sp.pre_b,            \
                     (int32_t)sp.pre_e, ctr, gen, qq, oo, lse, qstride, lstride, kpp, vpp,      \
                     pl->G,                                                                      \
                     pl->Hq,                                                                     \
                     pl->P, pl->log2P, c)
  const bool small_pages = pl->P < kBlockN;  // a 32-key block spans two pages
  if (pl->D == 128) {
    if (small_pages) SEGPAGED_LAUNCH_PREFILL(128, true); else SEGPAGED_LAUNCH_PREFILL(128, false);
  } else {
    if (small_pages) SEGPAGED_LAUNCH_PREFILL(64, true); else SEGPAGED_LAUNCH_PREFILL(64, false);
  }
#undef SEGPAGED_LAUNCH_PREFILL
  return check_launch();
}

SEGPAGED_API int segpaged_decode(const segpaged_plan* pl, int32_t layer, const void* q,
                                 const int32_t* d_table, const void* k_pool, const void* v_pool,
                                 float scale, void* o, float* lse, void* workspace,
                                 int64_t workspace_bytes, void* stream) {
  if (!pl || !q || !d_table || !pools_ok(pl, k_pool, v_pool) || !o) return SEGPAGED_EINVAL;
  if (!aligned16(q) || !aligned16(o) || !aligned16(k_pool) || !aligned16(v_pool) ||
      !aligned4(d_table) || (lse && !aligned4(lse)))
    return SEGPAGED_EINVAL;
  if (!(scale > 0.f) || !std::isfinite(scale)) return SEGPAGED_EINVAL;
  if (layer < -1 || layer >= pl->L) return SEGPAGED_ESTATE;
  const Span sp = span_of(pl, layer);
  const int64_t nitems = sp.dec_e - sp.dec_b;
  const int64_t rec_bytes = (int64_t)pl->G * (pl->D + 4) * 4;  // one partial (G columns)
  const int64_t need = nitems * rec_bytes;
  if (need > 0 && (!workspace || !aligned16(workspace))) return SEGPAGED_EINVAL;
  if (workspace_bytes < need) return SEGPAGED_ENOSPACE;
  // Parts per item, while a part keeps >= 256 keys and the workspace holds the
  // partials. A launch with fewer items than the chip holds waves at once (one
  // layer of a plan whose split was sized for all layers) deals each item's steps
  // to up to 16 waves, as many as fit in one round of resident waves (a second
  // round of short waves would cost more than it spreads). A launch of several
  // rounds deals its last items, one round of waves' worth, to kDecTailParts
  // waves each: the waves dispatched last are short, so the launch does not end
  // on a few long waves that cannot keep HBM busy.
  DecParts dp{(int32_t)nitems, 1, 1};
  if (nitems > 0) {
    const int64_t keys = layer < 0 ? pl->total.decode_tokens : pl->stats[layer].decode_tokens;
    const int64_t recs = workspace_bytes / rec_bytes;
    const int64_t resident = decode_resident_waves(pl->D);
    if (nitems < resident) {
      const int64_t nparts = std::min<int64_t>({kDecMaxParts, resident / nitems, recs / nitems,
                                                keys / (nitems * 256)});
      dp.nh = (int32_t)std::max<int64_t>(nparts, 1);
    } else if (recs > nitems && keys / (nitems * kDecTailParts) >= 256) {
      const int64_t x = std::min<int64_t>({nitems, resident / kDecTailParts,
                                           (recs - nitems) / (kDecTailParts - 1)});
      dp = DecParts{(int32_t)(nitems - x), 1, kDecTailParts};
    }
  }
  const int64_t nunits = sp.unit_e - sp.unit_b;
  if (nunits == 0) return SEGPAGED_OK;
  hipStream_t st = (hipStream_t)stream;
  const int64_t qstride = layer < 0 ? (int64_t)pl->B * pl->Hq * pl->D : 0;
  const float c = scale * kLog2e;
  auto* qq = (const uint16_t*)q;
  auto* kpp = (const uint16_t*)k_pool;
  auto* vpp = (const uint16_t*)v_pool;
  auto* ws = (float*)workspace;
  if (nitems > 0) {
    const dim3 grid((unsigned)((dp.waves_before((int32_t)nitems) + 3) / 4)), block(256);
    if (pl->D == 128)
      hipLaunchKernelGGL(decode_partial_kernel<128>, grid, block, 0, st, d_table,
                         (int32_t)pl->off_pages, (int32_t)pl->off_dec,
                         (int32_t)sp.dec_b, (int32_t)sp.dec_e, dp, qq, qstride, kpp, vpp,
                         ws, pl->G, pl->Hq, pl->P, pl->log2P, c);
    else
      hipLaunchKernelGGL(decode_partial_kernel<64>, grid, block, 0, st, d_table,
                         (int32_t)pl->off_pages, (int32_t)pl->off_dec,
                         (int32_t)sp.dec_b, (int32_t)sp.dec_e, dp, qq, qstride, kpp, vpp,
                         ws, pl->G, pl->Hq, pl->P, pl->log2P, c);
    int rc = check_launch();
    if (rc) return rc;
  }
  // Four waves per pair when some unit has many items and the pairs alone leave
  // the chip short of waves (under 64 per CU); otherwise four pairs per workgroup.
  const int64_t pairs = nunits * pl->G;
  const int wpp = sp.max_unit_items * std::max(dp.nh, dp.nt) > 16 && pairs < 64 * 256 ? 4 : 1;
  const int64_t per_wg = 4 / wpp;
  const dim3 grid((unsigned)((pairs + per_wg - 1) / per_wg)), block(256);
  auto* oo = (uint16_t*)o;
#define SEGPAGED_LAUNCH_COMBINE(DD, WW)                                                          \
  hipLaunchKernelGGL((decode_combine_kernel<DD, WW>), grid, block, 0, st, d_table,               \
                     (int32_t)pl->off_decunits, (int32_t)sp.unit_b, (int32_t)sp.unit_e,         \
                     (int32_t)sp.dec_b, dp, ws, pl->G, pl->Hq, pl->B,                           \
                     oo, lse,                                                                   \
                     (int32_t)(layer < 0))
  if (pl->D == 128) {
    if (wpp == 4) SEGPAGED_LAUNCH_COMBINE(128, 4); else SEGPAGED_LAUNCH_COMBINE(128, 1);
  } else {
    if (wpp == 4) SEGPAGED_LAUNCH_COMBINE(64, 4); else SEGPAGED_LAUNCH_COMBINE(64, 1);
  }
#undef SEGPAGED_LAUNCH_COMBINE
  return check_launch();
}

SEGPAGED_API int segpaged_decode_noalloc(const segpaged_plan* pl, int32_t layer, const void* q,
                                         const int32_t* d_table, const void* k_pool,
                                         const void* v_pool, float scale, void* o, float* lse,
                                         void* stream) {
  if (!pl) return SEGPAGED_EINVAL;
  void* ws = nullptr;
  const int rc = scratch_address(&ws);
  if (rc) return rc;
  return segpaged_decode(pl, layer, q, d_table, k_pool, v_pool, scale, o, lse, ws,
                         kNoAllocScratchBytes, stream);
}

}  // extern "C"
