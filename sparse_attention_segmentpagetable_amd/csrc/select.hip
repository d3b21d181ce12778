// Retrieval-set selection on the GPU: top-p by attention mass. Retrieval heads
// keep the tokens that carry the attention [runtime explainer, section 2;
// RedKnot summary: retrieval heads look up the important tokens on demand]. For
// each (sequence b, retrieval KV head h) of a layer: the decode row's (position
// N_b - 1) attention over every key of the dense history, averaged over the G
// query heads of the group, gives a mass per key; the set is the shortest
// mass-ordered prefix (larger first, equal masses by position) reaching p of the
// total, returned as sorted positions.
//
//   select_scores_kernel  scores of 256 keys x G heads per workgroup (bf16 MFMA,
//                         fp32, log2 units), with each block's max and exp-sum
//                         per head
//   select_mass_kernel    per chunk of 2048 keys of a pair: the pair's
//                         normalisers, the masses, and the histogram of their
//                         top 8 bits with each bin's mass in fixed point
//   select_topp_kernel    one workgroup per pair: the first radix pass from the
//                         chunk histograms, three more passes (8 bits each,
//                         larger values first) over the masses held in
//                         registers, then the positions taken in order by a
//                         block scan
// Every sum is taken in a fixed order or in exact integer arithmetic, so the set
// is the same on every call.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "plan.hpp"

using namespace segpaged;

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kSelKeys = 256;  // keys per scoring workgroup
constexpr int kSelThreads = 256;
constexpr float kLog2eSel = 1.4426950408889634f;


__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// Scores of 256 keys for the G query heads of (b, h) with v_mfma_f32_16x16x32_bf16:
// S[16 keys][16 cols] = K[keys][32 dims] . Q^T[32 dims][cols], the G query heads as
// columns (zero past G). A wave takes 64 keys, 16 per MFMA tile; lane (n, g) loads
// 8 dims (16 bytes) of key n of a tile straight from the dense K rows and holds
// the scores of keys 4g .. 4g + 3 for head n. Writes s[g] = c * q_g . k_j (log2
// units) and, per block and head, the max and the sum of exp2(s - max).
template <int D>
__global__ __launch_bounds__(kSelThreads) void select_scores_kernel(
    const int32_t* __restrict__ tab, int32_t off_seqs, int32_t off_units, int32_t layer, int32_t B,
    int32_t Hkv, int32_t G, int32_t Hq, int32_t T, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ kd, float c, float* __restrict__ ws_s,
    float* __restrict__ ws_part, int32_t nblk) {
  constexpr int KS = D / 32;  // 32-dim steps of the contraction
  const int b = blockIdx.y / Hkv, h = blockIdx.y % Hkv, blk = blockIdx.x;
  const int32_t* ur = tab + off_units + kUnitInts * ((layer * B + b) * Hkv + h);
  if (ur[U_KIND] != SEGPAGED_RETRIEVAL) return;
  const int32_t N = tab[off_seqs + kSeqInts * b + S_N];
  const int32_t kvo = tab[off_seqs + kSeqInts * b + S_KVOFF];
  if (blk * kSelKeys >= N) return;  // uniform over the workgroup
  __shared__ float ssc[kSelKeys][kMaxGroup + 1];  // padded: a thread's row in its own bank
  __shared__ float red[kMaxGroup][4][2];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  // Q^T operand: head n (zero past G), dims 32 ks + 8 g .. + 7
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (n < G) w = *reinterpret_cast<const u32x4*>(q + ((int64_t)b * Hq + h * G + n) * D + ks * 32 + g * 8);
    qf[ks] = __builtin_bit_cast(bf16x8, w);
  }
  // K operands of the wave's 4 tiles of 16 keys, every load in flight at once
  u32x4 kv[4][KS];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int32_t j = blk * kSelKeys + wave * 64 + t * 16 + n;
    const uint16_t* row = kd + ((int64_t)(kvo + min(j, N - 1)) * Hkv + h) * D + g * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kv[t][ks] = *reinterpret_cast<const u32x4*>(row + ks * 32);
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kv[t][ks]), qf[ks],
                                                    acc, 0, 0, 0);
    if (n < G) {
#pragma unroll
      for (int i = 0; i < 4; ++i) ssc[wave * 64 + t * 16 + 4 * g + i][n] = acc[i] * c;
    }
  }
  __syncthreads();
  // thread t: key t of the block. Per head, each wave's max and exp-sum in one
  // pass, then the four waves merged in order by thread g < G.
  const int32_t j = blk * kSelKeys + (int32_t)threadIdx.x;
  const bool ok = j < N;
  float* srow = ws_s + ((int64_t)h * T + kvo + j) * G;
#pragma unroll
  for (int g = 0; g < kMaxGroup; ++g) {
    if (g < G) {
      const float sv = ok ? ssc[threadIdx.x][g] : -INFINITY;
      if (ok) srow[g] = sv;
      const float m = wave_max(sv);  // -inf only for a wave past the last key
      const float l = wave_sum(ok ? exp2f(sv - (m == -INFINITY ? 0.f : m)) : 0.f);
      if (lane == 0) {
        red[g][wave][0] = m;
        red[g][wave][1] = l;
      }
    }
  }
  __syncthreads();
  if ((int)threadIdx.x < G) {
    const int g = threadIdx.x;
    float mb = red[g][0][0];
    for (int w = 1; w < 4; ++w) mb = fmaxf(mb, red[g][w][0]);
    float lb = 0.f;
    for (int w = 0; w < 4; ++w)
      if (red[g][w][0] != -INFINITY) lb += red[g][w][1] * exp2f(red[g][w][0] - mb);
    float* part = ws_part + (((int64_t)h * B + b) * nblk + blk) * G * 2 + 2 * g;
    part[0] = mb;
    part[1] = lb;
  }
}

// Top-p over the keys of (b, h), one workgroup of kTopThreads per pair: the
// masses come from the workspace (held in registers, row-major over the threads,
// up to kTopThreads * kRegKeys keys), the first radix pass from the
// merged chunk histograms, then three more passes on the masses' bits, 8 bits per
// pass, larger values first. Each bin's mass is summed
// in fixed point (mass * 2^40, 64-bit integer adds), so the sums are exact and
// the same on every call.
constexpr int kTopThreads = 1024;
constexpr int kTopWaves = kTopThreads / 64;
constexpr int kRegKeys = 32;  // keys per thread whose mass bits stay in registers

__device__ __forceinline__ unsigned long long to_fx(float m) {
  return (unsigned long long)(m * 1099511627776.0f);  // exact scaling, truncated
}

__device__ unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Radix-select step over 256 bins (counts hc, fixed-point masses hs), taken from
// the largest bin down: the chosen bin is the largest k whose bins k..255 hold a
// mass of at least R (that bin holds mass, so it is not empty); when all of them
// hold less (candidates below the fixed-point step) it is the lowest non-empty
// bin. acc is the mass of the bins above the chosen one. Threads 0..255 take one
// bin each, in reverse so that a prefix scan gives the sums from the top.
struct BinPick {
  unsigned long long wsum[4];
  int kstar, low, chosen;
  unsigned long long acc;
};
__device__ void choose_bin(const unsigned int* hc, const unsigned long long* hs,
                           unsigned long long R, BinPick& bp) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k = 255 - tid;
  unsigned long long v = 0, incl = 0;
  if (tid == 0) {
    bp.kstar = -1;
    bp.low = 256;
  }
  if (tid < 256) {
    v = hs[k];
    incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const unsigned long long y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    if (lane == 63) bp.wsum[wave] = incl;
  }
  __syncthreads();
  if (tid < 256) {
    for (int w = 0; w < wave; ++w) incl += bp.wsum[w];  // mass of bins k..255
    const unsigned long long ge = __ballot(incl >= R);  // holds for k <= kstar
    const unsigned long long ne = __ballot(hc[k] != 0u);
    if (lane == 0 && ge) atomicMax(&bp.kstar, 255 - (wave * 64 + __ffsll((long long)ge) - 1));
    if (lane == 0 && ne) atomicMin(&bp.low, 255 - (wave * 64 + 63 - __clzll((long long)ne)));
  }
  __syncthreads();
  const int chosen = bp.kstar >= 0 ? bp.kstar : bp.low;
  if (tid < 256 && k == chosen) {
    bp.chosen = chosen;
    bp.acc = incl - v;
  }
  __syncthreads();
}
// exclusive prefix sum in thread order
__device__ int block_scan_top(int v, int* wtot, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  __syncthreads();
  if (lane == 63) wtot[wave] = x;
  __syncthreads();
  int base = 0;
  total = 0;
  for (int w = 0; w < kTopWaves; ++w) {
    if (w < wave) base += wtot[w];
    total += wtot[w];
  }
  return base + x - v;
}

// (m, l) <- the merge of two (max, exp-sum) pairs in log2 units; empty is (-inf, 0)
__device__ __forceinline__ void merge_ml(float& m, float& l, float m2, float l2) {
  if (m2 == -INFINITY) return;
  if (m == -INFINITY) {
    m = m2;
    l = l2;
    return;
  }
  const float mx = fmaxf(m, m2);
  l = l * exp2f(m - mx) + l2 * exp2f(m2 - mx);
  m = mx;
}

// The G normalisers of a pair from the block partials of the scores kernel, with
// the threads of one workgroup of NT, into sm (max, log2 units) and sl (1/sum).
// One pass: each thread merges its share of the partials (all G heads' loads in
// flight at once); in each wave the max by a fixed xor tree, then every lane's sum
// rescaled to it and added by the same tree; then the waves in order.
template <int NT>
__device__ void pair_normalisers(const float* part, int nb, int G, float* sm, float* sl,
                                 float (*redm)[kMaxGroup], float (*redl)[kMaxGroup]) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float m[kMaxGroup], l[kMaxGroup];
#pragma unroll
  for (int g = 0; g < kMaxGroup; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
  }
  for (int k = tid; k < nb; k += NT) {
    float pm[kMaxGroup], pv[kMaxGroup];
#pragma unroll
    for (int g = 0; g < kMaxGroup; ++g) {  // heads past G re-read head G - 1, unused
      const int64_t e = ((int64_t)k * G + min(g, G - 1)) * 2;
      pm[g] = part[e];
      pv[g] = part[e + 1];
    }
#pragma unroll
    for (int g = 0; g < kMaxGroup; ++g)
      if (g < G) merge_ml(m[g], l[g], pm[g], pv[g]);
  }
#pragma unroll
  for (int g = 0; g < kMaxGroup; ++g) {
    if (g < G) {
      const float mw = wave_max(m[g]);
      const float lw = wave_sum(m[g] == -INFINITY ? 0.f : l[g] * exp2f(m[g] - mw));
      if (lane == 0) {
        redm[wave][g] = mw;
        redl[wave][g] = lw;
      }
    }
  }
  __syncthreads();
  if (tid < G) {
    float mt = redm[0][tid], lt = redl[0][tid];
    for (int w = 1; w < NW; ++w) merge_ml(mt, lt, redm[w][tid], redl[w][tid]);
    sm[tid] = mt;
    sl[tid] = 1.f / lt;
  }
  __syncthreads();
}

// Masses of keys [chunk * kSelChunk, +kSelChunk) of a pair (mean over the G heads
// of each head's softmax weight), into ws_m, and the chunk's histogram of the
// masses' top 8 bits: counts, and mass sums in fixed point (mass * 2^40) with the
// chunk's total in bin 256.
constexpr int kMassThreads = 256;
__global__ __launch_bounds__(kMassThreads) void select_mass_kernel(
    const int32_t* __restrict__ tab, int32_t off_seqs, int32_t off_units, int32_t layer, int32_t B,
    int32_t Hkv, int32_t G, int32_t T, const float* __restrict__ ws_s,
    const float* __restrict__ ws_part, int32_t nblk, float* __restrict__ ws_m,
    unsigned long long* __restrict__ hsum, unsigned int* __restrict__ hcnt, int32_t nchunk) {
  const int b = blockIdx.y / Hkv, h = blockIdx.y % Hkv, ch = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t* ur = tab + off_units + kUnitInts * ((layer * B + b) * Hkv + h);
  const int32_t N = tab[off_seqs + kSeqInts * b + S_N];
  const int32_t kvo = tab[off_seqs + kSeqInts * b + S_KVOFF];
  if (ur[U_KIND] != SEGPAGED_RETRIEVAL || ch * kSelChunk >= N) return;  // uniform
  __shared__ float sm[kMaxGroup], sl[kMaxGroup];
  __shared__ float redm[kMassThreads / 64][kMaxGroup], redl[kMassThreads / 64][kMaxGroup];
  // a bin's count (at most kSelChunk < 2^12) in bits 52..63 and its fixed-point mass
  // (below 2^52: the chunk's masses sum to at most about 1, i.e. 2^40) below: one
  // atomic per key
  static_assert(kSelChunk < (1 << 12), "bin counts take 12 bits");
  __shared__ unsigned long long hp[256];
  __shared__ unsigned long long redu[kMassThreads / 64];
  for (int k = tid; k < 256; k += kMassThreads) hp[k] = 0;
  const float* S = ws_s + ((int64_t)h * T + kvo) * G;
  float* Mg = ws_m + (int64_t)h * T + kvo;
  const float inv_g = 1.f / (float)G;
  unsigned long long tfx = 0;
  constexpr int kPer = kSelChunk / kMassThreads;  // keys per thread, all loads in flight
  const int32_t j0 = ch * kSelChunk + tid;
  // G a multiple of 4: the thread's scores (16-byte loads) are requested before the
  // normalisers, so their latency passes under those reductions
  const bool vec = (G & 3) == 0;
  float4 xs[kMaxGroup / 4][kPer];
  if (vec) {
#pragma unroll
    for (int gq = 0; gq < kMaxGroup / 4; ++gq)
      if (4 * gq < G)
#pragma unroll
        for (int u = 0; u < kPer; ++u)
          xs[gq][u] = *reinterpret_cast<const float4*>(
              S + (int64_t)min(j0 + u * kMassThreads, N - 1) * G + 4 * gq);
  }
  const int nb = (N + kSelKeys - 1) / kSelKeys;
  pair_normalisers<kMassThreads>(ws_part + ((int64_t)h * B + b) * nblk * G * 2, nb, G, sm, sl,
                                 redm, redl);
  float m[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) m[u] = 0.f;
  if (vec) {
#pragma unroll
    for (int gq = 0; gq < kMaxGroup / 4; ++gq) {
      if (4 * gq < G) {
        const int g = 4 * gq;
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
          m[u] += __builtin_amdgcn_exp2f(xs[gq][u].x - sm[g]) * sl[g];
          m[u] += __builtin_amdgcn_exp2f(xs[gq][u].y - sm[g + 1]) * sl[g + 1];
          m[u] += __builtin_amdgcn_exp2f(xs[gq][u].z - sm[g + 2]) * sl[g + 2];
          m[u] += __builtin_amdgcn_exp2f(xs[gq][u].w - sm[g + 3]) * sl[g + 3];
        }
      }
    }
  } else {
    for (int g = 0; g < G; ++g) {
      float x[kPer];
#pragma unroll
      for (int u = 0; u < kPer; ++u) x[u] = S[(int64_t)min(j0 + u * kMassThreads, N - 1) * G + g];
#pragma unroll
      for (int u = 0; u < kPer; ++u) m[u] += __builtin_amdgcn_exp2f(x[u] - sm[g]) * sl[g];
    }
  }
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int32_t j = j0 + u * kMassThreads;
    if (j < N) {
      const float mu = m[u] * inv_g;
      Mg[j] = mu;
      const unsigned long long fx = to_fx(mu);
      tfx += fx;
      const uint32_t bin = __float_as_uint(mu) >> 24;
      atomicAdd(&hp[bin], (1ull << 52) + fx);
    }
  }
  tfx = wave_sum_u64(tfx);
  if ((tid & 63) == 0) redu[tid >> 6] = tfx;
  __syncthreads();
  const int64_t rec = ((int64_t)h * B + b) * nchunk + ch;
  for (int k = tid; k < 256; k += kMassThreads) {
    hsum[rec * 257 + k] = hp[k] & ((1ull << 52) - 1);
    hcnt[rec * 256 + k] = (unsigned int)(hp[k] >> 52);
  }
  if (tid == 0) {
    unsigned long long t = 0;
    for (int w = 0; w < kMassThreads / 64; ++w) t += redu[w];
    hsum[rec * 257 + 256] = t;
  }
}

__global__ __launch_bounds__(kTopThreads) void select_topp_kernel(
    const int32_t* __restrict__ tab, int32_t off_seqs, int32_t off_units, int32_t layer, int32_t B,
    int32_t Hkv, int32_t T, const float* __restrict__ ws_m,
    const unsigned long long* __restrict__ hsum, const unsigned int* __restrict__ hcnt,
    int32_t nchunk, float p, int32_t* __restrict__ out_pos, int32_t* __restrict__ out_cnt) {
  const int b = blockIdx.x / Hkv, h = blockIdx.x % Hkv;
  const int tid = threadIdx.x;
  const int32_t* ur = tab + off_units + kUnitInts * ((layer * B + b) * Hkv + h);
  const int32_t N = tab[off_seqs + kSeqInts * b + S_N];
  const int32_t kvo = tab[off_seqs + kSeqInts * b + S_KVOFF];
  if (ur[U_KIND] != SEGPAGED_RETRIEVAL || N == 0) {
    if (tid == 0) out_cnt[b * Hkv + h] = 0;
    return;
  }
  __shared__ unsigned int hc[256];
  __shared__ unsigned long long hs[257];
  __shared__ int wtot[kTopWaves];
  __shared__ BinPick bp;
  __shared__ int rc[kRegKeys * kTopWaves];  // per (row, wave): counts, then their prefix
  const float* Mg = ws_m + (int64_t)h * T + kvo;
  const int lane = tid & 63, wave = tid >> 6;
  // Up to kTopThreads * kRegKeys keys, thread t holds the mass bits of keys
  // i * kTopThreads + t (row i) in registers for every pass (coalesced loads);
  // beyond that each thread takes a run of consecutive keys from the workspace.
  const bool in_reg = N <= kTopThreads * kRegKeys;
  uint32_t mu[kRegKeys];
  if (in_reg) {
#pragma unroll
    for (int i = 0; i < kRegKeys; ++i)
      mu[i] = __float_as_uint(Mg[min(i * kTopThreads + tid, N - 1)]);  // past N: unused
  }
  auto valid = [&](int i) { return i * kTopThreads + tid < N; };
  // the first radix pass and the total from the chunk histograms (integer sums)
  const int nch = (N + kSelChunk - 1) / kSelChunk;
  const int64_t rec0 = ((int64_t)h * B + b) * nchunk;
  if (tid < 257) {  // chunks 8 at a time, their loads in flight together
    unsigned long long t = 0;
    unsigned int c = 0;
    for (int q0 = 0; q0 < nch; q0 += 8) {
      unsigned long long a[8];
      unsigned int n8[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t r = rec0 + min(q0 + u, nch - 1);
        a[u] = hsum[r * 257 + tid];
        n8[u] = hcnt[r * 256 + min(tid, 255)];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (q0 + u < nch) { t += a[u]; c += n8[u]; }
    }
    hs[tid] = t;
    if (tid < 256) hc[tid] = c;
  }
  __syncthreads();
  const unsigned long long total = hs[256];
  unsigned long long R = (unsigned long long)((double)p * (double)total);  // still to take
  if (R == 0) R = 1;
  uint32_t prefix = 0, mask = 0;
  unsigned int c_eq = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (shift < 24) {  // the first pass's histogram came from the chunks
      for (int k = tid; k < 256; k += kTopThreads) { hc[k] = 0; hs[k] = 0; }
      __syncthreads();
      auto count = [&](uint32_t u) {
        if ((u & mask) == prefix) {
          const uint32_t bin = (u >> shift) & 255u;
          atomicAdd(&hc[bin], 1u);
          atomicAdd(&hs[bin], to_fx(__uint_as_float(u)));
        }
      };
      if (in_reg) {
#pragma unroll
        for (int i = 0; i < kRegKeys; ++i)
          if (valid(i)) count(mu[i]);
      } else {
        for (int32_t jb = 0; jb < N; jb += 4 * kTopThreads) {
          uint32_t u[4];
#pragma unroll
          for (int x = 0; x < 4; ++x) u[x] = __float_as_uint(Mg[min(jb + x * kTopThreads + tid, N - 1)]);
#pragma unroll
          for (int x = 0; x < 4; ++x)
            if (jb + x * kTopThreads + tid < N) count(u[x]);
        }
      }
      __syncthreads();
    }
    choose_bin(hc, hs, R, bp);
    R -= bp.acc;
    prefix |= (uint32_t)bp.chosen << shift;
    mask |= 255u << shift;
    c_eq = hc[bp.chosen];
    __syncthreads();
  }
  // keys of mass above the threshold, then the first t (by position) equal to it
  const unsigned long long tau_fx = to_fx(__uint_as_float(prefix));
  int t = (int)c_eq;
  if (tau_fx > 0) t = (int)min((unsigned long long)c_eq, max(1ull, (R + tau_fx - 1) / tau_fx));
  const bool all_ties = t >= (int)c_eq;  // uniform
  int32_t* out = out_pos + (int64_t)h * T + kvo;
  if (in_reg) {
    // Position order is row-major over (row i, lane t): a key's rank among the
    // flagged keys is the flagged count of the (row, wave) pairs before its own
    // plus its lanes below it in the wave's ballot.
    auto rank_base = [&](auto flag, int& total_out) {
#pragma unroll
      for (int i = 0; i < kRegKeys; ++i) {
        const unsigned long long bal = __ballot(flag(i));
        if (lane == 0) rc[i * kTopWaves + wave] = __popcll(bal);
      }
      __syncthreads();
      const int v = tid < kRegKeys * kTopWaves ? rc[tid] : 0;
      const int base = block_scan_top(v, wtot, total_out);
      __syncthreads();  // every count read before the prefixes overwrite them
      if (tid < kRegKeys * kTopWaves) rc[tid] = base;
      __syncthreads();
    };
    auto below = [&](unsigned long long bal) {
      return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                             __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
    };
    bool sel[kRegKeys];
    if (all_ties) {
#pragma unroll
      for (int i = 0; i < kRegKeys; ++i) sel[i] = valid(i) && mu[i] >= prefix;
    } else {  // the ties' ranks by position decide which of them are taken
      int ties_total;
      auto tie = [&](int i) { return valid(i) && mu[i] == prefix; };
      rank_base(tie, ties_total);
#pragma unroll
      for (int i = 0; i < kRegKeys; ++i) {
        const bool ti = tie(i);
        const int rank = rc[i * kTopWaves + wave] + below(__ballot(ti));
        sel[i] = valid(i) && (mu[i] > prefix || (ti && rank < t));
      }
      __syncthreads();  // ranks read before the selection counts overwrite them
    }
    int nsel_total;
    rank_base([&](int i) { return sel[i]; }, nsel_total);
#pragma unroll
    for (int i = 0; i < kRegKeys; ++i) {
      const unsigned long long bal = __ballot(sel[i]);
      if (sel[i]) out[rc[i * kTopWaves + wave] + below(bal)] = i * kTopThreads + tid;
    }
    if (tid == 0) out_cnt[b * Hkv + h] = nsel_total;
    return;
  }
  // runs of consecutive keys per thread, masses from the workspace
  const int32_t per = (N + kTopThreads - 1) / kTopThreads;
  const int32_t lo = min(N, tid * per), hi = min(N, lo + per);
  int tie_base = 0;
  if (!all_ties) {  // only the first t ties by position are taken: count them first
    int ties = 0;
    for (int32_t j = lo; j < hi; ++j) ties += __float_as_uint(Mg[j]) == prefix;
    int ties_total;
    tie_base = block_scan_top(ties, wtot, ties_total);
  }
  int nsel = 0, tr = tie_base;
  auto take = [&](uint32_t u) {  // in position order within the run
    const bool s_ = u > prefix || (u == prefix && tr < t);
    tr += u == prefix;
    return s_;
  };
  for (int32_t j = lo; j < hi; ++j) nsel += take(__float_as_uint(Mg[j]));
  int nsel_total;
  int pos = block_scan_top(nsel, wtot, nsel_total);
  tr = tie_base;
  for (int32_t j = lo; j < hi; ++j)
    if (take(__float_as_uint(Mg[j]))) out[pos++] = j;
  if (tid == 0) out_cnt[b * Hkv + h] = nsel_total;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

}  // namespace

extern "C" {

SEGPAGED_API int segpaged_select_topp(const segpaged_plan* pl, int32_t layer, const void* q,
                                      const void* k_dense, const int32_t* d_table, float scale,
                                      float p, int32_t* out_pos, int32_t* out_cnt, void* workspace,
                                      int64_t workspace_bytes, void* stream) {
  if (!pl || !q || !k_dense || !d_table || !out_pos || !out_cnt || !workspace)
    return SEGPAGED_EINVAL;
  if (!aligned16(q) || !aligned16(k_dense) || !aligned4(d_table) || !aligned4(out_pos) ||
      !aligned4(out_cnt) || !aligned16(workspace))
    return SEGPAGED_EINVAL;
  if (!(scale > 0.f) || !std::isfinite(scale) || !(p > 0.f) || !(p <= 1.f)) return SEGPAGED_EINVAL;
  if (layer < 0 || layer >= pl->L) return SEGPAGED_ESTATE;
  const int64_t B = pl->B, Hkv = pl->Hkv, G = pl->G, T = pl->kv_rows;
  int64_t nmax = 0;
  for (int64_t b = 0; b < B; ++b)
    nmax = std::max<int64_t>(nmax, pl->buf[pl->off_seqs + kSeqInts * b + S_N]);
  const int64_t nblk = std::max<int64_t>(1, (nmax + kSelKeys - 1) / kSelKeys);
  const int64_t s_floats = Hkv * T * G, m_floats = Hkv * T, part_floats = Hkv * B * nblk * G * 2;
  const int64_t nchunk = std::max<int64_t>(1, (nmax + kSelChunk - 1) / kSelChunk);
  const int64_t hist_off = (4 * (s_floats + m_floats + part_floats) + 15) / 16 * 16;
  const int64_t need = hist_off + Hkv * B * nchunk * (257 * 8 + 256 * 4);
  if (workspace_bytes < need) return SEGPAGED_ENOSPACE;
  float* ws_s = (float*)workspace;
  float* ws_m = ws_s + s_floats;
  float* ws_part = ws_m + m_floats;
  unsigned long long* hsum = (unsigned long long*)((char*)workspace + hist_off);
  unsigned int* hcnt = (unsigned int*)(hsum + Hkv * B * nchunk * 257);
  hipStream_t st = (hipStream_t)stream;
  const float c = scale * kLog2eSel;
  const dim3 g1((unsigned)nblk, (unsigned)(B * Hkv)), blk(kSelThreads);
  if (pl->D == 128)
    hipLaunchKernelGGL(select_scores_kernel<128>, g1, blk, 0, st, d_table, (int32_t)pl->off_seqs,
                       (int32_t)pl->off_units, layer, (int32_t)B, (int32_t)Hkv, (int32_t)G, pl->Hq,
                       (int32_t)T, (const uint16_t*)q, (const uint16_t*)k_dense, c, ws_s, ws_part,
                       (int32_t)nblk);
  else
    hipLaunchKernelGGL(select_scores_kernel<64>, g1, blk, 0, st, d_table, (int32_t)pl->off_seqs,
                       (int32_t)pl->off_units, layer, (int32_t)B, (int32_t)Hkv, (int32_t)G, pl->Hq,
                       (int32_t)T, (const uint16_t*)q, (const uint16_t*)k_dense, c, ws_s, ws_part,
                       (int32_t)nblk);
  if (hipGetLastError() != hipSuccess) return SEGPAGED_EHIP;
  hipLaunchKernelGGL(select_mass_kernel, dim3((unsigned)nchunk, (unsigned)(B * Hkv)),
                     dim3(kMassThreads), 0, st, d_table, (int32_t)pl->off_seqs,
                     (int32_t)pl->off_units, layer, (int32_t)B, (int32_t)Hkv, (int32_t)G,
                     (int32_t)T, ws_s, ws_part, (int32_t)nblk, ws_m, hsum, hcnt, (int32_t)nchunk);
  if (hipGetLastError() != hipSuccess) return SEGPAGED_EHIP;
  hipLaunchKernelGGL(select_topp_kernel, dim3((unsigned)(B * Hkv)), dim3(kTopThreads), 0, st,
                     d_table, (int32_t)pl->off_seqs, (int32_t)pl->off_units, layer, (int32_t)B,
                     (int32_t)Hkv, (int32_t)T, ws_m, hsum, hcnt, (int32_t)nchunk, p, out_pos,
                     out_cnt);
  return hipGetLastError() == hipSuccess ? SEGPAGED_OK : SEGPAGED_EHIP;
}

}  // extern "C"
