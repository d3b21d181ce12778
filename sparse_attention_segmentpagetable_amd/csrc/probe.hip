// Measurement probes (libsegpaged_probe.so): sustained dense bf16 MFMA rate and
// streaming HBM read rate on gfx950. Used to report the attention kernels'
// achieved rates against what the chip reaches, next to the published peaks.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "segpaged_probe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// 8 waves per workgroup (two per SIMD), four independent accumulator chains per
// wave; 8 MFMAs per iteration with the operand pairs rotating.
__global__ __launch_bounds__(512) void mfma_probe_kernel(const uint4* __restrict__ seed,
                                                         int32_t iters, float* __restrict__ out) {
  const int tid = threadIdx.x;
  bf16x8 a[4], b[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    a[r] = __builtin_bit_cast(bf16x8, seed[(2 * r) * 512 + tid]);
    b[r] = __builtin_bit_cast(bf16x8, seed[(2 * r + 1) * 512 + tid]);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int32_t it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[0], c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], b[1], c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2], b[2], c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[3], b[3], c3, 0, 0, 0);
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], b[2], c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2], b[3], c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[3], b[0], c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[1], c3, 0, 0, 0);
  }
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) r += (c0[i] + c1[i]) + (c2[i] + c3[i]);
  out[(int64_t)blockIdx.x * 512 + tid] = r;
}

// Grid-stride streaming read of n16 16-byte chunks, DEPTH loads in flight per
// thread; each workgroup writes the fp32 sum of what it read.
template <int DEPTH>
__global__ __launch_bounds__(256) void hbm_read_probe_kernel(const f32x4* __restrict__ src,
                                                             int64_t n16, float* __restrict__ out) {
  __shared__ float part[4];
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  float acc = 0.f;
  for (; i + (DEPTH - 1) * stride < n16; i += DEPTH * stride) {
    f32x4 v[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) v[d] = __builtin_nontemporal_load(src + i + d * stride);
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) acc += (v[d].x + v[d].y) + (v[d].z + v[d].w);
  }
  for (; i < n16; i += stride) {
    const f32x4 v = src[i];
    acc += (v.x + v.y) + (v.z + v.w);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = (part[0] + part[1]) + (part[2] + part[3]);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int launch_status() { return hipGetLastError() == hipSuccess ? SEGPAGED_OK : SEGPAGED_EHIP; }

}  // namespace

extern "C" {

SEGPAGED_API int segpaged_probe_mfma_bf16(const void* seed, int32_t iters, int32_t workgroups,
                                          float* out, void* stream) {
  if (!seed || !out || !aligned16(seed) || !aligned16(out) || iters < 1 || workgroups < 1)
    return SEGPAGED_EINVAL;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)workgroups), dim3(512), 0,
                     (hipStream_t)stream, (const uint4*)seed, iters, out);
  return launch_status();
}

SEGPAGED_API int segpaged_probe_hbm_read(const void* src, int64_t bytes, int32_t workgroups,
                                         int32_t depth, float* out, void* stream) {
  if (!src || !out || !aligned16(src) || bytes <= 0 || bytes % 16 != 0 || workgroups < 1 ||
      (depth != 4 && depth != 8 && depth != 16))
    return SEGPAGED_EINVAL;
  const dim3 grid((unsigned)workgroups), block(256);
  hipStream_t st = (hipStream_t)stream;
  const f32x4* s4 = (const f32x4*)src;
  if (depth == 4) hipLaunchKernelGGL(hbm_read_probe_kernel<4>, grid, block, 0, st, s4, bytes / 16, out);
  else if (depth == 8) hipLaunchKernelGGL(hbm_read_probe_kernel<8>, grid, block, 0, st, s4, bytes / 16, out);
  else hipLaunchKernelGGL(hbm_read_probe_kernel<16>, grid, block, 0, st, s4, bytes / 16, out);
  return launch_status();
}

}  // extern "C"
