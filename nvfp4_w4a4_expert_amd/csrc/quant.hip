// Per-expert NVFP4 activation quantiser for gfx950 (page 3, "NVFP4" section,
// runtime-order figure; SFScale[expert_idx] excerpt).
//
// Token-major: one thread owns one 16-element block of one source row.  It
// loads the 32 bytes once, forms amax/6 once, and then, for each of the row's
// topk destinations, applies that expert's SFScaleVal, encodes the 16 codes
// and stores 8 bytes of packed codes plus one E4M3 byte.  Consecutive threads
// own consecutive blocks, so loads and stores of a wavefront are contiguous.
// The kernel is HBM-bound: it reads each source row once and writes
// topk * (K/2 + K/16) bytes per row.
#include "internal.h"
#include "nvfp4_device.h"

namespace nvfp4 {

__global__ __launch_bounds__(256) void quantize_experts_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int32_t num_rows, int32_t nblk, int32_t topk,
    const int32_t* __restrict__ expert_idx, const int32_t* __restrict__ dst_row,
    int32_t num_experts, const float* __restrict__ gscale, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ sf, int32_t num_dst_rows) {
#pragma clang fp contract(off)
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= (int64_t)num_rows * nblk) return;
  const int32_t t = (int32_t)(g / nblk);
  const int32_t b = (int32_t)(g - (int64_t)t * nblk);

  const u32x4* src = reinterpret_cast<const u32x4*>(x + (int64_t)t * ldx + (int64_t)b * 16);
  const u32x4 v0 = __builtin_nontemporal_load(src);
  const u32x4 v1 = __builtin_nontemporal_load(src + 1);
  float xv[16];
  unpack_bf16x8(v0, xv);
  unpack_bf16x8(v1, xv + 8);
  const float a6 = absmax16(xv) / kE2M1Max;

  const int64_t row_bytes = (int64_t)nblk * 8;
  for (int32_t j = 0; j < topk; ++j) {
    const int64_t q = (int64_t)t * topk + j;
    const int32_t e = expert_idx ? expert_idx[q] : 0;
    const int32_t p = dst_row ? dst_row[q] : (int32_t)q;
    if ((uint32_t)p >= (uint32_t)num_dst_rows || (uint32_t)e >= (uint32_t)num_experts) continue;
    const float gs = gscale ? gscale[e] : 1.0f;
    const BlockScale bs = block_scale(a6, gs);
    uint2 w;
    w.x = encode8(xv, bs.inv);
    w.y = encode8(xv + 8, bs.inv);
    *reinterpret_cast<uint2*>(codes + (int64_t)p * row_bytes + (int64_t)b * 8) = w;
    sf[(int64_t)p * nblk + b] = (uint8_t)bs.sf;
  }
}

hipError_t launch_quantize(const uint16_t* x, int64_t ldx, int32_t num_rows, int32_t K,
                           int32_t topk, const int32_t* expert_idx, const int32_t* dst_row,
                           int32_t num_experts, const float* gscale, uint8_t* codes, uint8_t* sf,
                           int32_t num_dst_rows, hipStream_t stream) {
  const int32_t nblk = K / 16;
  const int64_t total = (int64_t)num_rows * nblk;
  if (total == 0) return hipSuccess;
  const int64_t grid = (total + 255) / 256;
  hipLaunchKernelGGL(quantize_experts_kernel, dim3((uint32_t)grid), dim3(256), 0, stream, x, ldx,
                     num_rows, nblk, topk, expert_idx, dst_row, num_experts, gscale, codes, sf,
                     num_dst_rows);
  return hipGetLastError();
}

// Calibration statistic: per-expert max |x| over its grouped rows.  One block
// folds 16 consecutive grouped rows; each row's maximum is published to its
// expert with an unsigned atomic max (non-negative floats order like their
// bit patterns), so the result does not depend on scheduling.
__device__ __forceinline__ int32_t expert_of_row(const int32_t* offsets, int32_t E, int32_t r) {
  int32_t lo = 0, hi = E - 1;          // last e with offsets[e] <= r
  while (lo < hi) {
    const int32_t mid = (lo + hi + 1) >> 1;
    if (offsets[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(256) void absmax_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                     int32_t K, const int32_t* __restrict__ src,
                                                     int32_t src_div,
                                                     const int32_t* __restrict__ offsets,
                                                     int32_t E, int32_t num_rows,
                                                     uint32_t* __restrict__ amax_bits) {
  __shared__ float red[256];
  const int32_t n8 = K / 8;
  for (int32_t rr = 0; rr < 16; ++rr) {
    const int32_t r = (int32_t)blockIdx.x * 16 + rr;
    if (r >= num_rows) break;
    const int64_t row = src ? (int64_t)(src[r] / src_div) : (int64_t)r;
    const uint4* p = reinterpret_cast<const uint4*>(x + row * ldx);
    float m = 0.0f;
    for (int32_t c = threadIdx.x; c < n8; c += blockDim.x) {
      float v[8];
      unpack_bf16x8(p[c], v);
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
    }
    red[threadIdx.x] = m;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
      if ((int)threadIdx.x < s) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + s]);
      __syncthreads();
    }
    if (threadIdx.x == 0) atomicMax(amax_bits + expert_of_row(offsets, E, r), __float_as_uint(red[0]));
    __syncthreads();
  }
}

__global__ void fill_u32_kernel(uint32_t* p, int32_t n, uint32_t v) {
  const int32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_absmax(const uint16_t* x, int64_t ldx, int32_t K, const int32_t* src,
                         int32_t src_div, const int32_t* offsets, int32_t E, int32_t num_rows,
                         float* amax, hipStream_t stream) {
  hipLaunchKernelGGL(fill_u32_kernel, dim3((E + 255) / 256), dim3(256), 0, stream,
                     reinterpret_cast<uint32_t*>(amax), E, 0u);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || num_rows == 0) return err;
  hipLaunchKernelGGL(absmax_kernel, dim3((uint32_t)((num_rows + 15) / 16)), dim3(256), 0, stream,
                     x, ldx, K, src, src_div, offsets, E, num_rows,
                     reinterpret_cast<uint32_t*>(amax));
  return hipGetLastError();
}

}  // namespace nvfp4
