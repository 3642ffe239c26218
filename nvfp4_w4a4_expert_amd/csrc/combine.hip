// Unpermute + top-k weighted combine (page 3, "矩阵融合" pipeline figure:
// restore token order and sum by routing weight).
//
// out[t, :] = bf16( residual[t, :] + sum_{j<k} w[t, j] * C2[inv[t*k + j], :] )
// with the sum taken in fp32, j ascending, and one rounding to bf16 at the
// end.  A gather (each token reads its k rows), not a scatter-add, so the
// result is deterministic.  One thread produces 4 consecutive outputs: one
// 16-byte load per source row and one 8-byte store (measured at 4096 tokens,
// top-8, hidden 2816 with the routed permutation: 78.3 -> 68.2 us against 8
// outputs per thread).  HBM-bound.
#include "internal.h"
#include "nvfp4_device.h"

namespace nvfp4 {

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ c2,
                                                      const float* __restrict__ w,
                                                      const int32_t* __restrict__ inv, int32_t T,
                                                      int32_t k, int32_t H,
                                                      const uint16_t* residual, uint16_t* out) {
  const int32_t h4 = H / 4;
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= (int64_t)T * h4) return;
  const int32_t t = (int32_t)(g / h4);
  const int32_t c = (int32_t)(g - (int64_t)t * h4) * 4;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  // Slots in groups of kU: the group's row indices first, then all its row
  // loads, then the sums in slot order (slots past k re-read row k-1 and are
  // not added), so each thread keeps kU loads in flight instead of a chain
  // of index load -> row load per slot.
  constexpr int kU = 8;
  const int64_t q0 = (int64_t)t * k;
  for (int32_t j0 = 0; j0 < k; j0 += kU) {
    int32_t row[kU];
    float wj[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int32_t j = min(j0 + u, k - 1);
      row[u] = inv[q0 + j];
      wj[u] = w[q0 + j];
    }
    f32x4 a[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u)
      a[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(c2 + (int64_t)row[u] * H + c));
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (j0 + u < k) {
        acc[0] += wj[u] * a[u].x; acc[1] += wj[u] * a[u].y;
        acc[2] += wj[u] * a[u].z; acc[3] += wj[u] * a[u].w;
      }
    }
  }
  if (residual) {
    const uint2 r = *reinterpret_cast<const uint2*>(residual + (int64_t)t * H + c);
    acc[0] += bf16_lo(r.x); acc[1] += bf16_hi(r.x);
    acc[2] += bf16_lo(r.y); acc[3] += bf16_hi(r.y);
  }
  uint2 o;
  o.x = f32_to_bf16(acc[0]) | (f32_to_bf16(acc[1]) << 16);
  o.y = f32_to_bf16(acc[2]) | (f32_to_bf16(acc[3]) << 16);
  *reinterpret_cast<uint2*>(out + (int64_t)t * H + c) = o;
}

hipError_t launch_combine(const float* c2, const float* w, const int32_t* inv, int32_t T,
                          int32_t k, int32_t H, const uint16_t* residual, uint16_t* out,
                          hipStream_t stream) {
  const int64_t total = (int64_t)T * (H / 4);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3((uint32_t)((total + 255) / 256)), dim3(256), 0, stream,
                     c2, w, inv, T, k, H, residual, out);
  return hipGetLastError();
}

}  // namespace nvfp4
