// Unpermute + top-k weighted combine (page 3, "矩阵融合" pipeline figure:
// restore token order and sum by routing weight).
//
// out[t, :] = bf16( residual[t, :] + sum_{j<k} w[t, j] * C2[inv[t*k + j], :] )
// with the sum taken in fp32, j ascending, and one rounding to bf16 at the
// end.  A gather (each token reads its k rows), not a scatter-add, so the
// result is deterministic.  One thread produces 8 consecutive outputs: two
// 16-byte loads per source row and one 16-byte store.  HBM-bound.
#include "internal.h"
#include "nvfp4_device.h"

namespace nvfp4 {

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ c2,
                                                      const float* __restrict__ w,
                                                      const int32_t* __restrict__ inv, int32_t T,
                                                      int32_t k, int32_t H,
                                                      const uint16_t* residual, uint16_t* out) {
  const int32_t h8 = H / 8;
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= (int64_t)T * h8) return;
  const int32_t t = (int32_t)(g / h8);
  const int32_t c = (int32_t)(g - (int64_t)t * h8) * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // Slots in groups of kU: the group's row indices first, then all its row
  // loads, then the sums in slot order (slots past k re-read row k-1 and are
  // not added), so each thread keeps 2 kU loads in flight instead of a chain
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
    f32x4 a[kU], b[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const f32x4* src = reinterpret_cast<const f32x4*>(c2 + (int64_t)row[u] * H + c);
      a[u] = __builtin_nontemporal_load(src);
      b[u] = __builtin_nontemporal_load(src + 1);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (j0 + u < k) {
        acc[0] += wj[u] * a[u].x; acc[1] += wj[u] * a[u].y;
        acc[2] += wj[u] * a[u].z; acc[3] += wj[u] * a[u].w;
        acc[4] += wj[u] * b[u].x; acc[5] += wj[u] * b[u].y;
        acc[6] += wj[u] * b[u].z; acc[7] += wj[u] * b[u].w;
      }
    }
  }
  if (residual) {
    const uint4 r = *reinterpret_cast<const uint4*>(residual + (int64_t)t * H + c);
    float rv[8];
    unpack_bf16x8(r, rv);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += rv[i];
  }
  uint4 o;
  o.x = f32_to_bf16(acc[0]) | (f32_to_bf16(acc[1]) << 16);
  o.y = f32_to_bf16(acc[2]) | (f32_to_bf16(acc[3]) << 16);
  o.z = f32_to_bf16(acc[4]) | (f32_to_bf16(acc[5]) << 16);
  o.w = f32_to_bf16(acc[6]) | (f32_to_bf16(acc[7]) << 16);
  *reinterpret_cast<uint4*>(out + (int64_t)t * H + c) = o;
}

hipError_t launch_combine(const float* c2, const float* w, const int32_t* inv, int32_t T,
                          int32_t k, int32_t H, const uint16_t* residual, uint16_t* out,
                          hipStream_t stream) {
  const int64_t total = (int64_t)T * (H / 8);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3((uint32_t)((total + 255) / 256)), dim3(256), 0, stream,
                     c2, w, inv, T, k, H, residual, out);
  return hipGetLastError();
}

}  // namespace nvfp4
