// Router top-k and the stable regrouping of (token, slot) pairs by expert.
//
// Page 3, "NVFP4" runtime figure: the router fixes expert_idx before the
// activation quantiser runs; "矩阵融合", MoE FFN paragraph: the backend
// reorders rows by routing so each expert's rows form one group of a grouped
// GEMM, and the pipeline figure ends by restoring token order and summing by
// routing weight.
//
// route_topk: one wavefront per token.  Lanes hold the token's logits
// (E <= 64 * EPL); k rounds of a wave-wide argmax, ordered by (logit
// descending, expert index ascending), pick the experts; the k weights are a
// softmax over the picked logits in fp32.
//
// permute: one workgroup per expert.  Each thread owns a contiguous segment
// of the pair array, so a block-wide exclusive scan of per-thread match
// counts gives every match its stable rank (token-major order) without
// atomics; the count of smaller expert ids gives the expert's offset.
#include <float.h>

#include "internal.h"

namespace nvfp4 {

template <int EPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits,
                                                         int32_t T, int32_t E, int32_t k,
                                                         int32_t* __restrict__ ids,
                                                         float* __restrict__ weights) {
  const int lane = threadIdx.x & 63;
  const int32_t t = (int32_t)blockIdx.x * 4 + (int32_t)(threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (int64_t)t * E;
  float v[EPL];
  bool taken[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? row[e] : -INFINITY;
    taken[i] = e >= E;
  }
  int32_t my_id = 0;
  float my_val = 0.0f;
  for (int r = 0; r < k; ++r) {
    float bv = -INFINITY;
    int32_t bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i;
      if (!taken[i] && (v[i] > bv || (v[i] == bv && e < bi))) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int32_t oi = __shfl_xor(bi, off, 64);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (bi == lane + 64 * i) taken[i] = true;
    if (lane == r) {
      my_id = bi;
      my_val = bv;
    }
  }
  const float mx = __shfl(my_val, 0, 64);                 // pick 0 is the largest
  float ex = lane < k ? expf(my_val - mx) : 0.0f;
  float sum = ex;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
  if (lane < k) {
    ids[(int64_t)t * k + lane] = my_id;
    weights[(int64_t)t * k + lane] = ex / sum;
  }
}

hipError_t launch_route(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* ids,
                        float* weights, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const dim3 grid((T + 3) / 4), block(256);
  if (E <= 64)
    hipLaunchKernelGGL(route_topk_kernel<1>, grid, block, 0, stream, logits, T, E, k, ids, weights);
  else if (E <= 128)
    hipLaunchKernelGGL(route_topk_kernel<2>, grid, block, 0, stream, logits, T, E, k, ids, weights);
  else if (E <= 256)
    hipLaunchKernelGGL(route_topk_kernel<4>, grid, block, 0, stream, logits, T, E, k, ids, weights);
  else if (E <= 512)
    hipLaunchKernelGGL(route_topk_kernel<8>, grid, block, 0, stream, logits, T, E, k, ids, weights);
  else
    hipLaunchKernelGGL(route_topk_kernel<16>, grid, block, 0, stream, logits, T, E, k, ids, weights);
  return hipGetLastError();
}

// Block-wide exclusive scan of one int per thread (256 threads).
__device__ __forceinline__ int32_t block_exclusive_scan(int32_t v, int32_t* total, int32_t* s_tmp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) s_tmp[wave] = incl;
  __syncthreads();
  int32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int32_t s = s_tmp[w];
    base += w < wave ? s : 0;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + incl - v;
}

__global__ __launch_bounds__(256) void permute_kernel(const int32_t* __restrict__ ids, int32_t P,
                                                      int32_t E, int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ src_pair,
                                                      int32_t* __restrict__ inv) {
  __shared__ int32_t s_tmp[4];
  const int32_t e = blockIdx.x;
  const int32_t seg = (P + 255) / 256;
  const int32_t q0 = min(P, (int32_t)threadIdx.x * seg);
  const int32_t q1 = min(P, q0 + seg);
  int32_t less = 0, eq = 0;
  for (int32_t q = q0; q < q1; ++q) {
    const int32_t id = ids[q];
    less += id < e;
    eq += id == e;
  }
  int32_t total_less, total_eq;
  (void)block_exclusive_scan(less, &total_less, s_tmp);
  const int32_t rank0 = block_exclusive_scan(eq, &total_eq, s_tmp);
  if (threadIdx.x == 0) {
    offsets[e] = total_less;
    if (e == E - 1) offsets[E] = total_less + total_eq;
  }
  if (eq == 0) return;
  int32_t p = total_less + rank0;
  for (int32_t q = q0; q < q1; ++q) {
    if (ids[q] == e) {
      src_pair[p] = q;
      inv[q] = p;
      ++p;
    }
  }
}

hipError_t launch_permute(const int32_t* ids, int32_t P, int32_t E, int32_t* offsets,
                          int32_t* src_pair, int32_t* inv, hipStream_t stream) {
  hipLaunchKernelGGL(permute_kernel, dim3(E), dim3(256), 0, stream, ids, P, E, offsets, src_pair,
                     inv);
  return hipGetLastError();
}

}  // namespace nvfp4
