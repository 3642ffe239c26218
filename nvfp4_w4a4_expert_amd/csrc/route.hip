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
// permute: workgroups own consecutive blocks of pairs; each histograms all
// ids, derives the expert offsets, and ranks its block's pairs stably with
// wavefront ballots (see permute_kernel).
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

constexpr int kPermThreads = 512;                 // 8 wavefronts
constexpr int kPermWaves = kPermThreads / 64;
constexpr int kPermMaxE = 1024;

// Exclusive scan over the workgroup of one int per thread; *total receives
// the sum.  s_tmp holds kPermWaves ints.
__device__ __forceinline__ int32_t perm_exclusive_scan(int32_t v, int32_t* total,
                                                       int32_t* s_tmp) {
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
  for (int w = 0; w < kPermWaves; ++w) {
    const int32_t s = s_tmp[w];
    base += w < wave ? s : 0;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + incl - v;
}

// One workgroup per block of `span` consecutive pairs.
//  1. Every workgroup histograms all P ids in LDS, split into pairs before
//     its block and pairs from its block on; the counts are the same in
//     every workgroup whatever the order of the LDS additions.
//  2. An exclusive scan over experts of the totals gives expert offsets;
//     adding the counts before the block gives each expert's first row in
//     this block.
//  3. The block's pairs are walked in token-major order, 512 at a time.
//     Inside a wavefront, lanes holding the same expert are found with one
//     ballot per id bit; a lane's rank among them is the popcount of the
//     equal lanes below it.  Per-expert counts of the 8 wavefronts are
//     turned into running bases by one thread per expert, so ranks follow
//     pair order across wavefronts and across steps: the result is the
//     stable order.
// Ids outside [0, E) are left out of every count and never written.
__global__ __launch_bounds__(kPermThreads) void permute_kernel(
    const int32_t* __restrict__ ids, int32_t P, int32_t E, int32_t id_bits, int32_t span,
    int32_t* __restrict__ offsets, int32_t* __restrict__ src_pair, int32_t* __restrict__ inv) {
  __shared__ int32_t s_before[kPermMaxE];
  __shared__ int32_t s_after[kPermMaxE];
  __shared__ int32_t s_base[kPermMaxE];
  __shared__ int32_t s_wave[kPermWaves][kPermMaxE];
  __shared__ int32_t s_tmp[kPermWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t q0 = (int32_t)blockIdx.x * span;
  const int32_t q1 = min(P, q0 + span);

  for (int e = tid; e < E; e += kPermThreads) {
    s_before[e] = 0;
    s_after[e] = 0;
#pragma unroll
    for (int w = 0; w < kPermWaves; ++w) s_wave[w][e] = 0;
  }
  __syncthreads();

  // 1. histogram of all pairs
  constexpr int kUnroll = 8;
  for (int64_t qb = 0; qb < P; qb += kPermThreads * kUnroll) {
    int32_t id[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t q = qb + u * kPermThreads + tid;
      id[u] = q < P ? ids[q] : -1;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t q = qb + u * kPermThreads + tid;
      if ((uint32_t)id[u] < (uint32_t)E) atomicAdd(q < q0 ? &s_before[id[u]] : &s_after[id[u]], 1);
    }
  }
  __syncthreads();

  // 2. expert offsets; running base of each expert at the start of the block
  const int per = (E + kPermThreads - 1) / kPermThreads;   // experts per thread (<= 2)
  int32_t local = 0;
  for (int i = 0; i < per; ++i) {
    const int e = tid * per + i;
    if (e < E) local += s_before[e] + s_after[e];
  }
  int32_t total;
  int32_t run = perm_exclusive_scan(local, &total, s_tmp);
  for (int i = 0; i < per; ++i) {
    const int e = tid * per + i;
    if (e < E) {
      if (blockIdx.x == 0) offsets[e] = run;
      s_base[e] = run + s_before[e];
      run += s_before[e] + s_after[e];
    }
  }
  if (blockIdx.x == 0 && tid == 0) offsets[E] = total;
  __syncthreads();

  // 3. stable ranks inside the block
  const uint64_t below = (1ull << lane) - 1ull;
  for (int64_t qs = q0; qs < q1; qs += kPermThreads) {
    const int32_t q = (int32_t)min(qs + tid, (int64_t)q1);
    const int32_t id = q < q1 ? ids[q] : -1;
    const bool valid = (uint32_t)id < (uint32_t)E;
    uint64_t same = __ballot(valid);
    for (int b = 0; b < id_bits; ++b) {
      const bool bit = (id >> b) & 1;
      const uint64_t ones = __ballot(bit);
      same &= bit ? ones : ~ones;
    }
    const bool leader = valid && (same & below) == 0;
    if (leader) s_wave[wave][id] = __popcll(same);
    __syncthreads();
    for (int e = tid; e < E; e += kPermThreads) {
      int32_t r = s_base[e];
#pragma unroll
      for (int w = 0; w < kPermWaves; ++w) {
        const int32_t c = s_wave[w][e];
        if (c != 0) s_wave[w][e] = r;
        r += c;
      }
      s_base[e] = r;
    }
    __syncthreads();
    if (valid) {
      const int32_t p = s_wave[wave][id] + __popcll(same & below);
      src_pair[p] = q;
      inv[q] = p;
    }
    // Only this wavefront touches row `wave` of s_wave until the next
    // barrier, and its LDS operations complete in program order, so the
    // leader clears its entry after every lane of the wavefront has read it.
    if (leader) s_wave[wave][id] = 0;
  }
}

hipError_t launch_permute(const int32_t* ids, int32_t P, int32_t E, int32_t* offsets,
                          int32_t* src_pair, int32_t* inv, hipStream_t stream) {
  if (E < 1 || E > kPermMaxE || P < 0) return hipErrorInvalidValue;
  // Blocks of at least 2048 pairs; at most 256 of them, so the all-pairs
  // histogram each workgroup builds stays a small multiple of P.
  int64_t span = ((int64_t)P + 255) / 256;
  span = (span + kPermThreads - 1) / kPermThreads * kPermThreads;
  if (span < 2048) span = 2048;
  const int32_t blocks = P == 0 ? 1 : (int32_t)(((int64_t)P + span - 1) / span);
  int32_t id_bits = 0;
  while ((1 << id_bits) < E) ++id_bits;
  hipLaunchKernelGGL(permute_kernel, dim3(blocks), dim3(kPermThreads), 0, stream, ids, P, E,
                     id_bits, (int32_t)span, offsets, src_pair, inv);
  return hipGetLastError();
}

}  // namespace nvfp4
