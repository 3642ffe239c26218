// Router top-k and the stable regrouping of (token, slot) pairs by expert.
//
// Page 3, "NVFP4" runtime figure: the router fixes expert_idx before the
// activation quantiser runs; "矩阵融合", MoE FFN paragraph: the backend
// reorders rows by routing so each expert's rows form one group of a grouped
// GEMM, and the pipeline figure ends by restoring token order and summing by
// routing weight.
//
// route_topk: one wavefront per token.  Lanes hold the token's logits
// (E <= 64 * EPL) as order-preserving 64-bit keys; k rounds of a wave-wide
// maximum (DPP steps in registers), ordered by (logit descending, expert
// index ascending), pick the experts; the k weights are a softmax over the
// picked logits in fp32.
//
// permute: workgroups own consecutive blocks of pairs; each histograms all
// ids, derives the expert offsets, and ranks its block's pairs stably with
// wavefront ballots (see permute_kernel).
#include <float.h>

#include <type_traits>

#include "internal.h"
#include "route_token.h"

namespace nvfp4 {

template <int EPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits,
                                                         int32_t T, int32_t E, int32_t k,
                                                         int32_t* __restrict__ ids,
                                                         float* __restrict__ weights) {
  const int lane = threadIdx.x & 63;
  const int32_t t = (int32_t)blockIdx.x * 4 + (int32_t)(threadIdx.x >> 6);
  if (t >= T) return;
  int32_t id;
  float w;
  route_token<EPL>(logits + (int64_t)t * E, E, k, lane, id, w);
  if (lane < k) {
    ids[(int64_t)t * k + lane] = id;
    weights[(int64_t)t * k + lane] = w;
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

  // the block's own ids (its first kOwn steps) are loaded first, so their
  // latency overlaps the histogram
  constexpr int kOwn = 4;
  int32_t own[kOwn];
#pragma unroll
  for (int u = 0; u < kOwn; ++u) {
    const int64_t q = (int64_t)q0 + u * kPermThreads + tid;
    own[u] = q < q1 ? ids[q] : -1;
  }

  for (int e = tid; e < E; e += kPermThreads) {
    s_before[e] = 0;
    s_after[e] = 0;
#pragma unroll
    for (int w = 0; w < kPermWaves; ++w) s_wave[w][e] = 0;
  }
  __syncthreads();

  // 1. histogram of all pairs (all loads of a round are issued before its
  // LDS additions)
  constexpr int kUnroll = 32;
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
  auto rank_step = [&](int64_t qs, int32_t id) {
    const int32_t q = (int32_t)min(qs + tid, (int64_t)q1);
    const bool valid = q < q1 && (uint32_t)id < (uint32_t)E;
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
  };
#pragma unroll
  for (int u = 0; u < kOwn; ++u) {
    const int64_t qs = (int64_t)q0 + u * kPermThreads;
    if (qs < q1) rank_step(qs, own[u]);        // uniform condition
  }
  for (int64_t qs = (int64_t)q0 + kOwn * kPermThreads; qs < q1; qs += kPermThreads) {
    const int64_t q = qs + tid;
    rank_step(qs, q < q1 ? ids[q] : -1);
  }
}

hipError_t launch_permute(const int32_t* ids, int32_t P, int32_t E, int32_t* offsets,
                          int32_t* src_pair, int32_t* inv, hipStream_t stream) {
  if (E < 1 || E > kPermMaxE || P < 0) return hipErrorInvalidValue;
  // Blocks of at least 512 pairs (one ranking step per workgroup: measured
  // 16.4 -> 13.3 us at 32768 pairs against 2048-pair blocks); at most 256 of
  // them, so the all-pairs histogram each workgroup builds stays a small
  // multiple of P.
  int64_t span = ((int64_t)P + 255) / 256;
  span = (span + kPermThreads - 1) / kPermThreads * kPermThreads;
  if (span < kPermThreads) span = kPermThreads;
  const int32_t blocks = P == 0 ? 1 : (int32_t)(((int64_t)P + span - 1) / span);
  int32_t id_bits = 0;
  while ((1 << id_bits) < E) ++id_bits;
  hipLaunchKernelGGL(permute_kernel, dim3(blocks), dim3(kPermThreads), 0, stream, ids, P, E,
                     id_bits, (int32_t)span, offsets, src_pair, inv);
  return hipGetLastError();
}

}  // namespace nvfp4
