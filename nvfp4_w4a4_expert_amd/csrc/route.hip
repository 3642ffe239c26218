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

namespace nvfp4 {

// Order-preserving 64-bit key of (logit, expert): the high word orders fp32
// values like the reals (-0.0 is folded onto +0.0 first, so the two tie), the
// low word is ~expert so that of two equal logits the lower expert index has
// the larger key.  Keys are distinct, so a maximum is unique.
__device__ __forceinline__ uint64_t route_key(float v, int32_t e) {
  const uint32_t u = __float_as_uint(v + 0.0f);
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)ord << 32) | (uint32_t)~(uint32_t)e;
}

__device__ __forceinline__ float route_key_value(uint64_t key) {
  const uint32_t ord = (uint32_t)(key >> 32);
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}

// One DPP step of a wave maximum over 64-bit keys: combine with the lane that
// DPP control `kCtrl` selects (rows outside `kRowMask` keep their own key).
template <int kCtrl, int kRowMask>
__device__ __forceinline__ uint64_t dpp_max_step(uint64_t k) {
  const uint32_t lo = (uint32_t)k, hi = (uint32_t)(k >> 32);
  const uint32_t olo = (uint32_t)__builtin_amdgcn_update_dpp((int)lo, (int)lo, kCtrl, kRowMask, 0xF, false);
  const uint32_t ohi = (uint32_t)__builtin_amdgcn_update_dpp((int)hi, (int)hi, kCtrl, kRowMask, 0xF, false);
  const uint64_t o = ((uint64_t)ohi << 32) | olo;
  return o > k ? o : k;
}

// Maximum key of the wavefront, returned uniformly: quad swaps, the 8- and
// 16-lane mirrors, then row broadcasts 15 and 31 leave the maximum in lane 63.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t k) {
  k = dpp_max_step<0xB1, 0xF>(k);      // quad_perm [1,0,3,2]
  k = dpp_max_step<0x4E, 0xF>(k);      // quad_perm [2,3,0,1]
  k = dpp_max_step<0x141, 0xF>(k);     // row_half_mirror
  k = dpp_max_step<0x140, 0xF>(k);     // row_mirror
  k = dpp_max_step<0x142, 0xA>(k);     // row_bcast:15 into rows 1 and 3
  k = dpp_max_step<0x143, 0xC>(k);     // row_bcast:31 into rows 2 and 3
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)k, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(k >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// Wave sum of one float per lane (same reduction pattern), returned uniformly.
__device__ __forceinline__ float wave_sum(float v) {
  auto step = [](float x, auto ctrl, auto rows) {
    constexpr int c = decltype(ctrl)::value, m = decltype(rows)::value;
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), c, m, 0xF, false));
  };
  using std::integral_constant;
  v = step(v, integral_constant<int, 0xB1>{}, integral_constant<int, 0xF>{});
  v = step(v, integral_constant<int, 0x4E>{}, integral_constant<int, 0xF>{});
  v = step(v, integral_constant<int, 0x141>{}, integral_constant<int, 0xF>{});
  v = step(v, integral_constant<int, 0x140>{}, integral_constant<int, 0xF>{});
  v = step(v, integral_constant<int, 0x142>{}, integral_constant<int, 0xA>{});
  v = step(v, integral_constant<int, 0x143>{}, integral_constant<int, 0xC>{});
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

template <int EPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits,
                                                         int32_t T, int32_t E, int32_t k,
                                                         int32_t* __restrict__ ids,
                                                         float* __restrict__ weights) {
  const int lane = threadIdx.x & 63;
  const int32_t t = (int32_t)blockIdx.x * 4 + (int32_t)(threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (int64_t)t * E;
  uint64_t key[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < E ? route_key(row[e], e) : 0ull;         // 0 is below every real key
  }
  int32_t my_id = 0;
  float my_val = 0.0f;
  for (int r = 0; r < k; ++r) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) best = key[i] > best ? key[i] : best;
    const uint64_t top = wave_max_key(best);
    const int32_t e = (int32_t)~(uint32_t)top;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (e == lane + 64 * i) key[i] = 0;                  // taken
    if (lane == r) {
      my_id = e;
      my_val = route_key_value(top);
    }
  }
  // softmax over the k picks, in fp32; pick 0 is the largest
  const float mx = __shfl(my_val, 0, 64);
  const float ex = lane < k ? expf(my_val - mx) : 0.0f;
  const float sum = wave_sum(ex);
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
