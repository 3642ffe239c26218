// Per-expert NVFP4 activation quantiser for gfx950 (page 3, "NVFP4" section,
// runtime-order figure; SFScale[expert_idx] excerpt).
//
// Token-major: a workgroup owns one source row, one 16-element block per
// lane.  The row, its topk destinations and their SFScaleVals are uniform
// (scalar loads); each lane loads its block once, forms amax/6 once, and for
// every destination applies that expert's SFScaleVal, encodes 16 codes and
// stores 8 bytes of packed codes plus its E4M3 byte.  A wavefront's loads and
// stores are contiguous.
// The kernel is HBM-bound: it reads each source row once and writes
// topk * (K/2 + K/16) bytes per row.
//
// UE8M0 mode (kMX; the template's UE8M0_SF switch in the same excerpt): a
// block is 32 elements, i.e. a pair of adjacent lanes, which exchange their
// 16-element maxima; both lanes form the same power-of-two scale.
// Scale bytes leave as 32-bit words gathered across lanes when the row's
// scale count is a multiple of 4 (byte stores otherwise).
#include "internal.h"
#include "nvfp4_device.h"
#include "route_token.h"

namespace nvfp4 {

// kE / kP / kG: expert_idx / dst_row / gscale are present (not null);
// kF16: the source rows are fp16 instead of bf16 (both convert exactly to fp32);
// kMX: UE8M0 scales per 32 elements instead of E4M3 scales per 16.
template <bool kE, bool kP, bool kG, bool kF16, bool kMX>
__global__ __launch_bounds__(1024) void quantize_experts_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int32_t num_rows, int32_t nblk, int32_t topk,
    const int32_t* __restrict__ expert_idx, const int32_t* __restrict__ dst_row,
    int32_t num_experts, const float* __restrict__ gscale, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ sf, int32_t num_dst_rows) {
#pragma clang fp contract(off)
  // One workgroup per source row (wave-uniform t); thread -> block b.  The
  // whole row, and so every destination row's codes and scale bytes, is
  // written from one CU and one L2.
  const int32_t t = (int32_t)blockIdx.x;
  const int32_t b = (int32_t)blockIdx.y * (int32_t)blockDim.x + (int32_t)threadIdx.x;
  const bool on = b < nblk;

  float xv[16];
  float a6 = 0.0f;
  if (on) {
    const u32x4* src = reinterpret_cast<const u32x4*>(x + (int64_t)t * ldx + (int64_t)b * 16);
    const u32x4 v0 = __builtin_nontemporal_load(src);
    const u32x4 v1 = __builtin_nontemporal_load(src + 1);
    if constexpr (kF16) {
      unpack_f16x8(v0, xv);
      unpack_f16x8(v1, xv + 8);
    } else {
      unpack_bf16x8(v0, xv);
      unpack_bf16x8(v1, xv + 8);
    }
    a6 = absmax16(xv);
  }
  if constexpr (kMX) a6 = fmaxf(a6, __shfl_xor(a6, 1, 64));   // the block's other half
  a6 = a6 / kE2M1Max;
  const int64_t row_bytes = (int64_t)nblk * 8;
  // whole 32-bit scale words per destination row (and an aligned array):
  // then every lane whose block starts a word has the word's other blocks
  const bool sf_words = (reinterpret_cast<uintptr_t>(sf) & 3) == 0 && (kMX ? nblk % 8 : nblk % 4) == 0;
  // Destinations in batches of 8 (scalar loads shared by the wavefront): the
  // batch's expert ids and rows, then their SFScaleVals, are fetched before
  // any encoding, so the load latencies overlap.
  constexpr int kBatch = 8;
  for (int32_t j0 = 0; j0 < topk; j0 += kBatch) {
    int32_t eb[kBatch], pb[kBatch];
    float gb[kBatch];
#pragma unroll
    for (int jj = 0; jj < kBatch; ++jj) {
      // slots past topk re-read the last slot (always in range) and are
      // skipped below, so every load is unconditional
      const int64_t q = (int64_t)t * topk + min(j0 + jj, topk - 1);
      eb[jj] = kE ? expert_idx[q] : 0;
      pb[jj] = kP ? dst_row[q] : (int32_t)q;
    }
#pragma unroll
    for (int jj = 0; jj < kBatch; ++jj) {
      const int32_t ec = min(max(eb[jj], 0), num_experts - 1);   // clamped for the load
      gb[jj] = kG ? gscale[ec] : 1.0f;
    }
#pragma unroll
    for (int jj = 0; jj < kBatch; ++jj) {
      const int32_t e = eb[jj], p = pb[jj];
      // wave-uniform skip (every lane sees the same destination), so the
      // whole wavefront takes part in the scale-byte exchange below
      if (j0 + jj >= topk || (uint32_t)p >= (uint32_t)num_dst_rows ||
          (uint32_t)e >= (uint32_t)num_experts)
        continue;
      const BlockScale bs = kMX ? block_scale_ue8m0(a6, gb[jj]) : block_scale(a6, gb[jj]);
      if (on) {
        uint2 w;
        w.x = encode8(xv, bs.inv);
        w.y = encode8(xv + 8, bs.inv);
        *reinterpret_cast<uint2*>(codes + (int64_t)p * row_bytes + (int64_t)b * 8) = w;
      }
      // Scale bytes, four per 32-bit store: lane b collects the bytes of the
      // next three blocks with two DPP moves (E4M3: lanes b+1..b+3; UE8M0,
      // where both lanes of a pair hold their block's byte: b+2, b+4, b+6).
      if (sf_words) {
        uint32_t v = bs.sf;
        if constexpr (kMX) {
          v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false) << 8;
          v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x104, 0xF, 0xF, false) << 16;
          if (on && (b & 7) == 0)
            *reinterpret_cast<uint32_t*>(sf + (int64_t)p * (nblk / 2) + b / 2) = v;
        } else {
          v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false) << 8;
          v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false) << 16;
          if (on && (b & 3) == 0) *reinterpret_cast<uint32_t*>(sf + (int64_t)p * nblk + b) = v;
        }
      } else if (on) {
        if constexpr (kMX) {
          if ((b & 1) == 0) sf[(int64_t)p * (nblk / 2) + b / 2] = (uint8_t)bs.sf;
        } else {
          sf[(int64_t)p * nblk + b] = (uint8_t)bs.sf;
        }
      }
    }
  }
}

// The layer's case of the kernel above (expert ids and scales given, bf16
// rows, E4M3 scales; destination rows given, or the identity when kP is
// false), specialised: the workgroup is exactly one lane per block of the
// row (no idle lanes, so no per-lane guards), destination offsets are 32-bit,
// and every scale word is whole.
//
// Lane b quantises block b of `x_row` once per slot j < topk with the
// SFScaleVal of expert tok_ids[j], writing destination row tok_dst[j] (kP)
// or q0 + j; a slot whose expert or destination row is out of range is
// skipped.  Slots go in batches of 8: the batch's codes and scale words are
// all computed first and its stores then issued back to back (measured on
// the 8192 x 2816 top-8 workload, destinations in (token, slot) order: 30.5
// -> 28.5 us; storing each slot as soon as it is encoded leaves the stores
// spread between the encoding instructions).  kTopk > 0 fixes the slot count
// at compile time.
// kMX: UE8M0 block scales, one per 32 elements (page 3, "NVFP4" section, the
// quantiser template's UE8M0_SF switch).  The two 16-element halves of a
// block are lanes b and b ^ 1, which share the block's absolute maximum; the
// lanes at multiples of 8 store the 4 scale bytes of blocks b/2 .. b/2 + 3
// as one 32-bit word (nblk must then be a multiple of 8).
template <bool kP, int kTopk, bool kMX = false>
__device__ __forceinline__ void quantize_token_slots(
    const uint16_t* __restrict__ x_row, int32_t nblk, int32_t b, int32_t topk_arg,
    const int32_t* tok_ids, const int32_t* tok_dst, int32_t q0, int32_t num_experts,
    const float* __restrict__ gscale, uint8_t* __restrict__ codes, uint8_t* __restrict__ sf,
    int32_t num_dst_rows) {
#pragma clang fp contract(off)
  const int32_t topk = kTopk > 0 ? kTopk : topk_arg;
  float xv[16];
  const u32x4* src = reinterpret_cast<const u32x4*>(x_row + (int64_t)b * 16);
  const u32x4 v0 = __builtin_nontemporal_load(src);
  const u32x4 v1 = __builtin_nontemporal_load(src + 1);
  unpack_bf16x8(v0, xv);
  unpack_bf16x8(v1, xv + 8);
  float am = absmax16(xv);
  if constexpr (kMX) am = fmaxf(am, __shfl_xor(am, 1, 64));   // the block's other half
  const float a6 = am / kE2M1Max;
  const uint32_t row_bytes = (uint32_t)nblk * 8u;
  constexpr int kBatch = 8;
  for (int32_t j0 = 0; j0 < topk; j0 += kBatch) {
    int32_t eb[kBatch], pb[kBatch];
    float gb[kBatch];
#pragma unroll
    for (int jj = 0; jj < kBatch; ++jj) {
      const int32_t j = min(j0 + jj, topk - 1);
      eb[jj] = tok_ids[j];
      pb[jj] = kP ? tok_dst[j] : q0 + j;
    }
#pragma unroll
    for (int jj = 0; jj < kBatch; ++jj) gb[jj] = gscale[min(max(eb[jj], 0), num_experts - 1)];
    // a slot is stored when it exists and both its expert and its
    // destination row are in range (uniform over the workgroup)
    bool keep[kBatch];
#pragma unroll
    for (int jj = 0; jj < kBatch; ++jj)
      keep[jj] = j0 + jj < topk && (uint32_t)pb[jj] < (uint32_t)num_dst_rows &&
                 (uint32_t)eb[jj] < (uint32_t)num_experts;
    uint2 w[kBatch];
    uint32_t sw[kBatch];
#pragma unroll
    for (int jj = 0; jj < kBatch; ++jj) {
      const BlockScale bs = kMX ? block_scale_ue8m0(a6, gb[jj]) : block_scale(a6, gb[jj]);
      w[jj].x = encode8(xv, bs.inv);
      w[jj].y = encode8(xv + 8, bs.inv);
      uint32_t v = bs.sf;
      if constexpr (kMX) {
        // lanes b + 2, b + 4 and b + 6 hold the next three blocks' scales
        v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false) << 8;
        v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x104, 0xF, 0xF, false) << 16;
      } else {
        v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false) << 8;
        v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false) << 16;
      }
      sw[jj] = v;
    }
#pragma unroll
    for (int jj = 0; jj < kBatch; ++jj)
      if (keep[jj])
        *reinterpret_cast<uint2*>(codes + ((uint32_t)pb[jj] * row_bytes + (uint32_t)b * 8u)) = w[jj];
    if constexpr (kMX) {
      if ((b & 7) == 0) {
#pragma unroll
        for (int jj = 0; jj < kBatch; ++jj)
          if (keep[jj])
            *reinterpret_cast<uint32_t*>(
                sf + ((uint32_t)pb[jj] * (uint32_t)(nblk / 2) + (uint32_t)(b / 2))) = sw[jj];
      }
    } else if ((b & 3) == 0) {
#pragma unroll
      for (int jj = 0; jj < kBatch; ++jj)
        if (keep[jj])
          *reinterpret_cast<uint32_t*>(sf + ((uint32_t)pb[jj] * (uint32_t)nblk + (uint32_t)b)) =
              sw[jj];
    }
  }
}

template <bool kP, int kTopk, bool kMX>
__global__ __launch_bounds__(1024) void quantize_pairs_fast_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int32_t nblk, int32_t topk,
    const int32_t* __restrict__ expert_idx, const int32_t* __restrict__ dst_row,
    int32_t num_experts, const float* __restrict__ gscale, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ sf, int32_t num_dst_rows) {
  const int32_t t = (int32_t)blockIdx.x;
  const int64_t q0 = (int64_t)t * (kTopk > 0 ? kTopk : topk);
  quantize_token_slots<kP, kTopk, kMX>(x + (int64_t)t * ldx, nblk, (int32_t)threadIdx.x, topk,
                                       expert_idx + q0, kP ? dst_row + q0 : nullptr, (int32_t)q0,
                                       num_experts, gscale, codes, sf, num_dst_rows);
}

// Routing and the A1 quantisation of the layer in one launch: workgroup t
// (exactly H/16 >= 64 lanes) routes token t with its first wavefront (the
// router's own code, route_token) and writes the token's k ids and weights;
// after a barrier every lane quantises its block of the row into rows
// t*k + j with the SFScaleVals of the picked experts.  This saves the
// router's launch.  kMX: UE8M0 block scales per 32 elements.
template <int EPL, int kTopk, bool kMX>
__global__ __launch_bounds__(1024) void route_quantize_kernel(
    const float* __restrict__ logits, int32_t E, int32_t k_arg, int32_t* __restrict__ ids,
    float* __restrict__ weights, const uint16_t* __restrict__ x, int32_t nblk,
    const float* __restrict__ gscale, uint8_t* __restrict__ codes, uint8_t* __restrict__ sf,
    int32_t num_dst_rows) {
  __shared__ int32_t s_ids[32];
  const int32_t k = kTopk > 0 ? kTopk : k_arg;
  const int32_t t = (int32_t)blockIdx.x;
  const int lane = threadIdx.x & 63;
  if (threadIdx.x < 64) {
    int32_t id;
    float w;
    route_token<EPL>(logits + (int64_t)t * E, E, k, lane, id, w);
    if (lane < k) {
      ids[(int64_t)t * k + lane] = id;
      weights[(int64_t)t * k + lane] = w;
      s_ids[lane] = id;
    }
  }
  __syncthreads();
  quantize_token_slots<false, kTopk, kMX>(x + (int64_t)t * nblk * 16, nblk, (int32_t)threadIdx.x,
                                          k, s_ids, nullptr, t * k, E, gscale, codes, sf,
                                          num_dst_rows);
}

// Gather form: one workgroup per destination row p (grid.x) and one 16-element
// block per lane.  Row p belongs to the expert e with offsets[e] <= p <
// offsets[e+1] (found by a wave-uniform binary search) and quantises source
// row src_row[p] / src_div of x (row p when src_row is null) with that
// expert's SFScaleVal.  Rows outside [offsets[0], offsets[E]) and rows whose
// source row falls outside [0, num_src_rows) are not written.  The row's code
// bytes and scale bytes are written by one workgroup, contiguously.
template <bool kS, bool kG, bool kF16, bool kMX>
__global__ __launch_bounds__(1024) void quantize_gather_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int32_t nblk, const int32_t* __restrict__ src_row,
    int32_t src_div, int32_t num_src_rows, const int32_t* __restrict__ offsets, int32_t E,
    const float* __restrict__ gscale, uint8_t* __restrict__ codes, uint8_t* __restrict__ sf) {
#pragma clang fp contract(off)
  const int32_t p = (int32_t)blockIdx.x;
  const int32_t b = (int32_t)blockIdx.y * (int32_t)blockDim.x + (int32_t)threadIdx.x;
  if (p < offsets[0] || p >= offsets[E]) return;             // uniform per workgroup
  int32_t lo = 0, hi = E - 1;                                // last e with offsets[e] <= p
  while (lo < hi) {
    const int32_t mid = (lo + hi + 1) >> 1;
    if (offsets[mid] <= p) lo = mid; else hi = mid - 1;
  }
  const int32_t s = kS ? src_row[p] : p;
  if (s < 0) return;
  const int64_t srow = kS ? (int64_t)(s / src_div) : (int64_t)p;
  if (srow >= num_src_rows) return;
  const float gs = kG ? gscale[lo] : 1.0f;
  const bool on = b < nblk;
  float xv[16];
  float a6 = 0.0f;
  if (on) {
    const u32x4* src = reinterpret_cast<const u32x4*>(x + srow * ldx + (int64_t)b * 16);
    const u32x4 v0 = __builtin_nontemporal_load(src);
    const u32x4 v1 = __builtin_nontemporal_load(src + 1);
    if constexpr (kF16) {
      unpack_f16x8(v0, xv);
      unpack_f16x8(v1, xv + 8);
    } else {
      unpack_bf16x8(v0, xv);
      unpack_bf16x8(v1, xv + 8);
    }
    a6 = absmax16(xv);
  }
  if constexpr (kMX) a6 = fmaxf(a6, __shfl_xor(a6, 1, 64));   // the block's other half
  a6 = a6 / kE2M1Max;
  const BlockScale bs = kMX ? block_scale_ue8m0(a6, gs) : block_scale(a6, gs);
  if (on) {
    uint2 w;
    w.x = encode8(xv, bs.inv);
    w.y = encode8(xv + 8, bs.inv);
    *reinterpret_cast<uint2*>(codes + (int64_t)p * nblk * 8 + (int64_t)b * 8) = w;
  }
  const bool sf_words = (reinterpret_cast<uintptr_t>(sf) & 3) == 0 && (kMX ? nblk % 8 : nblk % 4) == 0;
  if (sf_words) {
    uint32_t v = bs.sf;
    if constexpr (kMX) {
      v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false) << 8;
      v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x104, 0xF, 0xF, false) << 16;
      if (on && (b & 7) == 0)
        *reinterpret_cast<uint32_t*>(sf + (int64_t)p * (nblk / 2) + b / 2) = v;
    } else {
      v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false) << 8;
      v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false) << 16;
      if (on && (b & 3) == 0) *reinterpret_cast<uint32_t*>(sf + (int64_t)p * nblk + b) = v;
    }
  } else if (on) {
    if constexpr (kMX) {
      if ((b & 1) == 0) sf[(int64_t)p * (nblk / 2) + b / 2] = (uint8_t)bs.sf;
    } else {
      sf[(int64_t)p * nblk + b] = (uint8_t)bs.sf;
    }
  }
}

namespace {

template <bool kF16, bool kMX>
void launch_quantize_variant(int variant, dim3 grid, int32_t threads, hipStream_t stream,
                             const uint16_t* x, int64_t ldx, int32_t num_rows, int32_t nblk,
                             int32_t topk, const int32_t* expert_idx, const int32_t* dst_row,
                             int32_t num_experts, const float* gscale, uint8_t* codes,
                             uint8_t* sf, int32_t num_dst_rows) {
#define NVFP4_QUANT_CASE(v, ke, kp, kg)                                                         \
  case v:                                                                                       \
    hipLaunchKernelGGL((quantize_experts_kernel<ke, kp, kg, kF16, kMX>), grid, dim3(threads),   \
                       0, stream, x, ldx, num_rows, nblk, topk, expert_idx, dst_row,           \
                       num_experts, gscale, codes, sf, num_dst_rows);                           \
    break;
  switch (variant) {
    NVFP4_QUANT_CASE(0, false, false, false)
    NVFP4_QUANT_CASE(1, false, false, true)
    NVFP4_QUANT_CASE(2, false, true, false)
    NVFP4_QUANT_CASE(3, false, true, true)
    NVFP4_QUANT_CASE(4, true, false, false)
    NVFP4_QUANT_CASE(5, true, false, true)
    NVFP4_QUANT_CASE(6, true, true, false)
    NVFP4_QUANT_CASE(7, true, true, true)
  }
#undef NVFP4_QUANT_CASE
}

}  // namespace

hipError_t launch_quantize(const uint16_t* x, int64_t ldx, int32_t num_rows, int32_t K,
                           int32_t topk, const int32_t* expert_idx, const int32_t* dst_row,
                           int32_t num_experts, const float* gscale, uint8_t* codes, uint8_t* sf,
                           int32_t num_dst_rows, hipStream_t stream, bool fp16_input, bool mx) {
  const int32_t nblk = K / 16;
  if ((int64_t)num_rows * nblk == 0) return hipSuccess;
  // the layer's case: one workgroup of exactly nblk lanes per row, whole
  // scale words, 32-bit destination offsets
  if (expert_idx && gscale && !fp16_input && !mx && nblk <= 1024 && nblk % 4 == 0 &&
      (reinterpret_cast<uintptr_t>(sf) & 3) == 0 &&
      (int64_t)num_dst_rows * nblk * 8 <= (int64_t)UINT32_MAX) {
    // top-8, the layer's case, has its own instantiation (measured 29.9 ->
    // 28.8 us on the 8192 x 2816 workload with destinations in token-slot
    // order)
#define NVFP4_FAST(kp, kk)                                                                       \
  hipLaunchKernelGGL((quantize_pairs_fast_kernel<kp, kk, false>), dim3((uint32_t)num_rows),      \
                     dim3(nblk),                                                                 \
                     0, stream, x, ldx, nblk, topk, expert_idx, dst_row, num_experts, gscale,    \
                     codes, sf, num_dst_rows)
    if (dst_row) {
      if (topk == 8) NVFP4_FAST(true, 8);
      else NVFP4_FAST(true, 0);
    } else {
      if (topk == 8) NVFP4_FAST(false, 8);
      else NVFP4_FAST(false, 0);
    }
#undef NVFP4_FAST
    return hipGetLastError();
  }
  // 64-lane wavefronts covering the row's blocks, at most 1024 threads per
  // workgroup (longer rows take several workgroups; 1024 is even, so the two
  // halves of a 32-element block always share a wavefront)
  const int32_t threads = min(1024, (nblk + 63) / 64 * 64);
  const dim3 grid((uint32_t)num_rows, (uint32_t)((nblk + threads - 1) / threads));
  const int variant = (expert_idx ? 4 : 0) | (dst_row ? 2 : 0) | (gscale ? 1 : 0);
  if (mx)
    launch_quantize_variant<false, true>(variant, grid, threads, stream, x, ldx, num_rows, nblk,
                                         topk, expert_idx, dst_row, num_experts, gscale, codes,
                                         sf, num_dst_rows);
  else if (fp16_input)
    launch_quantize_variant<true, false>(variant, grid, threads, stream, x, ldx, num_rows, nblk,
                                         topk, expert_idx, dst_row, num_experts, gscale, codes,
                                         sf, num_dst_rows);
  else
    launch_quantize_variant<false, false>(variant, grid, threads, stream, x, ldx, num_rows, nblk,
                                          topk, expert_idx, dst_row, num_experts, gscale, codes,
                                          sf, num_dst_rows);
  return hipGetLastError();
}

namespace {

template <bool kF16, bool kMX>
void launch_gather_variant(int variant, dim3 grid, int32_t threads, hipStream_t stream,
                           const uint16_t* x, int64_t ldx, int32_t nblk, const int32_t* src_row,
                           int32_t src_div, int32_t num_src_rows, const int32_t* offsets,
                           int32_t E, const float* gscale, uint8_t* codes, uint8_t* sf) {
#define NVFP4_GATHER_CASE(v, ks, kg)                                                            \
  case v:                                                                                       \
    hipLaunchKernelGGL((quantize_gather_kernel<ks, kg, kF16, kMX>), grid, dim3(threads), 0,     \
                       stream, x, ldx, nblk, src_row, src_div, num_src_rows, offsets, E,        \
                       gscale, codes, sf);                                                      \
    break;
  switch (variant) {
    NVFP4_GATHER_CASE(0, false, false)
    NVFP4_GATHER_CASE(1, false, true)
    NVFP4_GATHER_CASE(2, true, false)
    NVFP4_GATHER_CASE(3, true, true)
  }
#undef NVFP4_GATHER_CASE
}

}  // namespace

hipError_t launch_quantize_gather(const uint16_t* x, int64_t ldx, int32_t K,
                                  const int32_t* src_row, int32_t src_div, int32_t num_src_rows,
                                  int32_t P, const int32_t* offsets, int32_t E,
                                  const float* gscale, uint8_t* codes, uint8_t* sf,
                                  hipStream_t stream, bool fp16_input, bool mx) {
  const int32_t nblk = K / 16;
  if ((int64_t)P * nblk == 0) return hipSuccess;
  // 64-lane wavefronts covering the row's blocks, at most 1024 threads per
  // workgroup (1024 is even, so a 32-element block never straddles two)
  const int32_t threads = min(1024, (nblk + 63) / 64 * 64);
  const dim3 grid((uint32_t)P, (uint32_t)((nblk + threads - 1) / threads));
  const int variant = (src_row ? 2 : 0) | (gscale ? 1 : 0);
  if (mx)
    launch_gather_variant<false, true>(variant, grid, threads, stream, x, ldx, nblk, src_row,
                                       src_div, num_src_rows, offsets, E, gscale, codes, sf);
  else if (fp16_input)
    launch_gather_variant<true, false>(variant, grid, threads, stream, x, ldx, nblk, src_row,
                                       src_div, num_src_rows, offsets, E, gscale, codes, sf);
  else
    launch_gather_variant<false, false>(variant, grid, threads, stream, x, ldx, nblk, src_row,
                                        src_div, num_src_rows, offsets, E, gscale, codes, sf);
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

// Calibration: per-expert input_scale = fl32(amax / 2688) from the absmax
// pass, and the `written` mask of experts that received at least one row.
// An expert without rows gets NaN and written = 0, so the load-time check
// reports it as unwritten instead of a reciprocal being taken of it.
__global__ void calibrate_finish_kernel(float* __restrict__ scale, uint8_t* __restrict__ written,
                                        const int32_t* __restrict__ offsets, int32_t E) {
#pragma clang fp contract(off)
  const int32_t e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  const bool any = offsets[e + 1] > offsets[e];
  scale[e] = any ? scale[e] / (kE2M1Max * kE4M3Max) : __builtin_nanf("");
  written[e] = any ? 1 : 0;
}

hipError_t launch_calibrate(const uint16_t* x, int64_t ldx, int32_t K, const int32_t* src,
                            int32_t src_div, const int32_t* offsets, int32_t E, int32_t num_rows,
                            float* scale, uint8_t* written, hipStream_t stream) {
  hipError_t err = launch_absmax(x, ldx, K, src, src_div, offsets, E, num_rows, scale, stream);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(calibrate_finish_kernel, dim3((E + 255) / 256), dim3(256), 0, stream, scale,
                     written, offsets, E);
  return hipGetLastError();
}

// Device self-check of the five conversion instructions the kernels rely
// on, each against a reference built from the format definitions:
//   count[0]: fp32 -> E2M1 encode (encode8) vs the midpoint comparisons of
//             e2m1_code(), over every non-NaN fp32 pattern (each positive
//             pattern and its negation form one pair);
//   count[1]: E2M1 byte -> fp16 pair (GEMM operand dequant) vs the E2M1 table,
//             all 256 bytes in all 4 byte positions, sign of zero included;
//   count[2]: E4M3 byte -> fp16 (block-scale decode) vs e4m3_decode(), all
//             256 codes except the two NaN patterns, in both halves.
typedef _Float16 st_half2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float e2m1_ref(uint32_t c) {
  const float mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
  const float v = mag[c & 7u];
  return (c & 8u) ? -v : v;
}

__device__ __forceinline__ bool same_f16(_Float16 h, float ref) {
  const float f = (float)h;
  return f == ref && (__float_as_uint(f) >> 31) == (__float_as_uint(ref) >> 31);
}

__global__ __launch_bounds__(256) void conversions_selftest_kernel(unsigned long long* count) {
  unsigned long long local = 0, local8 = 0;
  const uint32_t tid = blockIdx.x * blockDim.x + threadIdx.x;
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t u = tid; u < 0x80000000u; u += stride) {
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu)) continue;   // NaN
    const float f[2] = {__uint_as_float(u), __uint_as_float(u | 0x80000000u)};
    const uint32_t hw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, f[0], f[1], 1.0f, 0) & 0xFFu;
    const uint32_t sw = e2m1_code(f[0]) | (e2m1_code(f[1]) << 4);
    local += hw != sw;
    // E4M3 encode of a non-negative block scale (+inf included)
    local8 += e4m3_encode_hw(f[0]) != e4m3_encode(f[0]);
  }
  if (local) atomicAdd(count, local);
  if (local8) atomicAdd(count + 3, local8);
  if (tid < 256) {
    const uint32_t b = tid;
    unsigned long long bad = 0;
    const st_half2 d0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(b, 1.0f, 0);
    const st_half2 d1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(b << 8, 1.0f, 1);
    const st_half2 d2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(b << 16, 1.0f, 2);
    const st_half2 d3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(b << 24, 1.0f, 3);
    const st_half2 d[4] = {d0, d1, d2, d3};
    for (int i = 0; i < 4; ++i)
      bad += !same_f16(d[i].x, e2m1_ref(b & 15u)) + !same_f16(d[i].y, e2m1_ref(b >> 4));
    if (bad) atomicAdd(count + 1, bad);
    if ((b & 0x7Fu) != 0x7Fu) {
      const float ref = (b & 0x80u) ? -e4m3_decode(b & 0x7Fu) : e4m3_decode(b);
      const st_half2 lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b | (b << 8), 1.0f, false);
      const st_half2 hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((b << 16) | (b << 24), 1.0f, true);
      const unsigned long long bad8 = !same_f16(lo.x, ref) + !same_f16(lo.y, ref) +
                                      !same_f16(hi.x, ref) + !same_f16(hi.y, ref);
      if (bad8) atomicAdd(count + 2, bad8);
      if (b < 0x7Fu)
        atomicAdd(count + 4, (unsigned long long)(__float_as_uint(e4m3_decode_hw(b)) !=
                                                   __float_as_uint(e4m3_decode(b))));
    }
  }
}

__global__ void zero_u64_kernel(unsigned long long* p, int n) {
  if ((int)threadIdx.x < n) p[threadIdx.x] = 0;
}

hipError_t launch_conversions_selftest(unsigned long long* count, hipStream_t stream) {
  hipLaunchKernelGGL(zero_u64_kernel, dim3(1), dim3(64), 0, stream, count, 5);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(conversions_selftest_kernel, dim3(8192), dim3(256), 0, stream, count);
  return hipGetLastError();
}


hipError_t launch_route_quantize(const float* logits, int32_t T, int32_t E, int32_t k,
                                 int32_t* ids, float* weights, const uint16_t* x, int32_t H,
                                 const float* gscale, uint8_t* codes, uint8_t* sf,
                                 hipStream_t stream, bool mx) {
  const int32_t nblk = H / 16;
  // whole scale words: 4 E4M3 scales (H % 64), or 4 UE8M0 scales of 32
  // elements (H % 128)
  if (T < 1 || E < 1 || E > 1024 || k < 1 || k > 32 || k > E || H % (mx ? 128 : 64) ||
      nblk < 64 || nblk > 1024 || !gscale || (reinterpret_cast<uintptr_t>(sf) & 3) != 0 ||
      (int64_t)T * k * nblk * 8 > (int64_t)UINT32_MAX)
    return hipErrorNotSupported;
  const int32_t P = T * k;
#define NVFP4_RQ(epl, kk)                                                                        \
  if (mx)                                                                                        \
    hipLaunchKernelGGL((route_quantize_kernel<epl, kk, true>), dim3((uint32_t)T), dim3(nblk), 0,  \
                       stream, logits, E, k, ids, weights, x, nblk, gscale, codes, sf, P);       \
  else                                                                                           \
    hipLaunchKernelGGL((route_quantize_kernel<epl, kk, false>), dim3((uint32_t)T), dim3(nblk), 0, \
                       stream, logits, E, k, ids, weights, x, nblk, gscale, codes, sf, P)
#define NVFP4_RQ_E(kk)                                                                           \
  if (E <= 64) NVFP4_RQ(1, kk);                                                                  \
  else if (E <= 128) NVFP4_RQ(2, kk);                                                            \
  else if (E <= 256) NVFP4_RQ(4, kk);                                                            \
  else if (E <= 512) NVFP4_RQ(8, kk);                                                            \
  else NVFP4_RQ(16, kk);
  if (k == 8) {
    NVFP4_RQ_E(8)
  } else {
    NVFP4_RQ_E(0)
  }
#undef NVFP4_RQ_E
#undef NVFP4_RQ
  return hipGetLastError();
}

}  // namespace nvfp4
