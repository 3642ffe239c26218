// The router's per-token top-k (page 3, "NVFP4" runtime figure: the router
// fixes expert_idx before the activation quantiser runs), as device
// functions shared by the routing kernel and the fused routing + A1
// quantisation kernel, so both pick the same experts with the same weights.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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

// The k picks of one token and their softmax weights, by one wavefront
// (all 64 lanes active): lane j < k receives pick j; lanes >= k receive
// nothing meaningful.  Lanes hold the token's logits (E <= 64 * EPL) as
// order-preserving 64-bit keys; k rounds of a wave-wide maximum (DPP steps in
// registers), ordered by (logit descending, expert index ascending), pick the
// experts; the k weights are a softmax over the picked logits in fp32.
template <int EPL>
__device__ __forceinline__ void route_token(const float* __restrict__ row, int32_t E, int32_t k,
                                            int lane, int32_t& id, float& weight) {
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
  id = my_id;
  weight = ex / sum;
}

}  // namespace nvfp4
