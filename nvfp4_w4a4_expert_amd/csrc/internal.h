// Internal launchers shared between the kernel translation units and the
// C-ABI layer.  Not exported from the shared library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nvfp4 {

hipError_t launch_quantize(const uint16_t* x, int64_t ldx, int32_t num_rows, int32_t K,
                           int32_t topk, const int32_t* expert_idx, const int32_t* dst_row,
                           int32_t num_experts, const float* gscale, uint8_t* codes, uint8_t* sf,
                           int32_t num_dst_rows, hipStream_t stream, bool fp16_input = false,
                           bool mx = false);

// The quantiser's gather form: destination row p quantises source row
// src_row[p] / src_div (p when src_row is null) with the SFScaleVal of its
// expert (offsets[e] <= p < offsets[e+1]).
hipError_t launch_quantize_gather(const uint16_t* x, int64_t ldx, int32_t K,
                                  const int32_t* src_row, int32_t src_div, int32_t num_src_rows,
                                  int32_t P, const int32_t* offsets, int32_t E,
                                  const float* gscale, uint8_t* codes, uint8_t* sf,
                                  hipStream_t stream, bool fp16_input = false, bool mx = false);

hipError_t launch_route(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* ids,
                        float* weights, hipStream_t stream);

// The router and the layer's A1 quantisation (bf16 x [T, H], E4M3 scales per
// 16 elements, or UE8M0 scales per 32 when mx; rows in (token, slot) order)
// in one launch.  Returns hipErrorNotSupported, launching nothing, for shapes
// it does not cover (H/16 below 64 or above 1024, k above 32); the caller
// then launches the two kernels.
hipError_t launch_route_quantize(const float* logits, int32_t T, int32_t E, int32_t k,
                                 int32_t* ids, float* weights, const uint16_t* x, int32_t H,
                                 const float* gscale, uint8_t* codes, uint8_t* sf,
                                 hipStream_t stream, bool mx = false);

hipError_t launch_permute(const int32_t* ids, int32_t P, int32_t E, int32_t* offsets,
                          int32_t* src_pair, int32_t* inv, hipStream_t stream);

hipError_t launch_absmax(const uint16_t* x, int64_t ldx, int32_t K, const int32_t* src,
                         int32_t src_div, const int32_t* offsets, int32_t E, int32_t num_rows,
                         float* amax, hipStream_t stream);

hipError_t launch_calibrate(const uint16_t* x, int64_t ldx, int32_t K, const int32_t* src,
                            int32_t src_div, const int32_t* offsets, int32_t E, int32_t num_rows,
                            float* scale, uint8_t* written, hipStream_t stream);

hipError_t launch_conversions_selftest(unsigned long long* count, hipStream_t stream);

struct Gemm1Args {
  const uint8_t* a_codes;   // [P, H/2]
  const uint8_t* a_sf;      // [P, H/16]
  // weight-only variant (w16): A row p = a_rows[(a_src[p] / a_src_div) * lda], bf16
  const uint16_t* a_rows = nullptr;
  const int32_t* a_src = nullptr;
  int64_t lda = 0;
  int32_t a_src_div = 1;
  uint16_t* h_out = nullptr;  // [P, I] bf16 h (w16)
  bool w16 = false;
  bool mx = false;          // UE8M0 operands: a_sf [P, H/32], w_sf 32-element blocks, out_sf [P, I/32]
  const uint8_t* w_codes;   // [E, 2I, H/2]
  const uint8_t* w_sf;      // [E, 2I, H/16]
  const float* in_scale;    // [E] w13_input_scale
  const float* w_scale2;    // [E] w13_scale2
  const float* out_gscale;  // [E] a2_gscale (requant of h)
  const int32_t* offsets;   // [E+1]
  uint8_t* out_codes;       // [P, I/2]
  uint8_t* out_sf;          // [P, I/16]
  float* c1_dbg;            // [P, 2I] or null
  uint16_t* h_dbg;          // [P, I] or null
  // When set (only if gemm_map::fold_permutation(P, E)), GEMM1 regroups the
  // routed ids [P] itself instead of reading offsets / a_src, and writes the
  // permutation (offsets [E+1], src_pair [P], inv [P]) for the later stages;
  // a_src must still be non-null (it selects the gathered-row path).
  const int32_t* perm_ids = nullptr;
  int32_t* perm_offsets = nullptr;
  int32_t* perm_src = nullptr;
  int32_t* perm_inv = nullptr;
  int32_t P, E, H, I;
};

struct Gemm2Args {
  const uint8_t* a_codes;   // [P, I/2]
  const uint8_t* a_sf;      // [P, I/16]
  const uint16_t* a_rows = nullptr;  // w16: bf16 h [P, I]
  bool w16 = false;
  bool mx = false;          // UE8M0 operands (32-element blocks)
  const uint8_t* w_codes;   // [E, H, I/2]
  const uint8_t* w_sf;      // [E, H, I/16]
  const float* in_scale;    // [E] w2_input_scale
  const float* w_scale2;    // [E] w2_scale2
  const int32_t* offsets;   // [E+1]
  float* out;               // [P, H]
  int32_t P, E, H, I;
};

hipError_t launch_gemm1(const Gemm1Args& a, hipStream_t stream);
hipError_t launch_pack_weights(int32_t projection, const uint8_t* codes, const uint8_t* sf,
                               int32_t E, int32_t N, int32_t K, uint8_t* codes_out,
                               uint8_t* sf_out, hipStream_t stream, bool mx = false);
hipError_t launch_gemm2(const Gemm2Args& a, hipStream_t stream);

hipError_t launch_combine(const float* c2, const float* w, const int32_t* inv, int32_t T,
                          int32_t k, int32_t H, const uint16_t* residual, uint16_t* out,
                          hipStream_t stream);

}  // namespace nvfp4
