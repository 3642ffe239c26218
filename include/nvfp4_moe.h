/*
 * nvfp4_moe.h — C ABI of libnvfp4moe.so, the MI355X (gfx950) NVFP4 W4A4
 * routed-expert MoE block.
 *
 * What is computed comes from page 3, "Gemma 4 NVFP4 MoE 空输出"
 * (taking-lying-flat.github.io): its "NVFP4" section (E2M1 codes with one
 * E4M3 scale per 16 elements and an FP32 global scale; the runtime order of
 * the per-expert activation quantiser; the SFScale[expert_idx] lookup), its
 * "ROOT CAUSE" section (per-expert input scales whose reciprocals are taken
 * without checking that every slot was written) and its "矩阵融合" section
 * (fused gate/up w13, act(gate) x up, and the MoE pipeline: permute ->
 * quant(a1) -> grouped w13 -> SiLU/mul + quant(a2) -> grouped w2 -> restore
 * token order and sum by routing weight).
 *
 * Conventions shared by every entry point
 *  - Plain C types only.  "device" pointers are HIP device memory (for
 *    example torch tensors' data_ptr()); "host" pointers are ordinary memory.
 *  - The caller owns every buffer.  The library allocates nothing on the
 *    device and keeps no mutable global state, so calls on different streams
 *    are independent.  The one exception is nvfp4_moe_forward_noalloc, whose
 *    workspace is a fixed static buffer per device (see there).
 *  - Calls that take a stream only enqueue work on it (NULL = the default
 *    stream) and never synchronise the host.  A launch failure reported by the
 *    HIP runtime returns NVFP4_ERR_DEVICE; argument problems found on the host
 *    return NVFP4_ERR_INVALID_ARG before anything is enqueued.
 *  - bf16 tensors are 16-bit bit patterns (the top half of an IEEE fp32).
 *  - NVFP4 tensors are two arrays: packed codes uint8 [rows, K/2] (element
 *    2j in the low nibble of byte j, element 2j+1 in the high nibble; E2M1 =
 *    sign, 2 exponent bits, 1 mantissa bit) and block scales uint8
 *    [rows, K/16] (OCP E4M3, one per 16 consecutive elements of a row), both
 *    row-major.  Dequantised element = E2M1(code) * E4M3(scale) * global scale.
 *  - No exceptions, printing or aborts cross the boundary.
 */
#ifndef NVFP4_MOE_H
#define NVFP4_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(NVFP4_BUILDING_LIBRARY)
#define NVFP4_API __attribute__((visibility("default")))
#else
#define NVFP4_API
#endif

/* A hipStream_t, passed as an opaque pointer so this header needs no HIP. */
typedef void* nvfp4_stream_t;

typedef enum {
  NVFP4_OK = 0,
  NVFP4_ERR_INVALID_ARG = 1,  /* null required pointer, bad size or alignment   */
  NVFP4_ERR_BAD_SCALE = 2,    /* a per-expert input scale failed the load check */
  NVFP4_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required     */
  NVFP4_ERR_DEVICE = 4,       /* the HIP runtime reported an error              */
  NVFP4_ERR_UNSUPPORTED = 5,  /* valid request outside the built kernels' shapes */
  NVFP4_ERR_TOO_LARGE = 6     /* needs more than nvfp4_moe_forward_noalloc's fixed buffer */
} nvfp4_status_t;

/* Per-slot verdicts of nvfp4_validate_scales. */
enum {
  NVFP4_SLOT_OK = 0,
  NVFP4_SLOT_UNWRITTEN = 1,       /* the loader never wrote this expert's slot        */
  NVFP4_SLOT_NAN = 2,
  NVFP4_SLOT_INF = 3,
  NVFP4_SLOT_NONPOSITIVE = 4,     /* <= 0, including -0.0                              */
  NVFP4_SLOT_RECIP_OVERFLOW = 5   /* fp32 1/x is not finite (x below ~2.94e-39)        */
};

/* Human-readable name of a status code; never NULL. */
NVFP4_API const char* nvfp4_status_string(nvfp4_status_t status);

/* ABI revision of this header; bumped on any incompatible change. */
NVFP4_API int32_t nvfp4_abi_version(void);
#define NVFP4_ABI_VERSION 6

/*
 * nvfp4_validate_scales — the load-time completeness check (page 3, "ROOT
 * CAUSE": format conversion takes reciprocals of w13_input_scale and
 * w2_input_scale into a1_gscale / a2_gscale without verifying that every
 * expert slot was written, so stale bits become inf, NaN or garbage
 * quantisation parameters).  HOST memory, synchronous, needs no GPU.
 *
 *   input_scale  host fp32 [num_experts]: one projection's per-expert FP32
 *                activation global scale (input_scale).
 *   written      host uint8 [num_experts] or NULL: nonzero where the loader
 *                wrote the slot.  A stale value can look like a valid float,
 *                so without this mask only value checks are possible.
 *   gscale_out   host fp32 [num_experts] or NULL: receives fl32(1/x) per slot,
 *                and is written ONLY when every slot passes (the page's
 *                SFScaleVal, i.e. a1_gscale / a2_gscale).
 *   slot_status  host int32 [num_experts] or NULL: NVFP4_SLOT_* per slot.
 *   num_bad      host int32 or NULL: number of rejected slots.
 *
 * Returns NVFP4_OK when every slot passes, NVFP4_ERR_BAD_SCALE when any slot
 * is rejected (nothing written to gscale_out), NVFP4_ERR_INVALID_ARG for a
 * NULL input_scale or num_experts <= 0.
 */
NVFP4_API nvfp4_status_t nvfp4_validate_scales(const float* input_scale, const uint8_t* written,
                                               int32_t num_experts, float* gscale_out,
                                               int32_t* slot_status, int32_t* num_bad);

/*
 * nvfp4_quantize_experts — dynamic per-expert NVFP4 activation quantisation
 * (page 3, "NVFP4" section: runtime-order figure and the
 * SFScale[expert_idx] excerpt), over rows already grouped by expert.  Row p
 * of the output belongs to the expert e with expert_offsets[e] <= p <
 * expert_offsets[e+1] and quantises source row s = src_row ? src_row[p] : p
 * of x in blocks of 16 along K, with SFScaleVal = gscale ? gscale[e] : 1.0f:
 *     amax = max|x|;  s = fl32(SFScaleVal * fl32(amax / 6));
 *     sf = E4M3(s) (nearest, ties to even, saturating at 448);
 *     v = fl32(x * min(fl32(SFScaleVal / E4M3value(sf)), FLT_MAX)), or 0 when
 *     the E4M3 value is 0;  code = E2M1(v) (nearest, ties to even,
 *     saturating at 6, sign kept).
 *
 *   x_bf16          device bf16 [num_src_rows, ldx]; 16-byte aligned, ldx % 8 == 0.
 *   ldx             row stride of x in elements (>= K).
 *   K               elements per row; K % 16 == 0.
 *   src_row         device int32 [P] or NULL (identity: row p reads row p,
 *                   and then num_src_rows >= P is required).
 *   num_src_rows    rows of x; output rows whose source row falls outside
 *                   [0, num_src_rows) are not written.
 *   P               output rows; 0 is a no-op.
 *   expert_offsets  device int32 [E+1], non-decreasing; output rows outside
 *                   [expert_offsets[0], expert_offsets[E]) are not written.
 *   E               experts (length of gscale), >= 1.
 *   gscale          device fp32 [E] or NULL (=> 1.0f, the page's null-SFScale
 *                   case).  Values must come from nvfp4_validate_scales.
 *   codes           device uint8 [P, K/2], 8-byte aligned.
 *   sf              device uint8 [P, K/16].
 * NVFP4_ERR_INVALID_ARG for a bad size, a NULL required pointer or a
 * misaligned x / codes, before anything is enqueued.
 */
NVFP4_API nvfp4_status_t nvfp4_quantize_experts(const void* x_bf16, int64_t ldx, int32_t K,
                                                const int32_t* src_row, int32_t num_src_rows,
                                                int32_t P, const int32_t* expert_offsets,
                                                int32_t E, const float* gscale, uint8_t* codes,
                                                uint8_t* sf, nvfp4_stream_t stream);

/*
 * nvfp4_quantize_experts_fp16 — the same quantiser for fp16 source rows
 * (page 3, "NVFP4" runtime-order figure: the hidden state entering the
 * quantiser is BF16 or FP16).  Every fp16 value converts exactly to fp32, so
 * the arithmetic above applies unchanged.  Arguments, layouts, ownership and
 * errors as for nvfp4_quantize_experts, with x_fp16 device fp16
 * [num_src_rows, ldx], 16-byte aligned, ldx % 8 == 0.
 */
NVFP4_API nvfp4_status_t nvfp4_quantize_experts_fp16(const void* x_fp16, int64_t ldx, int32_t K,
                                                     const int32_t* src_row, int32_t num_src_rows,
                                                     int32_t P, const int32_t* expert_offsets,
                                                     int32_t E, const float* gscale,
                                                     uint8_t* codes, uint8_t* sf,
                                                     nvfp4_stream_t stream);

/*
 * nvfp4_quantize_pairs — the same quantisation, fused with the regrouping by
 * expert: the form the layer forward runs, which reads each token row once
 * for all of its topk destinations.  For every (row t, slot j) pair
 * q = t*topk + j, with e = expert_idx[q] (0 when expert_idx is NULL), row t of
 * x is quantised with SFScaleVal = gscale ? gscale[e] : 1.0f and written to
 * output row p = dst_row ? dst_row[q] : q.
 *
 *   x_bf16        device bf16 [num_rows, ldx]; 16-byte aligned, ldx % 8 == 0.
 *   num_rows      rows of x (tokens); 0 is a no-op.
 *   K             elements per row; K % 16 == 0.
 *   topk          destinations per source row (>= 1).
 *   expert_idx    device int32 [num_rows*topk] or NULL.
 *   dst_row       device int32 [num_rows*topk] or NULL (identity).  Distinct
 *                 destinations are the caller's contract; pairs whose p or e
 *                 falls outside [0, num_dst_rows) / [0, num_experts) are
 *                 skipped.
 *   num_experts   length of gscale (>= 1).
 *   gscale        device fp32 [num_experts] or NULL (=> 1.0f).
 *   codes         device uint8 [num_dst_rows, K/2], 8-byte aligned.
 *   sf            device uint8 [num_dst_rows, K/16].
 */
NVFP4_API nvfp4_status_t nvfp4_quantize_pairs(const void* x_bf16, int64_t ldx, int32_t num_rows,
                                              int32_t K, int32_t topk, const int32_t* expert_idx,
                                              const int32_t* dst_row, int32_t num_experts,
                                              const float* gscale, uint8_t* codes, uint8_t* sf,
                                              int32_t num_dst_rows, nvfp4_stream_t stream);

/*
 * nvfp4_route_topk — the router's choice of expert_idx (page 3, "NVFP4"
 * runtime figure: the router has fixed expert_idx before quantisation) and
 * the routing weights the final sum uses ("矩阵融合" pipeline figure).
 * Per token: the k largest fp32 logits, ordered by (logit descending, expert
 * index ascending); weights = softmax over those k logits, in fp32.
 *
 *   logits   device fp32 [num_tokens, num_experts], finite.
 *   ids      device int32 [num_tokens, k];  weights device fp32 [num_tokens, k].
 *   1 <= k <= num_experts <= 1024, k <= 32.
 */
NVFP4_API nvfp4_status_t nvfp4_route_topk(const float* logits, int32_t num_tokens,
                                          int32_t num_experts, int32_t k, int32_t* ids,
                                          float* weights, nvfp4_stream_t stream);

/*
 * nvfp4_permute — regroup the num_tokens*k (token, slot) pairs by expert so
 * every expert's rows are contiguous for the grouped GEMMs (page 3,
 * "矩阵融合", MoE FFN paragraph: the backend reorders inputs by routing so
 * the per-expert products form one grouped GEMM).  The order is stable:
 * sorted by (expert, token, slot).  Deterministic: the result does not depend
 * on the order in which the device's threads run.
 *
 *   ids             device int32 [num_tokens*k], each in [0, num_experts);
 *                   pairs with an id outside that range are left out (their
 *                   inv_pair entry is not written).  1 <= num_experts <= 1024.
 *   expert_offsets  device int32 [num_experts+1]: rows of expert e are
 *                   [offsets[e], offsets[e+1]).
 *   src_pair        device int32 [num_tokens*k]: permuted row p -> pair q.
 *   inv_pair        device int32 [num_tokens*k]: pair q -> permuted row p.
 */
NVFP4_API nvfp4_status_t nvfp4_permute(const int32_t* ids, int32_t num_tokens, int32_t k,
                                       int32_t num_experts, int32_t* expert_offsets,
                                       int32_t* src_pair, int32_t* inv_pair,
                                       nvfp4_stream_t stream);

/*
 * nvfp4_expert_absmax — calibration helper: per-expert max |x| over grouped
 * rows, the statistic behind the FP32 global scales (page 3, "NVFP4" section:
 * the stored global scale is based on the 6 x 448 = 2688 range; calibration
 * glossary entry: activation statistics gathered per expert).  Rows of expert
 * e are p in [expert_offsets[e], expert_offsets[e+1]); row p reads source row
 * src ? src[p] / src_div : p of x.  amax_out[e] = 0 for an expert with no rows.
 *
 *   x_bf16          device bf16 [*, ldx], 16-byte aligned, ldx % 8 == 0, K % 8 == 0.
 *   src             device int32 [num_rows] or NULL;  src_div >= 1.
 *   expert_offsets  device int32 [num_experts+1], non-decreasing, offsets[0] == 0.
 *   num_rows        expert_offsets[num_experts] (the grouped row count).
 *   amax_out        device fp32 [num_experts].
 */
NVFP4_API nvfp4_status_t nvfp4_expert_absmax(const void* x_bf16, int64_t ldx, int32_t K,
                                             const int32_t* src, int32_t src_div,
                                             const int32_t* expert_offsets, int32_t num_experts,
                                             int32_t num_rows, float* amax_out,
                                             nvfp4_stream_t stream);

/*
 * nvfp4_calibrate_input_scales — the calibration pass behind the per-expert
 * FP32 activation scales, with its coverage report (page 3, "ROOT CAUSE":
 * experts that saw no calibration token are left without a written
 * input_scale; "NVFP4" section: the stored global scale is based on the
 * 6 x 448 = 2688 range).  Over the grouped rows of each expert (as in
 * nvfp4_expert_absmax):
 *     input_scale[e] = fl32(max|x| / 2688), written[e] = 1   if e has rows,
 *     input_scale[e] = NaN,                 written[e] = 0   otherwise.
 * Passing both arrays to nvfp4_validate_scales then rejects exactly the
 * experts without calibration rows (NVFP4_SLOT_UNWRITTEN), before any
 * reciprocal is taken.
 *
 *   x_bf16, ldx, K, src, src_div, expert_offsets, num_experts, num_rows:
 *                    as for nvfp4_expert_absmax.
 *   input_scale_out  device fp32 [num_experts].
 *   written_out      device uint8 [num_experts].
 */
NVFP4_API nvfp4_status_t nvfp4_calibrate_input_scales(const void* x_bf16, int64_t ldx, int32_t K,
                                                      const int32_t* src, int32_t src_div,
                                                      const int32_t* expert_offsets,
                                                      int32_t num_experts, int32_t num_rows,
                                                      float* input_scale_out,
                                                      uint8_t* written_out,
                                                      nvfp4_stream_t stream);

/*
 * nvfp4_selftest_conversions — device self-check of the five gfx950
 * conversion instructions the kernels use, each against a reference built
 * from the format definitions (page 3, "NVFP4" section: the E2M1 code table;
 * encoding rounds to nearest with ties to even and saturates to 6; E4M3 block
 * scales).  mismatches: device uint64[5], written asynchronously:
 *   [0] fp32 -> E2M1 encode vs midpoint comparisons, every non-NaN fp32 input;
 *   [1] E2M1 byte -> fp16 pair vs the code table, all 256 bytes x 4 positions;
 *   [2] E4M3 -> fp16 vs the OCP E4M3 definition, all 254 non-NaN codes;
 *   [3] non-negative fp32 -> E4M3 block-scale encode (clamp to 448, then the
 *       FP8 conversion) vs nearest-even saturating rounding, every
 *       non-negative fp32 input and +inf;
 *   [4] E4M3 -> fp32 vs the OCP E4M3 definition, all 127 non-negative codes.
 * All five must read 0.
 */
NVFP4_API nvfp4_status_t nvfp4_selftest_conversions(unsigned long long* mismatches,
                                                    nvfp4_stream_t stream);

/*
 * nvfp4_moe_pack_weights — load-time layout conversion of one projection's
 * NVFP4 expert weights into the layout the grouped GEMMs read (page 3,
 * "Kernel Backend": once the backend is chosen, the packed weights and their
 * scales are converted to the layout that implementation requires, then
 * handed to the kernel).  A pure byte permutation within each block of 32
 * weight rows; sizes are unchanged.
 *
 *   projection  0 = w13 ([E, 2I, H]: codes [E, 2I, H/2], scales [E, 2I, H/16]),
 *               1 = w2  ([E, H, I]:  codes [E, H, I/2],  scales [E, H, I/16]).
 *   codes, sf   device, the checkpoint's row-major layout (16-byte aligned codes).
 *   codes_out, sf_out  device, same sizes, distinct from the inputs: the
 *               kernel layout nvfp4_moe_forward expects.
 *   Requires H % 128 == 0 and I % 64 == 0 (else NVFP4_ERR_UNSUPPORTED).
 */
NVFP4_API nvfp4_status_t nvfp4_moe_pack_weights(int32_t projection, const uint8_t* codes,
                                                const uint8_t* sf, int32_t num_experts,
                                                int32_t hidden, int32_t inter, uint8_t* codes_out,
                                                uint8_t* sf_out, nvfp4_stream_t stream);

/*
 * One MoE layer's NVFP4 expert weights and scales — the checkpoint fields of
 * page 3 ("ROOT CAUSE" and the glossary's static weight quantisation entry:
 * w13/w2 packed FP4 weights, weight_scale (E4M3 per 16), weight_scale_2
 * (FP32 per expert), w13_input_scale / w2_input_scale (FP32 per expert)),
 * plus the reciprocals a1_gscale / a2_gscale from nvfp4_validate_scales.
 * All device pointers, caller-owned.  w13/w13_sf and w2/w2_sf are in the
 * kernel layout produced by nvfp4_moe_pack_weights from the logical PyTorch
 * [out, in] layout: w13 [E, 2I, H] with rows [0, I) gate and [I, 2I) up
 * ("矩阵融合", gated FFN: gate and up fused into w13), w2 [E, H, I];
 * *_scale2, *_input_scale, a*_gscale [E].
 */
typedef struct {
  const uint8_t* w13;
  const uint8_t* w13_sf;
  const float* w13_scale2;
  const uint8_t* w2;
  const uint8_t* w2_sf;
  const float* w2_scale2;
  const float* w13_input_scale;
  const float* w2_input_scale;
  const float* a1_gscale;
  const float* a2_gscale;
  int32_t num_experts;  /* E */
  int32_t hidden;       /* H */
  int32_t inter;        /* I */
} nvfp4_moe_weights_t;

/* Optional device buffers that receive intermediates of nvfp4_moe_forward
 * (P = num_tokens*k).  Any member may be NULL.  stage_events, when set, is an
 * array of NVFP4_MOE_STAGES+1 hipEvent_t (created by the caller) recorded on
 * the stream before the first launch and after each stage: route, permute,
 * quantise A1, grouped w13 GEMM (+SiLU*mul+requant), grouped w2 GEMM,
 * combine.  In the W4A4 forwards, when H/16 lies in [64, 1024] (and H is a
 * multiple of 128 in the UE8M0 mode), routing and the A1 quantisation run as
 * one kernel: it is timed as the route stage and the quantise stage is
 * empty.  Batches of at most 512 pairs whose experts
 * average fewer than 32 rows (P < 32*E) launch no permutation kernel: the
 * w13 GEMM regroups the routed ids itself and writes expert_offsets,
 * src_pair and inv, so the permute stage is empty.  Buffer dumps are copied
 * after the last event. */
#define NVFP4_MOE_STAGES 6
typedef struct {
  int32_t* topk_ids;        /* [T, k]   */
  float* topk_weights;      /* [T, k]   */
  int32_t* expert_offsets;  /* [E+1]    */
  int32_t* src_pair;        /* [P]      */
  int32_t* inv_pair;        /* [P]      */
  uint8_t* a1_codes;        /* [P, H/2]  rows in (token, slot) order t*k + j */
  uint8_t* a1_sf;           /* [P, H/16] the same order */
  float* c1;                /* [P, 2I]  fp32 w13 output incl. alpha1 */
  uint16_t* h;              /* [P, I]   bf16 SiLU(gate)*up           */
  uint8_t* a2_codes;        /* [P, I/2] */
  uint8_t* a2_sf;           /* [P, I/16]*/
  float* c2;                /* [P, H]   fp32 w2 output incl. alpha2  */
  void** stage_events;      /* hipEvent_t[NVFP4_MOE_STAGES+1]        */
} nvfp4_moe_debug_t;

/* Bytes of device workspace nvfp4_moe_forward needs for these sizes. */
NVFP4_API nvfp4_status_t nvfp4_moe_workspace_size(int32_t num_tokens, int32_t k,
                                                  const nvfp4_moe_weights_t* w, size_t* bytes);

/*
 * nvfp4_moe_forward — one NVFP4 W4A4 routed-expert MoE layer (page 3,
 * "矩阵融合" pipeline figure), all on `stream`:
 *   route (top-k of fp32 logits, softmax over the k) -> permute by expert ->
 *   quantise x per expert with a1_gscale -> grouped w13 GEMM,
 *   C1 = alpha1[e] * A1 . W13[e]^T, alpha1 = w13_input_scale * w13_scale2
 *   ("NVFP4" runtime figure: the GEMM output scaling folds in both FP32
 *   global scales) -> h = bf16(silu(gate) * up) -> quantise h with a2_gscale ->
 *   grouped w2 GEMM, C2 = alpha2[e] * A2 . W2[e]^T (fp32) ->
 *   out[t] = bf16(residual[t] + sum_j w[t,j] * C2[row of (t,j)]), j ascending.
 *
 *   x_bf16         device bf16 [T, H], 16-byte aligned.
 *   router_logits  device fp32 [T, E], finite.
 *   residual_bf16  device bf16 [T, H] or NULL (treated as zero).
 *   out_bf16       device bf16 [T, H]; may alias residual_bf16 or x_bf16.
 *   workspace      device, 256-byte aligned, >= nvfp4_moe_workspace_size().
 *   debug          NULL or buffers for intermediates.
 * Requirements: H % 128 == 0, I % 64 == 0, 1 <= k <= min(E, 32), E <= 1024,
 * T*k <= 2^30, and (ceil(T*k/32) + min(T*k, E)) * max(ceil(I/128), ceil(H/256))
 * <= 2^31 - 1 (the GEMM tile count); else NVFP4_ERR_UNSUPPORTED.
 * T == 0 is a no-op.  Experts that receive no rows cost nothing.
 * The call only enqueues kernels: it allocates nothing, clears nothing with
 * memset and never synchronises the host.  With debug == NULL it may be
 * captured into a HIP graph and replayed; a replay reads whatever the input
 * buffers hold when it runs.  (Tested with one call on the device made
 * before the capture, which does the one-time occupancy lookup.)
 */
NVFP4_API nvfp4_status_t nvfp4_moe_forward(const nvfp4_moe_weights_t* w, const void* x_bf16,
                                           const float* router_logits, int32_t num_tokens,
                                           int32_t k, const void* residual_bf16, void* out_bf16,
                                           void* workspace, size_t workspace_bytes,
                                           const nvfp4_moe_debug_t* debug, nvfp4_stream_t stream);

/*
 * nvfp4_moe_forward_noalloc — nvfp4_moe_forward for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops
 * and harnesses that forbid hipMalloc.  The same layer, arguments, results,
 * debug buffers and errors as nvfp4_moe_forward, without the workspace
 * arguments: the workspace is a fixed buffer of NVFP4_NOALLOC_SCRATCH_BYTES
 * in static device memory that the library holds on every device it runs on
 * until the process ends.  Nothing is allocated or freed.
 *   Runs on the current device; `stream` must belong to it.
 *   Returns NVFP4_ERR_TOO_LARGE, before anything is enqueued, when
 *   nvfp4_moe_workspace_size(num_tokens, k, w) exceeds the buffer (at hidden
 *   2816, intermediate 704 and top-8: about 600 tokens).
 *   Every call on one device shares that device's buffer, which keeps the
 *   last call's contents: calls that overlap in time on one device (on two
 *   streams, or from two host threads) race, and the caller must serialise
 *   them.  No part of the buffer needs to start at zero.
 */
#define NVFP4_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
NVFP4_API nvfp4_status_t nvfp4_moe_forward_noalloc(const nvfp4_moe_weights_t* w,
                                                   const void* x_bf16,
                                                   const float* router_logits,
                                                   int32_t num_tokens, int32_t k,
                                                   const void* residual_bf16, void* out_bf16,
                                                   const nvfp4_moe_debug_t* debug,
                                                   nvfp4_stream_t stream);

/*
 * Weight-only (W4A16) forward of the same layer (page 3, "Kernel Backend" and
 * the "本案例：CUTLASS 与 Marlin" comparison: the MARLIN backend runs NVFP4
 * expert weights against bf16 activations — W4A16 — and sets the activation
 * scale to None, so w13_input_scale / w2_input_scale are never consumed).
 * Same weights and packed layout as nvfp4_moe_forward; on `stream`:
 *   route -> permute ->
 *   grouped w13 GEMM on bf16 rows, C1 = w13_scale2[e] * x[token(p)] . W13[e]^T
 *   -> h = bf16(silu(gate) * up), kept as bf16 ->
 *   grouped w2 GEMM, C2 = w2_scale2[e] * h . W2[e]^T (fp32) -> combine as in
 *   nvfp4_moe_forward.
 * Weight operands are dequantised exactly (E2M1 x E4M3 is a bf16 number);
 * activations are used as given.  w->w13_input_scale, w2_input_scale,
 * a1_gscale and a2_gscale may be NULL and are not read, so a layer whose
 * activation scales fail nvfp4_validate_scales still runs here.
 * Arguments and requirements as for nvfp4_moe_forward, with the workspace
 * from nvfp4_moe_workspace_size_w4a16.  debug: topk_ids, topk_weights,
 * expert_offsets, src_pair, inv_pair, c1, h, c2 are filled; the a1/a2 members
 * are ignored; stage event 3 follows event 2 directly (no quantisation).
 */
NVFP4_API nvfp4_status_t nvfp4_moe_workspace_size_w4a16(int32_t num_tokens, int32_t k,
                                                        const nvfp4_moe_weights_t* w,
                                                        size_t* bytes);
NVFP4_API nvfp4_status_t nvfp4_moe_forward_w4a16(const nvfp4_moe_weights_t* w,
                                                 const void* x_bf16, const float* router_logits,
                                                 int32_t num_tokens, int32_t k,
                                                 const void* residual_bf16, void* out_bf16,
                                                 void* workspace, size_t workspace_bytes,
                                                 const nvfp4_moe_debug_t* debug,
                                                 nvfp4_stream_t stream);

/*
 * ---- UE8M0 (MX-style) block-scale mode --------------------------------------
 * Page 3 ("NVFP4" section, quantiser excerpt) instantiates the per-expert
 * quantiser with a UE8M0_SF switch that selects UE8M0 (unsigned 8-bit
 * power-of-two exponent) block scales instead of E4M3.  The pages give only
 * the switch; this library's reading: the block-scale value is formed as in
 * the E4M3 mode, s = fl32(gs * fl32(amax / 6)), and encoded as the smallest
 * power of two >= s, code = log2 + 127 clamped to [1, 254]; a block is 32
 * consecutive elements; elements are normalised by fl32(gs / 2^(code-127))
 * (clamped to FLT_MAX) and rounded to E2M1 exactly as in the E4M3 mode.
 * Dequantised value: E2M1(code) * 2^(sf - 127) (times the FP32 global scale).
 */

/*
 * nvfp4_quantize_experts_mx / nvfp4_quantize_pairs_mx — nvfp4_quantize_experts
 * and nvfp4_quantize_pairs in the UE8M0 mode.  Same arguments and
 * behaviour, except: K % 32 == 0, and sf is [rows, K/32] UE8M0 codes (one per
 * 32 elements).
 */
NVFP4_API nvfp4_status_t nvfp4_quantize_experts_mx(const void* x_bf16, int64_t ldx, int32_t K,
                                                   const int32_t* src_row, int32_t num_src_rows,
                                                   int32_t P, const int32_t* expert_offsets,
                                                   int32_t E, const float* gscale, uint8_t* codes,
                                                   uint8_t* sf, nvfp4_stream_t stream);
NVFP4_API nvfp4_status_t nvfp4_quantize_pairs_mx(const void* x_bf16, int64_t ldx,
                                                 int32_t num_rows, int32_t K, int32_t topk,
                                                 const int32_t* expert_idx,
                                                 const int32_t* dst_row, int32_t num_experts,
                                                 const float* gscale, uint8_t* codes,
                                                 uint8_t* sf, int32_t num_dst_rows,
                                                 nvfp4_stream_t stream);

/*
 * nvfp4_moe_pack_weights_mx — nvfp4_moe_pack_weights for UE8M0 weights:
 * scales are [E, 2I, H/32] (projection 0) or [E, H, I/32] (projection 1);
 * codes as in the E4M3 mode (w13 with a 256-wide K step).  Same errors;
 * requires H % 256 == 0 and I % 64 == 0 (else NVFP4_ERR_UNSUPPORTED).
 */
NVFP4_API nvfp4_status_t nvfp4_moe_pack_weights_mx(int32_t projection, const uint8_t* codes,
                                                   const uint8_t* sf, int32_t num_experts,
                                                   int32_t hidden, int32_t inter,
                                                   uint8_t* codes_out, uint8_t* sf_out,
                                                   nvfp4_stream_t stream);

/*
 * nvfp4_moe_forward_mx — the W4A4 layer of nvfp4_moe_forward with every block
 * scale in the UE8M0 mode: weights packed by nvfp4_moe_pack_weights_mx, A1 and
 * A2 quantised with UE8M0 scales per 32 elements (a1_gscale / a2_gscale as
 * SFScaleVal), both grouped GEMMs on the gfx950 scaled FP4 matrix instruction
 * (the power-of-two block scales are applied by the instruction; nothing is
 * dequantised), alpha = input_scale * weight_scale_2 as in the E4M3 mode.
 * Same arguments, workspace (nvfp4_moe_workspace_size) and debug buffers as
 * nvfp4_moe_forward, plus H % 256 == 0; debug a1_sf / a2_sf receive
 * [P, H/32] and [P, I/32] UE8M0 codes.
 */
NVFP4_API nvfp4_status_t nvfp4_moe_forward_mx(const nvfp4_moe_weights_t* w, const void* x_bf16,
                                              const float* router_logits, int32_t num_tokens,
                                              int32_t k, const void* residual_bf16,
                                              void* out_bf16, void* workspace,
                                              size_t workspace_bytes,
                                              const nvfp4_moe_debug_t* debug,
                                              nvfp4_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_MOE_H */
