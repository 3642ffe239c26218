// C ABI of libnvfp4moe.so: argument checking, the load-time scale check,
// workspace layout and the launch sequence of one MoE layer.
#include <algorithm>
#include <cstdint>
#include <math.h>
#include <string.h>

#include <hip/hip_runtime.h>

#define NVFP4_BUILDING_LIBRARY 1
#include "../../include/nvfp4_moe.h"
#include "gemm_tiles.h"
#include "internal.h"

namespace {

using namespace nvfp4;

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

nvfp4_status_t device_status(hipError_t e) {
  return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_DEVICE;
}

// Byte layout of the forward pass's workspace.
// (The weight-only forward keeps no quantised activations: its a1/a2 regions
// are empty and h holds the bf16 GEMM1 output instead.)
struct Layout {
  size_t ids, wts, offsets, src_pair, inv, a1c, a1s, a2c, a2s, h, c2, total;
};

Layout layout(int64_t T, int64_t k, int64_t E, int64_t H, int64_t I, bool w16 = false) {
  const int64_t P = T * k;
  const int64_t Pq = w16 ? 0 : P, Ph = w16 ? P : 0;
  Layout L;
  size_t o = 0;
  L.ids = o;      o = align_up(o + (size_t)P * 4);
  L.wts = o;      o = align_up(o + (size_t)P * 4);
  L.offsets = o;  o = align_up(o + (size_t)(E + 1) * 4);
  L.src_pair = o; o = align_up(o + (size_t)P * 4);
  L.inv = o;      o = align_up(o + (size_t)P * 4);
  L.a1c = o;      o = align_up(o + (size_t)Pq * (H / 2));
  L.a1s = o;      o = align_up(o + (size_t)Pq * (H / 16));
  L.a2c = o;      o = align_up(o + (size_t)Pq * (I / 2));
  L.a2s = o;      o = align_up(o + (size_t)Pq * (I / 16));
  L.h = o;        o = align_up(o + (size_t)Ph * I * 2);
  L.c2 = o;       o = align_up(o + (size_t)P * H * 4);
  L.total = o;
  return L;
}

// The activation scales (input scales and their reciprocals) are required
// by the W4A4 forward only; the weight-only forward never reads them.
nvfp4_status_t check_weights(const nvfp4_moe_weights_t* w, bool w16 = false) {
  if (!w || !w->w13 || !w->w13_sf || !w->w13_scale2 || !w->w2 || !w->w2_sf || !w->w2_scale2)
    return NVFP4_ERR_INVALID_ARG;
  if (!w16 && (!w->w13_input_scale || !w->w2_input_scale || !w->a1_gscale || !w->a2_gscale))
    return NVFP4_ERR_INVALID_ARG;
  if (w->num_experts <= 0 || w->hidden <= 0 || w->inter <= 0) return NVFP4_ERR_INVALID_ARG;
  if (w->hidden % 16 || w->inter % 16) return NVFP4_ERR_INVALID_ARG;
  if (!aligned(w->w13, 16) || !aligned(w->w2, 16)) return NVFP4_ERR_INVALID_ARG;
  if (w->num_experts > 1024) return NVFP4_ERR_UNSUPPORTED;
  if (w->hidden % 128 || w->inter % 64) return NVFP4_ERR_UNSUPPORTED;
  return NVFP4_OK;
}

hipError_t copy_async(void* dst, const void* src, size_t bytes, hipStream_t s) {
  if (!dst || bytes == 0) return hipSuccess;
  return hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, s);
}

}  // namespace

extern "C" {

NVFP4_API const char* nvfp4_status_string(nvfp4_status_t status) {
  switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_INVALID_ARG: return "invalid argument";
    case NVFP4_ERR_BAD_SCALE: return "per-expert input scale failed the load-time check";
    case NVFP4_ERR_WORKSPACE: return "workspace missing or too small";
    case NVFP4_ERR_DEVICE: return "HIP runtime error";
    case NVFP4_ERR_UNSUPPORTED: return "shape not supported by the built kernels";
    case NVFP4_ERR_TOO_LARGE:
      return "request needs more workspace than the allocation-free forward's fixed buffer";
  }
  return "unknown status";
}

NVFP4_API int32_t nvfp4_abi_version(void) { return NVFP4_ABI_VERSION; }

NVFP4_API nvfp4_status_t nvfp4_validate_scales(const float* input_scale, const uint8_t* written,
                                               int32_t num_experts, float* gscale_out,
                                               int32_t* slot_status, int32_t* num_bad) {
  if (!input_scale || num_experts <= 0) return NVFP4_ERR_INVALID_ARG;
  int32_t bad = 0;
  for (int32_t e = 0; e < num_experts; ++e) {
    // read the bits, so a signalling pattern is never used as a float operand
    uint32_t bits;
    memcpy(&bits, input_scale + e, 4);
    const uint32_t mag = bits & 0x7FFFFFFFu;
    int32_t st = NVFP4_SLOT_OK;
    if (written && !written[e]) st = NVFP4_SLOT_UNWRITTEN;
    else if (mag > 0x7F800000u) st = NVFP4_SLOT_NAN;
    else if (mag == 0x7F800000u) st = NVFP4_SLOT_INF;
    else if ((bits >> 31) || mag == 0) st = NVFP4_SLOT_NONPOSITIVE;
    else {
      volatile float x = input_scale[e];
      const float r = 1.0f / x;
      if (!isfinite(r)) st = NVFP4_SLOT_RECIP_OVERFLOW;
    }
    if (slot_status) slot_status[e] = st;
    bad += st != NVFP4_SLOT_OK;
  }
  if (num_bad) *num_bad = bad;
  if (bad) return NVFP4_ERR_BAD_SCALE;
  if (gscale_out)
    for (int32_t e = 0; e < num_experts; ++e) gscale_out[e] = 1.0f / input_scale[e];
  return NVFP4_OK;
}

}  // extern "C"

namespace {

// The gather-form quantiser entry points (E4M3 bf16, E4M3 fp16, UE8M0 bf16).
nvfp4_status_t quantize_gather(const void* x, int64_t ldx, int32_t K, const int32_t* src_row,
                               int32_t num_src_rows, int32_t P, const int32_t* expert_offsets,
                               int32_t E, const float* gscale, uint8_t* codes, uint8_t* sf,
                               nvfp4_stream_t stream, bool fp16, bool mx) {
  if (P < 0 || K <= 0 || K % (mx ? 32 : 16) || E < 1 || num_src_rows < 0 || ldx < K || ldx % 8)
    return NVFP4_ERR_INVALID_ARG;
  if (P == 0) return NVFP4_OK;
  if (!x || !expert_offsets || !codes || !sf || !aligned(x, 16) || !aligned(codes, 8))
    return NVFP4_ERR_INVALID_ARG;
  if (!src_row && num_src_rows < P) return NVFP4_ERR_INVALID_ARG;
  return device_status(launch_quantize_gather(static_cast<const uint16_t*>(x), ldx, K, src_row, 1,
                                              num_src_rows, P, expert_offsets, E, gscale, codes,
                                              sf, static_cast<hipStream_t>(stream), fp16, mx));
}

// The scatter-form (token-slot pairs) entry points.
nvfp4_status_t quantize_pairs(const void* x_bf16, int64_t ldx, int32_t num_rows, int32_t K,
                              int32_t topk, const int32_t* expert_idx, const int32_t* dst_row,
                              int32_t num_experts, const float* gscale, uint8_t* codes,
                              uint8_t* sf, int32_t num_dst_rows, nvfp4_stream_t stream, bool mx) {
  if (num_rows < 0 || K <= 0 || K % (mx ? 32 : 16) || topk < 1 || num_experts < 1 ||
      num_dst_rows < 0 || ldx < K || ldx % 8)
    return NVFP4_ERR_INVALID_ARG;
  if (num_rows == 0) return NVFP4_OK;
  if (!x_bf16 || !codes || !sf || !aligned(x_bf16, 16) || !aligned(codes, 8))
    return NVFP4_ERR_INVALID_ARG;
  return device_status(launch_quantize(static_cast<const uint16_t*>(x_bf16), ldx, num_rows, K,
                                       topk, expert_idx, dst_row, num_experts, gscale, codes, sf,
                                       num_dst_rows, static_cast<hipStream_t>(stream), false, mx));
}

}  // namespace

extern "C" {

NVFP4_API nvfp4_status_t nvfp4_quantize_experts(const void* x_bf16, int64_t ldx, int32_t K,
                                                const int32_t* src_row, int32_t num_src_rows,
                                                int32_t P, const int32_t* expert_offsets,
                                                int32_t E, const float* gscale, uint8_t* codes,
                                                uint8_t* sf, nvfp4_stream_t stream) {
  return quantize_gather(x_bf16, ldx, K, src_row, num_src_rows, P, expert_offsets, E, gscale,
                         codes, sf, stream, false, false);
}

NVFP4_API nvfp4_status_t nvfp4_quantize_experts_fp16(const void* x_fp16, int64_t ldx, int32_t K,
                                                     const int32_t* src_row, int32_t num_src_rows,
                                                     int32_t P, const int32_t* expert_offsets,
                                                     int32_t E, const float* gscale,
                                                     uint8_t* codes, uint8_t* sf,
                                                     nvfp4_stream_t stream) {
  return quantize_gather(x_fp16, ldx, K, src_row, num_src_rows, P, expert_offsets, E, gscale,
                         codes, sf, stream, true, false);
}

NVFP4_API nvfp4_status_t nvfp4_quantize_experts_mx(const void* x_bf16, int64_t ldx, int32_t K,
                                                   const int32_t* src_row, int32_t num_src_rows,
                                                   int32_t P, const int32_t* expert_offsets,
                                                   int32_t E, const float* gscale, uint8_t* codes,
                                                   uint8_t* sf, nvfp4_stream_t stream) {
  return quantize_gather(x_bf16, ldx, K, src_row, num_src_rows, P, expert_offsets, E, gscale,
                         codes, sf, stream, false, true);
}

NVFP4_API nvfp4_status_t nvfp4_quantize_pairs(const void* x_bf16, int64_t ldx, int32_t num_rows,
                                              int32_t K, int32_t topk, const int32_t* expert_idx,
                                              const int32_t* dst_row, int32_t num_experts,
                                              const float* gscale, uint8_t* codes, uint8_t* sf,
                                              int32_t num_dst_rows, nvfp4_stream_t stream) {
  return quantize_pairs(x_bf16, ldx, num_rows, K, topk, expert_idx, dst_row, num_experts, gscale,
                        codes, sf, num_dst_rows, stream, false);
}

NVFP4_API nvfp4_status_t nvfp4_quantize_pairs_mx(const void* x_bf16, int64_t ldx,
                                                 int32_t num_rows, int32_t K, int32_t topk,
                                                 const int32_t* expert_idx,
                                                 const int32_t* dst_row, int32_t num_experts,
                                                 const float* gscale, uint8_t* codes,
                                                 uint8_t* sf, int32_t num_dst_rows,
                                                 nvfp4_stream_t stream) {
  return quantize_pairs(x_bf16, ldx, num_rows, K, topk, expert_idx, dst_row, num_experts, gscale,
                        codes, sf, num_dst_rows, stream, true);
}

NVFP4_API nvfp4_status_t nvfp4_route_topk(const float* logits, int32_t num_tokens,
                                          int32_t num_experts, int32_t k, int32_t* ids,
                                          float* weights, nvfp4_stream_t stream) {
  if (num_tokens < 0 || num_experts < 1 || k < 1 || k > num_experts) return NVFP4_ERR_INVALID_ARG;
  if (num_experts > 1024 || k > 32) return NVFP4_ERR_UNSUPPORTED;
  if (num_tokens == 0) return NVFP4_OK;
  if (!logits || !ids || !weights) return NVFP4_ERR_INVALID_ARG;
  return device_status(launch_route(logits, num_tokens, num_experts, k, ids, weights,
                                    static_cast<hipStream_t>(stream)));
}

NVFP4_API nvfp4_status_t nvfp4_permute(const int32_t* ids, int32_t num_tokens, int32_t k,
                                       int32_t num_experts, int32_t* expert_offsets,
                                       int32_t* src_pair, int32_t* inv_pair,
                                       nvfp4_stream_t stream) {
  if (num_tokens < 0 || k < 1 || num_experts < 1) return NVFP4_ERR_INVALID_ARG;
  if (num_experts > 1024) return NVFP4_ERR_UNSUPPORTED;
  if (!expert_offsets) return NVFP4_ERR_INVALID_ARG;
  if (num_tokens > 0 && (!ids || !src_pair || !inv_pair)) return NVFP4_ERR_INVALID_ARG;
  if ((int64_t)num_tokens * k > 0x7FFFFFFF) return NVFP4_ERR_UNSUPPORTED;
  return device_status(launch_permute(ids, num_tokens * k, num_experts, expert_offsets, src_pair,
                                      inv_pair, static_cast<hipStream_t>(stream)));
}

NVFP4_API nvfp4_status_t nvfp4_expert_absmax(const void* x_bf16, int64_t ldx, int32_t K,
                                             const int32_t* src, int32_t src_div,
                                             const int32_t* expert_offsets, int32_t num_experts,
                                             int32_t num_rows, float* amax_out,
                                             nvfp4_stream_t stream) {
  if (K <= 0 || K % 8 || ldx < K || ldx % 8 || src_div < 1 || num_experts < 1 || num_rows < 0)
    return NVFP4_ERR_INVALID_ARG;
  if (!expert_offsets || !amax_out) return NVFP4_ERR_INVALID_ARG;
  if (num_rows > 0 && (!x_bf16 || !aligned(x_bf16, 16))) return NVFP4_ERR_INVALID_ARG;
  return device_status(launch_absmax(static_cast<const uint16_t*>(x_bf16), ldx, K, src, src_div,
                                     expert_offsets, num_experts, num_rows, amax_out,
                                     static_cast<hipStream_t>(stream)));
}

NVFP4_API nvfp4_status_t nvfp4_calibrate_input_scales(const void* x_bf16, int64_t ldx, int32_t K,
                                                      const int32_t* src, int32_t src_div,
                                                      const int32_t* expert_offsets,
                                                      int32_t num_experts, int32_t num_rows,
                                                      float* input_scale_out,
                                                      uint8_t* written_out,
                                                      nvfp4_stream_t stream) {
  if (K <= 0 || K % 8 || ldx < K || ldx % 8 || src_div < 1 || num_experts < 1 || num_rows < 0)
    return NVFP4_ERR_INVALID_ARG;
  if (!expert_offsets || !input_scale_out || !written_out) return NVFP4_ERR_INVALID_ARG;
  if (num_rows > 0 && (!x_bf16 || !aligned(x_bf16, 16))) return NVFP4_ERR_INVALID_ARG;
  return device_status(launch_calibrate(static_cast<const uint16_t*>(x_bf16), ldx, K, src,
                                        src_div, expert_offsets, num_experts, num_rows,
                                        input_scale_out, written_out,
                                        static_cast<hipStream_t>(stream)));
}

NVFP4_API nvfp4_status_t nvfp4_selftest_conversions(unsigned long long* mismatches,
                                                    nvfp4_stream_t stream) {
  if (!mismatches) return NVFP4_ERR_INVALID_ARG;
  return device_status(launch_conversions_selftest(mismatches, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

nvfp4_status_t pack_weights(int32_t projection, const uint8_t* codes, const uint8_t* sf,
                            int32_t num_experts, int32_t hidden, int32_t inter,
                            uint8_t* codes_out, uint8_t* sf_out, nvfp4_stream_t stream, bool mx) {
  if (projection != 0 && projection != 1) return NVFP4_ERR_INVALID_ARG;
  if (num_experts < 1 || hidden <= 0 || inter <= 0 || hidden % 16 || inter % 16)
    return NVFP4_ERR_INVALID_ARG;
  if (hidden % 128 || inter % 64 || (mx && hidden % 256)) return NVFP4_ERR_UNSUPPORTED;
  if (!codes || !sf || !codes_out || !sf_out || codes == codes_out || sf == sf_out)
    return NVFP4_ERR_INVALID_ARG;
  if (!aligned(codes, 16) || !aligned(codes_out, 16)) return NVFP4_ERR_INVALID_ARG;
  const int32_t N = projection == 0 ? 2 * inter : hidden;
  const int32_t K = projection == 0 ? hidden : inter;
  return device_status(launch_pack_weights(projection, codes, sf, num_experts, N, K, codes_out,
                                           sf_out, static_cast<hipStream_t>(stream), mx));
}

}  // namespace

extern "C" {

NVFP4_API nvfp4_status_t nvfp4_moe_pack_weights(int32_t projection, const uint8_t* codes,
                                                const uint8_t* sf, int32_t num_experts,
                                                int32_t hidden, int32_t inter, uint8_t* codes_out,
                                                uint8_t* sf_out, nvfp4_stream_t stream) {
  return pack_weights(projection, codes, sf, num_experts, hidden, inter, codes_out, sf_out,
                      stream, false);
}

NVFP4_API nvfp4_status_t nvfp4_moe_pack_weights_mx(int32_t projection, const uint8_t* codes,
                                                   const uint8_t* sf, int32_t num_experts,
                                                   int32_t hidden, int32_t inter,
                                                   uint8_t* codes_out, uint8_t* sf_out,
                                                   nvfp4_stream_t stream) {
  return pack_weights(projection, codes, sf, num_experts, hidden, inter, codes_out, sf_out,
                      stream, true);
}

NVFP4_API nvfp4_status_t nvfp4_moe_workspace_size(int32_t num_tokens, int32_t k,
                                                  const nvfp4_moe_weights_t* w, size_t* bytes) {
  if (!bytes || !w || num_tokens < 0 || k < 1) return NVFP4_ERR_INVALID_ARG;
  if (w->num_experts <= 0 || w->hidden <= 0 || w->inter <= 0) return NVFP4_ERR_INVALID_ARG;
  *bytes = layout(num_tokens, k, w->num_experts, w->hidden, w->inter).total;
  return NVFP4_OK;
}

NVFP4_API nvfp4_status_t nvfp4_moe_workspace_size_w4a16(int32_t num_tokens, int32_t k,
                                                        const nvfp4_moe_weights_t* w,
                                                        size_t* bytes) {
  if (!bytes || !w || num_tokens < 0 || k < 1) return NVFP4_ERR_INVALID_ARG;
  if (w->num_experts <= 0 || w->hidden <= 0 || w->inter <= 0) return NVFP4_ERR_INVALID_ARG;
  *bytes = layout(num_tokens, k, w->num_experts, w->hidden, w->inter, true).total;
  return NVFP4_OK;
}

}  // extern "C"

namespace {

enum class Mode { kNV, kW16, kMX };

// One MoE layer: W4A4 with E4M3 scales (kNV), weight-only W4A16 (kW16), or
// W4A4 with UE8M0 scales per 32 elements (kMX).
nvfp4_status_t moe_forward(const nvfp4_moe_weights_t* w, const void* x_bf16,
                           const float* router_logits, int32_t num_tokens, int32_t k,
                           const void* residual_bf16, void* out_bf16, void* workspace,
                           size_t workspace_bytes, const nvfp4_moe_debug_t* debug,
                           nvfp4_stream_t stream, Mode mode) {
  const bool w16 = mode == Mode::kW16, mx = mode == Mode::kMX;
  const int32_t sblk = mx ? 32 : 16;                    // elements per block scale
  nvfp4_status_t st = check_weights(w, w16);
  if (st != NVFP4_OK) return st;
  const int32_t E = w->num_experts, H = w->hidden, I = w->inter;
  if (mx && H % 256) return NVFP4_ERR_UNSUPPORTED;
  if (num_tokens < 0 || k < 1 || k > E) return NVFP4_ERR_INVALID_ARG;
  if (k > 32) return NVFP4_ERR_UNSUPPORTED;
  if ((int64_t)num_tokens * k > (1 << 30)) return NVFP4_ERR_UNSUPPORTED;
  // the GEMM kernels number their (m-tile, n-tile) pairs in 32 bits: bound
  // them for the smallest tiles (32 rows; 128 h columns, 256 output columns)
  {
    const int64_t P = (int64_t)num_tokens * k;
    const int64_t m_tiles = (P + 31) / 32 + (P < E ? P : E);
    const int64_t n_tiles = std::max(((int64_t)I + 127) / 128, ((int64_t)H + 255) / 256);
    if (m_tiles * n_tiles > INT32_MAX) return NVFP4_ERR_UNSUPPORTED;
  }
  if (num_tokens == 0) return NVFP4_OK;
  if (!x_bf16 || !router_logits || !out_bf16) return NVFP4_ERR_INVALID_ARG;
  if (!aligned(x_bf16, 16) || !aligned(out_bf16, 16) ||
      (residual_bf16 && !aligned(residual_bf16, 16)))
    return NVFP4_ERR_INVALID_ARG;
  const Layout L = layout(num_tokens, k, E, H, I, w16);
  if (!workspace || workspace_bytes < L.total || !aligned(workspace, kAlign))
    return NVFP4_ERR_WORKSPACE;

  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int32_t T = num_tokens, P = T * k;
  char* ws = static_cast<char*>(workspace);
  int32_t* ids = reinterpret_cast<int32_t*>(ws + L.ids);
  float* wts = reinterpret_cast<float*>(ws + L.wts);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
  int32_t* src_pair = reinterpret_cast<int32_t*>(ws + L.src_pair);
  int32_t* inv = reinterpret_cast<int32_t*>(ws + L.inv);
  uint8_t* a1c = reinterpret_cast<uint8_t*>(ws + L.a1c);
  uint8_t* a1s = reinterpret_cast<uint8_t*>(ws + L.a1s);
  uint8_t* a2c = reinterpret_cast<uint8_t*>(ws + L.a2c);
  uint8_t* a2s = reinterpret_cast<uint8_t*>(ws + L.a2s);
  uint16_t* hbuf = reinterpret_cast<uint16_t*>(ws + L.h);
  float* c2 = reinterpret_cast<float*>(ws + L.c2);

  void** ev = debug ? debug->stage_events : nullptr;
  auto mark = [&](int i) -> hipError_t {
    return ev ? hipEventRecord(static_cast<hipEvent_t>(ev[i]), s) : hipSuccess;
  };
  hipError_t err = mark(0);
  // A1 rows are written in (token, slot) order q = t*k + j: each token's k
  // rows are contiguous, and GEMM1 reads them through src_pair.  Both W4A4
  // modes route and quantise in one kernel where the fused kernel covers
  // the shape (timed as the route stage; the quantise stage is then empty).
  bool fused = false;
  if (err == hipSuccess && !w16) {
    const hipError_t ferr = launch_route_quantize(
        router_logits, T, E, k, ids, wts, static_cast<const uint16_t*>(x_bf16), H,
        w->a1_gscale, a1c, a1s, s, mx);
    if (ferr == hipSuccess) fused = true;
    else if (ferr != hipErrorNotSupported) err = ferr;
  }
  if (err == hipSuccess && !fused) err = launch_route(router_logits, T, E, k, ids, wts, s);
  if (err == hipSuccess) err = mark(1);
  // Small batches: GEMM1 regroups the routed ids itself and writes offsets,
  // src_pair and inv (the permute stage is then empty).
  const bool fold = gemm_map::fold_permutation(P, E);
  if (err == hipSuccess && !fold) err = launch_permute(ids, P, E, offsets, src_pair, inv, s);
  if (err == hipSuccess) err = mark(2);
  if (err == hipSuccess && !w16 && !fused)
    err = launch_quantize(static_cast<const uint16_t*>(x_bf16), H, T, H, k, ids, nullptr, E,
                          w->a1_gscale, a1c, a1s, P, s, false, mx);
  if (err == hipSuccess) err = mark(3);
  if (err == hipSuccess) {
    Gemm1Args g1;
    g1.a_codes = a1c; g1.a_sf = a1s; g1.w_codes = w->w13; g1.w_sf = w->w13_sf;
    g1.in_scale = w->w13_input_scale; g1.w_scale2 = w->w13_scale2; g1.out_gscale = w->a2_gscale;
    g1.offsets = offsets; g1.out_codes = a2c; g1.out_sf = a2s;
    g1.c1_dbg = debug ? debug->c1 : nullptr;
    g1.h_dbg = debug && !w16 ? debug->h : nullptr;
    g1.mx = mx;
    g1.a_src = src_pair;
    g1.a_src_div = 1;
    if (fold) {
      g1.perm_ids = ids;
      g1.perm_offsets = offsets; g1.perm_src = src_pair; g1.perm_inv = inv;
    }
    if (w16) {
      g1.w16 = true;
      g1.a_rows = static_cast<const uint16_t*>(x_bf16);
      g1.a_src = src_pair; g1.a_src_div = k; g1.lda = H;
      g1.h_out = hbuf;
    }
    g1.P = P; g1.E = E; g1.H = H; g1.I = I;
    err = launch_gemm1(g1, s);
  }
  if (err == hipSuccess) err = mark(4);
  if (err == hipSuccess) {
    Gemm2Args g2;
    g2.a_codes = a2c; g2.a_sf = a2s; g2.w_codes = w->w2; g2.w_sf = w->w2_sf;
    g2.in_scale = w->w2_input_scale; g2.w_scale2 = w->w2_scale2; g2.offsets = offsets;
    if (w16) { g2.w16 = true; g2.a_rows = hbuf; }
    g2.mx = mx;
    g2.out = c2; g2.P = P; g2.E = E; g2.H = H; g2.I = I;
    err = launch_gemm2(g2, s);
  }
  if (err == hipSuccess) err = mark(5);
  if (err == hipSuccess)
    err = launch_combine(c2, wts, inv, T, k, H, static_cast<const uint16_t*>(residual_bf16),
                         static_cast<uint16_t*>(out_bf16), s);
  if (err == hipSuccess) err = mark(6);
  if (err == hipSuccess && debug) {
    err = copy_async(debug->topk_ids, ids, (size_t)P * 4, s);
    if (err == hipSuccess) err = copy_async(debug->topk_weights, wts, (size_t)P * 4, s);
    if (err == hipSuccess) err = copy_async(debug->expert_offsets, offsets, (size_t)(E + 1) * 4, s);
    if (err == hipSuccess) err = copy_async(debug->src_pair, src_pair, (size_t)P * 4, s);
    if (err == hipSuccess) err = copy_async(debug->inv_pair, inv, (size_t)P * 4, s);
    if (!w16) {
      if (err == hipSuccess) err = copy_async(debug->a1_codes, a1c, (size_t)P * (H / 2), s);
      if (err == hipSuccess) err = copy_async(debug->a1_sf, a1s, (size_t)P * (H / sblk), s);
      if (err == hipSuccess) err = copy_async(debug->a2_codes, a2c, (size_t)P * (I / 2), s);
      if (err == hipSuccess) err = copy_async(debug->a2_sf, a2s, (size_t)P * (I / sblk), s);
    } else {
      if (err == hipSuccess) err = copy_async(debug->h, hbuf, (size_t)P * I * 2, s);
    }
    if (err == hipSuccess) err = copy_async(debug->c2, c2, (size_t)P * H * 4, s);
  }
  return device_status(err);
}

}  // namespace

extern "C" {

NVFP4_API nvfp4_status_t nvfp4_moe_forward(const nvfp4_moe_weights_t* w, const void* x_bf16,
                                           const float* router_logits, int32_t num_tokens,
                                           int32_t k, const void* residual_bf16, void* out_bf16,
                                           void* workspace, size_t workspace_bytes,
                                           const nvfp4_moe_debug_t* debug, nvfp4_stream_t stream) {
  return moe_forward(w, x_bf16, router_logits, num_tokens, k, residual_bf16, out_bf16, workspace,
                     workspace_bytes, debug, stream, Mode::kNV);
}

NVFP4_API nvfp4_status_t nvfp4_moe_forward_mx(const nvfp4_moe_weights_t* w, const void* x_bf16,
                                              const float* router_logits, int32_t num_tokens,
                                              int32_t k, const void* residual_bf16,
                                              void* out_bf16, void* workspace,
                                              size_t workspace_bytes,
                                              const nvfp4_moe_debug_t* debug,
                                              nvfp4_stream_t stream) {
  return moe_forward(w, x_bf16, router_logits, num_tokens, k, residual_bf16, out_bf16, workspace,
                     workspace_bytes, debug, stream, Mode::kMX);
}

NVFP4_API nvfp4_status_t nvfp4_moe_forward_w4a16(const nvfp4_moe_weights_t* w,
                                                 const void* x_bf16, const float* router_logits,
                                                 int32_t num_tokens, int32_t k,
                                                 const void* residual_bf16, void* out_bf16,
                                                 void* workspace, size_t workspace_bytes,
                                                 const nvfp4_moe_debug_t* debug,
                                                 nvfp4_stream_t stream) {
  return moe_forward(w, x_bf16, router_logits, num_tokens, k, residual_bf16, out_bf16, workspace,
                     workspace_bytes, debug, stream, Mode::kW16);
}

}  // extern "C"
