// Host-side checks of the C ABI layer (api.cpp), built with g++ under
// AddressSanitizer and UndefinedBehaviorSanitizer and linked against recording
// stubs instead of the kernels and the HIP runtime: the load-time scale check,
// every entry point's argument checks, workspace sizing, and the launch
// sequence of a forward pass (which stage is launched with which buffers and
// sizes).  Nothing here touches a GPU; the stubs never dereference a pointer.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <string>
#include <vector>

#include <hip/hip_runtime.h>

#include "include/nvfp4_moe.h"
#include "nvfp4_w4a4_expert_amd/csrc/internal.h"

// ---- recording stubs ----------------------------------------------------------
static std::vector<std::string> g_calls;
static int g_quant_mx = -1, g_gemm1_mode = -1, g_gemm2_mode = -1;
static int32_t g_gemm1_P = -1, g_quant_dst_rows = -1;
// GEMM1 asked to regroup the routed ids itself (the permute kernel skipped)
static bool g_gemm1_fold = false;
// the fused routing + A1 quantisation launched in the UE8M0 mode
static bool g_rq_mx = false;
static int g_gather_src_div = -1;

namespace nvfp4 {
hipError_t launch_quantize(const uint16_t*, int64_t, int32_t, int32_t, int32_t, const int32_t*,
                           const int32_t*, int32_t, const float*, uint8_t*, uint8_t*,
                           int32_t num_dst_rows, hipStream_t, bool, bool mx) {
  g_calls.push_back("quantize");
  g_quant_mx = mx;
  g_quant_dst_rows = num_dst_rows;
  return hipSuccess;
}
hipError_t launch_quantize_gather(const uint16_t*, int64_t, int32_t, const int32_t*,
                                  int32_t src_div, int32_t, int32_t, const int32_t*, int32_t,
                                  const float*, uint8_t*, uint8_t*, hipStream_t, bool, bool mx) {
  g_calls.push_back("quantize_gather");
  g_quant_mx = mx;
  g_gather_src_div = src_div;
  return hipSuccess;
}
hipError_t launch_route(const float*, int32_t, int32_t, int32_t, int32_t*, float*, hipStream_t) {
  g_calls.push_back("route");
  return hipSuccess;
}
hipError_t launch_route_quantize(const float*, int32_t T, int32_t E, int32_t k, int32_t*,
                                 float*, const uint16_t*, int32_t H, const float* gscale,
                                 uint8_t* codes, uint8_t* sf, hipStream_t, bool mx) {
  // the shapes the real launcher covers; otherwise nothing is launched
  if (T < 1 || E > 1024 || k > 32 || H % (mx ? 128 : 64) || H / 16 < 64 || H / 16 > 1024)
    return hipErrorNotSupported;
  if (!gscale || !codes || !sf) abort();
  g_calls.push_back("route_quantize");
  g_rq_mx = mx;
  return hipSuccess;
}
hipError_t launch_permute(const int32_t*, int32_t, int32_t, int32_t*, int32_t*, int32_t*,
                          hipStream_t) {
  g_calls.push_back("permute");
  return hipSuccess;
}
hipError_t launch_absmax(const uint16_t*, int64_t, int32_t, const int32_t*, int32_t,
                         const int32_t*, int32_t, int32_t, float*, hipStream_t) {
  g_calls.push_back("absmax");
  return hipSuccess;
}
hipError_t launch_calibrate(const uint16_t*, int64_t, int32_t, const int32_t*, int32_t,
                            const int32_t*, int32_t, int32_t, float*, uint8_t*, hipStream_t) {
  g_calls.push_back("calibrate");
  return hipSuccess;
}
hipError_t launch_conversions_selftest(unsigned long long*, hipStream_t) {
  g_calls.push_back("selftest");
  return hipSuccess;
}
hipError_t launch_gemm1(const Gemm1Args& a, hipStream_t) {
  g_calls.push_back("gemm1");
  g_gemm1_mode = a.mx ? 2 : a.w16 ? 1 : 0;
  g_gemm1_P = a.P;
  g_gemm1_fold = a.perm_ids != nullptr;
  if (g_gemm1_fold && !(a.perm_offsets && a.perm_src && a.perm_inv && a.a_src)) abort();
  return hipSuccess;
}
hipError_t launch_pack_weights(int32_t, const uint8_t*, const uint8_t*, int32_t, int32_t, int32_t,
                               uint8_t*, uint8_t*, hipStream_t, bool) {
  g_calls.push_back("pack");
  return hipSuccess;
}
hipError_t launch_gemm2(const Gemm2Args& a, hipStream_t) {
  g_calls.push_back("gemm2");
  g_gemm2_mode = a.mx ? 2 : a.w16 ? 1 : 0;
  return hipSuccess;
}
hipError_t launch_combine(const float*, const float*, const int32_t*, int32_t, int32_t, int32_t,
                          const uint16_t*, uint16_t*, hipStream_t) {
  g_calls.push_back("combine");
  return hipSuccess;
}
}  // namespace nvfp4

extern "C" hipError_t hipEventRecord(hipEvent_t, hipStream_t) {
  g_calls.push_back("event");
  return hipSuccess;
}
extern "C" hipError_t hipMemcpyAsync(void*, const void*, size_t, hipMemcpyKind, hipStream_t) {
  g_calls.push_back("copy");
  return hipSuccess;
}

// ---- checks ---------------------------------------------------------------------
static int g_failures = 0;
#define CHECK(cond)                                                         \
  do {                                                                      \
    if (!(cond)) {                                                          \
      fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond);     \
      ++g_failures;                                                         \
    }                                                                       \
  } while (0)

static float f32(uint32_t bits) {
  float f;
  memcpy(&f, &bits, 4);
  return f;
}

static void validator_checks() {
  const float vals[] = {0.5f, f32(0x7FC00000u), f32(0x7F800000u), f32(0xFF800000u), 0.0f,
                        -0.0f, -1.0f, f32(0x00000001u), f32(0x00400000u), 3.0f};
  const int want[] = {NVFP4_SLOT_OK, NVFP4_SLOT_NAN, NVFP4_SLOT_INF, NVFP4_SLOT_INF,
                      NVFP4_SLOT_NONPOSITIVE, NVFP4_SLOT_NONPOSITIVE, NVFP4_SLOT_NONPOSITIVE,
                      NVFP4_SLOT_RECIP_OVERFLOW, NVFP4_SLOT_OK, NVFP4_SLOT_OK};
  const int E = 10;
  std::vector<float> gs(E, 123.0f);
  std::vector<int32_t> st(E, -1);
  int32_t bad = -1;
  CHECK(nvfp4_validate_scales(vals, nullptr, E, gs.data(), st.data(), &bad) ==
        NVFP4_ERR_BAD_SCALE);
  for (int e = 0; e < E; ++e) CHECK(st[e] == want[e]);
  CHECK(bad == 7);
  for (int e = 0; e < E; ++e) CHECK(gs[e] == 123.0f);  // nothing written on failure
  // valid-looking values that were never written
  const float good[] = {0.5f, 0.25f, 2.0f};
  const uint8_t written[] = {1, 0, 1};
  CHECK(nvfp4_validate_scales(good, written, 3, gs.data(), st.data(), &bad) ==
        NVFP4_ERR_BAD_SCALE);
  CHECK(st[1] == NVFP4_SLOT_UNWRITTEN && bad == 1 && gs[0] == 123.0f);
  // all good: reciprocals, every output optional
  CHECK(nvfp4_validate_scales(good, nullptr, 3, gs.data(), st.data(), &bad) == NVFP4_OK);
  CHECK(gs[0] == 2.0f && gs[1] == 4.0f && gs[2] == 0.5f && bad == 0);
  CHECK(nvfp4_validate_scales(good, nullptr, 3, nullptr, nullptr, nullptr) == NVFP4_OK);
  CHECK(nvfp4_validate_scales(nullptr, nullptr, 3, nullptr, nullptr, nullptr) ==
        NVFP4_ERR_INVALID_ARG);
  CHECK(nvfp4_validate_scales(good, nullptr, 0, nullptr, nullptr, nullptr) ==
        NVFP4_ERR_INVALID_ARG);
}

struct Buffers {  // host stand-ins for device buffers: aligned, never dereferenced by the stubs
  std::vector<uint8_t> mem;
  size_t used = 0;
  explicit Buffers(size_t bytes) : mem(bytes + 4096) {}
  void* get(size_t bytes) {
    uintptr_t base = reinterpret_cast<uintptr_t>(mem.data());
    uintptr_t p = (base + used + 255) & ~uintptr_t(255);
    used = p - base + bytes;
    if (used > mem.size()) abort();
    return reinterpret_cast<void*>(p);
  }
};

static void forward_checks() {
  const int32_t E = 8, H = 256, I = 128, T = 5, k = 3;
  Buffers b(64 << 20);
  nvfp4_moe_weights_t w;
  w.w13 = (const uint8_t*)b.get((size_t)E * 2 * I * H / 2);
  w.w13_sf = (const uint8_t*)b.get((size_t)E * 2 * I * H / 16);
  w.w13_scale2 = (const float*)b.get(E * 4);
  w.w2 = (const uint8_t*)b.get((size_t)E * H * I / 2);
  w.w2_sf = (const uint8_t*)b.get((size_t)E * H * I / 16);
  w.w2_scale2 = (const float*)b.get(E * 4);
  w.w13_input_scale = (const float*)b.get(E * 4);
  w.w2_input_scale = (const float*)b.get(E * 4);
  w.a1_gscale = (const float*)b.get(E * 4);
  w.a2_gscale = (const float*)b.get(E * 4);
  w.num_experts = E;
  w.hidden = H;
  w.inter = I;
  void* x = b.get((size_t)T * H * 2);
  float* logits = (float*)b.get((size_t)T * E * 4);
  void* out = b.get((size_t)T * H * 2);
  size_t ws_bytes = 0, ws16 = 0;
  CHECK(nvfp4_moe_workspace_size(T, k, &w, &ws_bytes) == NVFP4_OK && ws_bytes > 0);
  CHECK(nvfp4_moe_workspace_size_w4a16(T, k, &w, &ws16) == NVFP4_OK && ws16 > 0);
  void* ws = b.get(ws_bytes > ws16 ? ws_bytes : ws16);

  // the E4M3 forward: stages in order, the quantiser writing T*k rows; 15
  // pairs on 8 experts run the small-batch GEMMs, so GEMM1 regroups the
  // routed ids itself and the permute kernel is not launched
  g_calls.clear();
  CHECK(nvfp4_moe_forward(&w, x, logits, T, k, nullptr, out, ws, ws_bytes, nullptr, nullptr) ==
        NVFP4_OK);
  const std::vector<std::string> nv = {"route", "quantize", "gemm1", "gemm2", "combine"};
  CHECK(g_calls == nv);
  CHECK(g_quant_mx == 0 && g_quant_dst_rows == T * k && g_gemm1_P == T * k && g_gemm1_fold);
  CHECK(g_gemm1_mode == 0 && g_gemm2_mode == 0);
  // one byte short of the workspace, or misaligned
  g_calls.clear();
  CHECK(nvfp4_moe_forward(&w, x, logits, T, k, nullptr, out, ws, ws_bytes - 1, nullptr,
                          nullptr) == NVFP4_ERR_WORKSPACE);
  CHECK(nvfp4_moe_forward(&w, x, logits, T, k, nullptr, out, (char*)ws + 16, ws_bytes, nullptr,
                          nullptr) == NVFP4_ERR_WORKSPACE);
  CHECK(g_calls.empty());
  // stage events and debug copies
  nvfp4_moe_debug_t dbg;
  memset(&dbg, 0, sizeof(dbg));
  void* ev[NVFP4_MOE_STAGES + 1] = {};
  dbg.stage_events = ev;
  dbg.c2 = (float*)b.get((size_t)T * k * H * 4);
  g_calls.clear();
  CHECK(nvfp4_moe_forward(&w, x, logits, T, k, nullptr, out, ws, ws_bytes, &dbg, nullptr) ==
        NVFP4_OK);
  const std::vector<std::string> nvd = {"event", "route", "event", "event", "quantize",
                                        "event", "gemm1", "event", "gemm2", "event", "combine",
                                        "event", "copy"};
  CHECK(g_calls == nvd);

  // weight-only: no quantiser, no activation scale needed
  nvfp4_moe_weights_t w16 = w;
  w16.w13_input_scale = w16.w2_input_scale = w16.a1_gscale = w16.a2_gscale = nullptr;
  g_calls.clear();
  CHECK(nvfp4_moe_forward(&w16, x, logits, T, k, nullptr, out, ws, ws_bytes, nullptr, nullptr) ==
        NVFP4_ERR_INVALID_ARG);
  CHECK(nvfp4_moe_forward_w4a16(&w16, x, logits, T, k, nullptr, out, ws, ws16, nullptr,
                                nullptr) == NVFP4_OK);
  const std::vector<std::string> w16c = {"route", "gemm1", "gemm2", "combine"};
  CHECK(g_calls == w16c && g_gemm1_mode == 1 && g_gemm2_mode == 1 && g_gemm1_fold);

  // UE8M0 mode
  g_calls.clear();
  CHECK(nvfp4_moe_forward_mx(&w, x, logits, T, k, nullptr, out, ws, ws_bytes, nullptr, nullptr) ==
        NVFP4_OK);
  CHECK(g_calls == nv && g_quant_mx == 1 && g_gemm1_mode == 2 && g_gemm2_mode == 2);

  // hidden 1024 (H/16 = 64): routing and the A1 quantisation in one kernel,
  // timed as the route stage, in both W4A4 modes; the weight-only mode keeps
  // the separate router
  {
    nvfp4_moe_weights_t wf = w;
    const int32_t Hf = 1024;
    wf.hidden = Hf;
    wf.w13 = (const uint8_t*)b.get((size_t)E * 2 * I * Hf / 2);
    wf.w13_sf = (const uint8_t*)b.get((size_t)E * 2 * I * Hf / 16);
    wf.w2 = (const uint8_t*)b.get((size_t)E * Hf * I / 2);
    wf.w2_sf = (const uint8_t*)b.get((size_t)E * Hf * I / 16);
    size_t wsf = 0, wsf16 = 0;
    CHECK(nvfp4_moe_workspace_size(T, k, &wf, &wsf) == NVFP4_OK);
    CHECK(nvfp4_moe_workspace_size_w4a16(T, k, &wf, &wsf16) == NVFP4_OK);
    void* wsb = b.get(wsf > wsf16 ? wsf : wsf16);
    void* xf = b.get((size_t)T * Hf * 2);
    void* of = b.get((size_t)T * Hf * 2);
    g_calls.clear();
    CHECK(nvfp4_moe_forward(&wf, xf, logits, T, k, nullptr, of, wsb, wsf, nullptr, nullptr) ==
          NVFP4_OK);
    const std::vector<std::string> nvq = {"route_quantize", "gemm1", "gemm2", "combine"};
    CHECK(g_calls == nvq);
    g_calls.clear();
    CHECK(nvfp4_moe_forward(&wf, xf, logits, T, k, nullptr, of, wsb, wsf, &dbg, nullptr) ==
          NVFP4_OK);
    const std::vector<std::string> nvqd = {"event", "route_quantize", "event", "event",
                                           "event", "gemm1", "event", "gemm2",
                                           "event", "combine", "event", "copy"};
    CHECK(g_calls == nvqd && !g_rq_mx);
    // the UE8M0 mode fuses its routing and A1 quantisation the same way
    g_calls.clear();
    CHECK(nvfp4_moe_forward_mx(&wf, xf, logits, T, k, nullptr, of, wsb, wsf, nullptr,
                               nullptr) == NVFP4_OK);
    CHECK(g_calls == nvq && g_rq_mx && g_gemm1_mode == 2);
    nvfp4_moe_weights_t wf16 = wf;
    wf16.w13_input_scale = wf16.w2_input_scale = wf16.a1_gscale = wf16.a2_gscale = nullptr;
    g_calls.clear();
    CHECK(nvfp4_moe_forward_w4a16(&wf16, xf, logits, T, k, nullptr, of, wsb, wsf16, nullptr,
                                  nullptr) == NVFP4_OK);
    CHECK(g_calls == w16c);
  }

  // the permute kernel stays for batches the small-batch GEMM1 does not
  // regroup: the large-batch kernels (300 pairs on 8 experts) and more than
  // 512 pairs (640 on 64 experts)
  {
    const int32_t Tl = 100;
    void* xl = b.get((size_t)Tl * H * 2);
    void* ol = b.get((size_t)Tl * H * 2);
    float* ll = (float*)b.get((size_t)Tl * E * 4);
    size_t wsl = 0;
    CHECK(nvfp4_moe_workspace_size(Tl, k, &w, &wsl) == NVFP4_OK);
    void* wsb = b.get(wsl);
    g_calls.clear();
    CHECK(nvfp4_moe_forward(&w, xl, ll, Tl, k, nullptr, ol, wsb, wsl, nullptr, nullptr) ==
          NVFP4_OK);
    const std::vector<std::string> kept = {"route", "permute", "quantize", "gemm1", "gemm2",
                                           "combine"};
    CHECK(g_calls == kept && !g_gemm1_fold);

    nvfp4_moe_weights_t w64 = w;
    const int32_t E64 = 64, T64 = 40, k64 = 16;
    w64.num_experts = E64;
    w64.w13 = (const uint8_t*)b.get((size_t)E64 * 2 * I * H / 2);
    w64.w13_sf = (const uint8_t*)b.get((size_t)E64 * 2 * I * H / 16);
    w64.w2 = (const uint8_t*)b.get((size_t)E64 * H * I / 2);
    w64.w2_sf = (const uint8_t*)b.get((size_t)E64 * H * I / 16);
    w64.w13_scale2 = w64.w2_scale2 = w64.w13_input_scale = w64.w2_input_scale =
        w64.a1_gscale = w64.a2_gscale = (const float*)b.get(E64 * 4);
    void* x64 = b.get((size_t)T64 * H * 2);
    void* o64 = b.get((size_t)T64 * H * 2);
    float* l64 = (float*)b.get((size_t)T64 * E64 * 4);
    size_t ws64 = 0;
    CHECK(nvfp4_moe_workspace_size(T64, k64, &w64, &ws64) == NVFP4_OK);
    void* wsc = b.get(ws64);
    g_calls.clear();
    CHECK(nvfp4_moe_forward(&w64, x64, l64, T64, k64, nullptr, o64, wsc, ws64, nullptr,
                            nullptr) == NVFP4_OK);
    CHECK(g_calls == kept && !g_gemm1_fold && g_gemm1_P == T64 * k64);
  }

  // argument checks: nothing is launched
  g_calls.clear();
  CHECK(nvfp4_moe_forward(&w, x, logits, T, 0, nullptr, out, ws, ws_bytes, nullptr, nullptr) ==
        NVFP4_ERR_INVALID_ARG);
  CHECK(nvfp4_moe_forward(&w, x, logits, T, E + 1, nullptr, out, ws, ws_bytes, nullptr,
                          nullptr) == NVFP4_ERR_INVALID_ARG);
  CHECK(nvfp4_moe_forward(&w, (char*)x + 2, logits, T, k, nullptr, out, ws, ws_bytes, nullptr,
                          nullptr) == NVFP4_ERR_INVALID_ARG);
  CHECK(nvfp4_moe_forward(&w, x, logits, 0, k, nullptr, out, nullptr, 0, nullptr, nullptr) ==
        NVFP4_OK);
  nvfp4_moe_weights_t bad = w;
  bad.inter = 96;
  CHECK(nvfp4_moe_forward(&bad, x, logits, T, k, nullptr, out, ws, ws_bytes, nullptr, nullptr) ==
        NVFP4_ERR_UNSUPPORTED);
  bad = w;
  bad.hidden = 640;
  bad.inter = 320;
  CHECK(nvfp4_moe_forward_mx(&bad, x, logits, T, k, nullptr, out, ws, ws_bytes, nullptr,
                             nullptr) == NVFP4_ERR_UNSUPPORTED);
  // GEMM tile count past 32 bits (2^29 pairs, hidden 2^20): refused; the
  // largest pair count at this layer's widths passes that check and stops at
  // the workspace size
  bad = w;
  bad.hidden = 1 << 20;
  CHECK(nvfp4_moe_forward(&bad, x, logits, 1 << 26, k, nullptr, out, ws, ws_bytes, nullptr,
                          nullptr) == NVFP4_ERR_UNSUPPORTED);
  CHECK(nvfp4_moe_forward(&w, x, logits, (1 << 30) / k, k, nullptr, out, ws, ws_bytes, nullptr,
                          nullptr) == NVFP4_ERR_WORKSPACE);
  bad = w;
  bad.num_experts = 1025;
  CHECK(nvfp4_moe_forward(&bad, x, logits, T, k, nullptr, out, ws, ws_bytes, nullptr, nullptr) ==
        NVFP4_ERR_UNSUPPORTED);
  CHECK(g_calls.empty());
}

static void entry_point_checks() {
  Buffers b(1 << 20);
  void* x = b.get(4096);
  uint8_t* codes = (uint8_t*)b.get(4096);
  uint8_t* sf = (uint8_t*)b.get(4096);
  g_calls.clear();
  int32_t* offs = (int32_t*)b.get(64);
  int32_t* rows = (int32_t*)b.get(64);
  // scatter (pairs) form
  CHECK(nvfp4_quantize_pairs(x, 24, 1, 24, 1, nullptr, nullptr, 1, nullptr, codes, sf, 1,
                             nullptr) == NVFP4_ERR_INVALID_ARG);  // K % 16
  CHECK(nvfp4_quantize_pairs_mx(x, 48, 1, 48, 1, nullptr, nullptr, 1, nullptr, codes, sf, 1,
                                nullptr) == NVFP4_ERR_INVALID_ARG);  // K % 32
  CHECK(nvfp4_quantize_pairs((char*)x + 8, 16, 1, 16, 1, nullptr, nullptr, 1, nullptr, codes,
                             sf, 1, nullptr) == NVFP4_ERR_INVALID_ARG);  // x alignment
  // gather form
  CHECK(nvfp4_quantize_experts(x, 24, 24, rows, 4, 2, offs, 1, nullptr, codes, sf, nullptr) ==
        NVFP4_ERR_INVALID_ARG);  // K % 16
  CHECK(nvfp4_quantize_experts_mx(x, 48, 48, rows, 4, 2, offs, 1, nullptr, codes, sf,
                                  nullptr) == NVFP4_ERR_INVALID_ARG);  // K % 32
  CHECK(nvfp4_quantize_experts(x, 16, 16, rows, 4, 2, nullptr, 1, nullptr, codes, sf, nullptr) ==
        NVFP4_ERR_INVALID_ARG);  // offsets required
  CHECK(nvfp4_quantize_experts(x, 16, 16, nullptr, 1, 2, offs, 1, nullptr, codes, sf, nullptr) ==
        NVFP4_ERR_INVALID_ARG);  // identity rows need num_src_rows >= P
  CHECK(nvfp4_quantize_experts_fp16((char*)x + 8, 16, 16, rows, 4, 2, offs, 1, nullptr, codes,
                                    sf, nullptr) == NVFP4_ERR_INVALID_ARG);  // x alignment
  CHECK(nvfp4_quantize_experts(x, 16, 16, rows, 4, 2, offs, 0, nullptr, codes, sf, nullptr) ==
        NVFP4_ERR_INVALID_ARG);  // no experts
  CHECK(g_calls.empty());
  CHECK(nvfp4_quantize_experts(nullptr, 16, 16, nullptr, 0, 0, nullptr, 1, nullptr, nullptr,
                               nullptr, nullptr) == NVFP4_OK);  // P == 0 is a no-op
  CHECK(g_calls.empty());
  CHECK(nvfp4_quantize_pairs(x, 32, 2, 32, 1, nullptr, nullptr, 1, nullptr, codes, sf, 2,
                             nullptr) == NVFP4_OK);
  CHECK(g_calls.size() == 1 && g_calls[0] == "quantize" && g_quant_mx == 0);
  g_calls.clear();
  CHECK(nvfp4_quantize_experts_mx(x, 64, 64, rows, 4, 2, offs, 1, nullptr, codes, sf, nullptr) ==
        NVFP4_OK);
  CHECK(g_calls.size() == 1 && g_calls[0] == "quantize_gather" && g_quant_mx == 1 &&
        g_gather_src_div == 1);
  CHECK(nvfp4_route_topk((const float*)x, 4, 2000, 8, (int32_t*)codes, (float*)sf, nullptr) ==
        NVFP4_ERR_UNSUPPORTED);
  CHECK(nvfp4_route_topk((const float*)x, 4, 8, 9, (int32_t*)codes, (float*)sf, nullptr) ==
        NVFP4_ERR_INVALID_ARG);
  CHECK(nvfp4_moe_pack_weights(2, codes, sf, 1, 256, 128, codes + 1024, sf + 1024, nullptr) ==
        NVFP4_ERR_INVALID_ARG);
  CHECK(nvfp4_moe_pack_weights(0, codes, sf, 1, 256, 128, codes, sf + 1024, nullptr) ==
        NVFP4_ERR_INVALID_ARG);  // in place
  CHECK(nvfp4_moe_pack_weights_mx(0, codes, sf, 1, 384, 128, codes + 2048, sf + 2048, nullptr) ==
        NVFP4_ERR_UNSUPPORTED);  // hidden % 256 in the UE8M0 mode
  size_t n = 0;
  CHECK(nvfp4_moe_workspace_size(-1, 8, nullptr, &n) == NVFP4_ERR_INVALID_ARG);
  for (int s = 0; s <= 6; ++s) CHECK(strlen(nvfp4_status_string((nvfp4_status_t)s)) > 0);
  CHECK(strstr(nvfp4_status_string((nvfp4_status_t)99), "unknown") != nullptr);
  CHECK(nvfp4_abi_version() == NVFP4_ABI_VERSION);
}

int main() {
  validator_checks();
  forward_checks();
  entry_point_checks();
  if (g_failures) {
    fprintf(stderr, "%d check(s) failed\n", g_failures);
    return 1;
  }
  printf("abi host checks ok\n");
  return 0;
}
