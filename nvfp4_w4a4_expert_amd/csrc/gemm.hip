// Grouped NVFP4 x NVFP4 expert GEMMs for gfx950 (page 3, "矩阵融合": MoE FFN
// paragraph — per-expert products with different row counts M_e grouped into
// one launch; gated FFN paragraph — w13 holds gate and up, GEMM 1 produces
// both and act(gate) x up follows; "NVFP4" runtime figure — the GEMM's output
// scaling folds in the FP32 activation and weight global scales).
//
//   GEMM1: C1[p, n] = alpha1[e] * sum_k A1[p, k] * W13[e][n, k],  n < 2I
//          epilogue: h = bf16(silu(C1[:, gate]) * C1[:, up]), then h is
//          quantised per 16 columns with a2_gscale[e] into A2 codes + scales.
//   GEMM2: C2[p, n] = alpha2[e] * sum_k A2[p, k] * W2[e][n, k],  n < H (fp32)
//
// Operands are dequantised exactly: an E2M1 value times an E4M3 scale has at
// most 6 significant bits and lies in [2^-10, 2688], so it is an fp16 number.
// The contraction runs on v_mfma_f32_32x32x16_f16 with fp32 accumulation;
// alpha is applied once in the fp32 epilogue.
//
// Tiling: 256 threads (4 wavefronts, 2 x 2), a 128 x 128 output tile, K in
// steps of 64.  Each step, every thread loads 16 bytes of packed codes and
// 2 scale bytes of one A row and one B row, converts them to 32 fp16 values
// with the gfx950 FP4 -> fp16 conversion plus one packed fp16 multiply by
// the block scale, and stores them to LDS (double-buffered, rows padded by
// 16 bytes).  Each wavefront then issues 16 MFMAs on a 64 x 64 sub-tile.
// The K order inside a step is permuted identically for A and B so that each
// lane's MFMA operand is 16 contiguous LDS bytes; the sum is unchanged.
//
// Grouping: a tile is (expert e, m-tile of e's rows, n-tile).  The m-tiles of
// all experts are numbered consecutively; every workgroup recomputes the
// per-expert tile prefix from expert_offsets (E <= 1024) and finds its
// expert, so no host synchronisation is needed and experts with no rows cost
// nothing.  Rows past an expert's last row read a valid row and are not
// stored.  For GEMM1 an n-tile holds 64 gate columns and the matching 64 up
// columns, so SiLU*mul happens in registers.
#include "internal.h"
#include "nvfp4_device.h"

namespace nvfp4 {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBM = 128, kBN = 128, kBK = 64, kThreads = 256;
constexpr int kLd = kBK + 8;                         // fp16 per LDS row (16-byte pad)
constexpr int kStageHalves = (kBM + kBN) * kLd;      // A rows then B rows
constexpr int kLdsBytes = 2 * kStageHalves * 2;      // double buffered: 73728 B

// 32 consecutive E2M1 codes (16 bytes) with the E4M3 scales of their two
// 16-element blocks -> 32 exact fp16 values (16 half2, element order kept).
__device__ __forceinline__ void dequant32(const uint4 c, uint32_t sf2, half2_t* out) {
  const _Float16 s0 = (_Float16)e4m3_decode(sf2 & 0xFFu);
  const _Float16 s1 = (_Float16)e4m3_decode((sf2 >> 8) & 0xFFu);
  const half2_t h0 = {s0, s0}, h1 = {s1, s1};
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[4 * i + 0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 0) * (i < 2 ? h0 : h1);
    out[4 * i + 1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 1) * (i < 2 ? h0 : h1);
    out[4 * i + 2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 2) * (i < 2 ? h0 : h1);
    out[4 * i + 3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 3) * (i < 2 ? h0 : h1);
  }
}

// Block-wide search of the grouped m-tile `mt`: returns false when mt is past
// the last tile.  s_scan needs 6 ints of LDS.
__device__ __forceinline__ bool find_tile(const int32_t* __restrict__ offsets, int32_t E,
                                          int32_t mt, int32_t* s_scan, int32_t& e_out,
                                          int32_t& row0, int32_t& rows) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // thread tid owns experts [4 tid, 4 tid + 4)
  int32_t cnt[4], m[4], total = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int32_t e = 4 * tid + i;
    m[i] = e < E ? offsets[e + 1] - offsets[e] : 0;
    cnt[i] = (m[i] + kBM - 1) / kBM;
    total += cnt[i];
  }
  int32_t incl = total;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) s_scan[wave] = incl;
  if (tid == 0) s_scan[4] = -1;
  __syncthreads();
  int32_t base = incl - total;
  for (int w = 0; w < wave; ++w) base += s_scan[w];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (mt >= base && mt < base + cnt[i]) {
      s_scan[4] = 4 * tid + i;
      s_scan[5] = mt - base;
    }
    base += cnt[i];
  }
  __syncthreads();
  if (s_scan[4] < 0) return false;
  e_out = s_scan[4];
  const int32_t local = s_scan[5];
  row0 = offsets[e_out] + local * kBM;
  rows = min(kBM, offsets[e_out + 1] - row0);
  return true;
}

}  // namespace

template <bool kGated>
__global__ __launch_bounds__(kThreads, 2) void grouped_gemm_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_sf,
    const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_sf,
    const float* __restrict__ in_scale, const float* __restrict__ w_scale2,
    const int32_t* __restrict__ offsets, int32_t E, int32_t K, int32_t N_w, int32_t I,
    // GEMM2 output
    float* __restrict__ c_out, int32_t ldc,
    // GEMM1 epilogue
    const float* __restrict__ out_gscale, uint8_t* __restrict__ out_codes,
    uint8_t* __restrict__ out_sf, float* __restrict__ c1_dbg, uint16_t* __restrict__ h_dbg) {
  extern __shared__ __align__(16) _Float16 smem[];
  __shared__ int32_t s_scan[8];

  int32_t e, row0, rows;
  if (!find_tile(offsets, E, (int32_t)blockIdx.y, s_scan, e, row0, rows)) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int32_t nt = blockIdx.x;
  // n0: first output column of the tile (gate column for GEMM1)
  const int32_t n0 = kGated ? nt * 64 : nt * kBN;

  // this thread's load assignment: row r (0..127) of A and of B, K half hk
  const int r = tid >> 1, hk = tid & 1;
  const int64_t kb2 = K / 2, kb16 = K / 16;
  const int32_t a_row = row0 + min(r, rows - 1);
  const uint8_t* a_cp = a_codes + (int64_t)a_row * kb2 + 16 * hk;
  const uint8_t* a_sp = a_sf + (int64_t)a_row * kb16 + 2 * hk;
  int32_t w_row;
  if (kGated) w_row = r < 64 ? n0 + r : I + n0 + (r - 64);
  else w_row = n0 + r;
  const int64_t w_base = (int64_t)e * N_w + w_row;
  const uint8_t* b_cp = w_codes + w_base * kb2 + 16 * hk;
  const uint8_t* b_sp = w_sf + w_base * kb16 + 2 * hk;

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};

  const int nk = K / kBK;
  uint4 ac = *reinterpret_cast<const uint4*>(a_cp);
  uint32_t as = *reinterpret_cast<const uint16_t*>(a_sp);
  uint4 bc = *reinterpret_cast<const uint4*>(b_cp);
  uint32_t bs = *reinterpret_cast<const uint16_t*>(b_sp);

  auto stage_store = [&](int st) {
    half2_t v[16];
    _Float16* base = smem + st * kStageHalves;
    dequant32(ac, as, v);
    uint4* dst = reinterpret_cast<uint4*>(base + r * kLd + 32 * hk);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = *reinterpret_cast<const uint4*>(&v[4 * i]);
    dequant32(bc, bs, v);
    dst = reinterpret_cast<uint4*>(base + (kBM + r) * kLd + 32 * hk);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = *reinterpret_cast<const uint4*>(&v[4 * i]);
  };

  stage_store(0);
  __syncthreads();

  // A sub-tile rows of this wave, B sub-tile rows (in the LDS B block)
  const int a_r0 = wm * 64 + (lane & 31);
  const int b_r0 = kGated ? wn * 32 + (lane & 31) : wn * 64 + (lane & 31);
  const int b_r1 = kGated ? 64 + wn * 32 + (lane & 31) : wn * 64 + 32 + (lane & 31);
  const int kg = 32 * (lane >> 5);

  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) {
      const int64_t koff2 = (int64_t)(kt + 1) * (kBK / 2), koff16 = (kt + 1) * (kBK / 16);
      ac = *reinterpret_cast<const uint4*>(a_cp + koff2);
      as = *reinterpret_cast<const uint16_t*>(a_sp + koff16);
      bc = *reinterpret_cast<const uint4*>(b_cp + koff2);
      bs = *reinterpret_cast<const uint16_t*>(b_sp + koff16);
    }
    const _Float16* base = smem + st * kStageHalves;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int kk = kg + 8 * s;
      const half8_t a0 = *reinterpret_cast<const half8_t*>(base + a_r0 * kLd + kk);
      const half8_t a1 = *reinterpret_cast<const half8_t*>(base + (a_r0 + 32) * kLd + kk);
      const half8_t b0 = *reinterpret_cast<const half8_t*>(base + (kBM + b_r0) * kLd + kk);
      const half8_t b1 = *reinterpret_cast<const half8_t*>(base + (kBM + b_r1) * kLd + kk);
      acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b1, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b0, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b1, acc[1][1], 0, 0, 0);
    }
    if (kt + 1 < nk) stage_store(st ^ 1);
    __syncthreads();
  }

  const float alpha = in_scale[e] * w_scale2[e];
  // MFMA 32x32 output layout: lane holds column (lane & 31) and rows
  // 8 * (i / 4) + 4 * (lane / 32) + (i % 4) for accumulator element i.
  const int ccol = lane & 31, crow = 4 * (lane >> 5);

  if constexpr (!kGated) {
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = wm * 64 + mi * 32 + 8 * (i >> 2) + crow + (i & 3);
          const int col = n0 + wn * 64 + ni * 32 + ccol;
          if (row < rows) c_out[(int64_t)(row0 + row) * ldc + col] = alpha * acc[mi][ni][i];
        }
  } else {
    // SiLU(gate) * up -> bf16 tile [128][64] in LDS (reusing the stage buffers;
    // the loop's last barrier ordered every wave's final LDS reads before this)
    uint16_t* sh = reinterpret_cast<uint16_t*>(smem);
    constexpr int kLdh = 64 + 8;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = wm * 64 + mi * 32 + 8 * (i >> 2) + crow + (i & 3);
        const int col = wn * 32 + ccol;
        const float g = alpha * acc[mi][0][i];
        const float u = alpha * acc[mi][1][i];
        const float hv = g / (1.0f + __expf(-g)) * u;
        const uint32_t hb = f32_to_bf16(hv);
        sh[row * kLdh + col] = (uint16_t)hb;
        if (row < rows) {
          const int64_t p = row0 + row;
          if (c1_dbg) {
            c1_dbg[p * 2 * I + n0 + col] = g;
            c1_dbg[p * 2 * I + I + n0 + col] = u;
          }
          if (h_dbg) h_dbg[p * I + n0 + col] = (uint16_t)hb;
        }
      }
    __syncthreads();
    // requantise: 128 rows x 4 blocks of 16 columns; two blocks per thread
    const float gs = out_gscale[e];
    const int64_t ob2 = I / 2, ob16 = I / 16;
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int item = tid + kThreads * it;
      const int row = item >> 2, blk = item & 3;
      if (row < rows) {
        const uint4* src = reinterpret_cast<const uint4*>(sh + row * kLdh + 16 * blk);
        float xv[16];
        unpack_bf16x8(src[0], xv);
        unpack_bf16x8(src[1], xv + 8);
        const BlockScale bsc = block_scale(absmax16(xv) / kE2M1Max, gs);
        uint2 wv;
        wv.x = encode8(xv, bsc.inv);
        wv.y = encode8(xv + 8, bsc.inv);
        const int64_t p = row0 + row;
        *reinterpret_cast<uint2*>(out_codes + p * ob2 + (n0 + 16 * blk) / 2) = wv;
        out_sf[p * ob16 + n0 / 16 + blk] = (uint8_t)bsc.sf;
      }
    }
  }
}

static int32_t m_tiles_bound(int32_t P, int32_t E) {
  return (P + kBM - 1) / kBM + (P < E ? P : E);
}

hipError_t launch_gemm1(const Gemm1Args& a, hipStream_t stream) {
  if (a.P == 0) return hipSuccess;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t err = hipFuncSetAttribute((const void*)grouped_gemm_kernel<true>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (err != hipSuccess) return err;
    attr_set = true;
  }
  const dim3 grid(a.I / 64, m_tiles_bound(a.P, a.E));
  hipLaunchKernelGGL(grouped_gemm_kernel<true>, grid, dim3(kThreads), kLdsBytes, stream, a.a_codes,
                     a.a_sf, a.w_codes, a.w_sf, a.in_scale, a.w_scale2, a.offsets, a.E, a.H,
                     2 * a.I, a.I, (float*)nullptr, 0, a.out_gscale, a.out_codes, a.out_sf,
                     a.c1_dbg, a.h_dbg);
  return hipGetLastError();
}

hipError_t launch_gemm2(const Gemm2Args& a, hipStream_t stream) {
  if (a.P == 0) return hipSuccess;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t err = hipFuncSetAttribute((const void*)grouped_gemm_kernel<false>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (err != hipSuccess) return err;
    attr_set = true;
  }
  const dim3 grid(a.H / kBN, m_tiles_bound(a.P, a.E));
  hipLaunchKernelGGL(grouped_gemm_kernel<false>, grid, dim3(kThreads), kLdsBytes, stream,
                     a.a_codes, a.a_sf, a.w_codes, a.w_sf, a.in_scale, a.w_scale2, a.offsets, a.E,
                     a.I, a.H, a.I, a.out, a.H, (const float*)nullptr, (uint8_t*)nullptr,
                     (uint8_t*)nullptr, (float*)nullptr, (uint16_t*)nullptr);
  return hipGetLastError();
}

}  // namespace nvfp4
