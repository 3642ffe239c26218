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
// Work split.  A workgroup owns BM token rows of one expert (BM = 32 * kMB)
// and 64 * kWaves weight rows; wavefront w owns weight rows [64w, 64w + 64)
// of the tile and all BM token rows.  The last tile of an expert runs only
// its occupied 32-row sub-tiles (a separate instantiation of the tile body),
// so padding costs at most 31 rows per expert.
//  * The token operand A is shared by every wavefront: each K step it is
//    loaded once per workgroup, dequantised to fp16 and staged in LDS
//    (double buffered, rows padded by 16 bytes so the 16-byte fragment reads
//    of 16 consecutive lanes hit distinct banks).
//  * The weight operand B is private to its wavefront: each lane streams its
//    row's packed codes straight from global memory into a register ring
//    (kRing slots, loads kRing - 1 K steps ahead) and dequantises 8 values
//    per MFMA just before use (the
//    gfx950 FP4 -> fp16 pair conversion, then one packed fp16 multiply by the
//    block scale).  Weights never pass through LDS.
//  * K order inside a step is permuted identically for A and B so that each
//    lane's operand is contiguous: lane group g = lane / 32 covers k in
//    [g * BK/2, (g + 1) * BK/2) of a BK-wide step, 8 values per MFMA
//    (BK = 128 for w13, 64 for w2 whose K = I need not be a multiple of 128;
//    256 for the UE8M0 w13).
//
// Grouping and scheduling.  A tile is (expert, m-tile of the expert's rows,
// n-tile).  m-tiles of all experts are numbered consecutively; each
// workgroup recomputes the per-expert tile prefix from expert_offsets
// (E <= 1024) and finds its expert, so no host synchronisation is needed and
// experts without rows cost nothing.  The 1-D grid is remapped so that the
// workgroups the hardware sends to one XCD (round robin over 8) get a
// contiguous range of tiles: all n-tiles of an m-tile, and consecutive
// m-tiles of the same expert, share that XCD's L2.  Rows past an expert's
// last row read a valid row and are not stored.
//
// GEMM1 pairs columns: wavefront w's 64 weight rows are 32 gate rows and the
// 32 matching up rows, so SiLU*mul happens in registers and the tile's h
// columns are requantised from LDS in blocks of 16.  GEMM2 stages each
// 32 x 64 fp32 sub-tile in LDS and writes whole rows with 16-byte stores.
//
// Weight-only variant (kW16; page 3, "Kernel Backend": the Marlin backend
// runs the same NVFP4 weights as W4A16, bf16 activations, no activation
// scale).  A is bf16 rows — x gathered through src_pair for GEMM1, h for
// GEMM2 — staged into LDS unchanged; B is dequantised to bf16 exactly (FP4 ->
// fp32, times the E4M3 block scale in fp32, packed to bf16: the product has
// at most 6 significant bits); the contraction runs on
// v_mfma_f32_32x32x16_bf16; alpha is weight_scale_2 alone; GEMM1 writes h as
// bf16 rows instead of requantising it.
//
// UE8M0 variant (kModeMX; page 3, "NVFP4" section: the quantiser template's
// UE8M0_SF switch — power-of-two block scales, one per 32 elements).  Both
// operands stay packed E2M1: the gfx950 scaled matrix instruction
// v_mfma_scale_f32_32x32x64_f8f6f4 multiplies FP4 codes and applies one
// power-of-two scale per lane per 32-element block itself, so nothing is
// dequantised.  A's codes and scale bytes are staged in LDS as they are; the
// same K permutation gives each lane 32 consecutive elements (one block) per
// instruction; GEMM1 requantises h in the UE8M0 mode.
#include <type_traits>

#include "gemm_tiles.h"
#include "internal.h"
#include "nvfp4_device.h"

namespace nvfp4 {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

// Launch shapes, operand modes, tile mapping and global address arithmetic
// live in gemm_tiles.h, shared with the host-side range checker.
using namespace gemm_map;

template <int V>
using Int = std::integral_constant<int, V>;

// f(Int<0>{}), f(Int<1>{}), ..., f(Int<N-1>{}), in that order.
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(Int<N - 1>{});
  }
}

// 8 E2M1 codes (one 32-bit word) -> 8 exact fp16 values scaled by `s`.
__device__ __forceinline__ half8_t dequant8(uint32_t w, half2_t s) {
  const half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s;
  const half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s;
  const half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s;
  const half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s;
  return half8_t{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// Two E4M3 block scales (the low 16 bits of `w`, or the high 16 bits when
// kHi) -> their exact fp16 values, with the gfx950 FP8 -> fp16 conversion.
template <bool kHi>
__device__ __forceinline__ half2_t scales_f16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, kHi);
}

// 8 E2M1 codes -> 8 exact bf16 values scaled by the fp32 block scale `s`.
// (The conversion's own scale operand applies only a power of two, so the
// E4M3 scale is multiplied in fp32; every product is exact.)
__device__ __forceinline__ bf16x8_t dequant8_bf16(uint32_t w, float s) {
  const f32x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0) * s;
  const f32x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1) * s;
  const f32x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2) * s;
  const f32x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3) * s;
  return bf16x8_t{(__bf16)p0.x, (__bf16)p0.y, (__bf16)p1.x, (__bf16)p1.y,
                  (__bf16)p2.x, (__bf16)p2.y, (__bf16)p3.x, (__bf16)p3.y};
}

__device__ __forceinline__ half2_t bcast_lo(half2_t v) { return half2_t{v.x, v.x}; }
__device__ __forceinline__ half2_t bcast_hi(half2_t v) { return half2_t{v.y, v.y}; }

// Workgroup barrier that orders LDS accesses only.  Every barrier in these
// kernels hands LDS data between threads; none publishes global memory, so
// outstanding global loads (the register rings' prefetches) need not drain,
// which a full __syncthreads() fence would make the compiler wait for.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// A wave-uniform value the compiler cannot see through (it is kept in an
// SGPR and treated as produced at this point).
__device__ __forceinline__ int32_t opaque_sgpr(int32_t v) {
  asm volatile("" : "+s"(v));
  return v;
}

// Block-scale arrays are [.., K/16] E4M3 bytes, or [.., K/32] UE8M0 bytes in
// the UE8M0 mode.
struct GemmParams {
  const uint8_t* a_codes;   // [P, K/2]
  const uint8_t* a_sf;      // [P, K/16]
  // A row of grouped row p: row a_src[p] / a_src_div of the operand (p when
  // a_src is null) -- bf16 rows a_rows[.. * lda] (weight-only) or quantised
  // rows of a_codes / a_sf
  const uint16_t* a_rows;   // bf16
  const int32_t* a_src;
  int64_t lda;
  int32_t a_src_div;
  uint16_t* h_out;          // GEMM1: bf16 [P, I]
  const uint8_t* w_codes;   // [E, N_w, K/2]
  const uint8_t* w_sf;      // [E, N_w, K/16]
  const float* in_scale;    // [E]
  const float* w_scale2;    // [E]
  const int32_t* offsets;   // [E+1]
  int32_t E, K, N_w, I;     // N_w: weight rows per expert; I: GEMM1 h width
  int32_t n_tiles;
  // GEMM2 output
  float* c_out;             // [P, ldc]
  int32_t ldc;
  // GEMM1 epilogue
  const float* out_gscale;  // [E]
  uint8_t* out_codes;       // [P, I/2]
  uint8_t* out_sf;          // [P, I/16]
  float* c1_dbg;            // [P, 2I] or null
  uint16_t* h_dbg;          // [P, I] or null
  // small-batch GEMM1 only (gemm_map::fold_permutation): the routed expert
  // ids of the P pairs; when set, the kernel derives the grouping from them
  // instead of reading offsets / a_src, and writes the permutation out
  const int32_t* perm_ids;  // [P] or null
  int32_t perm_P;
  int32_t* perm_offsets;    // [E+1], written by workgroup 0
  int32_t* perm_src;        // [P] src_pair
  int32_t* perm_inv;        // [P] inv
};

}  // namespace

template <int kWaves, int kMB, int kBK, bool kGated, int kRing, int kOcc, int kMode>
__global__ __launch_bounds__(64 * kWaves, kOcc) void grouped_gemm_kernel(
    const GemmParams prm) {
  constexpr bool kW16 = kMode == kModeW16;
  constexpr bool kMX = kMode == kModeMX;
  constexpr int kThreads = 64 * kWaves;
  constexpr int kBM = 32 * kMB;
  constexpr int kLdA = kBK + 8;                          // fp16 per LDS row (16-byte pad)
  // UE8M0 mode LDS buffer: packed codes, rows padded by 16 bytes (the 16-byte
  // reads of 16 consecutive rows then start on distinct 4-bank groups), then
  // the rows' kBK/32 scale bytes
  constexpr int kLdAb = kBK / 2 + 16;
  constexpr int kScOff = kBM * kLdAb;
  constexpr int kMxBuf = kScOff + kBM * (kBK / 32);
  static_assert(!kMX || 2 * kMxBuf <= 2 * kBM * kLdA * 2, "UE8M0 stage fits the LDS buffer");
  constexpr int kVec = kBK / 64;                         // 16-byte B loads per block per step
  constexpr int kSteps = kBK / 16;                       // MFMA rounds per step
  __shared__ __align__(16) _Float16 smem[2 * kBM * kLdA];
  __shared__ int32_t s_off[kMaxExperts + 1];             // expert row offsets
  __shared__ int32_t s_mt[kMaxExperts + 1];              // m-tiles before each expert
  __shared__ int32_t s_scan[kWaves];
  // Small-batch GEMM1 regrouping the routed ids itself (prm.perm_ids set):
  // the ids, a second scan's wave totals, and the pair of each row of the
  // current tile.
  constexpr bool kFold = kGated && kMB == 1;
  __shared__ int32_t s_fids[kFold ? kFoldMaxPairs : 1];
  __shared__ int32_t s_fscan[kFold ? kWaves : 1];
  __shared__ int32_t s_fsrc[kFold ? 32 : 1];
  const bool fold = kFold && prm.perm_ids != nullptr;

  // ---- once per workgroup: per-expert m-tile prefix in LDS -----------------
  {
    // entries 0 .. E of the prefix (E + 1 <= kMaxExperts + 1 of them)
    constexpr int kPer = (kMaxExperts + 1 + kThreads - 1) / kThreads;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if constexpr (kFold) {
      if (fold) {
        // histogram of the routed ids (pairs with an id outside [0, E) are
        // left out, as the permutation kernel does); s_mt holds the counts
        // until every thread has read its entries below
        for (int e = tid; e < prm.E; e += kThreads) s_mt[e] = 0;
        lds_barrier();
        for (int32_t q = tid; q < prm.perm_P; q += kThreads) {
          const int32_t id = prm.perm_ids[q];
          s_fids[q] = id;
          if ((uint32_t)id < (uint32_t)prm.E) atomicAdd(&s_mt[id], 1);
        }
        lds_barrier();
      }
    }
    int32_t m[kPer], cnt[kPer], rcnt[kPer], total, rtotal;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int32_t e = kPer * tid + i;
      m[i] = 0;
      if (e < prm.E) {
        if (fold) {
          m[i] = s_mt[e];
        } else {
          const int32_t o0 = prm.offsets[e], o1 = prm.offsets[e + 1];
          s_off[e] = o0;
          if (e == prm.E - 1) s_off[prm.E] = o1;
          m[i] = o1 - o0;
        }
      }
    }
    // (the same per-thread counting as the host range checker repeats)
    thread_prefix_counts<kPer>(m, kBM, cnt, rcnt, total, rtotal);
    int32_t incl = total, rincl = rtotal;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int32_t o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
      if constexpr (kFold) {
        const int32_t ro = __shfl_up(rincl, off, 64);
        if (lane >= off) rincl += ro;
      }
    }
    if (lane == 63) {
      s_scan[wave] = incl;
      if constexpr (kFold) s_fscan[wave] = rincl;
    }
    lds_barrier();
    int32_t base = incl - total, rbase = rincl - rtotal;
    for (int w = 0; w < wave; ++w) {
      base += s_scan[w];
      if constexpr (kFold) rbase += s_fscan[w];
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int32_t e = kPer * tid + i;
      if (e <= prm.E) {
        s_mt[e] = base;
        if (fold) s_off[e] = rbase;     // expert offsets: exclusive prefix of the counts
      }
      base += cnt[i];
      rbase += rcnt[i];
    }
    lds_barrier();
    if (fold && blockIdx.x == 0)
      for (int e = tid; e <= prm.E; e += kThreads) prm.perm_offsets[e] = s_off[e];
  }
  const int32_t total_m = s_mt[prm.E];
  const int32_t total = total_m * prm.n_tiles;
  const int32_t xcd_tiles = per_xcd(total);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5;
  const int32_t K = prm.K;
  const int nk = K / kBK;

  // ---- persistent loop over tiles; the workgroups on one XCD walk a
  // contiguous range of (m-tile, n-tile) so they share that XCD's L2 --------
  for (int32_t t = blockIdx.x; t < xcd_tiles * kXcds; t += gridDim.x) {
  const int32_t logical = logical_tile(t, xcd_tiles);
  if (logical >= total) continue;
  const Tile tl = tile_of(logical, prm.n_tiles, s_mt, s_off, prm.E, kBM);
  const int32_t nt = tl.nt, e = tl.e, row0 = tl.row0, rows = tl.rows;
  if (rows <= 0) continue;                             // (uniform; never for consistent offsets)

  // Regrouping from the routed ids: the tile's rows are ranks
  // [row0 - offsets[e], + rows) among expert e's pairs in pair order (the
  // stable order of the permutation).  Wavefront 0 walks the ids 64 at a
  // time; a pair of expert e gets rank = matches before it, counted with a
  // ballot.  The tile with n-tile 0 writes its rows of src_pair and inv.
  if constexpr (kFold) {
    if (fold) {
      if (wave == 0) {
        const int32_t lo = row0 - s_off[e];
        const uint64_t below = (1ull << lane) - 1ull;
        int32_t seen = 0;
        for (int32_t c0 = 0; c0 < prm.perm_P; c0 += 64) {
          const int32_t q = c0 + lane;
          const bool match = q < prm.perm_P && s_fids[q] == e;
          const uint64_t mask = __ballot(match);
          if (match) {
            const int32_t r = seen + __popcll(mask & below) - lo;
            if (r >= 0 && r < rows) s_fsrc[r] = q;
          }
          seen += __popcll(mask);
        }
      }
      lds_barrier();
      if (nt == 0 && tid < rows) {
        const int32_t q = s_fsrc[tid];
        prm.perm_src[row0 + tid] = q;
        prm.perm_inv[q] = row0 + tid;
      }
    }
  }
  // pair index of tile row arow (row0 <= arow < row0 + rows)
  auto src_of = [&](int64_t arow) -> int32_t {
    if constexpr (kFold)
      if (fold) return s_fsrc[arow - row0];
    return prm.a_src[arow];
  };

  // ---- B streaming assignment: wave's 64 weight rows, 2 blocks of 32 ------
  // GEMM1: block 0 = gate rows, block 1 = the matching up rows.  Weights are
  // in the kernel layout (nvfp4_moe_pack_weights): inside each 32-row block,
  // K step kt holds, lane by lane, the 16-byte pieces each lane consumes, so a
  // wavefront's load is one contiguous 1 KB per piece (plus 64 contiguous
  // scale groups of kBK/32 bytes).
  const WaveBlocks wb = wave_blocks(kGated, kWaves, nt, wave, prm.I, prm.N_w);
  const int32_t n0 = wb.n0;                            // GEMM2: output column base
  const bool active = wb.active;                       // inactive waves read block 0
  const uint8_t* b_cp[2];
  const uint8_t* b_sp[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    b_cp[j] = prm.w_codes + b_codes_offset(e, prm.N_w, wb.row0[j], K, lane);
    // scale bytes per lane per K step: kBK/32 E4M3 scales (16-element
    // blocks) or kBK/64 UE8M0 scales (32-element blocks)
    b_sp[j] = prm.w_sf + b_scales_offset(e, prm.N_w, wb.row0[j], K, lane, kBK, kMX);
  }

  // The tile body, for kMBa = the number of 32-row sub-tiles that hold rows
  // (the last tile of an expert may be partly empty: its empty sub-tiles
  // are neither staged nor multiplied).
  auto tile = [&](auto mbc) {
  constexpr int kMBa = decltype(mbc)::value;
  // A is staged in chunks of 32 elements (16 code bytes + 2 scales), or of
  // 16 elements when that is what it takes to give every thread a chunk;
  // bf16 rows (kW16) in chunks of 8 elements (16 bytes); UE8M0 codes (kMX) in
  // chunks of one 32-element block (16 code bytes + 1 scale byte).
  constexpr int kCE = a_chunk_elems(kMode, kMBa, kBK, kThreads);
  constexpr int kCPR = kBK / kCE;                        // chunks per row per step
  constexpr int kChunks = 32 * kMBa * kCPR;
  constexpr int kChunksPerThread = (kChunks + kThreads - 1) / kThreads;
  using araw_t = std::conditional_t<kW16 || kMX || kCE == 32, u32x4, u32x2>;
  using op_t = std::conditional_t<kW16, bf16x8_t, half8_t>;

  // ---- A staging assignment: chunk c -> (row, kCE-wide k chunk) -------------
  const uint8_t* a_cp[kChunksPerThread];
  const uint8_t* a_sp[kChunksPerThread];
  int a_lds[kChunksPerThread];
  int a_lds_s[kChunksPerThread];                          // UE8M0 mode: scale byte offset
  bool a_on[kChunksPerThread];
#pragma unroll
  for (int i = 0; i < kChunksPerThread; ++i) {
    const int c = tid + i * kThreads;
    a_on[i] = kChunks % kThreads == 0 || c < kChunks;   // compile-time true when exact
    const int cc = a_on[i] ? c : 0;
    const int r = cc / kCPR, kc = cc % kCPR;
    const int64_t arow = a_row(row0, r, rows);
    if constexpr (kW16) {
      const int64_t srow = prm.a_src ? src_of(arow) / prm.a_src_div : arow;
      a_cp[i] = reinterpret_cast<const uint8_t*>(prm.a_rows + a_rows_offset(srow, prm.lda, kc, kCE));
      a_sp[i] = nullptr;
    } else {
      // GEMM1 reads A1 through the permutation (its rows are stored in
      // (token, slot) order); GEMM2's A2 rows are in grouped order
      const int64_t qrow = prm.a_src ? src_of(arow) / prm.a_src_div : arow;
      a_cp[i] = prm.a_codes + a_codes_offset(qrow, K, kc, kCE, kMX);
      a_sp[i] = prm.a_sf + a_scales_offset(qrow, K, kc, kCE, kMX);
    }
    a_lds[i] = kMX ? r * kLdAb + 16 * kc : r * kLdA + kCE * kc;
    a_lds_s[i] = kScOff + r * (kBK / 32) + kc;
  }

  // The tile's output scale.  The E4M3 w13 kernel loads it before the K loop,
  // so that its wait is absorbed there instead of draining every outstanding
  // load before the epilogue (w13 -1.3 us at the prefill layer); the other
  // kernels load it after the loop, where the extra live register would spill.
  constexpr bool kEarlyAlpha = kGated && kMode == kModeNV;
  float alpha_early = 0.0f;
  if constexpr (kEarlyAlpha) alpha_early = prm.in_scale[e] * prm.w_scale2[e];
  f32x16_t acc[kMBa][2];
#pragma unroll
  for (int i = 0; i < kMBa; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};

  // Register rings (kRing slots) for the packed codes of A and B: step kt's
  // loads are issued kRing - 1 steps before their use.
  araw_t a_raw[kRing][kChunksPerThread];
  uint32_t a_sraw[kRing][kChunksPerThread];
  u32x4 b_raw[kRing][2][kVec];    // [slot][block][16-byte piece]
  uint32_t b_sraw[kRing][2];      // [slot][block]: kBK/32 scale bytes (kBK/64 in UE8M0 mode)

  auto load_a = [&](int kt, auto slotc) {
    constexpr int slot = decltype(slotc)::value;
#pragma unroll
    for (int i = 0; i < kChunksPerThread; ++i) {
      if (!a_on[i]) continue;
      if constexpr (kW16) {
        a_raw[slot][i] = *reinterpret_cast<const araw_t*>(a_cp[i] + 2 * a_rows_step(kt, kBK));
        continue;
      }
      a_raw[slot][i] = *reinterpret_cast<const araw_t*>(a_cp[i] + a_codes_step(kt, kBK));
      if constexpr (kMX)
        a_sraw[slot][i] = a_sp[i][a_scales_step(kt, kBK, true)];
      else if constexpr (kCE == 32)
        a_sraw[slot][i] = *reinterpret_cast<const uint16_t*>(a_sp[i] + a_scales_step(kt, kBK, false));
      else
        a_sraw[slot][i] = a_sp[i][a_scales_step(kt, kBK, false)];
    }
  };
  // dequantise the A step held in register slot `slot` into LDS buffer `buf`
  auto store_a = [&](int buf, auto slotc) {
    constexpr int slot = decltype(slotc)::value;
    _Float16* base = smem + buf * (kBM * kLdA);
#pragma unroll
    for (int i = 0; i < kChunksPerThread; ++i) {
      if (!a_on[i]) continue;
      if constexpr (kW16) {
        *reinterpret_cast<u32x4*>(base + a_lds[i]) = a_raw[slot][i];
        continue;
      }
      if constexpr (kMX) {
        uint8_t* bb = reinterpret_cast<uint8_t*>(smem) + buf * kMxBuf;
        *reinterpret_cast<u32x4*>(bb + a_lds[i]) = a_raw[slot][i];
        bb[a_lds_s[i]] = (uint8_t)a_sraw[slot][i];
        continue;
      }
      const half2_t sp = scales_f16<false>(a_sraw[slot][i]);
      const half2_t s0 = bcast_lo(sp);
      half8_t* dst = reinterpret_cast<half8_t*>(base + a_lds[i]);
      dst[0] = dequant8(a_raw[slot][i].x, s0);
      dst[1] = dequant8(a_raw[slot][i].y, s0);
      if constexpr (kCE == 32) {
        const half2_t s1 = bcast_hi(sp);
        dst[2] = dequant8(a_raw[slot][i].z, s1);
        dst[3] = dequant8(a_raw[slot][i].w, s1);
      }
    }
  };
  auto load_b = [&](int kt, auto slotc) {
    constexpr int buf = decltype(slotc)::value;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint8_t* cbase = b_cp[j] + b_codes_step(kt, kBK);
#pragma unroll
      for (int v = 0; v < kVec; ++v)
        b_raw[buf][j][v] = *reinterpret_cast<const u32x4*>(cbase + 1024 * v);
      if constexpr (kMX) {
        const uint8_t* sp = b_sp[j] + b_scales_step(kt, kBK, true);
        if constexpr (kBK == 256) b_sraw[buf][j] = *reinterpret_cast<const uint32_t*>(sp);
        else if constexpr (kBK == 128) b_sraw[buf][j] = *reinterpret_cast<const uint16_t*>(sp);
        else b_sraw[buf][j] = *sp;
      } else {
        const uint8_t* sp = b_sp[j] + b_scales_step(kt, kBK, false);
        if constexpr (kBK == 128) b_sraw[buf][j] = *reinterpret_cast<const uint32_t*>(sp);
        else b_sraw[buf][j] = *reinterpret_cast<const uint16_t*>(sp);
      }
    }
  };
  // One K step: kSteps MFMA rounds of (kMBa x 2) 32x32x16 products on LDS
  // buffer `lbuf` and B ring slot `buf`.  The operands of round s+1 (B
  // dequantised from registers, A read from LDS) are produced while round
  // s's MFMAs run.
  // UE8M0 mode: kBK/64 rounds of (kMBa x 2) scaled 32x32x64 FP4 products.
  // Lane (row r = lane & 31, group g) supplies, for round st, the 32 codes
  // of its K block g * kBK/64 + st and that block's scale byte (operand
  // select st picks it from the lane's scale register).
  auto compute_mx = [&](int lbuf, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    const uint8_t* lb = reinterpret_cast<const uint8_t*>(smem) + lbuf * kMxBuf;
    const uint8_t* acod = lb + (lane & 31) * kLdAb + 16 * (kBK / 64) * g;
    const uint8_t* asc = lb + kScOff + (lane & 31) * (kBK / 32) + (kBK / 64) * g;
    int sa[kMBa];
#pragma unroll
    for (int i = 0; i < kMBa; ++i) {
      const uint8_t* q = asc + i * 32 * (kBK / 32);
      sa[i] = kBK == 256 ? (int)*reinterpret_cast<const uint32_t*>(q)
            : kBK == 128 ? (int)*reinterpret_cast<const uint16_t*>(q) : (int)*q;
    }
    auto round = [&](auto stc) {
      constexpr int st = decltype(stc)::value;
      i32x8_t bo[2], ao[kMBa];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x4 v = b_raw[buf][j][st];
        bo[j] = i32x8_t{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
      }
#pragma unroll
      for (int i = 0; i < kMBa; ++i) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(acod + i * 32 * kLdAb + 16 * st);
        ao[i] = i32x8_t{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
      }
#pragma unroll
      for (int i = 0; i < kMBa; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              ao[i], bo[j], acc[i][j], 4, 4, st, sa[i], st, (int)b_sraw[buf][j]);
    };
    static_assert(kBK == 64 || kBK == 128 || kBK == 256, "1, 2 or 4 scaled rounds per K step");
    round(Int<0>{});
    if constexpr (kBK >= 128) round(Int<1>{});
    if constexpr (kBK == 256) {
      round(Int<2>{});
      round(Int<3>{});
    }
  };
  auto compute = [&](int lbuf, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    if constexpr (kMX) {
      compute_mx(lbuf, bufc);
      return;
    }
    // the compiler's MFMA / LDS-read interleaving strategy for GEMM loops
    // (measured: about 1.5% off both GEMMs at the prefill layer)
    __builtin_amdgcn_iglp_opt(1);
    const _Float16* abase = smem + lbuf * (kBM * kLdA) + (lane & 31) * kLdA + (kBK / 2) * g;
    // block scales of this step: kBK/32 per block, as fp16 pairs
    // (8-value piece st of the lane's K range lies in block scale st / 2)
    half2_t sc[2][2];
    float scf[2][kBK / 32];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if constexpr (kW16) {
        const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)b_sraw[buf][j], false);
        scf[j][0] = lo.x;
        scf[j][1] = lo.y;
        if constexpr (kBK == 128) {
          const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)b_sraw[buf][j], true);
          scf[j][2] = hi.x;
          scf[j][3] = hi.y;
        }
      } else {
        sc[j][0] = scales_f16<false>(b_sraw[buf][j]);
        sc[j][1] = kBK == 128 ? scales_f16<true>(b_sraw[buf][j]) : sc[j][0];
      }
    }
    auto bdeq = [&](int st, int j) -> op_t {
      const u32x4& v = b_raw[buf][j][st >> 2];
      const uint32_t word = (st & 3) == 0 ? v.x : (st & 3) == 1 ? v.y : (st & 3) == 2 ? v.z : v.w;
      if constexpr (kW16) {
        return dequant8_bf16(word, scf[j][st >> 1]);
      } else {
        const half2_t pair = sc[j][(st >> 2) & 1];
        return dequant8(word, ((st >> 1) & 1) ? bcast_hi(pair) : bcast_lo(pair));
      }
    };
    auto aread = [&](int st, int i) -> op_t {
      return *reinterpret_cast<const op_t*>(abase + i * 32 * kLdA + 8 * st);
    };
    auto mfma = [](op_t a, op_t b, f32x16_t c) -> f32x16_t {
      if constexpr (kW16) return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
      else return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    };
    op_t bf[2], af[kMBa];
#pragma unroll
    for (int j = 0; j < 2; ++j) bf[j] = bdeq(0, j);
#pragma unroll
    for (int i = 0; i < kMBa; ++i) af[i] = aread(0, i);
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      op_t nbf[2], naf[kMBa];
      if (st + 1 < kSteps) {
#pragma unroll
        for (int j = 0; j < 2; ++j) nbf[j] = bdeq(st + 1, j);
#pragma unroll
        for (int i = 0; i < kMBa; ++i) naf[i] = aread(st + 1, i);
      }
#pragma unroll
      for (int i = 0; i < kMBa; ++i) {
        acc[i][0] = mfma(af[i], bf[0], acc[i][0]);
        acc[i][1] = mfma(af[i], bf[1], acc[i][1]);
      }
      if (st + 1 < kSteps) {
#pragma unroll
        for (int j = 0; j < 2; ++j) bf[j] = nbf[j];
#pragma unroll
        for (int i = 0; i < kMBa; ++i) af[i] = naf[i];
      }
    }
  };

  // ---- pipeline.  Ring slot of step x is x % kRing; LDS buffer is x & 1.
  // Step kt: issue A(kt+kRing) into the slot A(kt) left; in one basic block
  // dequantise A(kt+1) into LDS buffer (kt+1)&1 and run the MFMAs of step kt
  // (LDS buffer kt&1, B slot kt%kRing) so the scheduler interleaves them;
  // issue B(kt+kRing) into the slot just consumed; one barrier.  Whole groups
  // of kRing steps loop with no early exit (so accumulators stay in place);
  // the remaining steps follow.
  // prologue in the steady state's issue order (A then B of each step)
  static_assert(kRing >= 2, "at least two ring slots");
  static_for<kRing>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    load_a(min(i, nk - 1), Int<i>{});
    load_b(min(i, nk - 1), Int<i>{});
  });
  store_a(0, Int<0>{});
  lds_barrier();
  auto step = [&](int kt, auto rc) {
    constexpr int r = decltype(rc)::value;
    constexpr int rn = (r + 1) % kRing;
    // Loads are issued unconditionally (steps past the end re-read the last
    // step, which is harmless): a load under a branch makes the compiler's
    // wait counting fall back to waiting for every outstanding load, which
    // would defeat the ring.
    load_a(min(kt + kRing, nk - 1), Int<r>{});
    if (active) {
      // the large-batch w2 issues its MFMAs before staging the next token
      // step (the staging's load wait then overlaps them: 182 -> 178 us at the
      // prefill layer); w13 and the small-batch kernels measured better the
      // other way round
      if constexpr (kGated || kMB == 1) {
        store_a((kt + 1) & 1, Int<rn>{});
        compute(kt & 1, Int<r>{});
      } else {
        compute(kt & 1, Int<r>{});
        store_a((kt + 1) & 1, Int<rn>{});
      }
    } else {
      store_a((kt + 1) & 1, Int<rn>{});
    }
    load_b(min(kt + kRing, nk - 1), Int<r>{});
    lds_barrier();
  };
  const int nkr = nk - nk % kRing;
  for (int kt = 0; kt < nkr; kt += kRing)
    static_for<kRing>([&](auto ic) { step(kt + decltype(ic)::value, ic); });
  static_for<kRing - 1>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    if (nkr + i < nk) step(nkr + i, ic);
  });

  const float alpha = kEarlyAlpha ? alpha_early
                     : kW16 ? prm.w_scale2[e] : prm.in_scale[e] * prm.w_scale2[e];
  // MFMA 32x32 output layout: lane holds column (lane & 31) and rows
  // 8 * (i / 4) + 4 * (lane / 32) + (i % 4) for accumulator element i.
  const int ccol = lane & 31, crow = 4 * g;

  if constexpr (!kGated) {
    // Each wavefront stages one 32 x 64 fp32 sub-tile at a time in its own
    // LDS slice (rows padded to 72 floats: the two lane halves, 4 rows
    // apart, land on disjoint banks), then writes whole 256-byte row
    // segments with 16-byte stores.
    constexpr int kLdc = 72;
    constexpr bool kStaged = 2 * kBM * kLdA * 2 >= kWaves * 32 * kLdc * 4;
    if constexpr (kStaged) {
      float* sc = reinterpret_cast<float*>(smem) + wave * (32 * kLdc);
      const int rr = lane >> 4, c4 = 4 * (lane & 15);
      // row0 and ldc pass through an empty asm here so that the output
      // addresses are formed after the K loop instead of being hoisted above
      // it (where they would stay live across the loop).
      const int32_t ldc = opaque_sgpr(prm.ldc);
      const int32_t r0 = opaque_sgpr(row0);
      float* gout = prm.c_out + c_offset(r0, 0, ldc, n0, c4);
      if (active)
#pragma unroll
      for (int mi = 0; mi < kMBa; ++mi) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            sc[(8 * (i >> 2) + crow + (i & 3)) * kLdc + 32 * j + ccol] = alpha * acc[mi][j][i];
        // not unrolled: each row address is formed just before its store
#pragma unroll 1
        for (int q = 0; q < 8; ++q) {
          const int r = 4 * q + rr;
          const f32x4 v = *reinterpret_cast<const f32x4*>(sc + r * kLdc + c4);
          if (mi * 32 + r < rows)
            *reinterpret_cast<f32x4*>(gout + (mi * 32 + r) * ldc) = v;
        }
      }
    } else {
      if (active)
#pragma unroll
      for (int mi = 0; mi < kMBa; ++mi)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int row = mi * 32 + 8 * (i >> 2) + crow + (i & 3);
            if (row < rows)
              prm.c_out[(int64_t)(row0 + row) * prm.ldc + n0 + 32 * j + ccol] = alpha * acc[mi][j][i];
          }
    }
  } else {
    // SiLU(gate) * up -> bf16 tile [32 kMBa][32 * kWaves] in LDS (the stage
    // buffers are free: the loop's last barrier ordered all reads of them)
    constexpr int kHW = 32 * kWaves;
    constexpr int kLdh = kHW + 8;
    static_assert(kLdh <= 2 * kLdA, "h tile must fit the stage buffers");
    uint16_t* sh = reinterpret_cast<uint16_t*>(smem);
    const int32_t hbase = nt * kHW;
    const int32_t I = prm.I;
    if (active) {
#pragma unroll
      for (int mi = 0; mi < kMBa; ++mi)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = mi * 32 + 8 * (i >> 2) + crow + (i & 3);
          const int col = 32 * wave + ccol;
          const float gv = alpha * acc[mi][0][i];
          const float uv = alpha * acc[mi][1][i];
          // silu(g) = g / (1 + e^-g); the hardware reciprocal (1 ulp) is far
          // inside the bf16 rounding that follows
          const float hv = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
          const uint32_t hb = __builtin_bit_cast(uint16_t, (__bf16)hv);   // RNE, hardware
          sh[row * kLdh + col] = (uint16_t)hb;
          if (row < rows) {
            const int64_t p = row0 + row;
            if (prm.c1_dbg) {
              prm.c1_dbg[row_major(p, 2 * I, hbase + col)] = gv;
              prm.c1_dbg[row_major(p, 2 * I, I + hbase + col)] = uv;
            }
            if (prm.h_dbg) prm.h_dbg[row_major(p, I, hbase + col)] = (uint16_t)hb;
          }
        }
    }
    lds_barrier();
    if constexpr (kW16) {
      // h rows out as bf16, 16 bytes per store
      constexpr int kPieces = kHW / 8;
      for (int item = tid; item < 32 * kMBa * kPieces; item += kThreads) {
        const int row = item / kPieces, pc = item % kPieces;
        const int32_t hcol = hbase + 8 * pc;
        if (row < rows && hcol < I)
          *reinterpret_cast<u32x4*>(prm.h_out + a_rows_offset(row0 + row, I, hcol / 8, 8)) =
              *reinterpret_cast<const u32x4*>(sh + row * kLdh + 8 * pc);
      }
    } else if constexpr (kMX) {
      // requantise in the UE8M0 mode: rows x (kHW / 32) blocks of 32 columns
      constexpr int kItems = 32 * kMBa * (kHW / 32);
      const float gs = prm.out_gscale[e];
      for (int item = tid; item < kItems; item += kThreads) {
        const int row = item / (kHW / 32), blk = item % (kHW / 32);
        const int32_t hcol = hbase + 32 * blk;
        if (row < rows && hcol < I) {
          const u32x4* src = reinterpret_cast<const u32x4*>(sh + row * kLdh + 32 * blk);
          float xv[32];
#pragma unroll
          for (int q = 0; q < 4; ++q) unpack_bf16x8(src[q], xv + 8 * q);
          const float am = fmaxf(absmax16(xv), absmax16(xv + 16));
          const BlockScale bsc = block_scale_ue8m0(am / kE2M1Max, gs);
          u32x4 wv;
          wv.x = encode8(xv, bsc.inv);
          wv.y = encode8(xv + 8, bsc.inv);
          wv.z = encode8(xv + 16, bsc.inv);
          wv.w = encode8(xv + 24, bsc.inv);
          const int64_t p = row0 + row;
          *reinterpret_cast<u32x4*>(prm.out_codes + a_codes_offset(p, I, hcol / 32, 32, true)) = wv;
          prm.out_sf[a_scales_offset(p, I, hcol / 32, 32, true)] = (uint8_t)bsc.sf;
        }
      }
    } else {
    // requantise: rows x (kHW / 16) blocks of 16 columns
    constexpr int kItems = 32 * kMBa * (kHW / 16);
    const float gs = prm.out_gscale[e];
    for (int item = tid; item < kItems; item += kThreads) {
      const int row = item / (kHW / 16), blk = item % (kHW / 16);
      const int32_t hcol = hbase + 16 * blk;
      if (row < rows && hcol < I) {
        const u32x4* src = reinterpret_cast<const u32x4*>(sh + row * kLdh + 16 * blk);
        float xv[16];
        unpack_bf16x8(src[0], xv);
        unpack_bf16x8(src[1], xv + 8);
        const BlockScale bsc = block_scale(absmax16(xv) / kE2M1Max, gs);
        uint2 wv;
        wv.x = encode8(xv, bsc.inv);
        wv.y = encode8(xv + 8, bsc.inv);
        const int64_t p = row0 + row;
        *reinterpret_cast<uint2*>(prm.out_codes + a_codes_offset(p, I, hcol / 16, 16, false)) = wv;
        prm.out_sf[a_scales_offset(p, I, hcol / 16, 16, false)] = (uint8_t)bsc.sf;
      }
    }
    }
  }
  };  // tile

  const int sub = (rows + 31) >> 5;                  // 32-row sub-tiles holding rows
  static_assert(kMB >= 1 && kMB <= 4, "tile height is 32 to 128 rows");
  if (sub >= kMB) {
    tile(Int<kMB>{});
  } else {
    if constexpr (kMB == 4) {
      if (sub == 3) tile(Int<3>{});
      else if (sub == 2) tile(Int<2>{});
      else tile(Int<1>{});
    } else if constexpr (kMB == 3) {
      if (sub == 2) tile(Int<2>{});
      else tile(Int<1>{});
    } else if constexpr (kMB == 2) {
      tile(Int<1>{});
    }
  }
  lds_barrier();   // LDS is reused by the next tile
  }
}

namespace {

// Resident workgroups per CU for a kernel, and the CU count, for the current
// device (every device this library runs on is the same gfx950 part).
struct Residency {
  int cus = 0, per_cu = 0;
};

template <int kWaves, int kMB, int kBK, bool kGated, int kRing, int kOcc, int kMode>
hipError_t launch(GemmParams prm, int32_t P, hipStream_t stream) {
  constexpr int kBM = 32 * kMB;
  // looked up once per process (a function-local static is initialised once,
  // thread-safely); a failed lookup is retried on the next call
  static const Residency cached = [] {
    Residency r;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&r.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &r.per_cu, (const void*)grouped_gemm_kernel<kWaves, kMB, kBK, kGated, kRing, kOcc, kMode>,
            64 * kWaves, 0) != hipSuccess)
      return Residency{};
    if (r.per_cu < 1) r.per_cu = 1;
    return r;
  }();
  Residency res = cached;
  if (res.cus == 0) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err == hipSuccess) err = hipDeviceGetAttribute(&res.cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err == hipSuccess)
      err = hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &res.per_cu, (const void*)grouped_gemm_kernel<kWaves, kMB, kBK, kGated, kRing, kOcc, kMode>,
          64 * kWaves, 0);
    if (err != hipSuccess) return err;
    if (res.per_cu < 1) res.per_cu = 1;
  }
  const int64_t tiles = (int64_t)m_tiles_bound(P, prm.E, kBM) * prm.n_tiles;
  const int64_t slots = (int64_t)res.cus * res.per_cu;
  int64_t grid = tiles < slots ? tiles : slots;
  grid = (grid + kXcds - 1) / kXcds * kXcds;            // whole XCD rounds
  hipLaunchKernelGGL((grouped_gemm_kernel<kWaves, kMB, kBK, kGated, kRing, kOcc, kMode>), dim3((uint32_t)grid),
                     dim3(64 * kWaves), 0, stream, prm);
  return hipGetLastError();
}

}  // namespace

// The kernel instantiation for a gemm_map::Shape and operand mode.
template <int kMode, const Shape& S>
hipError_t launch_shape(const GemmParams& prm, int32_t P, hipStream_t stream) {
  return launch<S.waves, S.mb, S.bk, S.gated, S.ring, S.occ, kMode>(prm, P, stream);
}

// Shapes by batch (gemm_map::select_shape): the large-batch tiles when experts
// average at least 32 rows (prefill; the last tile of an expert runs only its
// occupied 32-row sub-tiles), else 32-row tiles (decode-like batches, weight
// streaming bound).
hipError_t launch_gemm1(const Gemm1Args& a, hipStream_t stream) {
  if (a.P == 0) return hipSuccess;
  GemmParams prm{};
  prm.a_codes = a.a_codes; prm.a_sf = a.a_sf; prm.w_codes = a.w_codes; prm.w_sf = a.w_sf;
  prm.a_rows = a.a_rows; prm.a_src = a.a_src; prm.a_src_div = a.a_src_div; prm.lda = a.lda;
  prm.h_out = a.h_out;
  prm.in_scale = a.in_scale; prm.w_scale2 = a.w_scale2; prm.offsets = a.offsets;
  prm.E = a.E; prm.K = a.H; prm.N_w = 2 * a.I; prm.I = a.I;
  prm.out_gscale = a.out_gscale; prm.out_codes = a.out_codes; prm.out_sf = a.out_sf;
  prm.c1_dbg = a.c1_dbg; prm.h_dbg = a.h_dbg;
  if (a.perm_ids) {
    // only the small-batch kernels regroup the ids themselves, and only up
    // to kFoldMaxPairs pairs (their LDS copy of the ids)
    if (!fold_permutation(a.P, a.E) || !a.perm_offsets || !a.perm_src || !a.perm_inv || !a.a_src)
      return hipErrorInvalidValue;
    prm.perm_ids = a.perm_ids; prm.perm_P = a.P;
    prm.perm_offsets = a.perm_offsets; prm.perm_src = a.perm_src; prm.perm_inv = a.perm_inv;
  }
  const int mode = a.mx ? kModeMX : a.w16 ? kModeW16 : kModeNV;
  prm.n_tiles = n_tiles(true, select_shape(true, mode, a.P, a.E).waves, a.I, a.H);
  if (large_batch(a.P, a.E)) {
    if (mode == kModeMX) return launch_shape<kModeMX, kG1LargeMx>(prm, a.P, stream);
    if (mode == kModeW16) return launch_shape<kModeW16, kG1LargeW16>(prm, a.P, stream);
    return launch_shape<kModeNV, kG1Large>(prm, a.P, stream);
  }
  if (mode == kModeMX) return launch_shape<kModeMX, kG1SmallMx>(prm, a.P, stream);
  if (mode == kModeW16) return launch_shape<kModeW16, kG1SmallW16>(prm, a.P, stream);
  return launch_shape<kModeNV, kG1Small>(prm, a.P, stream);
}

hipError_t launch_gemm2(const Gemm2Args& a, hipStream_t stream) {
  if (a.P == 0) return hipSuccess;
  GemmParams prm{};
  prm.a_codes = a.a_codes; prm.a_sf = a.a_sf; prm.w_codes = a.w_codes; prm.w_sf = a.w_sf;
  prm.a_rows = a.a_rows; prm.lda = a.I;
  prm.in_scale = a.in_scale; prm.w_scale2 = a.w_scale2; prm.offsets = a.offsets;
  prm.E = a.E; prm.K = a.I; prm.N_w = a.H; prm.I = a.I;
  prm.c_out = a.out; prm.ldc = a.H;
  const int mode = a.mx ? kModeMX : a.w16 ? kModeW16 : kModeNV;
  prm.n_tiles = n_tiles(false, select_shape(false, mode, a.P, a.E).waves, a.I, a.H);
  if (large_batch(a.P, a.E)) {
    if (mode == kModeMX) return launch_shape<kModeMX, kG2LargeMx>(prm, a.P, stream);
    if (mode == kModeW16) return launch_shape<kModeW16, kG2Large>(prm, a.P, stream);
    return launch_shape<kModeNV, kG2Large>(prm, a.P, stream);
  }
  if (mode == kModeMX) return launch_shape<kModeMX, kG2SmallMx>(prm, a.P, stream);
  if (mode == kModeW16) return launch_shape<kModeW16, kG2SmallW16>(prm, a.P, stream);
  return launch_shape<kModeNV, kG2Small>(prm, a.P, stream);
}

// ---- load-time weight layout conversion -----------------------------------
// Checkpoint layout: codes [E][N][K/2], scales [E][N][K/16], row-major.
// Kernel layout (same sizes): for each expert e, 32-row block nb and K step
// ks (kBK wide), the codes are stored lane by lane as the wavefront reads
// them: piece (v, lane) = 16 bytes of row nb*32 + (lane & 31), elements
// ks*kBK + (lane >> 5)*kBK/2 + 32v + [0, 32); the scales likewise hold, for
// each lane, the block scales of that row and K range (kBK/32 E4M3 scales,
// or kBK/64 UE8M0 scales in the 32-element-block mode).
__global__ __launch_bounds__(256) void pack_codes_kernel(const uint8_t* __restrict__ src,
                                                         uint8_t* __restrict__ dst, int64_t pieces,
                                                         int32_t N, int32_t K, int32_t bk) {
  const int64_t gi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gi >= pieces) return;
  const int32_t kvec = bk / 64, nks = K / bk, nb_per = N / 32;
  const int32_t lane = (int32_t)(gi % 64);
  int64_t t = gi / 64;
  const int32_t v = (int32_t)(t % kvec);
  t /= kvec;
  const int32_t ks = (int32_t)(t % nks);
  t /= nks;
  const int32_t nb = (int32_t)(t % nb_per);
  const int64_t e = t / nb_per;
  const int64_t row = e * N + nb * 32 + (lane & 31);
  const int64_t k0 = (int64_t)ks * bk + (lane >> 5) * (bk / 2) + 32 * v;
  *reinterpret_cast<uint4*>(dst + gi * 16) =
      *reinterpret_cast<const uint4*>(src + row * (K / 2) + k0 / 2);
}

__global__ __launch_bounds__(256) void pack_scales_kernel(const uint8_t* __restrict__ src,
                                                          uint8_t* __restrict__ dst, int64_t items,
                                                          int32_t N, int32_t K, int32_t bk,
                                                          int32_t blk_elems) {
  const int64_t gi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gi >= items) return;
  // per lane: the scales of the lane's bk/2 elements (blocks of blk_elems)
  const int32_t nks = K / bk, nb_per = N / 32, per = bk / 2 / blk_elems;
  const int32_t lane = (int32_t)(gi % 64);
  int64_t t = gi / 64;
  const int32_t ks = (int32_t)(t % nks);
  t /= nks;
  const int32_t nb = (int32_t)(t % nb_per);
  const int64_t e = t / nb_per;
  const int64_t row = e * N + nb * 32 + (lane & 31);
  const int64_t blk = ((int64_t)ks * bk + (lane >> 5) * (bk / 2)) / blk_elems;
  for (int32_t i = 0; i < per; ++i) dst[gi * per + i] = src[row * (K / blk_elems) + blk + i];
}

int32_t weight_step_k(int32_t projection, bool mx) {
  // every GEMM1 shape of a mode shares one K step, as every GEMM2 shape does
  static_assert(kG1Large.bk == kG1Small.bk && kG1Large.bk == kG1LargeW16.bk &&
                kG1Large.bk == kG1SmallW16.bk && kG1LargeMx.bk == kG1SmallMx.bk,
                "one w13 K step per mode");
  static_assert(kG2Large.bk == kG2Small.bk && kG2Large.bk == kG2LargeMx.bk &&
                kG2Large.bk == kG2SmallW16.bk && kG2Large.bk == kG2SmallMx.bk,
                "one w2 K step");
  return projection == 0 ? (mx ? kG1LargeMx.bk : kG1Large.bk) : kG2Large.bk;
}

hipError_t launch_pack_weights(int32_t projection, const uint8_t* codes, const uint8_t* sf,
                               int32_t E, int32_t N, int32_t K, uint8_t* codes_out,
                               uint8_t* sf_out, hipStream_t stream, bool mx) {
  const int32_t bk = weight_step_k(projection, mx);
  const int64_t pieces = (int64_t)E * N * K / 32;        // 16-byte pieces
  const int64_t items = (int64_t)E * (N / 32) * (K / bk) * 64;
  if (pieces == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_codes_kernel, dim3((uint32_t)((pieces + 255) / 256)), dim3(256), 0,
                     stream, codes, codes_out, pieces, N, K, bk);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(pack_scales_kernel, dim3((uint32_t)((items + 255) / 256)), dim3(256), 0,
                     stream, sf, sf_out, items, N, K, bk, mx ? 32 : 16);
  return hipGetLastError();
}

}  // namespace nvfp4
