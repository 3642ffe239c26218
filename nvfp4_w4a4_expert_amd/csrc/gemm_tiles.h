// Launch shapes, tile mapping and global address arithmetic of the grouped
// expert GEMMs (gemm.hip).  The kernel forms every global address it reads
// or writes through these functions, and a host-side checker
// (tests/host/gemm_ranges.cpp) runs the same functions over every tile,
// wavefront, lane and K step of a launch to prove each access lies inside
// its buffer; so the addresses the checker proves in bounds are the ones the
// kernel forms.  Plain integer arithmetic, no HIP types.
#pragma once

#include <stdint.h>

#if defined(__HIP__)
#define NVFP4_HD __host__ __device__ inline __attribute__((always_inline))
#else
#define NVFP4_HD inline
#endif

namespace nvfp4 {
namespace gemm_map {

// Operand modes of the grouped GEMM.
constexpr int kModeNV = 0;     // NVFP4 x NVFP4, fp16 MFMA on exact dequantised values
constexpr int kModeW16 = 1;    // bf16 activations x NVFP4 weights, bf16 MFMA
constexpr int kModeMX = 2;     // UE8M0 FP4 x UE8M0 FP4, scaled FP4 MFMA

constexpr int kXcds = 8;
constexpr int kMaxExperts = 1024;

// One instantiation of the grouped GEMM kernel.
struct Shape {
  int waves;   // wavefronts per workgroup
  int mb;      // 32-row sub-tiles per token tile (tile height 32 * mb)
  int bk;      // K elements per pipeline step
  int ring;    // register ring slots
  int occ;     // workgroups per CU the launch bounds ask for
  bool gated;  // GEMM1 (w13 + SiLU*mul epilogue) or GEMM2 (w2, fp32 C)
};

// Launch shapes for batches with at least 32 rows per expert on average
// (chosen by measurement on MI355X at the 4096-token prefill layer):
//   w13: 8 wavefronts (256 h columns), 64-row tiles, K step 128, 3-slot
//        register rings, one workgroup per CU: the staged token tile serves
//        twice the weight columns of a 4-wavefront workgroup
//   w2:  4 wavefronts (256 output columns), 128-row tiles, K step 64, 2-slot
//        register rings, 2 workgroups per CU
// (two wavefronts per SIMD, at most 256 VGPRs per lane; 96- or 128-row w13
// tiles either do not fit with 3-slot rings or lose more to latency with
// 2-slot rings than they save in dequantisation.)
constexpr Shape kG1Large{8, 2, 128, 3, 1, true};
// UE8M0 mode w13: K step 256 (nothing to dequantise, so a 128-wide step is
// too little matrix work per barrier and per prefetch slot); 96-row tiles
// with a 2-slot register ring, which reuse each weight fragment over a third
// more rows for the same registers as 64-row tiles with 3 slots (measured
// 140 -> 129 us at the prefill layer)
constexpr Shape kG1LargeMx{8, 3, 256, 2, 1, true};
// weight-only mode w13: 96-row tiles with a 2-slot ring as well (its weights
// cost twice the dequantisation instructions of the E4M3 mode, so reusing each
// fragment over more rows pays: measured 342 -> 321 us at the prefill layer)
constexpr Shape kG1LargeW16{8, 3, 128, 2, 1, true};
constexpr Shape kG2Large{4, 4, 64, 2, 2, false};
// UE8M0 mode w2: 3 ring slots (no dequantisation registers, so the deeper
// ring fits in 247 VGPRs; measured 138 -> 136 us; in the other modes it spills)
constexpr Shape kG2LargeMx{4, 4, 64, 3, 2, false};
// Batches with fewer than 32 rows per expert on average (decode): one 32-row
// sub-tile and 4 wavefronts; each tile streams one expert's weight slice, so
// the more workgroups a CU holds, the more of those streams are in flight.
// E4M3 mode: w13 with a 2-slot ring at 3 workgroups per CU (164 VGPRs), w2
// with a 3-slot ring at 4 per CU (128 VGPRs), so that the 16-token decode
// layer's ~880 w2 tiles (80 hit experts x 11 column tiles) run in one round
// of 1024 slots instead of 768 (measured: decode step 68.7 -> 65.7 us).
constexpr Shape kG1Small{4, 1, 128, 2, 3, true};
constexpr Shape kG2Small{4, 1, 64, 3, 4, false};
// UE8M0 mode: w2 with a 2-slot ring at 4 workgroups per CU (125 VGPRs;
// decode step 58.6 -> 56.8 us); its w13 keeps a 3-slot ring at 2 per CU (a
// 2-slot ring at 3 per CU spills and was slower).  Weight-only mode: 3-slot
// rings at 2 workgroups per CU (2-slot rings at 3 and 4 per CU spill and
// gained nothing measurable).
constexpr Shape kG1SmallMx{4, 1, 256, 3, 2, true};
constexpr Shape kG2SmallMx{4, 1, 64, 2, 4, false};
constexpr Shape kG1SmallW16{4, 1, 128, 3, 2, true};
constexpr Shape kG2SmallW16{4, 1, 64, 3, 2, false};

// The large-batch kernels run when experts average at least 32 rows.
NVFP4_HD bool large_batch(int32_t P, int32_t E) { return P >= 32 * E; }

// Small batches of at most kFoldMaxPairs (token, slot) pairs skip the
// permutation kernel: the small-batch GEMM1 regroups the routed ids itself
// (every workgroup histograms them in LDS for the expert offsets and ranks
// its own tile's pairs) and writes offsets, src_pair and inv for GEMM2, the
// combine and the debug dumps.
constexpr int kFoldMaxPairs = 512;
NVFP4_HD bool fold_permutation(int32_t P, int32_t E) {
  return !large_batch(P, E) && P <= kFoldMaxPairs;
}

NVFP4_HD Shape select_shape(bool gemm1, int mode, int32_t P, int32_t E) {
  if (large_batch(P, E)) {
    if (gemm1) return mode == kModeMX ? kG1LargeMx : mode == kModeW16 ? kG1LargeW16 : kG1Large;
    return mode == kModeMX ? kG2LargeMx : kG2Large;
  }
  if (gemm1) return mode == kModeMX ? kG1SmallMx : mode == kModeW16 ? kG1SmallW16 : kG1Small;
  return mode == kModeMX ? kG2SmallMx : mode == kModeW16 ? kG2SmallW16 : kG2Small;
}

// n-tiles of a launch: GEMM1 tiles cover 32 h columns per wavefront (32 gate
// plus 32 up weight rows), GEMM2 tiles 64 output columns per wavefront.
NVFP4_HD int32_t n_tiles(bool gated, int waves, int32_t I, int32_t H) {
  return gated ? (I + 32 * waves - 1) / (32 * waves) : (H + 64 * waves - 1) / (64 * waves);
}

// m-tiles of an expert with `rows` rows.
NVFP4_HD int32_t m_tiles(int32_t rows, int32_t bm) { return (rows + bm - 1) / bm; }

// Upper bound on the m-tiles of all experts together (sizes the grid).
NVFP4_HD int32_t m_tiles_bound(int32_t P, int32_t E, int32_t bm) {
  return (P + bm - 1) / bm + (P < E ? P : E);
}

// Persistent-loop position t -> logical tile.  The workgroups the hardware
// sends to one XCD (round robin over kXcds) get a contiguous range of logical
// tiles: all n-tiles of an m-tile, and consecutive m-tiles of an expert,
// share that XCD's L2.  t runs over [0, per_xcd * kXcds); logical tiles at or
// past `total` are skipped.
NVFP4_HD int32_t per_xcd(int32_t total) { return (total + kXcds - 1) / kXcds; }
NVFP4_HD int32_t logical_tile(int32_t t, int32_t per_xcd_tiles) {
  return (t % kXcds) * per_xcd_tiles + t / kXcds;
}

struct Tile {
  int32_t mt, nt;   // m-tile (over all experts) and n-tile
  int32_t e;        // expert
  int32_t row0;     // first grouped row of the tile
  int32_t rows;     // rows of the tile that belong to e (<= 32 * mb)
};

// Logical tile -> (expert, rows).  mt_prefix[e] is the number of m-tiles of
// experts before e (mt_prefix[E] = all of them), offsets[e] the expert's
// first grouped row (offsets[E] = P).
NVFP4_HD Tile tile_of(int32_t logical, int32_t n_tiles_, const int32_t* mt_prefix,
                      const int32_t* offsets, int32_t E, int32_t bm) {
  Tile c;
  c.mt = logical / n_tiles_;
  c.nt = logical - c.mt * n_tiles_;
  int32_t lo = 0, hi = E - 1;                      // last e with mt_prefix[e] <= mt
  while (lo < hi) {
    const int32_t mid = (lo + hi + 1) >> 1;
    if (mt_prefix[mid] <= c.mt) lo = mid; else hi = mid - 1;
  }
  c.e = lo;
  c.row0 = offsets[c.e] + (c.mt - mt_prefix[c.e]) * bm;
  const int32_t left = offsets[c.e + 1] - c.row0;
  c.rows = left < bm ? left : bm;
  return c;
}

// Per-thread part of a workgroup's expert prefix pass: a thread owns kPer
// consecutive experts with m[i] rows each (0 past the last expert).  cnt[i]
// is the expert's m-tiles of bm rows; rcnt[i] its rows (the second scan, run
// when the small-batch GEMM1 regroups the routed ids).  The totals feed the
// workgroup's exclusive scans.
template <int kPer>
NVFP4_HD void thread_prefix_counts(const int32_t (&m)[kPer], int32_t bm, int32_t (&cnt)[kPer],
                                   int32_t (&rcnt)[kPer], int32_t& total, int32_t& rtotal) {
  total = 0;
  rtotal = 0;
  for (int i = 0; i < kPer; ++i) {
    cnt[i] = m_tiles(m[i], bm);
    rcnt[i] = m[i];
    total += cnt[i];
    rtotal += rcnt[i];
  }
}

// The two 32-row weight blocks a wavefront streams.  GEMM1: block 0 = the
// gate rows of h columns [hc0, hc0 + 32), block 1 = the matching up rows
// (I + hc0); GEMM2: output columns [n0, n0 + 64) as two blocks.  A wavefront
// past the last column is inactive and points both blocks at block 0 of the
// expert (it loads, never multiplies or stores), so no base is negative.
struct WaveBlocks {
  bool active;
  int32_t hc0;       // GEMM1: first h column of the wavefront
  int32_t n0;        // GEMM2: first output column of the wavefront
  int32_t row0[2];   // first weight row of each 32-row block
};

NVFP4_HD WaveBlocks wave_blocks(bool gated, int waves, int32_t nt, int32_t wave, int32_t I,
                                int32_t N_w) {
  WaveBlocks b;
  b.hc0 = gated ? nt * (32 * waves) + 32 * wave : 0;
  b.n0 = gated ? 0 : nt * (64 * waves) + 64 * wave;
  b.active = gated ? b.hc0 < I : b.n0 < N_w;
  for (int j = 0; j < 2; ++j) {
    int32_t r = gated ? (j == 0 ? b.hc0 : I + b.hc0) : b.n0 + 32 * j;
    b.row0[j] = b.active ? r : 0;
  }
  return b;
}

// ---- B (weights, kernel layout of nvfp4_moe_pack_weights) -----------------
// Inside a 32-row block the codes of K step kt are stored lane by lane: lane
// `lane` reads 16-byte piece v at block base + kt * (bk/64) * 1024 + 1024 v
// + 16 lane (v < bk/64); its block scales are bk/32 E4M3 bytes (bk/64 UE8M0
// bytes) at scale base + kt * 64 * that + that * lane.
NVFP4_HD int64_t b_codes_offset(int32_t e, int32_t N_w, int32_t blk_row0, int32_t K, int lane) {
  return ((int64_t)e * N_w + blk_row0) * (K / 2) + 16 * lane;
}
NVFP4_HD int64_t b_codes_step(int32_t kt, int bk) { return (int64_t)kt * ((bk / 64) * 1024); }
NVFP4_HD int b_scale_bytes(int bk, bool mx) { return mx ? bk / 64 : bk / 32; }
NVFP4_HD int64_t b_scales_offset(int32_t e, int32_t N_w, int32_t blk_row0, int32_t K, int lane,
                                 int bk, bool mx) {
  const int64_t rbase = (int64_t)e * N_w + blk_row0;
  return mx ? rbase * (K / 32) + (bk / 64) * lane : rbase * (K / 16) + (bk / 32) * lane;
}
NVFP4_HD int64_t b_scales_step(int32_t kt, int bk, bool mx) {
  return (int64_t)kt * (64 * b_scale_bytes(bk, mx));
}

// ---- A (token rows) staging ---------------------------------------------------
// Each K step the workgroup stages the tile's occupied rows: chunk c of
// `chunk_elems` elements covers row c / (bk / chunk_elems) and k-chunk
// c % (bk / chunk_elems).  A is staged in chunks of 32 elements (16 code bytes
// + 2 scales), or of 16 elements when that is what it takes to give every
// thread a chunk; bf16 rows (kW16) in chunks of 8 elements (16 bytes); UE8M0
// codes (kMX) in chunks of one 32-element block (16 code bytes + 1 scale).
constexpr NVFP4_HD int a_chunk_elems(int mode, int mba, int bk, int threads) {
  return mode == kModeW16 ? 8 : mode == kModeMX ? 32 : 32 * mba * (bk / 32) >= threads ? 32 : 16;
}
// Rows past the expert's last row re-read its last row (never stored).
NVFP4_HD int64_t a_row(int32_t row0, int32_t r, int32_t rows) {
  return row0 + (r < rows - 1 ? r : rows - 1);
}
// Byte offsets of chunk (row arow, k-chunk kc) at K step 0 in the quantised
// operand's codes [P, K/2] and block scales [P, K/16] ([P, K/32] UE8M0), and
// per K step.
NVFP4_HD int64_t a_codes_offset(int64_t arow, int32_t K, int kc, int chunk_elems, bool mx) {
  return arow * (K / 2) + (mx ? 16 * kc : (chunk_elems / 2) * kc);
}
NVFP4_HD int64_t a_scales_offset(int64_t arow, int32_t K, int kc, int chunk_elems, bool mx) {
  return mx ? arow * (K / 32) + kc : arow * (K / 16) + (chunk_elems / 16) * kc;
}
NVFP4_HD int64_t a_codes_step(int32_t kt, int bk) { return (int64_t)kt * (bk / 2); }
NVFP4_HD int64_t a_scales_step(int32_t kt, int bk, bool mx) {
  return (int64_t)kt * (mx ? bk / 32 : bk / 16);
}
// Weight-only mode: element offset of chunk (source row srow, k-chunk kc) in
// bf16 rows of stride lda, and per K step.
NVFP4_HD int64_t a_rows_offset(int64_t srow, int64_t lda, int kc, int chunk_elems) {
  return srow * lda + (int64_t)chunk_elems * kc;
}
NVFP4_HD int64_t a_rows_step(int32_t kt, int bk) { return (int64_t)kt * bk; }

// ---- outputs ---------------------------------------------------------------------
// GEMM2: float offset of the 4 outputs lane (rr = lane / 16, c4 = 4 * (lane % 16))
// writes for tile row `row` of a wavefront's 64-column slab.
NVFP4_HD int64_t c_offset(int32_t row0, int32_t row, int32_t ldc, int32_t n0, int c4) {
  return ((int64_t)row0 + row) * ldc + n0 + c4;
}

// Element offset of column `col` of row `p` in a row-major matrix with `ld`
// columns (the GEMM1 debug dumps of C1 and h).
NVFP4_HD int64_t row_major(int64_t p, int32_t ld, int32_t col) { return p * ld + col; }

}  // namespace gemm_map
}  // namespace nvfp4
