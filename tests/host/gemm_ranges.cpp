// Host-side range check of every global access the grouped expert GEMMs
// form (gemm.hip), built with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer.  The tile mapping and every address come from
// gemm_tiles.h, the header the kernel itself uses; this program walks them
// the way a launch does (every persistent-loop position, wavefront, lane,
// staging chunk, K step and output element) and checks that each access lies
// inside its buffer.  It also checks that the tiles of a launch cover every
// (grouped row, column block) exactly once.
//
// Input (stdin), one case per line:
//   label mode E H I k T count_0 ... count_{E-1}
// mode 0 = E4M3 W4A4, 1 = weight-only (bf16 rows), 2 = UE8M0 W4A4; counts
// are the grouped rows of each expert (sum = T * k).  Prints one line per
// case and "gemm ranges ok" when every case passes; exits nonzero otherwise.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <string>
#include <vector>

#include "nvfp4_w4a4_expert_amd/csrc/gemm_tiles.h"

using namespace nvfp4::gemm_map;

namespace {

int g_failures = 0;
std::string g_label;

// [lo, hi) must lie inside [0, size)
void check_range(const char* what, int64_t lo, int64_t hi, int64_t size) {
  if (lo < 0 || hi > size || lo > hi) {
    if (g_failures < 20)
      fprintf(stderr, "%s: %s access [%lld, %lld) outside [0, %lld)\n", g_label.c_str(), what,
              (long long)lo, (long long)hi, (long long)size);
    ++g_failures;
  }
}

void check(bool ok, const char* what) {
  if (!ok) {
    if (g_failures < 20) fprintf(stderr, "%s: %s\n", g_label.c_str(), what);
    ++g_failures;
  }
}

struct Case {
  std::string label;
  int mode;
  int32_t E, H, I, k, T;
  std::vector<int32_t> counts;
};

// The kernel's expert prefix pass, repeated on the host: each of `threads`
// threads owns kPer experts and counts them with the kernel's own
// thread_prefix_counts; an exclusive scan over the threads' totals (what the
// kernel's wavefront scans and cross-wavefront sums compute) gives each
// thread's bases, then each owned expert's entries.
template <int kPer>
void kernel_prefix(const std::vector<int32_t>& counts, int32_t E, int32_t bm, int threads,
                   std::vector<int32_t>& pre, std::vector<int32_t>& rpre) {
  check(kPer * threads >= E + 1, "the prefix pass covers experts 0 .. E");
  pre.assign((size_t)E + 1, -1);
  rpre.assign((size_t)E + 1, -1);
  int32_t base = 0, rbase = 0;
  for (int tid = 0; tid < threads; ++tid) {
    int32_t m[kPer], cnt[kPer], rcnt[kPer], total, rtotal;
    for (int i = 0; i < kPer; ++i) {
      const int32_t e = kPer * tid + i;
      m[i] = e < E ? counts[e] : 0;
    }
    thread_prefix_counts<kPer>(m, bm, cnt, rcnt, total, rtotal);
    int32_t b = base, rb = rbase;
    for (int i = 0; i < kPer; ++i) {
      const int32_t e = kPer * tid + i;
      if (e <= E) {
        pre[e] = b;
        rpre[e] = rb;
      }
      b += cnt[i];
      rb += rcnt[i];
    }
    base += total;
    rbase += rtotal;
  }
}

// One GEMM launch of a case: GEMM1 (w13, gated) or GEMM2 (w2).
void check_gemm(const Case& c, bool gemm1) {
  const bool mx = c.mode == kModeMX, w16 = c.mode == kModeW16;
  const int32_t E = c.E, H = c.H, I = c.I, T = c.T;
  const int32_t P = T * c.k;
  const Shape sh = select_shape(gemm1, c.mode, P, E);
  check(sh.gated == gemm1, "shape kind");
  const int32_t bm = 32 * sh.mb, threads = 64 * sh.waves, bk = sh.bk;
  const int32_t K = gemm1 ? H : I, N_w = gemm1 ? 2 * I : H;
  const int32_t blk = mx ? 32 : 16;                  // elements per block scale
  check(K % bk == 0, "K is a whole number of pipeline steps");
  const int32_t nk = K / bk;
  const int32_t nt_count = n_tiles(gemm1, sh.waves, I, H);

  // buffer sizes (bytes, or elements for the typed outputs)
  const int64_t a_codes_bytes = (int64_t)P * K / 2, a_sf_bytes = (int64_t)P * K / blk;
  const int64_t w_codes_bytes = (int64_t)E * N_w * K / 2;
  const int64_t w_sf_bytes = (int64_t)E * N_w * K / blk;
  const int64_t c_elems = (int64_t)P * H;                         // GEMM2 fp32 C
  const int64_t out_codes_bytes = (int64_t)P * I / 2, out_sf_bytes = (int64_t)P * I / blk;
  const int64_t h_elems = (int64_t)P * I, c1_elems = (int64_t)P * 2 * I;
  // weight-only A rows: GEMM1 reads x [T, H] through src_pair / k, GEMM2 h [P, I]
  const int64_t a_row_count = w16 && gemm1 ? T : P;

  std::vector<int32_t> offsets(E + 1, 0), mt_prefix(E + 1, 0);
  for (int32_t e = 0; e < E; ++e) {
    offsets[e + 1] = offsets[e] + c.counts[e];
    mt_prefix[e + 1] = mt_prefix[e] + m_tiles(c.counts[e], bm);
  }
  check(offsets[E] == P, "counts sum to T * k");
  check(mt_prefix[E] <= m_tiles_bound(P, E, bm), "m-tile bound sizes the grid");
  const int32_t total = mt_prefix[E] * nt_count;
  const int32_t xcd_tiles = per_xcd(total);
  // the m-tile prefix and (small-batch GEMM1) the expert offsets as the
  // kernel's own prefix pass computes them
  {
    std::vector<int32_t> kpre, krpre;
    const int per = (kMaxExperts + 1 + threads - 1) / threads;
    if (per == 3) kernel_prefix<3>(c.counts, E, bm, threads, kpre, krpre);
    else if (per == 5) kernel_prefix<5>(c.counts, E, bm, threads, kpre, krpre);
    else check(false, "experts per thread of the prefix pass");
    check(kpre == mt_prefix, "kernel prefix pass: m-tiles");
    check(krpre == offsets, "kernel prefix pass: expert offsets");
  }

  // Small batches: GEMM1 regroups the routed ids itself.  The ids are laid out
  // here as an interleaving of the experts' pairs (consistent with the
  // counts); the per-tile ranking below repeats the kernel's walk (64 ids at a
  // time, rank = matches before the pair) and checks that every row of every
  // tile gets exactly one pair and every pair exactly one inverse entry.
  const bool fold = gemm1 && fold_permutation(P, E);
  std::vector<int32_t> ids;
  std::vector<uint8_t> inv_written;
  if (fold) {
    check(sh.mb == 1 && bm == 32, "regrouping runs in the 32-row small-batch kernel");
    check(P <= kFoldMaxPairs, "routed ids fit the workgroup's LDS copy");
    std::vector<int32_t> left(c.counts);
    for (int32_t q = 0, e = 0; q < P; ++q) {
      while (left[e] == 0) e = (e + 1) % E;
      ids.push_back(e);
      --left[e];
      e = (e + 7) % E;
    }
    inv_written.assign((size_t)P, 0);
  }

  // coverage: each (m-tile, n-tile) once
  std::vector<uint8_t> seen((size_t)total, 0);
  int64_t rows_covered = 0;
  for (int32_t t = 0; t < xcd_tiles * kXcds; ++t) {
    const int32_t logical = logical_tile(t, xcd_tiles);
    if (logical >= total) continue;
    check(logical >= 0, "logical tile >= 0");
    if (seen[logical]++) check(false, "logical tile visited twice");
    const Tile tl = tile_of(logical, nt_count, mt_prefix.data(), offsets.data(), E, bm);
    check(tl.e >= 0 && tl.e < E, "expert in range");
    check(tl.rows >= 1 && tl.rows <= bm, "tile rows in [1, tile height]");
    check(tl.row0 >= offsets[tl.e] && tl.row0 + tl.rows <= offsets[tl.e + 1],
          "tile rows inside the expert's rows");
    if (tl.nt == 0) rows_covered += tl.rows;
    if (fold) {
      check_range("routed ids read", 0, P, (int64_t)ids.size());
      check_range("offsets written", 0, E + 1, (int64_t)offsets.size());
      check(tl.rows <= 32, "tile rows fit the per-tile pair list");
      const int32_t lo = tl.row0 - offsets[tl.e];
      std::vector<int32_t> src((size_t)tl.rows, -1);
      int32_t matches = 0;
      for (int32_t c0 = 0; c0 < P; c0 += 64)
        for (int lane = 0; lane < 64; ++lane) {
          const int32_t q = c0 + lane;
          if (q >= P || ids[q] != tl.e) continue;
          const int32_t r = matches++ - lo;
          if (r >= 0 && r < tl.rows) {
            check(src[r] < 0, "tile row ranked once");
            src[r] = q;
          }
        }
      for (int32_t r = 0; r < tl.rows; ++r) {
        check(src[r] >= 0 && src[r] < P, "every tile row has a pair in [0, P)");
        if (tl.nt == 0 && src[r] >= 0 && src[r] < P) {
          check_range("src_pair written", tl.row0 + r, tl.row0 + r + 1, P);
          check(inv_written[src[r]]++ == 0, "inv entry written once");
        }
      }
    }
    const int sub = (tl.rows + 31) >> 5;
    const int mba = sub >= sh.mb ? sh.mb : sub;   // occupied 32-row sub-tiles staged

    // ---- B: every wavefront streams two 32-row blocks (inactive ones too)
    for (int wave = 0; wave < sh.waves; ++wave) {
      const WaveBlocks wb = wave_blocks(gemm1, sh.waves, tl.nt, wave, I, N_w);
      for (int j = 0; j < 2; ++j) {
        check(wb.row0[j] >= 0 && wb.row0[j] + 32 <= N_w, "weight block inside the expert");
        for (int lane = 0; lane < 64; ++lane) {
          const int64_t cb = b_codes_offset(tl.e, N_w, wb.row0[j], K, lane);
          check_range("B codes", cb + b_codes_step(0, bk),
                      cb + b_codes_step(nk - 1, bk) + 1024 * (bk / 64 - 1) + 16, w_codes_bytes);
          const int64_t sb = b_scales_offset(tl.e, N_w, wb.row0[j], K, lane, bk, mx);
          check_range("B scales", sb + b_scales_step(0, bk, mx),
                      sb + b_scales_step(nk - 1, bk, mx) + b_scale_bytes(bk, mx), w_sf_bytes);
        }
      }
      // ---- outputs of active wavefronts, rows < tile rows
      if (!wb.active) continue;
      if (gemm1) {
        check(wb.hc0 + 32 <= I, "h column block inside I");
        for (int row = 0; row < tl.rows; ++row)
          for (int ccol = 0; ccol < 32; ccol += 31) {
            const int32_t col = tl.nt * 32 * sh.waves + 32 * wave + ccol;
            const int64_t p = tl.row0 + row;
            check_range("C1 gate dump", row_major(p, 2 * I, col), row_major(p, 2 * I, col) + 1,
                        c1_elems);
            check_range("C1 up dump", row_major(p, 2 * I, I + col),
                        row_major(p, 2 * I, I + col) + 1, c1_elems);
            check_range("h dump", row_major(p, I, col), row_major(p, I, col) + 1, h_elems);
          }
      } else {
        for (int row = 0; row < tl.rows; ++row)
          for (int c4 = 0; c4 < 64; c4 += 4) {
            const int64_t o = c_offset(tl.row0, row, H, wb.n0, c4);
            check_range("C2", o, o + 4, c_elems);
          }
      }
    }

    // ---- A: staging chunks of the occupied sub-tiles, every K step
    const int ce = a_chunk_elems(c.mode, mba, bk, threads);
    const int cpr = bk / ce, chunks = 32 * mba * cpr;
    for (int ch = 0; ch < chunks; ++ch) {
      const int r = ch / cpr, kc = ch % cpr;
      const int64_t arow = a_row(tl.row0, r, tl.rows);
      check(arow >= tl.row0 && arow < tl.row0 + tl.rows, "staged row belongs to the tile");
      if (w16) {
        // the row index goes through src_pair (a permutation of [0, P)) / k
        // for GEMM1, so it stays below T; the check is the in-row range
        check(arow >= 0 && arow < P, "grouped row in range");
        const int64_t lo = a_rows_offset(0, K, kc, ce) + a_rows_step(0, bk);
        const int64_t hi = a_rows_offset(0, K, kc, ce) + a_rows_step(nk - 1, bk) + ce;
        check_range("A bf16 row", lo, hi, K);
        check_range("A bf16 rows", (a_row_count - 1) * (int64_t)K + lo,
                    (a_row_count - 1) * (int64_t)K + hi, a_row_count * (int64_t)K);
      } else {
        // GEMM1 reads A1 row src_pair[arow] (a permutation of [0, P), so
        // any row of it), GEMM2 reads A2 row arow
        const int64_t rows_read[3] = {arow, 0, (int64_t)P - 1};
        for (int ri = 0; ri < (gemm1 ? 3 : 1); ++ri) {
          const int64_t qrow = rows_read[ri];
          const int64_t co = a_codes_offset(qrow, K, kc, ce, mx);
          check_range("A codes", co + a_codes_step(0, bk),
                      co + a_codes_step(nk - 1, bk) + (mx ? 16 : ce / 2), a_codes_bytes);
          const int64_t so = a_scales_offset(qrow, K, kc, ce, mx);
          check_range("A scales", so + a_scales_step(0, bk, mx),
                      so + a_scales_step(nk - 1, bk, mx) + (mx ? 1 : ce / 16), a_sf_bytes);
        }
      }
    }

    // ---- GEMM1 epilogue: h rows (weight-only) or the A2 requantisation
    if (gemm1) {
      const int32_t hw = 32 * sh.waves, hbase = tl.nt * hw;
      const int piece = w16 ? 8 : mx ? 32 : 16;
      for (int row = 0; row < 32 * mba; ++row)
        for (int b = 0; b < hw / piece; ++b) {
          const int32_t hcol = hbase + piece * b;
          if (!(row < tl.rows && hcol < I)) continue;
          const int64_t p = tl.row0 + row;
          if (w16) {
            const int64_t o = a_rows_offset(p, I, hcol / 8, 8);
            check_range("h rows", o, o + 8, h_elems);
          } else {
            const int64_t o = a_codes_offset(p, I, hcol / piece, piece, mx);
            check_range("A2 codes", o, o + piece / 2, out_codes_bytes);
            const int64_t so = a_scales_offset(p, I, hcol / piece, piece, mx);
            check_range("A2 scales", so, so + 1, out_sf_bytes);
          }
        }
    }
  }
  for (int32_t i = 0; i < total; ++i) check(seen[i] == 1, "every tile visited once");
  check(rows_covered == P, "n-tile 0 covers every grouped row once");
  for (size_t q = 0; q < inv_written.size(); ++q) check(inv_written[q] == 1, "every pair gets inv");
}

}  // namespace

int main() {
  char line[1 << 16];
  int cases = 0;
  while (fgets(line, sizeof line, stdin)) {
    Case c;
    char label[256];
    int n = 0;
    if (sscanf(line, "%255s %d %d %d %d %d %d%n", label, &c.mode, &c.E, &c.H, &c.I, &c.k, &c.T,
               &n) != 7)
      continue;
    c.label = label;
    const char* p = line + n;
    for (int32_t e = 0; e < c.E; ++e) {
      char* end = nullptr;
      const long v = strtol(p, &end, 10);
      if (end == p) {
        fprintf(stderr, "%s: %d counts, expected %d\n", label, e, c.E);
        return 2;
      }
      c.counts.push_back((int32_t)v);
      p = end;
    }
    for (int gemm = 1; gemm <= 2; ++gemm) {
      g_label = c.label + (gemm == 1 ? " w13" : " w2") + " mode " + std::to_string(c.mode);
      const int before = g_failures;
      check_gemm(c, gemm == 1);
      printf("%s: %s\n", g_label.c_str(), g_failures == before ? "in bounds" : "FAILED");
    }
    ++cases;
  }
  if (cases == 0) {
    fprintf(stderr, "no cases\n");
    return 2;
  }
  if (g_failures) {
    fprintf(stderr, "%d failed checks\n", g_failures);
    return 1;
  }
  printf("gemm ranges ok (%d cases)\n", cases);
  return 0;
}
