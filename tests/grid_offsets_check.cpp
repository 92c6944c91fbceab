// Host-side range check of the grid kernels' work-unit mapping and 32-bit
// per-lane load offsets (post_bit_weight_awq_amd/csrc/grid_index.h, the same
// functions the kernels call: the fused kernels and the contraction).  For
// shapes up to the largest the library accepts (tokens <= 2^24, in/out
// features <= 2^20, in*out <= 2^34, grid launches <= 2^23 blocks) it checks
// that
//   * every offset equals its exact 64-bit value (no 32-bit wrap) and every
//     16-byte load it addresses lies inside its buffer, on the first and last
//     token and output tiles of every kernel form;
//   * the blocks of a launch that pass the kernels' early returns cover each
//     (grid point, tile) unit exactly once (each token half once when split),
//     with the tile's first token and output row inside the layer.
// Prints "ok" and exits 0, or prints the first violation and exits 1.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "grid_index.h"

using namespace awq::gidx;

static int fails = 0;
#define CHECK(cond, ...)                                  \
  do {                                                    \
    if (!(cond)) {                                        \
      if (fails++ < 10) {                                 \
        printf("violation: %s: ", #cond);                 \
        printf(__VA_ARGS__);                              \
        printf("\n");                                     \
      }                                                   \
    }                                                     \
  } while (0)

static int64_t align256(int64_t v) { return (v + 255) / 256 * 256; }
static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// k_grid_pp<BM>: offsets of the tile starting at token t0 and output o0
static void check_pp_tile(int BM, int t0, int o0, int64_t N, int64_t K, int64_t OUT, int n_grid,
                          int GC) {
  const int WMT = BM / 8, ALD = WMT / 8;
  const int64_t nch = K / 64;
  const int64_t x_bytes = 2 * N * K, w_bytes = 2 * OUT * K;
  for (int wave = 0; wave < 8; ++wave)
    for (int lane = 0; lane < 64; ++lane) {
      for (int i = 0; i < ALD; ++i) {
        const uint32_t off = pp_act_offset(t0, (int)N, (int)K, wave, WMT, i, lane);
        const int r = 8 * i + (lane >> 3);
        int64_t row = t0 + wave * WMT + r;
        if (row > N - 1) row = N - 1;
        const int64_t exact = 2 * ((row - t0) * K + 8 * ((lane & 7) ^ (r & 7)));
        CHECK((int64_t)off == exact, "pp act N=%lld K=%lld t0=%d w%d l%d i%d", (long long)N,
              (long long)K, t0, wave, lane, i);
        const int64_t last = 2 * t0 * K + (nch - 1) * 128 + exact + 16;
        CHECK(last <= x_bytes, "pp act end N=%lld K=%lld t0=%d", (long long)N, (long long)K, t0);
      }
      const int grp = wave >> 2, pc = wave & 3;
      for (int i = 0; i < 2; ++i) {
        const uint32_t off = pp_w_offset(o0, (int)OUT, (int)K, grp, pc, i, lane);
        const int r = 64 * grp + 16 * pc + 8 * i + (lane >> 3);
        int64_t go = o0 + r;
        if (go > OUT - 1) go = OUT - 1;
        const int64_t exact = 2 * ((go - o0) * K + 8 * ((lane & 7) ^ (r & 7)));
        CHECK((int64_t)off == exact, "pp w OUT=%lld K=%lld o0=%d", (long long)OUT, (long long)K, o0);
        CHECK(2 * o0 * K + (nch - 1) * 128 + exact + 16 <= w_bytes, "pp w end OUT=%lld o0=%d",
              (long long)OUT, o0);
      }
      // group parameters: [grid point][group][row] records of 16 bytes
      const int64_t ngroups = K / GC;
      const uint32_t poff = pp_param_offset(o0, (int)OUT, grp, lane);
      int64_t prow = o0 + 64 * grp + lane;
      if (prow > OUT - 1) prow = OUT - 1;
      CHECK((int64_t)poff == 16 * prow, "pp param");
      const int64_t pend = ((int64_t)(n_grid - 1) * ngroups + (ngroups - 1)) * OUT * 16 + poff + 16;
      CHECK(pend <= (int64_t)n_grid * ngroups * OUT * 16, "pp param end");
      // scales: the scale table [n_grid][K] floats, then the reciprocal table
      // on the next 256-byte boundary
      const int64_t inv_minus_s = align256(4 * (int64_t)n_grid * K);
      CHECK(inv_minus_s < ((int64_t)1 << 32), "scale table distance");
      const uint32_t soff = pp_scale_offset(lane, GC, (uint32_t)inv_minus_s);
      const int sl4 = lane % (GC / 2);
      const int64_t sexact = 16 * (sl4 % (GC / 4)) + (sl4 < GC / 4 ? 0 : inv_minus_s);
      CHECK((int64_t)soff == sexact, "pp scale");
      const int64_t send = 4 * ((int64_t)(n_grid - 1) * K + (ngroups - 1) * GC) + soff + 16;
      CHECK(send <= inv_minus_s + 4 * (int64_t)n_grid * K, "pp scale end");
      CHECK(sl4 < GC / 4 ? send <= 4 * (int64_t)n_grid * K : send > inv_minus_s, "pp scale table");
    }
}

// k_grid<128, 128, 4, GS>: offsets of the tile starting at t0, o0
static void check_g_tile(int t0, int o0, int64_t N, int64_t K, int64_t OUT) {
  const int BM = 128, NW = 4, NT = 256, WMT = BM / NW, MBW = WMT / 16, PR = 128 * 4 / NT;
  const int64_t nk = K / 32;
  for (int tid = 0; tid < NT; ++tid) {
    const int lane = tid & 63, wave = tid >> 6;
    for (int m = 0; m < MBW; ++m) {
      const uint32_t off = g_act_offset(t0, (int)N, (int)K, wave, WMT, m, lane);
      int64_t row = t0 + wave * WMT + m * 16 + (lane & 15);
      if (row > N - 1) row = N - 1;
      const int64_t exact = (row - t0) * K + 8 * (lane >> 4);
      CHECK((int64_t)off == exact, "g act N=%lld K=%lld t0=%d", (long long)N, (long long)K, t0);
      CHECK(t0 * K + exact + (nk - 1) * 32 + 8 <= N * K, "g act end");
    }
    for (int j = 0; j < PR; ++j) {
      const uint32_t off = g_w_offset(o0, (int)OUT, (int)K, tid, NT, j);
      int64_t go = o0 + (tid >> 2) + (NT / 4) * j;
      if (go > OUT - 1) go = OUT - 1;
      const int64_t exact = (go - o0) * K + 8 * (tid & 3);
      CHECK((int64_t)off == exact, "g w");
      CHECK(o0 * K + exact + (nk - 1) * 32 + 8 <= OUT * K, "g w end");
      const int prow0 = (wave >> 2) * 64 + lane;
      const uint32_t poff = g_param_offset(o0, (int)OUT, prow0, NT, j);
      int64_t pr = o0 + prow0 + (NT / 4) * j;
      if (pr > OUT - 1) pr = OUT - 1;
      CHECK((int64_t)poff == pr - o0, "g param");
    }
  }
}

// Blocks [0, blocks) of a launch with the given unit base and split: every
// block that passes the early returns has a tile inside the layer; the units
// [unit_base, unit_end) are covered once per token half.  Enumerates every
// block when `all`, else the first and last 4096.
static void check_units(int64_t N, int64_t OUT, int BM, int split, int n_grid, int64_t unit_base,
                        int64_t unit_end, bool all) {
  const int64_t nt = cdiv(N, (int64_t)BM * split), no = cdiv(OUT, 128);
  const int64_t n_tiles = nt * no;
  const int64_t blocks = (unit_end - unit_base) * split;
  std::vector<uint8_t> seen;
  if (all) seen.assign((size_t)((unit_end - unit_base) * 2), 0);
  for (int64_t b = 0; b < blocks; ++b) {
    if (!all && b >= 4096 && b < blocks - 4096) b = blocks - 4096;
    const Unit un = unit_of_block((int)b, (int)unit_base, split, n_grid, (int)no, BM);
    const int64_t u = unit_base + (split == 1 ? b : (b & 7) + 8 * (b >> 4));
    CHECK(u >= unit_base && u < unit_end, "unit %lld outside [%lld, %lld)", (long long)u,
          (long long)unit_base, (long long)unit_end);
    CHECK(un.ai >= 0 && un.ai < n_grid, "grid point");
    if (un.T >= n_tiles) continue;
    CHECK(un.tt >= 0 && un.tt < nt && un.ot >= 0 && un.ot < no, "tile index");
    if (un.t0 >= N) continue;  // the empty second half of a ragged last token tile
    CHECK(un.t0 >= 0 && un.o0 >= 0 && un.o0 < OUT, "tile origin t0=%d o0=%d", un.t0, un.o0);
    if (all) {
      const size_t slot = (size_t)((u - unit_base) * 2 + un.h);
      CHECK(slot < seen.size() && !seen[slot], "unit %lld half %d twice", (long long)u, un.h);
      if (slot < seen.size()) seen[slot] = 1;
    }
  }
  if (all) {
    // every unit whose tile exists (and whose half has rows) was seen
    for (int64_t u = unit_base; u < unit_end; ++u) {
      const int64_t jb = u >> 3, T = (jb / n_grid) * 8 + (u & 7);
      if (T >= n_tiles) continue;
      for (int h = 0; h < split; ++h) {
        const int64_t t0 = (T / no) * BM * split + h * BM;
        if (t0 < N) CHECK(seen[(size_t)((u - unit_base) * 2 + h)], "unit %lld half %d missed", (long long)u, h);
      }
    }
  }
}

// k_grid_gemm: offsets of the 256 x 256 tile starting at token t0 and output
// o0 of grid point ai; the weight error is [n_grid][OUT][K] fp16
static void check_gemm_tile(int t0, int o0, int64_t N, int64_t K, int64_t OUT) {
  const int LOADS = 256 * 64 * 2 / 1024 / 8;
  const int64_t nk = K / 64;
  for (int w = 0; w < 8; ++w)
    for (int lane = 0; lane < 64; ++lane)
      for (int i = 0; i < LOADS; ++i) {
        const int r = (w * LOADS + i) * 8 + (lane >> 3);
        const uint32_t oa = gemm_offset(t0, (int)N, (int)K, w, LOADS, i, lane);
        int64_t row = t0 + r;
        if (row > N - 1) row = N - 1;
        const int64_t ea = 2 * ((row - t0) * K + 8 * ((lane & 7) ^ (r & 7)));
        CHECK((int64_t)oa == ea, "gemm act N=%lld K=%lld t0=%d", (long long)N, (long long)K, t0);
        CHECK(2 * t0 * K + ea + (nk - 1) * 128 + 16 <= 2 * N * K, "gemm act end");
        const uint32_t ob = gemm_offset(o0, (int)OUT, (int)K, w, LOADS, i, lane);
        int64_t orow = o0 + r;
        if (orow > OUT - 1) orow = OUT - 1;
        const int64_t eb = 2 * ((orow - o0) * K + 8 * ((lane & 7) ^ (r & 7)));
        CHECK((int64_t)ob == eb, "gemm dw OUT=%lld K=%lld o0=%d", (long long)OUT, (long long)K, o0);
        CHECK(2 * o0 * K + eb + (nk - 1) * 128 + 16 <= 2 * OUT * K, "gemm dw end");
        CHECK(r < 256, "gemm tile row");
      }
}

// every (pair, token tile) of the contraction launch is taken by exactly one
// block that passes the early return, with its tile inside the layer
static int64_t gemm_blocks64(int64_t nt, int64_t pairs) { return cdiv(pairs, 8) * nt * 8; }

static void check_gemm_units(int64_t N, int64_t OUT, int n_grid, bool all) {
  const int64_t nt = cdiv(N, 256), no = cdiv(OUT, 128 * 2), pairs = n_grid * no;
  const int64_t blocks = gemm_blocks64(nt, pairs);
  CHECK(blocks == gemm_blocks((int)nt, (int)pairs), "gemm block count");
  std::vector<uint8_t> seen;
  if (all) seen.assign((size_t)(pairs * nt), 0);
  for (int64_t b = 0; b < blocks; ++b) {
    if (!all && b >= 4096 && b < blocks - 4096) b = blocks - 4096;
    const GemmUnit un = gemm_unit_of_block((int)b, (int)nt, (int)no, (int)pairs);
    CHECK(un.tt >= 0 && un.tt < nt, "gemm token tile of block %lld", (long long)b);
    if (un.pair >= pairs) {
      // idle blocks only in the last group of 4 pairs (XCDs with a pair fewer)
      const int64_t ppx = cdiv(pairs, 8), first_last = (ppx - 1) / 4 * 4 * nt;
      CHECK(b / 8 >= first_last, "gemm idle block %lld before the last group", (long long)b);
      continue;
    }
    CHECK(un.ai >= 0 && un.ai < n_grid && un.ot >= 0 && un.ot < no && un.tt >= 0 && un.tt < nt,
          "gemm unit %lld", (long long)b);
    CHECK(un.t0 < N && un.o0 < OUT, "gemm tile origin");
    if (all) {
      const size_t slot = (size_t)(un.pair * nt + un.tt);
      CHECK(!seen[slot], "gemm unit twice");
      seen[slot] = 1;
    }
  }
  if (all)
    for (size_t i = 0; i < seen.size(); ++i) CHECK(seen[i], "gemm unit %zu missed", i);
}

int main() {
  const int64_t MAXT = (int64_t)1 << 24, MAXF = (int64_t)1 << 20, MAXW = (int64_t)1 << 34;
  const int64_t MAXBLOCKS = (int64_t)1 << 23;
  const int64_t Ns[] = {1, 127, 128, 129, 255, 256, 257, 511, 512, 513, 1024, 1025, 1500, 2048,
                        2049, 3000, 4096, MAXT - 1, MAXT};
  const int64_t Ks[] = {128, 4096, 13824, MAXF / 2, MAXF};
  const int64_t OUTs[] = {1, 127, 128, 129, 27648, (int64_t)1 << 14, MAXF};
  const int grids[] = {1, 20, 64};
  const int GCs[] = {32, 64, 128};
  int shapes = 0;
  for (int64_t N : Ns)
    for (int64_t K : Ks)
      for (int64_t OUT : OUTs) {
        if (OUT * K > MAXW) continue;
        for (int n_grid : grids)
          for (int BM : {512, 256, 128}) {
            const int64_t nt = cdiv(N, BM), no = cdiv(OUT, 128);
            const int64_t units = cdiv(nt * no, 8) * 8 * n_grid;
            if (units > MAXBLOCKS) continue;  // the plan rejects the layer
            ++shapes;
            const int64_t tts[] = {0, nt - 1}, ots[] = {0, no - 1};
            for (int64_t tt : tts)
              for (int64_t ot : ots) {
                if (BM == 128) {
                  check_g_tile((int)(tt * BM), (int)(ot * 128), N, K, OUT);
                  // the halves of a split 256-token tile (k_grid on 128 rows)
                  const int64_t t2 = cdiv(N, 256);
                  for (int h = 0; h < 2; ++h) {
                    const int64_t t0 = (t2 - 1) * 256 + h * 128;
                    if (t0 < N) check_g_tile((int)t0, (int)(ot * 128), N, K, OUT);
                  }
                } else {
                  for (int GC : GCs) {
                    if (K % GC) continue;
                    check_pp_tile(BM, (int)(tt * BM), (int)(ot * 128), N, K, OUT, n_grid, GC);
                    if (BM == 256) {  // halves of a split 512-token tile
                      const int64_t t5 = cdiv(N, 512);
                      for (int h = 0; h < 2; ++h) {
                        const int64_t t0 = (t5 - 1) * 512 + h * 256;
                        if (t0 < N)
                          check_pp_tile(256, (int)t0, (int)(ot * 128), N, K, OUT, n_grid, GC);
                      }
                    }
                  }
                }
              }
            // unit mapping: the whole launch, and a last round split in token
            // halves (the leftover units from `whole` on, whole a multiple of 8)
            const bool all = units <= ((int64_t)1 << 20);
            check_units(N, OUT, BM, 1, n_grid, 0, units, all);
            if (BM > 128 && units >= 16) {
              const int64_t whole = units / 16 * 8;
              check_units(N, OUT, BM / 2, 2, n_grid, whole, units, all);
            }
          }
      }
  // the contraction path (layers of at least five 256-token tiles)
  for (int64_t N : Ns)
    for (int64_t K : Ks)
      for (int64_t OUT : OUTs) {
        if (OUT * K > MAXW || N < 1025) continue;
        for (int n_grid : grids) {
          const int64_t nt = cdiv(N, 256), no = cdiv(OUT, 256);
          if (gemm_blocks64(nt, n_grid * no) > MAXBLOCKS) continue;
          ++shapes;
          for (int64_t tt : {(int64_t)0, nt - 1})
            for (int64_t ot : {(int64_t)0, no - 1}) check_gemm_tile((int)(tt * 256), (int)(ot * 256), N, K, OUT);
          check_gemm_units(N, OUT, n_grid, n_grid * no * nt <= ((int64_t)1 << 20));
        }
      }
  // the contraction's block order on its own, for any token-tile count (whole
  // and ragged runs of 8 tiles, whole and ragged groups of 4 pairs)
  for (int64_t nt = 1; nt <= 40; ++nt)
    for (int64_t OUT : {(int64_t)1, (int64_t)256, (int64_t)700, (int64_t)5120, (int64_t)15360})
      for (int n_grid : {1, 3, 7, 20, 33, 64}) {
        ++shapes;
        check_gemm_units(nt * 256 - (nt % 3) * 50, OUT, n_grid, true);
      }
  if (fails) {
    printf("%d violations over %d shapes\n", fails, shapes);
    return 1;
  }
  printf("ok: %d shapes\n", shapes);
  return 0;
}
