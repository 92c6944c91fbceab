// Work-unit mapping and per-lane load offsets of the grid kernels (the fused
// kernels of search_grid.hip and the contraction of search_gemm.hip), written
// once for the device code and for a host-side range check.  The kernels address their loads as a wavefront-uniform 64-bit
// base plus a per-lane 32-bit offset; every offset below is computed in 32
// bits, and the host check evaluates them at the largest shapes the library
// accepts to show none of them wraps or leaves its buffer.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define AWQ_HD __host__ __device__ __forceinline__
#else
#define AWQ_HD inline
#endif

namespace awq {
namespace gidx {

AWQ_HD int imin(int a, int b) { return a < b ? a : b; }

// One block's work: grid point ai of tile T = tt * n_o_tiles + ot, token rows
// from t0 (BM of them, or the half h of a split 2*BM-token tile) and output
// rows from o0.  Whole tiles take one block per unit; a split launch gives
// blocks b and b + 8 (same XCD) the two token halves of unit
// unit_base + b % 8 + 8 (b / 16).  The j-th unit an XCD receives (block b runs
// on XCD b % 8) is grid point j % n_grid of tile 8 (j / n_grid) + xcd.
struct Unit {
  int ai, T, tt, ot, t0, o0, h;
};

AWQ_HD Unit unit_of_block(int b, int unit_base, int split, int n_grid, int n_o_tiles, int BM) {
  Unit r;
  const int u = unit_base + (split == 1 ? b : (b & 7) + 8 * (b >> 4));
  r.h = split == 1 ? 0 : (b >> 3) & 1;
  const int jb = u >> 3;
  r.ai = jb % n_grid;
  r.T = (jb / n_grid) * 8 + (u & 7);
  r.tt = r.T / n_o_tiles;
  r.ot = r.T - r.tt * n_o_tiles;
  r.t0 = r.tt * BM * split + r.h * BM;
  r.o0 = r.ot * 128;
  return r;
}

// ---- k_grid_pp (8 wavefronts; rows of 64-column chunks, whole-line loads)
// Byte offset from the tile's first activation row of lane `lane`'s piece of
// load i of wavefront `wave` (WMT rows per wavefront); the 16-byte piece p of
// row r sits at position p ^ (r & 7).
AWQ_HD uint32_t pp_act_offset(int t0, int N, int K, int wave, int WMT, int i, int lane) {
  const int r = 8 * i + (lane >> 3);
  const int row = imin(t0 + wave * WMT + r, N - 1) - t0;
  return 2u * ((uint32_t)row * (uint32_t)K + 8 * ((lane & 7) ^ (r & 7)));
}
// Byte offset from the tile's first weight row of weight load i (0, 1) of
// piece pc of wavefront group grp.
AWQ_HD uint32_t pp_w_offset(int o0, int OUT, int K, int grp, int pc, int i, int lane) {
  const int r = 64 * grp + 16 * pc + 8 * i + (lane >> 3);
  const int go = imin(o0 + r, OUT - 1) - o0;
  return 2u * ((uint32_t)go * (uint32_t)K + 8 * ((lane & 7) ^ (r & 7)));
}
// Byte offset of the lane's 16-byte group-parameter record within one
// (grid point, column group) slice of the table [grid point][group][row].
AWQ_HD uint32_t pp_param_offset(int o0, int OUT, int grp, int lane) {
  return 16u * (uint32_t)imin(o0 + 64 * grp + lane, OUT - 1);
}
// Byte offset from a column group's first scale of the lane's 16 bytes: lanes
// 0 .. GC/4-1 the group's GC scales, the next GC/4 lanes its reciprocals
// (reached through inv_minus_s, the distance in bytes from the scale table to
// the reciprocal table), further lanes repeating them.
AWQ_HD uint32_t pp_scale_offset(int lane, int GC, uint32_t inv_minus_s) {
  const int sl4 = lane % (GC / 2);
  return 16 * (sl4 % (GC / 4)) + (sl4 < GC / 4 ? 0u : inv_minus_s);
}

// ---- k_grid (4 wavefronts on the 128-token tile; fragment-shaped loads)
// Element offset from the tile's first activation row of the lane's A
// fragment m (16 rows x 64 bytes per fragment load).
AWQ_HD uint32_t g_act_offset(int t0, int N, int K, int wave, int WMT, int m, int lane) {
  const int row = imin(t0 + wave * WMT + m * 16 + (lane & 15), N - 1) - t0;
  return (uint32_t)row * (uint32_t)K + 8 * (lane >> 4);
}
// Element offset from the tile's first weight row of thread tid's raw-weight
// load j (NT threads, four per 64-byte row segment).
AWQ_HD uint32_t g_w_offset(int o0, int OUT, int K, int tid, int NT, int j) {
  const int go = imin(o0 + (tid >> 2) + (NT / 4) * j, OUT - 1) - o0;
  return (uint32_t)go * (uint32_t)K + 8 * (tid & 3);
}
// Record offset (in records) from the tile's first row of the parameters of
// produced row prow0 + (NT / 4) j.
AWQ_HD uint32_t g_param_offset(int o0, int OUT, int prow0, int NT, int j) {
  return (uint32_t)(imin(o0 + prow0 + (NT / 4) * j, OUT - 1) - o0);
}

// ---- k_grid_gemm (8 wavefronts; 256 x 256 tiles of the produced weight
// error, K steps of 64 columns, whole-line loads)
// Blocks run on XCD b % 8.  The pairs (grid point, output tile), pair index =
// grid point * no + output tile, are dealt to the XCDs (pair 8 m + xcd is the
// XCD's m-th), and an XCD's j-th block takes a unit of its pairs in groups of
// 4: group j / (4 nt), and within the group, runs of up to 8 token tiles
// (the last run ragged) whose units go token tile fastest, so the 32 blocks
// an XCD holds at a time share the group's weight-error tiles and the run's
// activation tiles in its L2.  Every block has work, but for the last group's
// units of a pair that an XCD lacks (when the pairs are not a multiple of 8):
// idle blocks in a fixed pattern (runs padded to 8 tiles) loaded some shader
// engines twice as much as others on layers of 5-7 token tiles.
struct GemmUnit {
  int pair, ai, ot, tt, t0, o0;
};
constexpr int kGemmRunTiles = 8;    // token tiles per run
constexpr int kGemmGroupPairs = 4;  // pairs per group
AWQ_HD int gemm_blocks(int nt, int pairs) { return (pairs + 7) / 8 * nt * 8; }
AWQ_HD GemmUnit gemm_unit_of_block(int b, int nt, int no, int pairs) {
  constexpr int T = kGemmRunTiles, P = kGemmGroupPairs;
  const int j = b >> 3, ppx = (pairs + 7) / 8;
  const int g = j / (P * nt), q = j - g * P * nt;
  const int pc = imin(P, ppx - g * P);  // pairs of this group
  const int tb = q / (pc * T), r = q - tb * pc * T;
  const int tc = imin(T, nt - tb * T);  // token tiles of this run
  const int p = r / tc;
  GemmUnit u;
  u.tt = tb * T + (r - p * tc);
  u.pair = (g * P + p) * 8 + (b & 7);
  u.ai = u.pair / no;
  u.ot = u.pair - u.ai * no;
  u.t0 = u.tt * 256;
  u.o0 = u.ot * 256;
  return u;
}
// Byte offset, from the first row of a 256-row tile, of the lane's 16-byte
// piece of load i of wavefront w (8 rows x 128 bytes per load, row r of the
// tile's rows clamped to the layer's last row, piece p stored at p ^ (r & 7)).
AWQ_HD uint32_t gemm_offset(int row0, int rows, int K, int w, int loads_per_wave, int i,
                            int lane) {
  const int r = (w * loads_per_wave + i) * 8 + (lane >> 3);
  const int row = imin(row0 + r, rows - 1) - row0;
  return 2u * ((uint32_t)row * (uint32_t)K + 8 * ((lane & 7) ^ (r & 7)));
}

}  // namespace gidx
}  // namespace awq
