// Work mapping and index arithmetic of the pack kernel (pack.hip), in one
// place so that a host-side check evaluates the very functions the kernel
// calls (tests/pack_index_check.cpp).
//
// A (row, group) pair p = row * (K/G) + group covers the G contiguous weights
// from weight p * G, i.e. the 16-byte pieces p * G/8 ... p * G/8 + G/8 - 1
// (and the code words of the same indices).  A team of G/32 lanes takes a
// pair, 32 weights per lane: lane l of the team holds the pieces l, l + G/32,
// l + 2G/32 and l + 3G/32.  Wavefront w's teams take the pairs w * T + team
// (T teams per wavefront) and then step by S pairs per sweep; S is a
// multiple of both T and K/G, so the S pairs of a sweep are dealt out once
// each and a lane's group (hence its columns and scales) never changes.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define AWQ_PK_HD __host__ __device__ __forceinline__
#else
#define AWQ_PK_HD inline
#endif

namespace awq {
namespace pidx {

constexpr int kPieces = 4;            // 16-byte pieces (32 weights) per lane and pair
constexpr int64_t kWaves = 2048;      // wavefronts aimed for (8 per compute unit)
constexpr int kWavesPerBlock = 4;     // blocks of 256 threads

AWQ_PK_HD int team_lanes(int G) { return G / (8 * kPieces); }
AWQ_PK_HD int teams_per_wave(int G) { return 64 / team_lanes(G); }

AWQ_PK_HD int64_t gcd(int64_t a, int64_t b) {
  while (b) {
    const int64_t t = a % b;
    a = b;
    b = t;
  }
  return a;
}

struct Plan {
  int64_t pairs_per_sweep;  // S
  int64_t waves;            // S / teams per wavefront
  int64_t blocks;           // ceil(waves / 4)
};

// S = lcm(T, K/G) * m, with m chosen for about kWaves wavefronts and no more
// sweeps' worth of wavefronts than the pairs need.
AWQ_PK_HD Plan plan(int64_t K, int64_t OUT, int G) {
  const int64_t teams = teams_per_wave(G), ng = K / G, pairs = OUT * ng;
  const int64_t unit = teams / gcd(teams, ng) * ng;
  int64_t m = kWaves * teams / unit;
  if (m < 1) m = 1;
  const int64_t need = (pairs + unit - 1) / unit;
  if (m > need) m = need;
  Plan pl;
  pl.pairs_per_sweep = unit * m;
  pl.waves = pl.pairs_per_sweep / teams;
  pl.blocks = (pl.waves + kWavesPerBlock - 1) / kWavesPerBlock;
  return pl;
}

// The first pair of lane `lane` of wavefront `wid`.
AWQ_PK_HD int64_t first_pair(int64_t wid, int lane, int G) {
  return wid * teams_per_wave(G) + lane / team_lanes(G);
}
// Index of the lane's first 16-byte piece of pair p (its code word has the
// same index); the lane's other pieces follow at steps of G/32.
AWQ_PK_HD int64_t piece_index(int64_t p, int lane, int G) {
  return p * (G / 8) + lane % team_lanes(G);
}
// The first column of the lane's first piece of group g.
AWQ_PK_HD int64_t first_column(int64_t g, int lane, int G) {
  return g * G + (int64_t)(lane % team_lanes(G)) * 8;
}
// The lane's first piece in the last row of its group g: loads of sweeps past
// the end are clamped to it.
AWQ_PK_HD int64_t last_piece_index(int64_t pairs, int64_t ng, int64_t g, int lane, int G) {
  return piece_index(pairs - ng + g, lane, G);
}

}  // namespace pidx
}  // namespace awq
