// Host-side check of the pack kernel's work mapping and index arithmetic
// (post_bit_weight_awq_amd/csrc/pack_index.h, the functions the kernel
// calls).  For every group size and shapes up to the largest the library
// accepts (in/out features <= 2^20, in * out <= 2^34) it checks that
//   * the plan's sweep S is a multiple of the teams per wavefront and of the
//     groups per row, its wavefronts deal out each pair of a sweep once, and
//     the grid fits a launch;
//   * every lane's loads (clamped to its last in-range piece) and stores lie
//     inside W / qweight, and its scale reads inside s;
// and, on shapes small enough to enumerate, it runs the kernel's loop on the
// host and checks that every (row, group) pair is packed exactly once, by a
// team whose lanes hold each of its pieces once.  Prints "ok" and exits 0, or
// prints the first violations and exits 1.
#include <stdint.h>
#include <stdio.h>

#include <vector>

#include "pack_index.h"

using namespace awq::pidx;

static int fails = 0;
#define CHECK(cond, ...)                      \
  do {                                        \
    if (!(cond)) {                            \
      if (fails++ < 10) {                     \
        printf("violation: %s: ", #cond);     \
        printf(__VA_ARGS__);                  \
        printf("\n");                         \
      }                                       \
    }                                         \
  } while (0)

// Bounds of every lane's first pair in a launch (closed form: the lanes of
// wavefront w start at w * T ... w * T + T - 1).
static void check_plan(int64_t K, int64_t OUT, int G) {
  const Plan pl = plan(K, OUT, G);
  const int64_t T = teams_per_wave(G), TL = team_lanes(G), ng = K / G, pairs = OUT * ng;
  const int64_t S = pl.pairs_per_sweep;
  CHECK(S > 0 && S % T == 0 && S % ng == 0, "K=%lld OUT=%lld G=%d S=%lld", (long long)K,
        (long long)OUT, G, (long long)S);
  CHECK(pl.waves * T == S, "K=%lld OUT=%lld G=%d", (long long)K, (long long)OUT, G);
  CHECK(pl.blocks * kWavesPerBlock >= pl.waves && (pl.blocks - 1) * kWavesPerBlock < pl.waves,
        "K=%lld OUT=%lld G=%d", (long long)K, (long long)OUT, G);
  CHECK(pl.blocks >= 1 && pl.blocks < ((int64_t)1 << 31), "blocks %lld", (long long)pl.blocks);
  CHECK(S < pairs + T * ng, "S %lld for %lld pairs", (long long)S, (long long)pairs);
  const int64_t pieces = pairs * (G / 8);  // 16-byte pieces of W = code words
  // the extreme lanes: first and last lane of the first and last wavefront
  const int64_t wids[2] = {0, pl.waves - 1};
  for (int64_t wid : wids)
    for (int lane : {0, (int)TL - 1, 63 - (int)TL + 1, 63}) {
      const int64_t p = first_pair(wid, lane, G);
      CHECK(p >= 0 && p < S, "first pair %lld of S %lld", (long long)p, (long long)S);
      if (p >= pairs) continue;  // that team has no work
      const int64_t g = p % ng;
      const int64_t k0 = first_column(g, lane, G);
      CHECK(k0 >= 0 && k0 + 8 * TL * (kPieces - 1) + 8 <= K, "scale column %lld of %lld",
            (long long)k0, (long long)K);
      const int64_t w0 = piece_index(p, lane, G), wl = last_piece_index(pairs, ng, g, lane, G);
      CHECK(w0 >= 0 && w0 <= wl, "first piece %lld last %lld", (long long)w0, (long long)wl);
      CHECK(wl + TL * (kPieces - 1) < pieces, "last piece %lld + %lld of %lld", (long long)wl,
            (long long)(TL * (kPieces - 1)), (long long)pieces);
    }
}

// The kernel's loop on the host: every pair once, every piece of a packed
// pair held by exactly one lane of its team, loads and stores in bounds.
static void enumerate(int64_t K, int64_t OUT, int G) {
  const Plan pl = plan(K, OUT, G);
  const int64_t TL = team_lanes(G), ng = K / G, pairs = OUT * ng, pieces = pairs * (G / 8);
  const int64_t S = pl.pairs_per_sweep, wstep = S * (G / 8);
  const int depth = 2;
  std::vector<uint8_t> pair_seen(pairs, 0), piece_seen(pieces, 0);
  for (int64_t wid = 0; wid < pl.blocks * kWavesPerBlock; ++wid) {
    if (wid >= pl.waves) continue;
    for (int lane = 0; lane < 64; ++lane) {
      int64_t p = first_pair(wid, lane, G);
      if (p >= pairs) continue;
      const int64_t g = p % ng;
      int64_t widx = piece_index(p, lane, G);
      const int64_t wlast = last_piece_index(pairs, ng, g, lane, G);
      for (int d = 0; d < depth; ++d) {
        const int64_t wi = widx + d * wstep < wlast ? widx + d * wstep : wlast;
        CHECK(wi >= 0 && wi + TL * (kPieces - 1) < pieces, "load %lld", (long long)wi);
      }
      while (p < pairs) {
        for (int d = 0; d < depth; ++d) {
          if (p < pairs) {
            CHECK(p % ng == g, "group changed: pair %lld", (long long)p);
            CHECK(widx == piece_index(p, lane, G), "piece index drift at pair %lld", (long long)p);
            if (lane % TL == 0) pair_seen[p]++;
            for (int h = 0; h < kPieces; ++h) {
              const int64_t q = widx + TL * h;
              CHECK(q >= p * (G / 8) && q < (p + 1) * (G / 8), "piece %lld outside pair %lld",
                    (long long)q, (long long)p);
              piece_seen[q]++;
            }
          }
          const int64_t wi = widx + depth * wstep < wlast ? widx + depth * wstep : wlast;
          CHECK(wi >= 0 && wi + TL * (kPieces - 1) < pieces, "load %lld", (long long)wi);
          p += S;
          widx += wstep;
        }
      }
    }
  }
  for (int64_t p = 0; p < pairs; ++p)
    CHECK(pair_seen[p] == 1, "K=%lld OUT=%lld G=%d pair %lld packed %d times", (long long)K,
          (long long)OUT, G, (long long)p, pair_seen[p]);
  for (int64_t q = 0; q < pieces; ++q)
    CHECK(piece_seen[q] == 1, "K=%lld OUT=%lld G=%d piece %lld held %d times", (long long)K,
          (long long)OUT, G, (long long)q, piece_seen[q]);
}

int main() {
  int shapes = 0;
  const int64_t Ks[] = {128, 256, 384, 512, 640, 1024, 1280, 4096, 5120, 10368, 11008, 13824,
                        27648, 65536, 1 << 20};
  const int64_t OUTs[] = {1, 2, 3, 7, 48, 64, 77, 200, 300, 513, 1000, 4096, 5120, 12288, 27648,
                          65537, 1 << 20};
  for (int G : {32, 64, 128})
    for (int64_t K : Ks)
      for (int64_t OUT : OUTs) {
        if (K * OUT > ((int64_t)1 << 34)) continue;
        check_plan(K, OUT, G);
        ++shapes;
        if (K * OUT <= ((int64_t)1 << 24)) enumerate(K, OUT, G);
      }
  if (fails) {
    printf("%d violations\n", fails);
    return 1;
  }
  printf("ok: %d shapes\n", shapes);
  return 0;
}
