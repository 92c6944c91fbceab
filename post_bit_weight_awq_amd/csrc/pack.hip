// Packing of the chosen codes (esaholic.com "What is AWQ Quantization?",
// pipeline step "INT4 Weight Packing & Export": 4-bit codes in INT32
// containers; dev.to page, quant_config: zero point, groups of 128, 4 bit;
// "AWQ > Salient Weight Preservation", step-size equation).
//
// HBM-bound: 2 bytes of W in, 0.5 + 4/G bytes out per weight.  Per group, in
// binary32 (qmax = 2^b - 1):
//   ws = w * s, step = (max - min) / qmax (1 for a zero range),
//   zero = rint(-min / step), q = clamp(rint(ws / step) + zero, 0, qmax);
// the symmetric variant takes step = max|ws| / 2^(b-1) and zero = 2^(b-1).
// The codes and the zero need the correctly rounded quotients ws / step and
// -min / step.  They are formed as products with 1/step, which lie within
// 2.5 ulp of those quotients; a product and its quotient can round to
// different integers only when the product lies that close to a
// half-integer, so such values (about 1e-5 of them) take the IEEE division.
// The clamp is one median, and the eight codes of a word are gathered by
// exact fp32 multiply-adds (two 16-bit halves).
//
// Work layout (pack_index.h).  A group of G columns takes a team of G/32
// lanes with 32 weights per lane, in four 16-byte pieces, so each of the
// lane's four load instructions reads whole contiguous runs across the team.
// Each wavefront sweeps the pairs p, p + S, p + 2S, ... with S a multiple of
// K/G, so a lane's columns, and the 32 scales it holds in registers, never
// change; two sweeps' loads are in flight while a third is packed.  On the
// 13B-block weights this ran 7-11 % faster than one pair set per launch slot
// with all loads issued first (which held 16 weights per lane and reloaded
// its scales).
#include "awq_device.h"
#include "awq_internal.h"
#include "pack_index.h"

namespace awq {

constexpr int kPackPieces = pidx::kPieces;  // 16-byte pieces (32 weights) per lane and pair
constexpr int kPackDepth = 2;               // sweeps whose loads are in flight

// Minimum and maximum over a team of TL aligned lanes (TL = 1, 2 or 4) by DPP
// lane swaps within the VALU instructions: swap neighbours, then pairs.
// After each step every lane holds the extreme of a set twice as large, so
// all TL lanes end with the team's extreme.  The order of the operands differs
// from lane to lane only in which of two equal-valued zeros may win, and the
// sign of a zero extreme changes none of the outputs (step uses max - min, the
// zero point rounds -min and adds +0).
template <int CTRL, bool MAX>
__device__ __forceinline__ float dpp_extreme(float v) {
  const float o = __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
  return MAX ? fmaxf(v, o) : fminf(v, o);
}
template <int TL, bool MAX>
__device__ __forceinline__ float team_extreme(float v) {
  static_assert(TL == 1 || TL == 2 || TL == 4, "teams of 1, 2 or 4 lanes");
  if constexpr (TL >= 2) v = dpp_extreme<0xB1, MAX>(v);   // quad_perm [1,0,3,2]
  if constexpr (TL >= 4) v = dpp_extreme<0x4E, MAX>(v);   // quad_perm [2,3,0,1]
  return v;
}

// The codes of one lane's 32 weights of a (row, group) pair, packed into
// four words, and the group's step and zero point.  w: the lane's pieces;
// sv: the scales of its 32 columns.
template <int G>
__device__ __forceinline__ void pack_codes(const uint4 (&w)[kPackPieces],
                                           const float (&sv)[8 * kPackPieces], float qmax,
                                           int symmetric, float nz, uint32_t (&word)[kPackPieces],
                                           float& step_out, float& zero_out) {
  constexpr int WPL = 8 * kPackPieces, TL = G / WPL;
  float ws[WPL];
#pragma unroll
  for (int h = 0; h < kPackPieces; ++h) {
    const uint32_t wv[4] = {w[h].x, w[h].y, w[h].z, w[h].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ws[8 * h + 2 * j] = mul_f16_f32<false>(wv[j], sv[8 * h + 2 * j], nz);
      ws[8 * h + 2 * j + 1] = mul_f16_f32<true>(wv[j], sv[8 * h + 2 * j + 1], nz);
    }
  }
  // three-operand chains: the compiler forms v_min3 / v_max3 (products are
  // canonical, so no canonicalizing instructions)
  float mn = fminf(ws[0], ws[1]), mx = fmaxf(ws[0], ws[1]);
#pragma unroll
  for (int j = 2; j < WPL; j += 2) {
    mn = fminf(fminf(mn, ws[j]), ws[j + 1]);
    mx = fmaxf(fmaxf(mx, ws[j]), ws[j + 1]);
  }
  mn = team_extreme<TL, false>(mn);
  mx = team_extreme<TL, true>(mx);
  float step;
  if (symmetric) {
    step = fmaxf(fabsf(mn), fabsf(mx)) / (0.5f * (qmax + 1.0f));
  } else {
    step = (mx - mn) / qmax;
  }
  if (step == 0.0f) step = 1.0f;
  const float inv_step = 1.0f / step;
  // A product v * (1/step) lies within 2.5 ulp of the quotient v / step, so
  // the two can round to different integers only within 2^-21 |x| of a
  // half-integer.  Products round monotonically, so every quotient of the
  // group (the codes' and the zero's) is at most M = max(|min|, |max|) *
  // (1/step) in magnitude: one margin per group, twice that window for the
  // margin's own roundings, flags every such value, and those take the
  // IEEE division.
  const float margin = 0.5f - fmaxf(fabsf(mn), fabsf(mx)) * inv_step * 0x1p-20f;
  float z;
  if (symmetric) {
    z = 0.5f * (qmax + 1.0f);
  } else {
    const float zx = -mn * inv_step;
    z = rintf(zx);
    if (fabsf(zx - z) >= margin) z = rintf(-mn / step);
    z += 0.0f;  // -0 -> +0
  }
  // the largest distance from an integer, one comparison for the lane (a
  // NaN distance is skipped by fmaxf, as it fails the comparison)
  float r[WPL];
  float dmax = 0.0f;
#pragma unroll
  for (int j = 0; j < WPL; ++j) {
    const float xf = ws[j] * inv_step;
    r[j] = rintf(xf);
    dmax = fmaxf(dmax, fabsf(xf - r[j]));
  }
  if (dmax >= margin) {  // rare: take the exact quotient where the margin flags it
    // the products again (the same values), so ws need not stay live
#pragma unroll
    for (int h = 0; h < kPackPieces; ++h) {
      const uint32_t wv[4] = {w[h].x, w[h].y, w[h].z, w[h].w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float v = (j & 1) ? mul_f16_f32<true>(wv[j / 2], sv[8 * h + j], nz)
                                : mul_f16_f32<false>(wv[j / 2], sv[8 * h + j], nz);
        const float xf = v * inv_step;
        if (fabsf(xf - r[8 * h + j]) >= margin) r[8 * h + j] = rintf(v / step);
      }
    }
  }
  // Codes are exact integers 0..qmax in binary32; four of them make the
  // exact 16-bit value q0 + 16 q1 + 256 q2 + 4096 q3, two of those a word.
  // q = clamp(r + z, 0, qmax) = clamp(r, -z, qmax - z) + z, so with the
  // zero point moved out of the clamp the four codes sum to
  // c0 + 16 c1 + 256 c2 + 4096 c3 + 4369 z (c = the clamped r).  For
  // |z| <= 2048 every bound, product and partial sum of that form is an
  // integer below 2^24 in magnitude, so it is exact and saves the add per
  // code; a larger zero point (a narrow group far from zero) adds first.
  if (fabsf(z) <= 2048.0f) {
    const float lo = -z, hi = qmax - z, zz = 4369.0f * z;
#pragma unroll
    for (int h = 0; h < kPackPieces; ++h) {
      float half16[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float* rr = r + 8 * h + 4 * e;
        float acc = med3(rr[0], lo, hi) + zz;
        acc = fmaf(med3(rr[1], lo, hi), 16.0f, acc);
        acc = fmaf(med3(rr[2], lo, hi), 256.0f, acc);
        acc = fmaf(med3(rr[3], lo, hi), 4096.0f, acc);
        half16[e] = acc;
      }
      word[h] = (uint32_t)half16[0] | ((uint32_t)half16[1] << 16);
    }
  } else {
#pragma unroll
    for (int h = 0; h < kPackPieces; ++h) {
      float half16[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float* rr = r + 8 * h + 4 * e;
        float acc = med3(rr[0] + z, 0.0f, qmax);
        acc = fmaf(med3(rr[1] + z, 0.0f, qmax), 16.0f, acc);
        acc = fmaf(med3(rr[2] + z, 0.0f, qmax), 256.0f, acc);
        acc = fmaf(med3(rr[3] + z, 0.0f, qmax), 4096.0f, acc);
        half16[e] = acc;
      }
      word[h] = (uint32_t)half16[0] | ((uint32_t)half16[1] << 16);
    }
  }
  step_out = step;
  zero_out = z;
}

// S: pairs per sweep (a multiple of K/G and of the teams per wavefront);
// n_waves = S / teams per wavefront.  Blocks of four wavefronts; a wavefront
// past n_waves, or a team whose first pair is past the end, has no work.  At
// 174 registers two wavefronts share a SIMD, so the 2048 of a launch are all
// resident at once.
template <int G>
__global__ void __launch_bounds__(256)
k_pack(const uint4* __restrict__ W, const float* __restrict__ s, int64_t OUT, int64_t K,
       float qmax, int symmetric, uint32_t* __restrict__ qweight, _Float16* __restrict__ step16,
       _Float16* __restrict__ zero16, int64_t S, int64_t n_waves) {
  constexpr int TL = G / (8 * kPackPieces);  // lanes per team
  const int64_t ng = K / G, pairs = OUT * ng;
  const int lane = threadIdx.x % kWave;
  const int64_t wid = (int64_t)blockIdx.x * pidx::kWavesPerBlock + threadIdx.x / kWave;
  if (wid >= n_waves) return;
  const int lt = lane % TL;
  int64_t p = pidx::first_pair(wid, lane, G);
  if (p >= pairs) return;
  const int64_t g = p % ng;  // the same for every sweep (S is a multiple of K/G)
  const int64_t k0 = pidx::first_column(g, lane, G);
  // the lane's first piece (and code word), its advance per sweep, and its
  // last in-range value (a load past the end re-reads the lane's piece of
  // the last row; nothing is stored for it)
  int64_t widx = pidx::piece_index(p, lane, G);
  const int64_t wstep = S * (G / 8);
  const int64_t wlast = pidx::last_piece_index(pairs, ng, g, lane, G);
  float sv[8 * kPackPieces];
#pragma unroll
  for (int h = 0; h < kPackPieces; ++h) {
    const float* sp = s + k0 + 8 * TL * h;
    const float4 sa = *(const float4*)sp, sb = *(const float4*)(sp + 4);
    sv[8 * h + 0] = sa.x; sv[8 * h + 1] = sa.y; sv[8 * h + 2] = sa.z; sv[8 * h + 3] = sa.w;
    sv[8 * h + 4] = sb.x; sv[8 * h + 5] = sb.y; sv[8 * h + 6] = sb.z; sv[8 * h + 7] = sb.w;
  }
  uint4 buf[kPackDepth][kPackPieces];
#pragma unroll
  for (int d = 0; d < kPackDepth; ++d) {
    const int64_t wi = min(widx + d * wstep, wlast);
#pragma unroll
    for (int h = 0; h < kPackPieces; ++h) buf[d][h] = W[wi + TL * h];
  }
  const float nz = opaque_neg_zero();
  while (p < pairs) {
#pragma unroll
    for (int d = 0; d < kPackDepth; ++d) {
      if (p < pairs) {
        uint32_t word[kPackPieces];
        float step, z;
        pack_codes<G>(buf[d], sv, qmax, symmetric, nz, word, step, z);
#pragma unroll
        for (int h = 0; h < kPackPieces; ++h) qweight[widx + TL * h] = word[h];
        if (lt == 0) {
          step16[p] = (_Float16)step;
          zero16[p] = (_Float16)z;
        }
      }
      // this slot's next sweep
      const int64_t wi = min(widx + kPackDepth * wstep, wlast);
#pragma unroll
      for (int h = 0; h < kPackPieces; ++h) buf[d][h] = W[wi + TL * h];
      p += S;
      widx += wstep;
    }
  }
}

hipError_t launch_pack(const void* W, const float* s, int64_t K, int64_t OUT, const QuantSpec& qs,
                       int32_t* qweight, void* step16, void* zero16, hipStream_t stream) {
  const pidx::Plan pl = pidx::plan(K, OUT, qs.group);
  const float qmax = (float)((1 << qs.w_bit) - 1);
  const int sym = qs.zero_point ? 0 : 1;
  const dim3 grid((unsigned)pl.blocks);
  const uint4* Wv = (const uint4*)W;
  uint32_t* qw = (uint32_t*)qweight;
  _Float16* st = (_Float16*)step16;
  _Float16* zr = (_Float16*)zero16;
  if (qs.group == 32)
    hipLaunchKernelGGL(k_pack<32>, grid, dim3(256), 0, stream, Wv, s, OUT, K, qmax, sym, qw, st,
                       zr, pl.pairs_per_sweep, pl.waves);
  else if (qs.group == 64)
    hipLaunchKernelGGL(k_pack<64>, grid, dim3(256), 0, stream, Wv, s, OUT, K, qmax, sym, qw, st,
                       zr, pl.pairs_per_sweep, pl.waves);
  else
    hipLaunchKernelGGL(k_pack<128>, grid, dim3(256), 0, stream, Wv, s, OUT, K, qmax, sym, qw, st,
                       zr, pl.pairs_per_sweep, pl.waves);
  return hipGetLastError();
}

}  // namespace awq
