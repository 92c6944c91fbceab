// Packing of the chosen codes (esaholic.com "What is AWQ Quantization?",
// pipeline step "INT4 Weight Packing & Export": 4-bit codes in INT32
// containers; dev.to page, quant_config: zero point, groups of 128, 4 bit;
// "AWQ > Salient Weight Preservation", step-size equation).
//
// HBM-bound: 2 bytes of W in, 0.5 + 4/G bytes out per weight.  A team of G/16
// lanes owns a (row, group of G columns) at a time; each lane loads its 16
// weights with two 16-byte loads, so a wavefront streams 2 KiB of W per pair
// set it holds, and the per-group work (reductions, divisions) is spread over
// 16 weights per lane.  Per group, in binary32 (qmax = 2^b - 1):
//   ws = w * s, step = (max - min) / qmax (1 for a zero range),
//   zero = rint(-min / step), q = clamp(rint(ws / step) + zero, 0, qmax);
// the symmetric variant takes step = max|ws| / 2^(b-1) and zero = 2^(b-1).
// The codes and the zero need the correctly rounded quotients ws / step and
// -min / step.  They are formed as products with 1/step, which lie within
// 2.5 ulp of those quotients; a product and its quotient can round to
// different integers only when the product lies that close to a
// half-integer, so such values (about 1e-5 of them) take the IEEE division.
// The clamp is one median, and the eight codes of a lane are gathered into
// its 32-bit word by exact fp32 multiply-adds (two 16-bit halves).
#include "awq_device.h"
#include "awq_internal.h"

namespace awq {

// Each team takes kPackPerTeam (row, group) pairs, a block's worth of teams
// apart, and issues all their loads before any arithmetic.  A group of G
// columns takes a team of G/16 lanes, 16 weights per lane: lane l of the team
// holds the 16-byte pieces l and l + G/16 of the group, so each of its two
// load instructions reads whole contiguous runs across the team.  The code
// range and zero follow the quantizer settings: qmax = 2^b - 1, and either
// step = (max - min) / qmax with zero = rint(-min/step), or (symmetric)
// step = max|w| / 2^(b-1) with zero = 2^(b-1).
constexpr int kPackPerTeam = 2;

template <int G>
__global__ void __launch_bounds__(256)
k_pack(const uint4* __restrict__ W, const float* __restrict__ s, int64_t OUT, int64_t K,
       float qmax, int symmetric, uint32_t* __restrict__ qweight, _Float16* __restrict__ step16,
       _Float16* __restrict__ zero16) {
  constexpr int TL = G / 16;             // lanes per team
  constexpr int TEAMS = 256 / TL;        // teams per block
  const int64_t ng = K / G;
  const int64_t pairs = OUT * ng;
  const int lt = threadIdx.x % TL;
  const int64_t p0 = (int64_t)blockIdx.x * (TEAMS * kPackPerTeam) + threadIdx.x / TL;
  uint4 w[kPackPerTeam][2];
  int64_t k0[kPackPerTeam], widx[kPackPerTeam];
#pragma unroll
  for (int u = 0; u < kPackPerTeam; ++u) {
    const int64_t p = min(p0 + TEAMS * u, pairs - 1);  // a tail team re-reads the last pair
    const int64_t o = p / ng, g = p - o * ng;
    k0[u] = g * G + lt * 8;            // first column of the lane's first piece
    widx[u] = (o * K + k0[u]) / 8;     // its 16-byte (and 8-code word) index
    w[u][0] = W[widx[u]];
    w[u][1] = W[widx[u] + TL];
  }
  const float nz = opaque_neg_zero();
#pragma unroll
  for (int u = 0; u < kPackPerTeam; ++u) {
    float ws[16];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float* sp = s + k0[u] + 8 * TL * h;
      const float4 sa = *(const float4*)sp, sb = *(const float4*)(sp + 4);
      const float sv[8] = {sa.x, sa.y, sa.z, sa.w, sb.x, sb.y, sb.z, sb.w};
      const uint32_t wv[4] = {w[u][h].x, w[u][h].y, w[u][h].z, w[u][h].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ws[8 * h + 2 * j] = mul_f16_f32<false>(wv[j], sv[2 * j], nz);
        ws[8 * h + 2 * j + 1] = mul_f16_f32<true>(wv[j], sv[2 * j + 1], nz);
      }
    }
    // three-operand chains: the compiler forms v_min3 / v_max3 (products are
    // canonical, so no canonicalizing instructions)
    float mn = fminf(ws[0], ws[1]), mx = fmaxf(ws[0], ws[1]);
#pragma unroll
    for (int j = 2; j < 16; j += 2) {
      mn = fminf(fminf(mn, ws[j]), ws[j + 1]);
      mx = fmaxf(fmaxf(mx, ws[j]), ws[j + 1]);
    }
#pragma unroll
    for (int d = TL / 2; d >= 1; d >>= 1) {
      mn = fminf(mn, __shfl_xor(mn, d, TL));
      mx = fmaxf(mx, __shfl_xor(mx, d, TL));
    }
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
    float r[16];
    bool redo = false;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float xf = ws[j] * inv_step;
      r[j] = rintf(xf);
      redo |= fabsf(xf - r[j]) >= margin;
    }
    if (redo) {  // rare: take the exact quotient where the margin flags it
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float xf = ws[j] * inv_step;
        if (fabsf(xf - r[j]) >= margin) r[j] = rintf(ws[j] / step);
      }
    }
    // codes are exact integers 0..qmax in binary32; four of them make the
    // exact 16-bit value q0 + 16 q1 + 256 q2 + 4096 q3, two of those a word
    uint32_t word[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
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
    const int64_t p = p0 + TEAMS * u;
    if (p < pairs) {
      qweight[widx[u]] = word[0];
      qweight[widx[u] + TL] = word[1];
      if (lt == 0) {
        step16[p] = (_Float16)step;
        zero16[p] = (_Float16)z;
      }
    }
  }
}

hipError_t launch_pack(const void* W, const float* s, int64_t K, int64_t OUT, const QuantSpec& qs,
                       int32_t* qweight, void* step16, void* zero16, hipStream_t stream) {
  const int64_t pairs = OUT * (K / qs.group);
  const float qmax = (float)((1 << qs.w_bit) - 1);
  const int sym = qs.zero_point ? 0 : 1;
  const int per_block = 256 / (qs.group / 16) * kPackPerTeam;
  const dim3 grid((unsigned)((pairs + per_block - 1) / per_block));
  const uint4* Wv = (const uint4*)W;
  uint32_t* qw = (uint32_t*)qweight;
  _Float16* st = (_Float16*)step16;
  _Float16* zr = (_Float16*)zero16;
  if (qs.group == 32)
    hipLaunchKernelGGL(k_pack<32>, grid, dim3(256), 0, stream, Wv, s, OUT, K, qmax, sym, qw, st, zr);
  else if (qs.group == 64)
    hipLaunchKernelGGL(k_pack<64>, grid, dim3(256), 0, stream, Wv, s, OUT, K, qmax, sym, qw, st, zr);
  else
    hipLaunchKernelGGL(k_pack<128>, grid, dim3(256), 0, stream, Wv, s, OUT, K, qmax, sym, qw, st,
                       zr);
  return hipGetLastError();
}

}  // namespace awq
