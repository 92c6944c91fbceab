// Packing of the chosen codes (esaholic.com "What is AWQ Quantization?",
// pipeline step "INT4 Weight Packing & Export": 4-bit codes in INT32
// containers; dev.to page, quant_config: zero point, groups of 128, 4 bit;
// "AWQ > Salient Weight Preservation", step-size equation).
//
// HBM-bound: 2 bytes of W in, 0.5 + 4/G bytes out per weight.  A team of G/8
// lanes owns a (row, group of G columns) at a time; each lane loads its 8
// weights with one 16-byte load, so a wavefront streams 1 KiB of W per pair
// set it holds.  Per group, in binary32 (qmax = 2^b - 1):
//   ws = w * s, step = (max - min) / qmax (1 for a zero range),
//   zero = rint(-min / step), q = clamp(rint(ws / step) + zero, 0, qmax);
// the symmetric variant takes step = max|ws| / 2^(b-1) and zero = 2^(b-1).
// The code needs the correctly rounded quotient ws / step.  It is formed as
// ws * (1/step), which is within 2.5 ulp of that quotient; the two can round
// to different integers only when the product lies that close to a
// half-integer, so such elements (about 1e-5 of them) take the IEEE division.
#include "awq_device.h"
#include "awq_internal.h"

namespace awq {

// Each team takes kPackPerTeam (row, group) pairs, a block's worth of teams
// apart, and issues all their loads before any arithmetic, so every lane
// keeps 32 bytes of W in flight (two pairs measured faster than four or eight
// on the 7B q_proj layer, 16.0 against 17.5 and 20 us, and equal on the 13B
// block: more, smaller blocks start their arithmetic and stores sooner).  A group of G columns takes a team of G/8
// lanes.  The code range and zero follow the quantizer settings: qmax =
// 2^b - 1, and either step = (max - min) / qmax with zero = rint(-min/step),
// or (symmetric) step = max|w| / 2^(b-1) with zero = 2^(b-1).
constexpr int kPackPerTeam = 2;

template <int G>
__global__ void __launch_bounds__(256)
k_pack(const uint4* __restrict__ W, const float* __restrict__ s, int64_t OUT, int64_t K,
       float qmax, int symmetric, uint32_t* __restrict__ qweight, _Float16* __restrict__ step16,
       _Float16* __restrict__ zero16) {
  constexpr int TL = G / 8;              // lanes per team
  constexpr int TEAMS = 256 / TL;        // teams per block
  const int64_t ng = K / G;
  const int64_t pairs = OUT * ng;
  const int lt = threadIdx.x % TL;
  const int64_t p0 = (int64_t)blockIdx.x * (TEAMS * kPackPerTeam) + threadIdx.x / TL;
  uint4 w[kPackPerTeam];
  int64_t k0[kPackPerTeam], widx[kPackPerTeam];
#pragma unroll
  for (int u = 0; u < kPackPerTeam; ++u) {
    const int64_t p = min(p0 + TEAMS * u, pairs - 1);  // a tail team re-reads the last pair
    const int64_t o = p / ng, g = p - o * ng;
    k0[u] = g * G + lt * 8;
    widx[u] = (o * K + k0[u]) / 8;
    w[u] = W[widx[u]];
  }
  const float nz = opaque_neg_zero();
#pragma unroll
  for (int u = 0; u < kPackPerTeam; ++u) {
    const float4 sa = *(const float4*)(s + k0[u]), sb = *(const float4*)(s + k0[u] + 4);
    const float sv[8] = {sa.x, sa.y, sa.z, sa.w, sb.x, sb.y, sb.z, sb.w};
    const uint32_t wv[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
    float ws[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ws[2 * j] = mul_f16_f32<false>(wv[j], sv[2 * j], nz);
      ws[2 * j + 1] = mul_f16_f32<true>(wv[j], sv[2 * j + 1], nz);
    }
    float mn = ws[0], mx = ws[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) {
      mn = fminf(mn, ws[j]);
      mx = fmaxf(mx, ws[j]);
    }
#pragma unroll
    for (int d = TL / 2; d >= 1; d >>= 1) {
      mn = fminf(mn, __shfl_xor(mn, d, TL));
      mx = fmaxf(mx, __shfl_xor(mx, d, TL));
    }
    float step, z;
    if (symmetric) {
      const float half = 0.5f * (qmax + 1.0f);
      step = fmaxf(fabsf(mn), fabsf(mx)) / half;
      if (step == 0.0f) step = 1.0f;
      z = half;
    } else {
      step = (mx - mn) / qmax;
      if (step == 0.0f) step = 1.0f;
      z = rintf(-mn / step) + 0.0f;
    }
    const float inv_step = 1.0f / step;
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float xf = ws[j] * inv_step;
      float r = rintf(xf);
      // near a half-integer: redo with the exact quotient
      if (0.5f - fabsf(xf - r) <= fabsf(xf) * 0x1p-21f) r = rintf(ws[j] / step);
      const float q = fminf(fmaxf(r + z, 0.0f), qmax);
      word |= (uint32_t)q << (4 * j);
    }
    const int64_t p = p0 + TEAMS * u;
    if (p < pairs) {
      qweight[widx[u]] = word;
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
  const int per_block = 256 / (qs.group / 8) * kPackPerTeam;
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
