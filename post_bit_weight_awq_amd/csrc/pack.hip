// Packing of the chosen codes (esaholic.com "What is AWQ Quantization?",
// pipeline step "INT4 Weight Packing & Export": 4-bit codes in INT32
// containers; dev.to page, quant_config: zero point, groups of 128, 4 bit;
// "AWQ > Salient Weight Preservation", step-size equation).
//
// HBM-bound: 2 bytes of W in, 0.5 + 4/128 bytes out per weight.  A team of 16
// lanes owns a (row, group) at a time; each lane loads its 8 weights with one
// 16-byte load, so a wavefront streams 1 KiB of W per pair it holds.  Per
// group, in binary32:
//   ws = w * s, step = (max - min) / 15 (1 for a zero range),
//   zero = rint(-min / step), q = clamp(rint(ws / step) + zero, 0, 15).
// The code needs the correctly rounded quotient ws / step.  It is formed as
// ws * (1/step), which is within 2.5 ulp of that quotient; the two can round
// to different integers only when the product lies that close to a
// half-integer, so such elements (about 1e-5 of them) take the IEEE division.
#include "awq_device.h"
#include "awq_internal.h"

namespace awq {

// Each team takes kPackPerTeam (row, group) pairs, 16 teams apart, and issues
// all their loads before any arithmetic, so every lane keeps 64 bytes of W in
// flight.
constexpr int kPackPerTeam = 4;
constexpr int kPackPairsPerBlock = 16 * kPackPerTeam;

__global__ void __launch_bounds__(256)
k_pack(const uint4* __restrict__ W, const float* __restrict__ s, int64_t OUT, int64_t K,
       uint32_t* __restrict__ qweight, _Float16* __restrict__ step16,
       _Float16* __restrict__ zero16) {
  const int64_t ng = K / kGroup;
  const int64_t pairs = OUT * ng;
  const int l16 = threadIdx.x % 16;
  const int64_t p0 = (int64_t)blockIdx.x * kPackPairsPerBlock + threadIdx.x / 16;
  uint4 w[kPackPerTeam];
  int64_t k0[kPackPerTeam], widx[kPackPerTeam];
#pragma unroll
  for (int u = 0; u < kPackPerTeam; ++u) {
    const int64_t p = min(p0 + 16 * u, pairs - 1);  // a tail team re-reads the last pair
    const int64_t o = p / ng, g = p - o * ng;
    k0[u] = g * kGroup + l16 * 8;
    widx[u] = (o * K + k0[u]) / 8;
    w[u] = W[widx[u]];
  }
  const float nz = neg_zero();
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
    for (int d = 8; d >= 1; d >>= 1) {
      mn = fminf(mn, __shfl_xor(mn, d, 16));
      mx = fmaxf(mx, __shfl_xor(mx, d, 16));
    }
    float step = (mx - mn) / 15.0f;
    if (step == 0.0f) step = 1.0f;
    const float z = rintf(-mn / step) + 0.0f;
    const float inv_step = 1.0f / step;
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float xf = ws[j] * inv_step;
      float r = rintf(xf);
      // near a half-integer: redo with the exact quotient
      if (0.5f - fabsf(xf - r) <= fabsf(xf) * 0x1p-21f) r = rintf(ws[j] / step);
      const float q = fminf(fmaxf(r + z, 0.0f), 15.0f);
      word |= (uint32_t)q << (4 * j);
    }
    const int64_t p = p0 + 16 * u;
    if (p < pairs) {
      qweight[widx[u]] = word;
      if (l16 == 0) {
        step16[p] = (_Float16)step;
        zero16[p] = (_Float16)z;
      }
    }
  }
}

hipError_t launch_pack(const void* W, const float* s, int64_t K, int64_t OUT, int32_t* qweight,
                       void* step16, void* zero16, hipStream_t stream) {
  const int64_t pairs = OUT * (K / kGroup);
  hipLaunchKernelGGL(k_pack, dim3((unsigned)((pairs + kPackPairsPerBlock - 1) / kPackPairsPerBlock)),
                     dim3(256), 0, stream, (const uint4*)W, s, OUT, K, (uint32_t*)qweight,
                     (_Float16*)step16, (_Float16*)zero16);
  return hipGetLastError();
}

}  // namespace awq
