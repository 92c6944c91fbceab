// Inference with the packed weights: y = x Wdq^T for fp16 activations and the
// 4-bit codes of awq_pack, Wdq[o, k] = (q[o, k] - z[o, g]) * step[o, g] with
// g = k / 128 (dev.to "AWQ: How Activation-Aware Quantization Saves 4-bit
// LLMs", "What do you actually deploy": W4A16 with groups of 128, where decode
// streams a quarter of the fp16 weight bytes; esaholic.com "What is AWQ
// Quantization?", INT4 codes in INT32 containers and W4A16 GEMM kernels;
// "AWQ > Salient Weight Preservation", step-size equation).
//
// HBM-bound at decode sizes: 0.5 byte of codes + 4/128 byte of step and zero
// per weight, read once.  A block owns 16 output rows and 16 token rows; its
// 16 wavefronts split the groups of 128 columns evenly and their partial
// outputs are added in LDS at the end (fixed order, no atomics).
//   * Lane l holds output row o0 + l % 16 and the 32-column slice l / 16 of the
//     current group: one 16-byte load of 32 codes.  Each of its four words
//     feeds one v_mfma_f32_16x16x32_f16 as the B operand; lane l's A operand is
//     the matching 8 activations of token t0 + l % 16.
//   * Codes become exact fp16 integers by bit placement: (nibble | 0x6400)
//     is the fp16 value 1024 + nibble, and one packed fp16 subtraction of 1024
//     leaves the code itself.  Two bit-select steps put them in column order.
//   * Per group, the MFMAs give A = sum_k x q and, with an all-ones B, the
//     activation sum S = sum_k x, both accumulated in fp32 from exact fp16
//     products; the group adds step * (A - z S) to the output.  The zero
//     point enters as one multiply per group, so it may be any stored fp16
//     value.
#include "awq_device.h"
#include "awq_internal.h"

namespace awq {

constexpr int kW4Slices = 16;  // wavefronts per block, each a share of the groups

__device__ __forceinline__ uint32_t lo_lo(uint32_t a, uint32_t b) {
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t hi_hi(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xffff0000u);
}

__global__ void __launch_bounds__(kW4Slices * 64)
k_w4a16(const _Float16* __restrict__ X, int M, int K, int OUT, const uint4* __restrict__ qw,
        const _Float16* __restrict__ step16, const _Float16* __restrict__ zero16,
        float* __restrict__ Y) {
  __shared__ float red[kW4Slices][256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int o0 = blockIdx.x * 16, t0 = blockIdx.y * 16;
  const int r16 = lane & 15, j4 = lane >> 4;
  const int orow = min(o0 + r16, OUT - 1);  // rows past the end re-read the last row
  const int tok = t0 + r16;
  const bool tok_ok = tok < M;
  const int ng = K >> 7;
  const int g0 = (int)((int64_t)wave * ng / kW4Slices);
  const int g1 = (int)((int64_t)(wave + 1) * ng / kW4Slices);
  const uint4* qrow = qw + (size_t)orow * (K >> 5) + j4;  // group g at qrow[4 g]
  const _Float16* xrow = X + (size_t)(tok_ok ? tok : 0) * K + 32 * j4;
  const _Float16* srow = step16 + (size_t)orow * ng;
  const _Float16* zrow = zero16 + (size_t)orow * ng;
  constexpr uint32_t kBias = 0x64006400u;  // fp16 1024 in both halves
  half8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (_Float16)1.0f;
  floatx4 y = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int g = g0; g < g1; ++g) {
    const uint4 q = qrow[4 * g];
    uint4 xv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      xv[j] = tok_ok ? *(const uint4*)(xrow + 128 * g + 8 * j) : make_uint4(0, 0, 0, 0);
    const float st = (float)srow[g];
    const float zf = (float)zrow[g];
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    floatx4 aq = {0.0f, 0.0f, 0.0f, 0.0f}, as = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // codes (c0, c4), (c1, c5), (c2, c6), (c3, c7) as exact fp16 pairs
      const uint32_t p0 = sub_f16x2((w[j] & 0x000F000Fu) | kBias, kBias);
      const uint32_t p1 = sub_f16x2(((w[j] >> 4) & 0x000F000Fu) | kBias, kBias);
      const uint32_t p2 = sub_f16x2(((w[j] >> 8) & 0x000F000Fu) | kBias, kBias);
      const uint32_t p3 = sub_f16x2(((w[j] >> 12) & 0x000F000Fu) | kBias, kBias);
      const uint4 bv = make_uint4(lo_lo(p0, p1), lo_lo(p2, p3), hi_hi(p0, p1), hi_hi(p2, p3));
      const half8 a = __builtin_bit_cast(half8, xv[j]);
      const half8 b = __builtin_bit_cast(half8, bv);
      aq = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, aq, 0, 0, 0);
      as = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, ones, as, 0, 0, 0);
    }
    // register r of lane l: token t0 + 4 (l / 16) + r, output row o0 + l % 16
#pragma unroll
    for (int r = 0; r < 4; ++r) y[r] = fmaf(st, fmaf(-zf, as[r], aq[r]), y[r]);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) red[wave][lane * 4 + r] = y[r];
  __syncthreads();
  if (threadIdx.x < 256) {
    const int e = threadIdx.x;
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < kW4Slices; ++w) s += red[w][e];
    const int l = e >> 2, r = e & 3;
    const int t = t0 + 4 * (l >> 4) + r, o = o0 + (l & 15);
    if (t < M && o < OUT) Y[(size_t)t * OUT + o] = s;
  }
}

hipError_t launch_w4a16(const void* X, int64_t M, int64_t K, int64_t OUT, const int32_t* qweight,
                        const void* step16, const void* zero16, float* Y, hipStream_t stream) {
  const dim3 grid((unsigned)((OUT + 15) / 16), (unsigned)((M + 15) / 16));
  hipLaunchKernelGGL(k_w4a16, grid, dim3(kW4Slices * 64), 0, stream, (const _Float16*)X, (int)M,
                     (int)K, (int)OUT, (const uint4*)qweight, (const _Float16*)step16,
                     (const _Float16*)zero16, Y);
  return hipGetLastError();
}

}  // namespace awq
