// Folding the inverse scale into the producer of the layer's input channels
// ("AWQ > Salient Weight Preservation": the preceding normalization's
// per-channel scale is multiplied by 1/s_j; "AWQ > Summary", per-channel
// scaling: the inverse is fused into preceding layers).  Row j of an fp16
// array (a norm's gain or bias, or a preceding linear's weight row and bias)
// is divided by s_j: dst = fp16(fp32(src) / s_j), IEEE division.
//
// HBM-bound elementwise pass: 2 bytes in and 2 bytes out per element.  When
// the row length is a multiple of 8 and both arrays are 16-byte aligned, each
// thread moves 8 elements of one row with 16-byte accesses; otherwise one
// element per thread.
#include "awq_device.h"
#include "awq_internal.h"

namespace awq {

__global__ void __launch_bounds__(256)
k_fold_vec8(const uint4* __restrict__ src, const float* __restrict__ s, int64_t n8, int64_t cols8,
            uint4* __restrict__ dst) {
  const int64_t T = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += T) {
    const float sj = s[i / cols8];
    const uint4 v = src[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const _Float16 lo = (_Float16)(f16_lo(w[e]) / sj);
      const _Float16 hi = (_Float16)(f16_hi(w[e]) / sj);
      o[e] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
             ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    dst[i] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

__global__ void __launch_bounds__(256)
k_fold_scalar(const _Float16* __restrict__ src, const float* __restrict__ s, int64_t n,
              int64_t cols, _Float16* __restrict__ dst) {
  const int64_t T = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += T)
    dst[i] = (_Float16)((float)src[i] / s[i / cols]);
}

hipError_t launch_fold(const void* src, const float* s, int64_t rows, int64_t cols, void* dst,
                       hipStream_t stream) {
  const int64_t n = rows * cols;
  const bool vec = cols % 8 == 0 && ((uintptr_t)src & 15u) == 0 && ((uintptr_t)dst & 15u) == 0;
  const int64_t items = vec ? n / 8 : n;
  const int64_t want = (items + 255) / 256;
  const unsigned blocks = (unsigned)(want < 8192 ? (want > 0 ? want : 1) : 8192);
  if (vec)
    hipLaunchKernelGGL(k_fold_vec8, dim3(blocks), dim3(256), 0, stream, (const uint4*)src, s,
                       items, cols / 8, (uint4*)dst);
  else
    hipLaunchKernelGGL(k_fold_scalar, dim3(blocks), dim3(256), 0, stream, (const _Float16*)src, s,
                       items, cols, (_Float16*)dst);
  return hipGetLastError();
}

}  // namespace awq
