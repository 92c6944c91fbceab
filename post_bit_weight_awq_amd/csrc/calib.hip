// Measured-peak references for the benchmark (not part of the search library):
// an MFMA-only loop with the grid kernel's instruction and wavefront shape, and
// a plain streaming read of a device buffer.  Built as libawq_calib.so.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// 8 wavefronts per block, each with 4 x 8 independent 16x16 fp32 accumulators
// fed by v_mfma_f32_16x16x32_f16 from registers: 32 MFMAs per iteration.
__global__ void __launch_bounds__(512) k_mfma_loop(float* __restrict__ out, int n_iter) {
  const int lane = threadIdx.x & 63;
  floatx4 acc[4][8];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[m][n] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  half8 a[4], b[8];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int e = 0; e < 8; ++e) a[m][e] = (_Float16)(0.001f * (lane + m + e));
#pragma unroll
  for (int n = 0; n < 8; ++n)
#pragma unroll
    for (int e = 0; e < 8; ++e) b[n][e] = (_Float16)(0.001f * (lane - n + e));
  for (int it = 0; it < n_iter; ++it) {
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int n = 0; n < 8; ++n)
        acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[m], b[n], acc[m][n], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 8; ++n) s += acc[m][n][0] + acc[m][n][1] + acc[m][n][2] + acc[m][n][3];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Grid-strided 16-byte loads, four in flight per lane; the XOR of everything
// read is written only if it matches an arbitrary constant (keeps the loads).
__global__ void __launch_bounds__(256)
k_read_stream(const uint4* __restrict__ x, int64_t n16, uint32_t* __restrict__ out) {
  const int64_t T = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * T < n16; i += 4 * T) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = x[i + u * T];
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += T) {
    const uint4 v = x[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) out[0] = acc;
}

// The fastest plain read measured here: one shot per block (each block reads
// 256 x 8 contiguous 16-byte pieces, all eight loads of a lane in flight at
// once) with nontemporal loads.  On a 283 MB buffer after a last-level-cache
// clear it moved 6.3 TB/s, against 5.2 TB/s for the grid-strided read above.
constexpr int kOneShotPieces = 8;
__global__ void __launch_bounds__(256)
k_read_oneshot(const uint4* __restrict__ x, int64_t n16, uint32_t* __restrict__ out) {
  const int64_t base = (int64_t)blockIdx.x * 256 * kOneShotPieces + threadIdx.x;
  uint4 v[kOneShotPieces];
#pragma unroll
  for (int u = 0; u < kOneShotPieces; ++u) {
    const int64_t i = base + u * 256 < n16 ? base + u * 256 : n16 - 1;
    v[u].x = __builtin_nontemporal_load(&x[i].x);
    v[u].y = __builtin_nontemporal_load(&x[i].y);
    v[u].z = __builtin_nontemporal_load(&x[i].z);
    v[u].w = __builtin_nontemporal_load(&x[i].w);
  }
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < kOneShotPieces; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  if (acc == 0x9e3779b9u) out[0] = acc;
}

}  // namespace

extern "C" {

// Flops of one awq_calib_mfma launch: n_blocks x 8 wavefronts x n_iter x 32
// MFMAs x 16384 flops.  out: n_blocks * 512 floats (device).  Returns 0, or
// -1 for bad arguments, -4 for a launch error.
int awq_calib_mfma(float* out, int n_blocks, int n_iter, void* stream) {
  if (!out || n_blocks <= 0 || n_iter <= 0) return -1;
  hipLaunchKernelGGL(k_mfma_loop, dim3(n_blocks), dim3(512), 0, (hipStream_t)stream, out, n_iter);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// Reads `bytes` (a multiple of 16, 16-byte aligned) of device memory once.
// out: one uint32 of device memory (written only by chance).  Returns 0, -1,
// or -4.
int awq_calib_read(const void* buf, int64_t bytes, uint32_t* out, int n_blocks, void* stream) {
  if (!buf || !out || bytes <= 0 || bytes % 16 != 0 || ((uintptr_t)buf & 15) || n_blocks <= 0)
    return -1;
  hipLaunchKernelGGL(k_read_stream, dim3(n_blocks), dim3(256), 0, (hipStream_t)stream,
                     (const uint4*)buf, bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// Reads `bytes` (a multiple of 16, 16-byte aligned) of device memory once with
// k_read_oneshot.  out: one uint32 of device memory (written only by chance).
// Returns 0, -1, or -4.
int awq_calib_read_oneshot(const void* buf, int64_t bytes, uint32_t* out, void* stream) {
  if (!buf || !out || bytes <= 0 || bytes % 16 != 0 || ((uintptr_t)buf & 15)) return -1;
  const int64_t n16 = bytes / 16, per_block = 256 * kOneShotPieces;
  hipLaunchKernelGGL(k_read_oneshot, dim3((unsigned)((n16 + per_block - 1) / per_block)), dim3(256),
                     0, (hipStream_t)stream, (const uint4*)buf, n16, out);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
