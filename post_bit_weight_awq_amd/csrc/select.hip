// Top-n channel selection for the saliency ablations (dev.to "AWQ: How
// Activation-Aware Quantization Saves 4-bit LLMs", "How does AWQ decide which
// weights to protect?": protecting about 1% of the channels; esaholic.com
// "What is AWQ Quantization?": the top 1% channels are the ones scaled).
// out[k] = sal[k] for the n_keep largest saliencies (equal values: lower
// channel index first) and 1 elsewhere, so that s = 1^alpha = 1 there.
//
// One block: an MSB-first radix select over the order-preserving 32-bit keys
// of the floats (four passes of 8-bit histograms in LDS) finds the key T of
// the n_keep-th largest value and how many keys equal to T are kept; a last
// pass keeps keys above T and ranks the keys equal to T by index with a
// wavefront ballot and a block prefix over the 16 wavefronts.  Tiny work
// (n <= 2^20 values, read five times).
#include "awq_device.h"
#include "awq_internal.h"

namespace awq {

constexpr int kSelThreads = 1024;

// Monotone map of a float to an unsigned key (for non-NaN values); -0 and +0
// share a key.
__device__ __forceinline__ uint32_t order_key(float v) {
  const uint32_t b = __float_as_uint(v + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__global__ void __launch_bounds__(kSelThreads)
k_select_top(const float* __restrict__ sal, int64_t n, int64_t n_keep, float* out) {
  __shared__ unsigned int hist[256];
  __shared__ unsigned int wave_cnt[kSelThreads / 64];
  __shared__ uint32_t sh_prefix;
  __shared__ long long sh_remaining;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (n_keep == 0 || n_keep >= n) {
    for (int64_t k = tid; k < n; k += kSelThreads) out[k] = n_keep == 0 ? 1.0f : sal[k];
    return;
  }
  uint32_t prefix = 0, mask = 0;
  long long remaining = n_keep;  // still to keep among the keys that match prefix
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0u;
    __syncthreads();
    for (int64_t k = tid; k < n; k += kSelThreads) {
      const uint32_t key = order_key(sal[k]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 0xFFu], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      long long above = 0;
      int d = 255;
      for (; d > 0; --d) {
        if (above + (long long)hist[d] >= remaining) break;
        above += hist[d];
      }
      sh_prefix = prefix | ((uint32_t)d << shift);
      sh_remaining = remaining - above;
    }
    __syncthreads();
    prefix = sh_prefix;
    remaining = sh_remaining;
    mask |= 0xFFu << shift;
  }
  // prefix is now the key of the n_keep-th largest value
  long long base = 0;  // keys equal to it in earlier chunks
  for (int64_t c0 = 0; c0 < n; c0 += kSelThreads) {
    const int64_t k = c0 + tid;
    const bool valid = k < n;
    const float v = valid ? sal[k] : 0.0f;
    const uint32_t key = order_key(v);
    const bool eq = valid && key == prefix;
    const unsigned long long bal = __ballot(eq);
    const unsigned rank = (unsigned)__popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wave_cnt[wave] = (unsigned)__popcll(bal);
    __syncthreads();
    unsigned before = 0, total = 0;
    for (int w = 0; w < kSelThreads / 64; ++w) {
      before += w < wave ? wave_cnt[w] : 0u;
      total += wave_cnt[w];
    }
    if (valid) {
      const bool keep = key > prefix || (eq && base + before + rank < remaining);
      out[k] = keep ? v : 1.0f;
    }
    base += total;
    __syncthreads();  // wave_cnt is rewritten by the next chunk
  }
}

hipError_t launch_select_top(const float* sal, int64_t n, int64_t n_keep, float* out,
                             hipStream_t stream) {
  hipLaunchKernelGGL(k_select_top, dim3(1), dim3(kSelThreads), 0, stream, sal, n, n_keep, out);
  return hipGetLastError();
}

}  // namespace awq
