// Step 1 of the AWQ search: per-input-channel activation saliency
// sal_k = mean_t |X[t,k]|   (dev.to "AWQ: How Activation-Aware Quantization
// Saves 4-bit LLMs", channel_importance listing; "AWQ > Summary", salient
// weight identification: average absolute activation over the calibration set).
//
// HBM-bound column reduction.  Each lane owns 8 consecutive columns and reads
// them with one 16-byte load per token row, so a wavefront reads 1 KiB of a row
// contiguously.  The block's four wavefronts take interleaved rows of one row
// chunk, sixteen rows in flight per lane.  |x| of an fp16 value is an integer
// multiple of 2^-24 below 2^16, so the per-lane binary64 sums are exact (at
// most 8192 rows per chunk); the block's column totals are stored as 64-bit
// integers in units of 2^-24, one row of partials per chunk.  A second kernel
// adds each column's partials (integer adds: exact, in a fixed order) and
// divides once.  Two launches, no atomics, no state kept between calls.
// Non-finite inputs follow IEEE sums of |x|: a column holding a NaN gets NaN,
// else one holding an infinity +inf.  The partials carry them as the two
// largest 64-bit values, which no finite column sum reaches (at most
// 2^24 tokens x 65504 x 2^24 < 2^64 - 2).
// Inputs of at most 4M elements take one launch instead (k_act_stats_1p): the
// whole input is then in flight at once, and a second launch would cost more
// than the parallelism it adds (measured 8.8 -> 6.4 us on 512 x 4096; on
// 4096 x 5120 the two-pass form is faster, 15 vs 23 us).
#include <map>
#include <mutex>

#include "awq_device.h"
#include "awq_internal.h"

// Scratch of the allocation-free entry point (awq_act_stats_noalloc): the
// two-pass path's partial column sums, in a fixed array of which each GPU
// holds its own copy until the process ends.  Host code never uses this name
// as an address: it asks the runtime for the current device's copy once
// (scratch_address) and passes that pointer to the kernels.
static __device__ __align__(256) unsigned char scratch[awq::kStatsScratchBytes];

namespace awq {

constexpr unsigned long long kPartInf = ~0ull - 1;  // some term was +inf, none NaN
constexpr unsigned long long kPartNaN = ~0ull;      // some term was NaN

constexpr int kStatsThreads = 256;
constexpr int kStatsCols = kWave * 8;  // columns per block

__global__ void __launch_bounds__(kStatsThreads)
k_act_stats(const uint4* __restrict__ X, int64_t n_tokens, int64_t in_features,
            int64_t rows_per_chunk, unsigned long long* __restrict__ part) {
  __shared__ double red[kStatsThreads / kWave][kStatsCols];
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int64_t col = (int64_t)blockIdx.x * kStatsCols + lane * 8;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_chunk;
  const int64_t r1 = min(r0 + rows_per_chunk, n_tokens);
  const int64_t row_vecs = in_features / 8;  // uint4 per row
  double s[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) s[j] = 0.0;
  if (col < in_features) {
    const uint4* p = X + r0 * row_vecs + col / 8;
    int64_t r = r0 + wave;
    // sixteen rows in flight per lane: a 64-row chunk is one round of loads
    for (; r + 60 < r1; r += 64) {
      uint4 v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = p[(r - r0 + 4 * u) * row_vecs];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          s[2 * j] += (double)fabsf(f16_lo(w[j]));
          s[2 * j + 1] += (double)fabsf(f16_hi(w[j]));
        }
      }
    }
    // a ragged last chunk: four rows in flight, then one
    for (; r + 12 < r1; r += 16) {
      uint4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = p[(r - r0 + 4 * u) * row_vecs];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          s[2 * j] += (double)fabsf(f16_lo(w[j]));
          s[2 * j + 1] += (double)fabsf(f16_hi(w[j]));
        }
      }
    }
    for (; r < r1; r += 4) {
      const uint4 v = p[(r - r0) * row_vecs];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s[2 * j] += (double)fabsf(f16_lo(w[j]));
        s[2 * j + 1] += (double)fabsf(f16_hi(w[j]));
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) red[wave][lane * 8 + j] = s[j];
  __syncthreads();
  // 512 column totals, two per thread; the four wave partials are exact, so
  // their sum is exact as well.
  unsigned long long* prow = part + (int64_t)blockIdx.y * in_features;
  for (int c = threadIdx.x; c < kStatsCols; c += kStatsThreads) {
    const int64_t gc = (int64_t)blockIdx.x * kStatsCols + c;
    if (gc < in_features) {
      const double t = red[0][c] + red[1][c] + red[2][c] + red[3][c];
      // exact: a finite t is a multiple of 2^-24
      prow[gc] = t != t ? kPartNaN : t == INFINITY ? kPartInf : (unsigned long long)(t * 16777216.0);
    }
  }
}

// One block per 64 columns; its 16 wavefronts add every 16th chunk's partials
// (lanes on consecutive columns), then wavefront 0 adds the 16 sums.  Integer
// adds, so the total is exact whatever the order.
__global__ void __launch_bounds__(1024)
k_stats_finalize(const unsigned long long* __restrict__ part, int64_t row_chunks,
                 int64_t in_features, int64_t n_tokens, float* __restrict__ sal) {
  __shared__ unsigned long long sh[16][64];
  __shared__ unsigned long long shf[16][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t k = (int64_t)blockIdx.x * 64 + lane;
  unsigned long long acc = 0, flag = 0;  // flag: the largest non-finite code seen
  if (k < in_features)
    for (int64_t c = wave; c < row_chunks; c += 16) {
      const unsigned long long v = part[c * in_features + k];
      if (v >= kPartInf)
        flag = v > flag ? v : flag;
      else
        acc += v;
    }
  sh[wave][lane] = acc;
  shf[wave][lane] = flag;
  __syncthreads();
  if (wave == 0 && k < in_features) {
    unsigned long long tot = 0, fl = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      tot += sh[w][lane];
      fl = shf[w][lane] > fl ? shf[w][lane] : fl;
    }
    // binary64 value of the exact sum (rounded only beyond 2^53 units), then
    // the binary64 quotient, then binary32.
    const double total = (double)tot * 0x1p-24;
    sal[k] = fl == kPartNaN ? __builtin_nanf("") : fl == kPartInf ? INFINITY
                                                                  : (float)(total / (double)n_tokens);
  }
}

// Single pass for small inputs: one block per 64-column strip reads every
// row of its strip (8 lanes per row, 128 contiguous bytes; 8 rows per
// wavefront load, 64 per block, eight loads in flight per lane) and writes the
// saliency directly.  The binary64 sums are exact for n_tokens <= 8192 (the
// same bound as above), so the result equals the two-pass one bit for bit.
constexpr int kStats1Threads = 512;
constexpr int64_t kStats1MaxElems = (int64_t)1 << 22;
__global__ void __launch_bounds__(kStats1Threads)
k_act_stats_1p(const uint4* __restrict__ X, int64_t n_tokens, int64_t in_features,
               float* __restrict__ sal) {
  __shared__ double red[kStats1Threads / kWave][64];
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int64_t col = (int64_t)blockIdx.x * 64 + 8 * (lane & 7);
  const int64_t row_vecs = in_features / 8;
  const int rsub = 8 * wave + (lane >> 3);  // row within a block round of 64
  double s[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) s[j] = 0.0;
  if (col < in_features) {
    const uint4* p = X + col / 8;
    int64_t r = rsub;
    for (; r + 448 < n_tokens; r += 512) {
      uint4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = p[(r + 64 * u) * row_vecs];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          s[2 * j] += (double)fabsf(f16_lo(w[j]));
          s[2 * j + 1] += (double)fabsf(f16_hi(w[j]));
        }
      }
    }
    for (; r < n_tokens; r += 64) {
      const uint4 v = p[r * row_vecs];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s[2 * j] += (double)fabsf(f16_lo(w[j]));
        s[2 * j + 1] += (double)fabsf(f16_hi(w[j]));
      }
    }
  }
  // lanes l, l^8, l^16, ... hold the same columns: exact fp64 adds
#pragma unroll
  for (int d = 8; d < kWave; d <<= 1)
#pragma unroll
    for (int j = 0; j < 8; ++j) s[j] += __shfl_xor(s[j], d, kWave);
  if (lane < 8)
#pragma unroll
    for (int j = 0; j < 8; ++j) red[wave][8 * lane + j] = s[j];
  __syncthreads();
  if (threadIdx.x < 64) {
    const int64_t k = (int64_t)blockIdx.x * 64 + threadIdx.x;
    if (k < in_features) {
      double total = 0.0;
#pragma unroll
      for (int w = 0; w < kStats1Threads / kWave; ++w) total += red[w][threadIdx.x];
      sal[k] = (float)(total / (double)n_tokens);
    }
  }
}

StatsPlan stats_plan(int64_t n_tokens, int64_t in_features) {
  StatsPlan p;
  p.col_blocks = (in_features + kStatsCols - 1) / kStatsCols;
  // about four blocks per compute unit, each streaming a multiple of 64 rows
  // (sixteen rows per wavefront per round of loads)
  const int64_t want = (1024 + p.col_blocks - 1) / p.col_blocks;
  const int64_t max_chunks = (n_tokens + 63) / 64;
  p.row_chunks = want < max_chunks ? want : max_chunks;
  if (p.row_chunks < 1) p.row_chunks = 1;
  p.rows_per_chunk = (n_tokens + p.row_chunks - 1) / p.row_chunks;
  p.rows_per_chunk = (p.rows_per_chunk + 63) / 64 * 64;
  if (p.rows_per_chunk > 8192) {  // keep the per-lane binary64 sums exact
    p.rows_per_chunk = 8192;
  }
  p.row_chunks = (n_tokens + p.rows_per_chunk - 1) / p.rows_per_chunk;
  p.workspace_bytes = (size_t)p.row_chunks * in_features * sizeof(unsigned long long);
  return p;
}

static bool one_pass(int64_t n_tokens, int64_t in_features) {
  return n_tokens <= 8192 && n_tokens * in_features <= kStats1MaxElems;
}

size_t stats_scratch_need(int64_t n_tokens, int64_t in_features) {
  return one_pass(n_tokens, in_features) ? 0 : stats_plan(n_tokens, in_features).workspace_bytes;
}

// Device address of the current GPU's copy of `scratch`, looked up once per
// device (with that device current) and kept.
hipError_t scratch_address(void** out) {
  static std::mutex mu;
  static std::map<int, void*> addr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  auto it = addr.find(dev);
  if (it == addr.end()) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    it = addr.emplace(dev, p).first;
  }
  *out = it->second;
  return hipSuccess;
}

hipError_t launch_act_stats(const void* X, int64_t n_tokens, int64_t in_features, float* sal,
                            void* workspace, hipStream_t stream) {
  const StatsPlan p = stats_plan(n_tokens, in_features);
  if (one_pass(n_tokens, in_features)) {
    hipLaunchKernelGGL(k_act_stats_1p, dim3((unsigned)((in_features + 63) / 64)),
                       dim3(kStats1Threads), 0, stream, (const uint4*)X, n_tokens, in_features,
                       sal);
    return hipGetLastError();
  }
  unsigned long long* part = (unsigned long long*)workspace;
  hipLaunchKernelGGL(k_act_stats, dim3((unsigned)p.col_blocks, (unsigned)p.row_chunks),
                     dim3(kStatsThreads), 0, stream, (const uint4*)X, n_tokens, in_features,
                     p.rows_per_chunk, part);
  hipLaunchKernelGGL(k_stats_finalize, dim3((unsigned)((in_features + 63) / 64)), dim3(1024), 0,
                     stream, part, p.row_chunks, in_features, n_tokens, sal);
  return hipGetLastError();
}

}  // namespace awq
