// Steps 2-5 of the AWQ search for one linear layer, all grid points in one pass.
//
// dev.to "AWQ: How Activation-Aware Quantization Saves 4-bit LLMs", search_scale
// listing: for alpha_i = i / n_grid, s = max(sal, 1e-4)^alpha_i scales the weight
// columns, the scaled weight is quantized, divided by s again, and the mean
// squared difference of the layer output against the unquantized layer's output
// is the loss; the first strict minimum wins.  The quantizer is the asymmetric
// group quantizer of "AWQ > Salient Weight Preservation" (step-size equation),
// groups of 128 along in_features with a zero point (quant_config of the dev.to
// page's "What do you actually deploy").
//
// Kernels, in launch order:
//   k_scale_table   s[i,k] = fp32(pow(fp64 max(sal_k, floor), i/n)), inv_s = fp32(1/s)
//   k_group_params  per (i, row, group): step, 1/step, -zero, 15-zero of W diag(s_i)
//   k_tile<REF>     reference output X W^T (fp32, into the workspace)
//   k_tile<SEARCH>  per (i, token tile, output tile): builds the fake-quantized
//                   fp16 weight tile in LDS, contracts it with the activation tile
//                   on the MFMA units (fp16 x fp16 -> fp32), and reduces
//                   (Y_q - Y_ref)^2 over the tile in registers; Y_q never leaves
//                   the chip.  One partial sum per tile.
//   k_argmin        fixed-order sum of the partials per grid point, mean, and a
//                   wavefront-shuffle argmin (lowest index wins ties).
#include "awq_device.h"
#include "awq_internal.h"

namespace awq {

// ---------------------------------------------------------------- scale table
__global__ void __launch_bounds__(256)
k_scale_table(const float* __restrict__ sal, float* __restrict__ s_tab,
              float* __restrict__ inv_tab, int64_t K, int n_grid, float floor_v) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)n_grid * K) return;
  const int i = (int)(idx / K);
  const int64_t k = idx - (int64_t)i * K;
  const float v = sal[k];
  const double base = (double)(v > floor_v ? v : floor_v);
  const double alpha = (double)i / (double)n_grid;
  const float s = (float)pow(base, alpha);
  s_tab[idx] = s;
  inv_tab[idx] = 1.0f / s;  // IEEE division
}

// ------------------------------------------------- per-group quantizer params
// A team of 16 lanes owns one (row, group); each lane holds 8 of its 128 weights
// and the team loops over the grid.  step = (max - min) / 15 with IEEE division,
// zero = rint(-min / step) (+0 for a zero), a zero range takes step = 1.
struct GroupParams {
  float step, inv_step, lo, hi;  // lo = -zero, hi = 15 - zero
};

__global__ void __launch_bounds__(256)
k_group_params(const uint4* __restrict__ W, const float* __restrict__ s_tab,
               GroupParams* __restrict__ prm, int64_t OUT, int64_t K, int n_grid) {
  const int64_t ng = K / kGroup;
  const int64_t team = (int64_t)blockIdx.x * 16 + threadIdx.x / 16;
  const int l16 = threadIdx.x % 16;
  const bool live = team < OUT * ng;
  const int64_t o = live ? team / ng : 0;
  const int64_t g = live ? team - o * ng : 0;
  const int64_t k0 = g * kGroup + l16 * 8;
  const uint4 w = W[(o * K + k0) / 8];
  const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
  const float nz = neg_zero();
  for (int i = 0; i < n_grid; ++i) {
    const float4* sp = (const float4*)(s_tab + (int64_t)i * K + k0);
    const float4 sa = sp[0], sb = sp[1];
    const float sv[8] = {sa.x, sa.y, sa.z, sa.w, sb.x, sb.y, sb.z, sb.w};
    float mn = INFINITY, mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = mul_f16_f32<false>(wv[j], sv[2 * j], nz);
      const float b = mul_f16_f32<true>(wv[j], sv[2 * j + 1], nz);
      mn = fminf(mn, fminf(a, b));
      mx = fmaxf(mx, fmaxf(a, b));
    }
#pragma unroll
    for (int d = 8; d >= 1; d >>= 1) {
      mn = fminf(mn, __shfl_xor(mn, d, 16));
      mx = fmaxf(mx, __shfl_xor(mx, d, 16));
    }
    if (live && l16 == 0) {
      float step = (mx - mn) / 15.0f;
      if (step == 0.0f) step = 1.0f;
      const float z = rintf(-mn / step) + 0.0f;
      GroupParams p;
      p.step = step;
      p.inv_step = 1.0f / step;
      p.lo = -z;
      p.hi = 15.0f - z;
      prm[((int64_t)i * OUT + o) * ng + g] = p;
    }
  }
}

// ------------------------------------------------------------ the tile kernel
// 256 threads = 4 wavefronts in a 2x2 arrangement; each wavefront computes a
// (BM/2) x (BN/2) block of the output tile with v_mfma_f32_32x32x16_f16.
// MFMA operand layout (32x32x16, fp16): lane l supplies row (l % 32) and the
// eight k values 8*(l/32) .. 8*(l/32)+7 of both A (tokens x k) and B^T
// (outputs x k); accumulator register r of lane l holds
// C[8*(r/4) + 4*(l/32) + r%4][l % 32].
constexpr int kTileThreads = 256;

template <int BM, int BN, int KC, bool REF>
__global__ void __launch_bounds__(kTileThreads)
k_tile(const _Float16* __restrict__ X, const _Float16* __restrict__ W,
       const float* __restrict__ s_tab, const float* __restrict__ inv_tab,
       const GroupParams* __restrict__ prm, float* __restrict__ yref,
       double* __restrict__ partials, int64_t N, int64_t K, int64_t OUT) {
  constexpr int PAD = 8;
  constexpr int LD = KC + PAD;          // LDS row stride in halves
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int MB = WM / 32, NB = WN / 32;
  constexpr int XV = BM * KC / 8 / kTileThreads;  // uint4 per thread per X tile
  constexpr int WV = BN * KC / 8 / kTileThreads;
  static_assert(XV >= 1 && WV >= 1, "tile too small for the block");
  __shared__ __attribute__((aligned(16))) _Float16 xs[BM * LD];
  __shared__ __attribute__((aligned(16))) _Float16 wsh[BN * LD];
  __shared__ double red[kTileThreads / kWave];

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int wm = wave / 2, wn = wave % 2;
  const int64_t ot = blockIdx.x, tt = blockIdx.y;
  const int ai = REF ? 0 : (int)blockIdx.z;
  const int64_t t0 = tt * BM, o0 = ot * BN;
  const int64_t ng = K / kGroup;
  const float nz = neg_zero();

  floatx16 acc[MB][NB];
#pragma unroll
  for (int a = 0; a < MB; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

  for (int64_t k0 = 0; k0 < K; k0 += KC) {
    // activation tile -> LDS (rows past the end re-read the last row; their
    // outputs are masked in the epilogue)
#pragma unroll
    for (int v = 0; v < XV; ++v) {
      const int idx = tid + v * kTileThreads;
      const int row = idx / (KC / 8), c8 = idx % (KC / 8);
      const int64_t gr = min(t0 + row, N - 1);
      const uint4 x = *(const uint4*)(X + gr * K + k0 + c8 * 8);
      *(uint4*)(xs + row * LD + c8 * 8) = x;
    }
    // weight tile -> (fake-quantized) fp16 -> LDS
#pragma unroll
    for (int v = 0; v < WV; ++v) {
      const int idx = tid + v * kTileThreads;
      const int row = idx / (KC / 8), c8 = idx % (KC / 8);
      const int64_t go = min(o0 + row, OUT - 1);
      const int64_t kk = k0 + c8 * 8;
      const uint4 w = *(const uint4*)(W + go * K + kk);
      uint4 out;
      if (REF) {
        out = w;
      } else {
        const GroupParams p = prm[((int64_t)ai * OUT + go) * ng + kk / kGroup];
        const float4* sp = (const float4*)(s_tab + (int64_t)ai * K + kk);
        const float4* ip = (const float4*)(inv_tab + (int64_t)ai * K + kk);
        const float4 sa = sp[0], sb = sp[1], ia = ip[0], ib = ip[1];
        const float sv[8] = {sa.x, sa.y, sa.z, sa.w, sb.x, sb.y, sb.z, sb.w};
        const float iv[8] = {ia.x, ia.y, ia.z, ia.w, ib.x, ib.y, ib.z, ib.w};
        const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
        uint32_t ov[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float a = mul_f16_f32<false>(wv[j], sv[2 * j], nz);
          const float b = mul_f16_f32<true>(wv[j], sv[2 * j + 1], nz);
          const float ca = med3(rintf(a * p.inv_step), p.lo, p.hi) * p.step;
          const float cb = med3(rintf(b * p.inv_step), p.lo, p.hi) * p.step;
          ov[j] = mul_f32_to_f16x2(ca, iv[2 * j], cb, iv[2 * j + 1], nz);
        }
        out = make_uint4(ov[0], ov[1], ov[2], ov[3]);
      }
      *(uint4*)(wsh + row * LD + c8 * 8) = out;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < KC; ks += 16) {
      half8 a[MB], b[NB];
#pragma unroll
      for (int m = 0; m < MB; ++m)
        a[m] = *(const half8*)(xs + (wm * WM + m * 32 + lane % 32) * LD + ks + (lane / 32) * 8);
#pragma unroll
      for (int n = 0; n < NB; ++n)
        b[n] = *(const half8*)(wsh + (wn * WN + n * 32 + lane % 32) * LD + ks + (lane / 32) * 8);
#pragma unroll
      for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int n = 0; n < NB; ++n)
          acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[m], b[n], acc[m][n], 0, 0, 0);
    }
    __syncthreads();
  }

  // epilogue
  float sq = 0.0f;
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const int64_t o = o0 + wn * WN + n * 32 + lane % 32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t t = t0 + wm * WM + m * 32 + 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
        if (t < N && o < OUT) {
          if (REF) {
            yref[t * OUT + o] = acc[m][n][r];
          } else {
            const float d = acc[m][n][r] - yref[t * OUT + o];
            sq += d * d;
          }
        }
      }
    }
  if (!REF) {
    double ds = (double)sq;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) ds += __shfl_xor(ds, d, kWave);
    if (lane == 0) red[wave] = ds;
    __syncthreads();
    if (tid == 0) {
      const double tot = (red[0] + red[1]) + (red[2] + red[3]);
      partials[((int64_t)ai * gridDim.y + tt) * gridDim.x + ot] = tot;
    }
  }
}

// -------------------------------------------------------------------- argmin
__global__ void __launch_bounds__(256)
k_argmin(const double* __restrict__ partials, int64_t n_tiles, int n_grid, double count,
         const float* __restrict__ s_tab, int64_t K, double* __restrict__ losses,
         int32_t* __restrict__ best_idx, float* __restrict__ s_best) {
  __shared__ double red[256];
  __shared__ double lsh[64];
  __shared__ int best_sh;
  const int tid = threadIdx.x;
  for (int i = 0; i < n_grid; ++i) {
    double acc = 0.0;
    for (int64_t t = tid; t < n_tiles; t += 256) acc += partials[(int64_t)i * n_tiles + t];
    red[tid] = acc;
    __syncthreads();
    for (int w = 128; w >= 1; w >>= 1) {
      if (tid < w) red[tid] += red[tid + w];
      __syncthreads();
    }
    if (tid == 0) lsh[i] = red[0] / count;
    __syncthreads();
  }
  if (tid < kWave) {
    // a finite loss competes; NaN and infinities never win.  Ties go to the
    // lower index, i.e. the first minimum along the grid.
    double v = (tid < n_grid) ? lsh[tid] : INFINITY;
    const bool ok = tid < n_grid && isfinite(v);
    if (!ok) v = INFINITY;
    int idx = ok ? tid : 0x7fffffff;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
      const double ov = __shfl_xor(v, d, kWave);
      const int oi = __shfl_xor(idx, d, kWave);
      if (ov < v || (ov == v && oi < idx)) {
        v = ov;
        idx = oi;
      }
    }
    if (tid < n_grid) losses[tid] = lsh[tid];
    if (tid == 0) {
      const int b = (idx == 0x7fffffff) ? -1 : idx;
      *best_idx = b;
      best_sh = b;
    }
  }
  __syncthreads();
  const int b = best_sh;
  for (int64_t k = tid; k < K; k += 256)
    s_best[k] = b >= 0 ? s_tab[(int64_t)b * K + k] : __builtin_nanf("");
}

// ------------------------------------------------------------------ host side
namespace {
constexpr int kBM = 128, kBN = 128, kKC = 32;
size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }
}  // namespace

SearchPlan search_plan(int64_t n_tokens, int64_t in_features, int64_t out_features, int n_grid) {
  SearchPlan p;
  p.tile_m = kBM;
  p.tile_n = kBN;
  p.kernel = 0;
  p.n_t_tiles = (n_tokens + kBM - 1) / kBM;
  p.n_o_tiles = (out_features + kBN - 1) / kBN;
  size_t off = 0;
  p.off_partials = off;
  off = align256(off + sizeof(double) * (size_t)n_grid * p.n_t_tiles * p.n_o_tiles);
  p.off_yref = off;
  off = align256(off + sizeof(float) * (size_t)n_tokens * out_features);
  p.off_s = off;
  off = align256(off + sizeof(float) * (size_t)n_grid * in_features);
  p.off_inv_s = off;
  off = align256(off + sizeof(float) * (size_t)n_grid * in_features);
  p.off_params = off;
  off = align256(off + sizeof(GroupParams) * (size_t)n_grid * out_features * (in_features / kGroup));
  p.bytes = off;
  return p;
}

hipError_t launch_search(const void* X, const void* W, const float* sal, int64_t N, int64_t K,
                         int64_t OUT, int n_grid, float sal_floor, double* losses,
                         int32_t* best_idx, float* s_best, void* workspace, const SearchPlan& p,
                         int stage_mask, hipStream_t stream) {
  char* ws = (char*)workspace;
  double* partials = (double*)(ws + p.off_partials);
  float* yref = (float*)(ws + p.off_yref);
  float* s_tab = (float*)(ws + p.off_s);
  float* inv_tab = (float*)(ws + p.off_inv_s);
  GroupParams* prm = (GroupParams*)(ws + p.off_params);
  const int64_t ng = K / kGroup;
  const _Float16* Xh = (const _Float16*)X;
  const _Float16* Wh = (const _Float16*)W;

  if (stage_mask & 1) {  // prepare
    const int64_t nst = (int64_t)n_grid * K;
    hipLaunchKernelGGL(k_scale_table, dim3((unsigned)((nst + 255) / 256)), dim3(256), 0, stream,
                       sal, s_tab, inv_tab, K, n_grid, sal_floor);
    const int64_t teams = OUT * ng;
    hipLaunchKernelGGL(k_group_params, dim3((unsigned)((teams + 15) / 16)), dim3(256), 0, stream,
                       (const uint4*)W, s_tab, prm, OUT, K, n_grid);
    const dim3 grid_ref((unsigned)p.n_o_tiles, (unsigned)p.n_t_tiles, 1);
    hipLaunchKernelGGL((k_tile<kBM, kBN, kKC, true>), grid_ref, dim3(kTileThreads), 0, stream, Xh,
                       Wh, s_tab, inv_tab, prm, yref, partials, N, K, OUT);
  }
  if (stage_mask & 2) {  // grid
    const dim3 grid((unsigned)p.n_o_tiles, (unsigned)p.n_t_tiles, (unsigned)n_grid);
    hipLaunchKernelGGL((k_tile<kBM, kBN, kKC, false>), grid, dim3(kTileThreads), 0, stream, Xh,
                       Wh, s_tab, inv_tab, prm, yref, partials, N, K, OUT);
  }
  if (stage_mask & 4) {  // select
    hipLaunchKernelGGL(k_argmin, dim3(1), dim3(256), 0, stream, partials,
                       p.n_t_tiles * p.n_o_tiles, n_grid, (double)N * (double)OUT, s_tab, K,
                       losses, best_idx, s_best);
  }
  return hipGetLastError();
}

}  // namespace awq
