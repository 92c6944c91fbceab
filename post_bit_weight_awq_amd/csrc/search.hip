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
//   k_group_params  per (i, group, row): step, 1/step, -zero, 15-zero of W diag(s_i)
//   k_grid          per (i, token tile, output tile): builds the fp16 weight-error
//                   tile fp16(Wq - W) in LDS, contracts it with the activation tile
//                   on the MFMA units (fp16 x fp16 -> fp32), which gives
//                   Y_q - Y_ref = X (Wq - W)^T directly, and reduces its square
//                   over the tile in registers; no output ever leaves the chip.
//                   One partial sum per tile (search_grid.hip).
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
  // the floor as a maximum that keeps a NaN saliency (pow(NaN, 0) is still 1)
  const double base = (double)(v < floor_v ? floor_v : v);
  const double alpha = (double)i / (double)n_grid;
  const float s = (float)pow(base, alpha);
  s_tab[idx] = s;
  inv_tab[idx] = 1.0f / s;  // IEEE division
}

// ------------------------------------------------- per-group quantizer params
// A team of 4 lanes owns one (row, group of G = 32, 64 or 128 columns); each
// lane holds G/4 of the group's weights for the whole grid loop.  The 16 teams of a wavefront share
// the group and take consecutive rows; a block covers 64 rows.  The block first
// copies the group's scales for every grid point into LDS (one coalesced pass
// over the scale table), so the grid loop only reads LDS.
// Per grid point: ws = fp32(w s), min and max over the group, then with
// qmax = 2^b - 1 and IEEE divisions (a zero range takes step 1):
//   zero point:  step = (max - min) / qmax, zero = rint(-min / step) (+0 for 0)
//   symmetric:   step = max(|min|, |max|) / 2^(b-1), zero = 2^(b-1)
// then 1/step and the clamp bounds -zero and qmax - zero.
// Grid points go in blocks of four: after the team's min/max reductions every
// lane of the team holds all four (min, max) pairs, and lane j of the team
// finishes grid point i0 + j, so the three divisions run on all lanes at once.
// Records are written in the layout [grid point][group][row].
constexpr int kParamsRows = 64;
// LDS copy of the group's G scales (and reciprocals) for every grid point,
// [grid point][G] floats.  Lane j of a team owns the 8-column pieces j, j + 4,
// j + 8, ... of the group, so the four lanes of a team read (and the
// producer writes) 64 contiguous bytes per instruction, and their scale
// reads cover 128 contiguous bytes of a row (every bank once).
template <int G>
struct ParamsLds {
  static constexpr int kPerGrid = G;
};

__device__ __forceinline__ float min3f(float a, float b, float c) {
  float r;
  asm("v_min3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
// min / max with a lane of the same quad (DPP quad permutation CTRL).  The
// operations are written out (min3/max3 above) because the compiler's own
// min/max would first canonicalize operands it cannot prove canonical.
template <int CTRL>
__device__ __forceinline__ float quad_min_step(float x) {
  const float y = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
  return min3f(x, y, y);
}
template <int CTRL>
__device__ __forceinline__ float quad_max_step(float x) {
  const float y = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
  return max3f(x, y, y);
}
// the value of lane CTRL & 3 of the lane's quad (CTRL a quad_perm [j, j, j, j])
template <int CTRL>
__device__ __forceinline__ float quad_bcast(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

// DW = false writes the parameter records (the fused grid kernel's input).
// DW = true instead produces, for every grid point, the lane's part of the
// fp16 weight error dW_i = fp16(Wq_i - W) of the layer into [grid point][OUT][K]
// (the contraction kernel's input): codes rint(ws / step) clamped to
// [-zero, qmax - zero], (q - zero) * step, times fp32(1/s) rounded once to
// fp16, minus the fp16 weight rounded once.  The quotient is formed as
// ws * (1/step), within 2.5 ulp of ws / step; where a per-group margin flags
// it as that close to a half-integer, the code takes the IEEE division, so
// every code equals the correctly rounded one (the fused kernel, which
// rebuilds codes per token tile, keeps the product).  The parameters of four
// grid points, finished by the four lanes of a team, reach every lane of the
// team by DPP broadcasts.
template <int G, bool DW>
__global__ void __launch_bounds__(256)
k_group_params(const _Float16* __restrict__ W, const float* __restrict__ s_tab,
               const float* __restrict__ inv_tab, GroupParams* __restrict__ prm,
               _Float16* __restrict__ dw, int OUT, int K, int n_grid, float qmax, int symmetric) {
  constexpr int PL = G / 4;   // weights per lane
  constexpr int NP = PL / 8;  // 8-column pieces per lane: j, j + 4, ... of the group
  constexpr int C4 = G / 4;   // float4 of scales per group and grid point
  extern __shared__ float4 s_lds4[];               // [n_grid][G / 4] float4 (x2 for DW)
  float4* i_lds4 = s_lds4 + (size_t)n_grid * C4;   // DW: the reciprocals, same layout
  const int ngroups = K / G;
  const int g = blockIdx.y;
  const int tid = threadIdx.x;
  const int l4 = tid & 3;
  const int o_raw = blockIdx.x * kParamsRows + (tid >> 2);
  const bool live = o_raw < OUT;
  const int o = live ? o_raw : OUT - 1;

  // scales of this group, every grid point: element e = (i, 16-byte column c4)
  for (int e = tid; e < n_grid * C4; e += 256) {
    const int i = e / C4, c4 = e - i * C4;
    s_lds4[e] = ((const float4*)(s_tab + (size_t)i * K + g * G))[c4];
    if (DW) i_lds4[e] = ((const float4*)(inv_tab + (size_t)i * K + g * G))[c4];
  }
  // the lane's weights (pieces l4 + 4 v), widened to fp32 once (exact) for the
  // whole grid loop
  const uint4* wp = (const uint4*)(W + (size_t)o * K + (size_t)g * G);
  float wf[PL];
  uint32_t wr[PL / 2];  // DW: the same weights as packed fp16 pairs
#pragma unroll
  for (int v = 0; v < NP; ++v) {
    const uint4 t = wp[4 * v + l4];
    const uint32_t u[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      wf[8 * v + 2 * e] = f16_lo(u[e]);
      wf[8 * v + 2 * e + 1] = f16_hi(u[e]);
      wr[4 * v + e] = u[e];
    }
  }
  const float half = 0.5f * (qmax + 1.0f);  // 2^(b-1)
  const float nz = opaque_neg_zero();
  __syncthreads();
  for (int i0 = 0; i0 < n_grid; i0 += 4) {
    float mnv[4], mxv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = min(i0 + j, n_grid - 1);
      // the scales of piece l4 + 4 (v / 2), half v % 2
      const float4* sp = s_lds4 + i * C4 + 2 * l4;
      // ws = fp32(w * s): the product of the exact fp32 widening, rounded once.
      // The compiler knows products are canonical, so fminf / fmaxf chains
      // become v_min3 / v_max3 with no canonicalizing instructions.
      float mn, mx;
#pragma unroll
      for (int v = 0; v < PL / 4; ++v) {
        const float4 sv = sp[8 * (v >> 1) + (v & 1)];
        const float a = wf[4 * v] * sv.x;
        const float b = wf[4 * v + 1] * sv.y;
        const float c = wf[4 * v + 2] * sv.z;
        const float d = wf[4 * v + 3] * sv.w;
        if (v == 0) {
          mn = fminf(fminf(a, b), fminf(c, d));
          mx = fmaxf(fmaxf(a, b), fmaxf(c, d));
        } else {
          mn = fminf(fminf(mn, a), fminf(b, fminf(c, d)));
          mx = fmaxf(fmaxf(mx, a), fmaxf(b, fmaxf(c, d)));
        }
      }
      mnv[j] = mn;
      mxv[j] = mx;
    }
    // team reductions, all eight values per DPP step (keeps DPP reads away
    // from the writes they depend on)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      mnv[j] = quad_min_step<0xB1>(mnv[j]);
      mxv[j] = quad_max_step<0xB1>(mxv[j]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      mnv[j] = quad_min_step<0x4E>(mnv[j]);
      mxv[j] = quad_max_step<0x4E>(mxv[j]);
    }
    const float mn = l4 == 0 ? mnv[0] : l4 == 1 ? mnv[1] : l4 == 2 ? mnv[2] : mnv[3];
    const float mx = l4 == 0 ? mxv[0] : l4 == 1 ? mxv[1] : l4 == 2 ? mxv[2] : mxv[3];
    const int i = i0 + l4;
    float step, z;
    if (symmetric) {
      step = fmaxf(fabsf(mn), fabsf(mx)) / half;
      if (step == 0.0f) step = 1.0f;
      z = half;
    } else {
      step = (mx - mn) / qmax;
      if (step == 0.0f) step = 1.0f;
      z = rintf(-mn / step) + 0.0f;
    }
    GroupParams p;
    p.step = step;
    p.inv_step = 1.0f / step;
    p.lo = -z;
    p.hi = qmax - z;
    if (!DW) {
      if (live && i < n_grid) prm[((size_t)i * ngroups + g) * OUT + o] = p;
      continue;
    }
    // products round monotonically, so every |ws / step| of the group is at
    // most max(|min|, |max|) * (1/step): one margin (twice the 2^-21 |x|
    // window, for its own roundings) flags the quotients near a tie
    const float margin = 0.5f - fmaxf(fabsf(mn), fabsf(mx)) * p.inv_step * 0x1p-20f;
    // every lane takes the four grid points' parameters from their lanes
    GroupParams pj[4];
    float mj[4];
    pj[0] = {quad_bcast<0x00>(p.step), quad_bcast<0x00>(p.inv_step), quad_bcast<0x00>(p.lo),
             quad_bcast<0x00>(p.hi)};
    pj[1] = {quad_bcast<0x55>(p.step), quad_bcast<0x55>(p.inv_step), quad_bcast<0x55>(p.lo),
             quad_bcast<0x55>(p.hi)};
    pj[2] = {quad_bcast<0xAA>(p.step), quad_bcast<0xAA>(p.inv_step), quad_bcast<0xAA>(p.lo),
             quad_bcast<0xAA>(p.hi)};
    pj[3] = {quad_bcast<0xFF>(p.step), quad_bcast<0xFF>(p.inv_step), quad_bcast<0xFF>(p.lo),
             quad_bcast<0xFF>(p.hi)};
    mj[0] = quad_bcast<0x00>(margin);
    mj[1] = quad_bcast<0x55>(margin);
    mj[2] = quad_bcast<0xAA>(margin);
    mj[3] = quad_bcast<0xFF>(margin);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ij = i0 + j;
      if (ij >= n_grid) break;
      const float4* sp = s_lds4 + ij * C4 + 2 * l4;
      const float4* ip = i_lds4 + ij * C4 + 2 * l4;
      uint32_t out[PL / 2];
#pragma unroll
      for (int v = 0; v < PL / 4; ++v) {
        const float4 sv = sp[8 * (v >> 1) + (v & 1)], iv = ip[8 * (v >> 1) + (v & 1)];
        const float ss[4] = {sv.x, sv.y, sv.z, sv.w};
        const float is[4] = {iv.x, iv.y, iv.z, iv.w};
        float c[4];
        bool redo = false;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = (wf[4 * v + e] * ss[e]) * pj[j].inv_step;
          c[e] = rintf(x);
          redo |= fabsf(x - c[e]) >= mj[j];
        }
        if (redo) {  // rare: the exact quotient where the margin flags it
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float ws = wf[4 * v + e] * ss[e];
            if (fabsf(ws * pj[j].inv_step - c[e]) >= mj[j]) c[e] = rintf(ws / pj[j].step);
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) c[e] = med3(c[e], pj[j].lo, pj[j].hi) * pj[j].step;
        out[2 * v] = sub_f16x2(mul_f32_to_f16x2(c[0], is[0], c[1], is[1], nz), wr[2 * v]);
        out[2 * v + 1] = sub_f16x2(mul_f32_to_f16x2(c[2], is[2], c[3], is[3], nz), wr[2 * v + 1]);
      }
      if (live) {
        uint4* dst = (uint4*)(dw + ((size_t)ij * OUT + o) * K + (size_t)g * G);
#pragma unroll
        for (int v = 0; v < NP; ++v)
          dst[4 * v + l4] = make_uint4(out[4 * v], out[4 * v + 1], out[4 * v + 2], out[4 * v + 3]);
      }
    }
  }
}

// -------------------------------------------------------------------- argmin
// 1024 threads: wavefront w sums the partials of grid points w, w+16, ... in
// a fixed order (lane-strided with eight loads in flight, then a shuffle
// tree), so the losses are bitwise reproducible.  Wavefront 0 then picks the
// first minimum.
constexpr int kArgminThreads = 1024;

__global__ void __launch_bounds__(kArgminThreads)
k_argmin(const double* __restrict__ partials, int64_t n_tiles, int n_grid, double count,
         const float* __restrict__ s_tab, int64_t K, double* __restrict__ losses,
         int32_t* __restrict__ best_idx, float* __restrict__ s_best) {
  __shared__ double lsh[64];
  __shared__ int best_sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = wave; i < n_grid; i += kArgminThreads / kWave) {
    const double* pp = partials + (int64_t)i * n_tiles;
    double acc = 0.0;
    int64_t t = lane;
    for (; t + 7 * kWave < n_tiles; t += 8 * kWave) {
      double v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = pp[t + kWave * u];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += v[u];
    }
    for (; t < n_tiles; t += kWave) acc += pp[t];
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) acc += __shfl_xor(acc, d, kWave);
    if (lane == 0) lsh[i] = acc / count;
  }
  __syncthreads();
  if (wave == 0) {
    // a finite loss competes; NaN and infinities never win.  Ties go to the
    // lower index, i.e. the first minimum along the grid.
    double v = (lane < n_grid) ? lsh[lane] : INFINITY;
    const bool ok = lane < n_grid && isfinite(v);
    if (!ok) v = INFINITY;
    int idx = ok ? lane : 0x7fffffff;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
      const double ov = __shfl_xor(v, d, kWave);
      const int oi = __shfl_xor(idx, d, kWave);
      if (ov < v || (ov == v && oi < idx)) {
        v = ov;
        idx = oi;
      }
    }
    if (lane < n_grid) losses[lane] = lsh[lane];
    if (lane == 0) {
      const int b = (idx == 0x7fffffff) ? -1 : idx;
      *best_idx = b;
      best_sh = b;
    }
  }
  __syncthreads();
  const int b = best_sh;
  for (int64_t k = tid; k < K; k += kArgminThreads)
    s_best[k] = b >= 0 ? s_tab[(int64_t)b * K + k] : __builtin_nanf("");
}

// ------------------------------------------------------------------ host side
namespace {
size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }
}  // namespace

SearchPlan search_plan(int64_t n_tokens, int64_t in_features, int64_t out_features, int n_grid,
                       const QuantSpec& qs) {
  SearchPlan p;
  p.quant = qs;
  // many token tiles: produce each grid point's weight error once and contract
  // it (a fused kernel would rebuild it per token tile)
  const bool gemm = (n_tokens + 255) / 256 >= kGemmMinTokenTiles;
  if (gemm) {
    p.kernel = kGridGemm;
    p.tile_m = 256;
    p.tile_n = 256;
    p.n_t_tiles = (n_tokens + 255) / 256;
    p.n_o_tiles = (out_features + 255) / 256;
    p.grid_blocks = grid_gemm_blocks(p.n_t_tiles, p.n_o_tiles, n_grid);
  } else {
    p.kernel = kGridFused;
    p.tile_m = grid_tile_m(n_tokens, out_features, n_grid);
    p.tile_n = kGridBN;
    p.n_t_tiles = (n_tokens + p.tile_m - 1) / p.tile_m;
    p.n_o_tiles = (out_features + p.tile_n - 1) / p.tile_n;
    p.grid_blocks = (p.n_t_tiles * p.n_o_tiles + 7) / 8 * 8 * n_grid;
  }
  size_t off = 0;
  p.off_partials = off;
  off = align256(off + sizeof(double) * 2 * (size_t)n_grid * p.n_t_tiles * p.n_o_tiles);
  p.off_s = off;
  off = align256(off + sizeof(float) * (size_t)n_grid * in_features);
  p.off_inv_s = off;
  off = align256(off + sizeof(float) * (size_t)n_grid * in_features);
  p.off_params = off;
  if (gemm)  // fp16 weight error [grid point][out][in]
    off = align256(off + sizeof(_Float16) * (size_t)n_grid * out_features * in_features);
  else       // parameter records [grid point][group][out]
    off = align256(off + sizeof(GroupParams) * (size_t)n_grid * out_features *
                             (in_features / qs.group));
  p.bytes = off;
  return p;
}

hipError_t launch_search(const void* X, const void* W, const float* sal, int64_t N, int64_t K,
                         int64_t OUT, int n_grid, float sal_floor, double* losses,
                         int32_t* best_idx, float* s_best, void* workspace, const SearchPlan& p,
                         int stage_mask, hipStream_t stream) {
  char* ws = (char*)workspace;
  double* partials = (double*)(ws + p.off_partials);
  float* s_tab = (float*)(ws + p.off_s);
  float* inv_tab = (float*)(ws + p.off_inv_s);
  GroupParams* prm = (GroupParams*)(ws + p.off_params);
  const int G = p.quant.group;
  const int64_t ng = K / G;
  const float qmax = (float)((1 << p.quant.w_bit) - 1);
  const int sym = p.quant.zero_point ? 0 : 1;

  const bool gemm = p.kernel == kGridGemm;
  _Float16* dw = (_Float16*)(ws + p.off_params);
  if (stage_mask & 1) {  // prepare
    const int64_t nst = (int64_t)n_grid * K;
    hipLaunchKernelGGL(k_scale_table, dim3((unsigned)((nst + 255) / 256)), dim3(256), 0, stream,
                       sal, s_tab, inv_tab, K, n_grid, sal_floor);
    const dim3 pgrid((unsigned)((OUT + kParamsRows - 1) / kParamsRows), (unsigned)ng);
    const _Float16* Wh = (const _Float16*)W;
    // LDS: the group's scales for every grid point (and, producing the weight
    // error, their reciprocals)
    const int tables = gemm ? 2 : 1;
    if (G == 32) {
      const size_t lds = sizeof(float) * ParamsLds<32>::kPerGrid * n_grid * tables;
      if (gemm)
        hipLaunchKernelGGL((k_group_params<32, true>), pgrid, dim3(256), lds, stream, Wh, s_tab,
                           inv_tab, prm, dw, (int)OUT, (int)K, n_grid, qmax, sym);
      else
        hipLaunchKernelGGL((k_group_params<32, false>), pgrid, dim3(256), lds, stream, Wh, s_tab,
                           inv_tab, prm, dw, (int)OUT, (int)K, n_grid, qmax, sym);
    } else if (G == 64) {
      const size_t lds = sizeof(float) * ParamsLds<64>::kPerGrid * n_grid * tables;
      if (gemm)
        hipLaunchKernelGGL((k_group_params<64, true>), pgrid, dim3(256), lds, stream, Wh, s_tab,
                           inv_tab, prm, dw, (int)OUT, (int)K, n_grid, qmax, sym);
      else
        hipLaunchKernelGGL((k_group_params<64, false>), pgrid, dim3(256), lds, stream, Wh, s_tab,
                           inv_tab, prm, dw, (int)OUT, (int)K, n_grid, qmax, sym);
    } else {
      const size_t lds = sizeof(float) * ParamsLds<128>::kPerGrid * n_grid * tables;
      if (gemm)
        hipLaunchKernelGGL((k_group_params<128, true>), pgrid, dim3(256), lds, stream, Wh, s_tab,
                           inv_tab, prm, dw, (int)OUT, (int)K, n_grid, qmax, sym);
      else
        hipLaunchKernelGGL((k_group_params<128, false>), pgrid, dim3(256), lds, stream, Wh, s_tab,
                           inv_tab, prm, dw, (int)OUT, (int)K, n_grid, qmax, sym);
    }
  }
  if (stage_mask & 2) {  // grid
    if (gemm)
      launch_grid_gemm(X, dw, partials, N, K, OUT, p.n_t_tiles, p.n_o_tiles, n_grid, stream);
    else
      launch_grid((int)p.tile_m, G, X, W, s_tab, inv_tab, prm, partials, N, K, OUT, p.n_t_tiles,
                  p.n_o_tiles, n_grid, stream);
  }
  if (stage_mask & 4) {  // select
    hipLaunchKernelGGL(k_argmin, dim3(1), dim3(kArgminThreads), 0, stream, partials,
                       2 * p.n_t_tiles * p.n_o_tiles, n_grid, (double)N * (double)OUT, s_tab, K,
                       losses, best_idx, s_best);
  }
  return hipGetLastError();
}

}  // namespace awq
