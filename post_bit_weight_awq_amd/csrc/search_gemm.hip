// Contraction and squared error of the AWQ search on layers with many token
// tiles: the weight error of every grid point, dW_i = fp16(Wq_i - W), has
// been produced once per layer (k_group_params<G, true>: the codes of
// W diag(s_i) of the step-size equation of "AWQ > Salient Weight
// Preservation", dequantized and divided by s_i as the dev.to page's
// search_scale listing does), so this kernel is a plain MFMA contraction
// X dW_i^T whose squares are summed in registers: the quantized layer's
// output error, never written out.  All grid points run in one launch.
//
// Why a separate producer pays here: the fused kernel (search_grid.hip)
// rebuilds each weight-error tile once per token tile, and its block phases
// alternate between the producing VALU work and the MFMAs.  With dW in
// memory, all eight wavefronts only multiply, the tile is square (256 x 256:
// 32 KB of operands per 32 columns against 40 KB for the fused 512 x 128
// tile), and each dW tile is read by the token tiles of its pair while it
// sits in one XCD's L2.  The producer writes the weight error once (2 bytes
// per weight and grid point).
//
// Layout: block tile 256 tokens x 256 outputs, 8 wavefronts as 4 (tokens) x 2
// (outputs), each 64 x 128 as 4 x 8 16x16 tiles of v_mfma_f32_16x16x32_f16
// with fp32 accumulators in registers for the whole K loop.  K steps of 64
// columns: both operand tiles (256 rows x 128 bytes each) move into LDS by
// direct loads of 8 rows x 128 bytes per instruction (16-byte piece p of row
// r stored at p ^ (r & 7), so the fragment reads hit every bank once), one
// barrier per step.  The weight-error tile has two LDS stages and is loaded
// for step s + 1 at the start of step s; the activation tile has three and is
// loaded for step s + 2 in the middle of step s, between the MFMAs of its two
// 32-column halves (160 KB of LDS).  The load instructions stall the
// wavefront that issues them; with half of them out of the step's start the
// kernel ran 2-3 % faster on the 13B shapes than with them after all the
// MFMAs, and that 0.5-2.6 % faster than with all loads at the start (a third
// activation stage loaded at the start lost 3-5 %).  The gain depends on the
// exact order the compiler emits: the loads sit between two separate MFMA
// loops, pinned by scheduling barriers.  A step reads both halves' fragments
// first, then issues the MFMAs.  Rows past the last token or
// output re-read the last row and are masked in the epilogue.  Each tile
// writes its sum of squares (fp32 per lane, fp64 across the block) to its
// grid point's partial slot.  Block order: the 32 blocks an XCD holds at a
// time take 4 (grid point, output tile) pairs x 8 token tiles (grid_index.h),
// so they share both operand tiles in the XCD's L2; on the 13B shapes this
// order ran at 1314-1342 TFLOP/s against 1245-1305 for all 16 token tiles of
// 2 pairs at a time, whose activation re-reads missed L2 about half the time.
#include "awq_device.h"
#include "awq_internal.h"
#include "grid_index.h"

namespace awq {

constexpr int kGemmBM = 256, kGemmBN = 256, kGemmKC = 64;
constexpr int kGemmWM = 4, kGemmWN = 2;  // wavefront grid (tokens x outputs)
constexpr int kGemmXS = 3, kGemmWS = 2;  // LDS stages: activations, weight error

__global__ void __launch_bounds__(512, 1)
k_grid_gemm(const _Float16* __restrict__ X, const _Float16* __restrict__ dW,
            double* __restrict__ partials, int N, int K, int OUT, int nt, int no, int n_grid) {
  constexpr int KC = kGemmKC;
  constexpr int TM = kGemmBM / kGemmWM, TN = kGemmBN / kGemmWN;  // 64 x 128 per wavefront
  constexpr int MT = TM / 16, NT = TN / 16;
  constexpr int LOADS = kGemmBM * KC * 2 / 1024 / 8;  // per operand, wavefront and step
  static_assert(LOADS == 4, "the loop's vmcnt(4) counts one step's activation loads");
  constexpr int XS = kGemmXS, WS = kGemmWS;
  // all of the LDS: XS activation stages, then WS weight-error stages; the
  // epilogue's 8 partial sums reuse its start once the loop is done
  __shared__ __attribute__((aligned(16))) _Float16 lds[(XS * kGemmBM + WS * kGemmBN) * KC];
  _Float16* const sa = lds;
  _Float16* const sb = lds + XS * kGemmBM * KC;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / kGemmWN, wn = wave % kGemmWN;
  const gidx::GemmUnit un = gidx::gemm_unit_of_block(blockIdx.x, nt, no, n_grid * no);
  if (un.pair >= n_grid * no) return;
  const _Float16* xa = X + (size_t)un.t0 * K;
  const _Float16* xb = dW + ((size_t)un.ai * OUT + un.o0) * K;
  uint32_t oa[LOADS], ob[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    oa[i] = gidx::gemm_offset(un.t0, N, K, wave, LOADS, i, lane);
    ob[i] = gidx::gemm_offset(un.o0, OUT, K, wave, LOADS, i, lane);
  }
  auto dma = [&](const void* base, uint32_t off, const void* l) {
    const uint32_t la = (uint32_t)(uintptr_t)l;
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(off), "s"(base), "s"(la)
                 : "memory", "m0");
  };
  // step s's tiles go to stage s % XS (activations) and s % WS (weight error)
  auto load_x = [&](int s) {
    const _Float16* pa = xa + s * KC;
    _Float16* d = sa + (s % XS) * kGemmBM * KC;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) dma(pa, oa[i], d + (wave * LOADS + i) * 8 * KC);
  };
  auto load_w = [&](int s) {
    const _Float16* pb = xb + s * KC;
    _Float16* d = sb + (s % WS) * kGemmBN * KC;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) dma(pb, ob[i], d + (wave * LOADS + i) * 8 * KC);
  };
  // the lane's 16 bytes of a 16-row fragment: row (lane % 16), k half kh,
  // 8-column piece 4 kh + lane / 16 of the step
  auto frag = [&](const _Float16* base, int row, int kh) -> half8 {
    const int piece = 4 * kh + (lane >> 4);
    return *(const half8*)(&base[row * KC + 8 * (piece ^ (row & 7))]);
  };
  floatx4 acc[MT][NT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[m][n] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

  const int nk = K / KC;  // K is a multiple of 128, so nk >= 2
  load_x(0);
  load_x(1);
  load_w(0);
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  __syncthreads();
  half8 a0[MT], b0[NT], a1[MT], b1[NT];
  for (int s = 0; s < nk; ++s) {
    // the weight-error stage of step s + 1 last held step s - 1, which every
    // wavefront finished reading before the previous barrier
    if (s + 1 < nk) load_w(s + 1);
    const _Float16* ta = sa + (s % XS) * kGemmBM * KC;
    const _Float16* tb = sb + (s % WS) * kGemmBN * KC;
#pragma unroll
    for (int m = 0; m < MT; ++m) a0[m] = frag(ta, wm * TM + m * 16 + (lane & 15), 0);
#pragma unroll
    for (int n = 0; n < NT; ++n) b0[n] = frag(tb, wn * TN + n * 16 + (lane & 15), 0);
#pragma unroll
    for (int m = 0; m < MT; ++m) a1[m] = frag(ta, wm * TM + m * 16 + (lane & 15), 1);
#pragma unroll
    for (int n = 0; n < NT; ++n) b1[n] = frag(tb, wn * TN + n * 16 + (lane & 15), 1);
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int n = 0; n < NT; ++n)
        acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0[m], b0[n], acc[m][n], 0, 0, 0);
    // the activation stage of step s + 2 also last held step s - 1; its loads
    // go out between the two halves' MFMAs (the scheduling barriers keep them
    // there)
    const bool more = s + 2 < nk;
    if (more) {
      __builtin_amdgcn_sched_barrier(0);
      load_x(s + 2);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int n = 0; n < NT; ++n)
        acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1[m], b1[n], acc[m][n], 0, 0, 0);
    // step s + 1's tiles have landed (this wavefront's loads: the weight error
    // issued this step, the activations last step; this step's activation
    // loads, the last 4 issued, may stay in flight), and no wavefront still
    // reads this step's stages (the barrier)
    if (more)
      __builtin_amdgcn_s_waitcnt(0x0f74);  // vmcnt(4)
    else
      __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    __syncthreads();
  }

  // epilogue: register r of lane l is C[4 (l / 16) + r][l % 16] of its 16x16
  // tile; rows past the last token or output are masked
  const int tb = un.t0 + wm * TM + 4 * (lane >> 4);
  const int oc = un.o0 + wn * TN + (lane & 15);
  const bool full = (un.t0 + kGemmBM <= N) && (un.o0 + kGemmBN <= OUT);
  float sq = 0.0f;
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float d = acc[m][n][r];
        if (full || (tb + m * 16 + r < N && oc + n * 16 < OUT)) sq = fmaf(d, d, sq);
      }
  double dsum = (double)sq;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) dsum += __shfl_xor(dsum, d, kWave);
  double* const red = (double*)lds;  // the loop's last barrier ended every read and load
  if (lane == 0) red[wave] = dsum;
  __syncthreads();
  if (tid == 0) {
    double tot = 0.0;
#pragma unroll
    for (int w = 0; w < 8; ++w) tot += red[w];
    double* slot = partials + 2 * ((size_t)un.ai * nt * no + (size_t)un.tt * no + un.ot);
    slot[0] = tot;
    slot[1] = 0.0;
  }
}

int64_t grid_gemm_blocks(int64_t nt, int64_t no, int n_grid) {
  // in 64 bits first: the plan rejects layers above the launch limit
  return ((int64_t)n_grid * no + 7) / 8 * nt * 8;
}

void launch_grid_gemm(const void* X, const void* dW, double* partials, int64_t N, int64_t K,
                      int64_t OUT, int64_t nt, int64_t no, int n_grid, hipStream_t stream) {
  const int64_t blocks = gidx::gemm_blocks((int)nt, (int)(n_grid * no));
  hipLaunchKernelGGL(k_grid_gemm, dim3((unsigned)blocks), dim3(512), 0, stream,
                     (const _Float16*)X, (const _Float16*)dW, partials, (int)N, (int)K, (int)OUT,
                     (int)nt, (int)no, n_grid);
}

}  // namespace awq
