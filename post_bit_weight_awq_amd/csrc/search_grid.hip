// The fused grid kernels of the AWQ search, for layers of at most four
// 256-token tiles (layers of more tokens produce the weight error once and
// contract it: search_gemm.hip): for one (grid point i, token tile, output
// tile) a block quantizes and dequantizes the weight tile of W diag(s_i)
// (asymmetric INT4, groups of 128; "AWQ > Salient Weight Preservation",
// step-size equation), divides it by s_i again (dev.to "AWQ: How
// Activation-Aware Quantization Saves 4-bit LLMs", search_scale listing),
// and reduces the squared output error over the tile in registers.
//
// The output error of the quantized layer is X Wq^T - X W^T = X (Wq - W)^T.
// The kernel contracts X with the weight error dW = fp16(Wq - W) (both
// operands fp16, the difference of two fp16 values rounded once) on the MFMA
// units, so neither the quantized output nor a reference output X W^T is ever
// formed: there is no reference GEMM and no N x OUT buffer.  The one rounding
// of dW has relative size <= 2^-11 and zero mean; it changes a loss by a
// second-order amount (measured ~1e-6 relative).
//
// Two kernels share this file.  k_grid_pp (after k_grid) runs the 512- and
// 256-token tiles, for groups of 32, 64 and 128 columns; k_grid runs the
// 128-token tile (the whole tile of small layers, and the halves of a split
// 256-token round).  The notes below describe k_grid; those of k_grid_pp
// stand above it.
//
// Layout (BM tokens x BN outputs per block, NW wavefronts, K steps of 32):
//   * NW = 4 wavefronts stacked along tokens, one per SIMD; each owns BM/NW
//     tokens x BN outputs as 16x16 tiles of v_mfma_f32_16x16x32_f16, whose
//     fp32 accumulators stay in registers for the whole K loop.
//   * Activations go from global memory straight into each wavefront's
//     A-fragment registers, one K step ahead.  The 16x16x32 fragment is 16
//     rows x 64 contiguous bytes, so each load instruction touches 16 cache
//     sectors: half as many as a 32x32 fragment, which matters because the
//     vector data-return path, not bandwidth, limits these loads.
//   * Weights take two LDS stages.  A coalesced load (four lanes per 64-byte
//     row segment) lands the raw fp16 tile in LDS; then wavefront w turns the
//     8-column chunk (w % 4) of rows (w / 4) * 64 + lane into the fake-
//     quantized fp16 tile that all wavefronts read as B fragments.  The
//     step's 32 scales and reciprocals travel with the raw tile into LDS and
//     are read as wavefront-wide broadcasts (no scalar loads in the loop:
//     they would share the LDS wait counter and force full drains); each
//     row's group parameters load once per quantization group (GS steps of
//     32 columns: a whole group ahead for groups of 128, one step ahead in
//     two rolling register sets for groups of 32 and 64).
//     The production cost is spread over the BM tokens of the tile.
//   * Pipeline at K step q: MFMAs on (A(q), Wq(q)), interleaved one MFMA to
//     two VALU instructions with producing Wq(q+1) from raw W(q+1); store raw
//     W(q+2) (loaded one step earlier); load raw W(q+3) and A(q+1).  Every
//     stage is double-buffered; one barrier per step.  The 512-token tile
//     gives each wavefront 32 MFMAs per step, enough to hide the production.
//   * Operand k mapping: lane l holds k0 + 8*(l/16) .. +7 of row (l % 16) for
//     both A (tokens) and B (outputs), so each MFMA sums matching k pairs.
//     Accumulator register r of lane l holds C[4*(l/16) + r][l % 16].
//   * Block order: linear block b runs on XCD b % 8.  Work unit u (one grid
//     point of one tile) is taken by the u-th block; the j-th unit an XCD
//     receives is grid point j % n_grid of tile 8*(j / n_grid) + xcd, so the
//     blocks resident on one XCD at a time are the grid points of one or two
//     tiles and share the tiles' activation and weight rows in that XCD's L2.
//   * Last round: when the units do not fill the chip a whole number of
//     times and the leftover units fill at most half of it, the leftover
//     units run as a second launch of the half-height kernel, two blocks per
//     unit (the halves of the tile's tokens, on the unit's XCD), so the last
//     round takes about half as long.  Each unit owns two partial-sum slots;
//     a whole-tile block writes its sum and a zero, a half-tile block its half.
#include <map>
#include <mutex>

#include "awq_device.h"
#include "awq_internal.h"
#include "grid_index.h"

namespace awq {

template <int BM, int BN, int NW, int GS>
__global__ void __launch_bounds__(NW * 64, 1)
k_grid(const _Float16* __restrict__ X, const _Float16* __restrict__ W,
       const float* __restrict__ s_tab, const float* __restrict__ inv_tab,
       const GroupParams* __restrict__ prm, double* __restrict__ partials, int N, int K,
       int OUT, int n_t_tiles, int n_o_tiles, int n_grid, int unit_base, int split) {
  constexpr int NT = NW * 64;
  constexpr int KC = 32;            // k per step (one 16x16x32 MFMA deep)
  constexpr int WMT = BM / NW;      // tokens per wavefront
  constexpr int MBW = WMT / 16;     // 16-row MFMA tiles per wavefront
  constexpr int NBW = BN / 16;      // 16-column MFMA tiles
  constexpr int NH = NBW / 2;       // B fragments are read in two halves
  constexpr int LDW = KC + 8;       // LDS row stride (halves): conflict-free 16-byte reads
  constexpr int PR = BN * 4 / NT;   // raw rows stored and produced per thread per step
  static_assert(MBW >= 1 && NBW % 2 == 0 && PR >= 1 && WMT % 16 == 0, "tile shape");
  __shared__ __attribute__((aligned(16))) _Float16 wq[2][BN * LDW];   // weight error fp16(Wq - W)
  __shared__ __attribute__((aligned(16))) _Float16 wraw[2][BN * LDW]; // raw fp16 weights
  __shared__ __attribute__((aligned(16))) float scl[2][2 * KC];       // s | 1/s of a step
  __shared__ double red[NW];

  static_assert(BN == 128, "the unit mapping assumes 128-row output tiles");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_tiles = n_t_tiles * n_o_tiles;
  // unit and token half of this block (whole tiles: one block per unit)
  const gidx::Unit un =
      gidx::unit_of_block(blockIdx.x, unit_base, split, n_grid, n_o_tiles, BM);
  const int ai = un.ai, T = un.T, h = un.h;
  if (T >= n_tiles) return;
  const int t0 = un.t0, o0 = un.o0;
  if (t0 >= N) {  // second half of a ragged last token tile: no rows
    if (threadIdx.x == 0) partials[2 * ((size_t)ai * n_tiles + T) + h] = 0.0;
    return;
  }
  const int ngroups = K / (KC * GS);  // quantization groups of 32 * GS columns
  const int nk = K / KC;               // a multiple of 4
  const float nz = opaque_neg_zero();

  // activation rows of this lane, as 32-bit offsets from the tile's first row
  // (rows past the end re-read the last row; their outputs are masked in the
  // epilogue)
  const _Float16* xt = X + (size_t)t0 * K;
  uint32_t pa[MBW];
#pragma unroll
  for (int m = 0; m < MBW; ++m) pa[m] = gidx::g_act_offset(t0, N, K, wave, WMT, m, lane);
  // coalesced raw-weight loads: thread t covers 16 bytes of row t/4 (+ NT/4 j),
  // as 32-bit offsets from the tile's first row
  const _Float16* wt = W + (size_t)o0 * K;
  uint32_t pwl[PR];
#pragma unroll
  for (int j = 0; j < PR; ++j) pwl[j] = gidx::g_w_offset(o0, OUT, K, tid, NT, j);
  // production: the wavefront-uniform chunk pc of rows prow0 + (NT/4) j
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int pc = wv & 3;
  const int prow0 = (wv >> 2) * 64 + lane;
  // parameters, layout [grid point][group][row]: uniform base + row offset
  const GroupParams* pt = prm + (size_t)ai * ngroups * OUT + o0;
  uint32_t pp[PR];
#pragma unroll
  for (int j = 0; j < PR; ++j) pp[j] = gidx::g_param_offset(o0, OUT, prow0, NT, j);
  // scale staging: threads 0..15 copy the step's 32 scales and 32 reciprocals
  const float* pst = s_tab + (size_t)ai * K;
  const float* pit = inv_tab + (size_t)ai * K;

  floatx4 acc[MBW][NBW];
#pragma unroll
  for (int m = 0; m < MBW; ++m)
#pragma unroll
    for (int n = 0; n < NBW; ++n) acc[m][n] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

  // Pipeline state is held in small by-value structs with fixed names (no
  // arrays indexed by step parity), so every stage stays in registers.
  struct AF {
    half8 v[MBW];  // activation fragments of one step
  };
  struct WR {
    uint4 v[PR];   // raw weights of one step, in flight
    float4 sc;     // threads 0..15: four of the step's scales or reciprocals
  };
  auto load_a = [&](int step) {
    AF r;
#pragma unroll
    for (int m = 0; m < MBW; ++m) r.v[m] = *(const half8*)(xt + pa[m] + step * KC);
    return r;
  };
  auto load_w = [&](int step) {
    WR r;
#pragma unroll
    for (int j = 0; j < PR; ++j) r.v[j] = *(const uint4*)(wt + pwl[j] + step * KC);
    if (tid < 16)
      r.sc = *(const float4*)((tid < 8 ? pst : pit) + 4 * (tid & 7) + step * KC);
    return r;
  };
  auto store_raw = [&](int buf, WR src) {
#pragma unroll
    for (int j = 0; j < PR; ++j)
      *(uint4*)(&wraw[buf][((tid >> 2) + (NT / 4) * j) * LDW + 8 * (tid & 3)]) = src.v[j];
    if (tid < 16) *(float4*)(&scl[buf][(tid < 8 ? 0 : KC) + 4 * (tid & 7)]) = src.sc;
  };
  // group parameters as float4: x = step, y = 1/step, z = -zero, w = 15 - zero
  struct GP {
    float4 v[PR];
  };
  auto load_params = [&](int grp) {
    GP g;
#pragma unroll
    for (int j = 0; j < PR; ++j) g.v[j] = *(const float4*)(pt + pp[j] + (size_t)grp * OUT);
    return g;
  };
  // dW(step) from raw buffer `buf` (weights and the step's scales) into LDS
  // buffer `buf`; the wavefront's 8 scales are broadcast reads
  auto produce = [&](int buf, GP gp) {
    const float4 s0 = *(const float4*)(&scl[buf][8 * pc]);
    const float4 s1 = *(const float4*)(&scl[buf][8 * pc + 4]);
    const float4 i0 = *(const float4*)(&scl[buf][KC + 8 * pc]);
    const float4 i1 = *(const float4*)(&scl[buf][KC + 8 * pc + 4]);
    const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
    const float iv[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
#pragma unroll
    for (int j = 0; j < PR; ++j) {
      const int row = prow0 + (NT / 4) * j;
      const uint4 r = *(const uint4*)(&wraw[buf][row * LDW + 8 * pc]);
      const float4 g = gp.v[j];  // step, 1/step, -zero, 15 - zero
      const uint32_t w[4] = {r.x, r.y, r.z, r.w};
      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float fa = mul_f16_f32<false>(w[e], sv[2 * e], nz);
        const float fb = mul_f16_f32<true>(w[e], sv[2 * e + 1], nz);
        const float ca = med3(rintf(fa * g.y), g.z, g.w) * g.x;
        const float cb = med3(rintf(fb * g.y), g.z, g.w) * g.x;
        // fp16 Wq pair, then the weight error dW = fp16(Wq - W) (one rounding
        // of the difference of two fp16 values)
        const uint32_t wq2 = mul_f32_to_f16x2(ca, iv[2 * e], cb, iv[2 * e + 1], nz);
        o[e] = sub_f16x2(wq2, w[e]);
      }
      *(uint4*)(&wq[buf][row * LDW + 8 * pc]) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  };
  auto mfma_half = [&](const AF& av, int buf, int h) {
    half8 bf[NH];
#pragma unroll
    for (int n = 0; n < NH; ++n)
      bf[n] = *(const half8*)(&wq[buf][((h * NH + n) * 16 + (lane & 15)) * LDW + 8 * (lane >> 4)]);
#pragma unroll
    for (int m = 0; m < MBW; ++m)
#pragma unroll
      for (int n = 0; n < NH; ++n)
        acc[m][h * NH + n] =
            __builtin_amdgcn_mfma_f32_16x16x32_f16(av.v[m], bf[n], acc[m][h * NH + n], 0, 0, 0);
  };
  // one K step: MFMAs on `cur` and Wq buffer `buf`, interleaved with producing
  // Wq(step+1) into the other buffer; then the raw store of `wst` into raw
  // buffer `buf` and a barrier.  The scheduler is asked for one MFMA, then two
  // VALU instructions, repeated, so the production work issues while the
  // matrix pipe runs instead of after it.
  auto step_body = [&](const AF& cur, int buf, GP gprod, WR wst) {
    mfma_half(cur, buf, 0);
    produce(buf ^ 1, gprod);
    mfma_half(cur, buf, 1);
    store_raw(buf, wst);
#pragma unroll
    for (int i = 0; i < MBW * NBW; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // VALU
    }
    __syncthreads();
  };

  // Pipeline at step q: MFMAs on A(q) and Wq(q) (LDS buffer q % 2),
  // interleaved with producing Wq(q+1) from raw W(q+1); store raw W(q+2)
  // (loaded during step q-1) into raw buffer q % 2; load raw W(q+3) and
  // A(q+1).  Loads past the last step re-read step nk - 1 (never used), which
  // keeps the body branch-free and every wait count exact.
  GP gcur = load_params(0);
  GP gnxt = load_params(min(GS == 4 ? 1 : 1 / GS, ngroups - 1));
  WR w = load_w(0);
  store_raw(0, w);
  w = load_w(1);
  store_raw(1, w);
  w = load_w(min(2, nk - 1));
  AF a0 = load_a(0), a1;
  __syncthreads();
  produce(0, gcur);
  __syncthreads();
  if constexpr (GS == 4) {
    // groups of 128 columns: the parameters change every 4 steps and load a
    // whole group ahead
    for (int gi = 0; gi < ngroups; ++gi) {
      const int q = 4 * gi;
      a1 = load_a(q + 1);
      step_body(a0, 0, gcur, w);  // produces Wq(q+1) from raw buffer 1
      w = load_w(min(q + 3, nk - 1));
      a0 = load_a(q + 2);
      step_body(a1, 1, gcur, w);
      w = load_w(min(q + 4, nk - 1));
      a1 = load_a(q + 3);
      step_body(a0, 0, gcur, w);
      w = load_w(min(q + 5, nk - 1));
      a0 = load_a(min(q + 4, nk - 1));
      step_body(a1, 1, gnxt, w);  // Wq(q+4): first step of the next group
      w = load_w(min(q + 6, nk - 1));
      gcur = gnxt;
      gnxt = load_params(min(gi + 2, ngroups - 1));
    }
  } else {
    // groups of 32 or 64 columns: step q produces Wq(q+1) with the parameters
    // of group (q+1)/GS; two register sets roll one step ahead
    GP ga = gnxt;  // group of step 1
    for (int b4 = 0; b4 < nk / 4; ++b4) {
      const int q = 4 * b4;
      GP gb = load_params(min((q + 2) / GS, ngroups - 1));
      a1 = load_a(q + 1);
      step_body(a0, 0, ga, w);
      w = load_w(min(q + 3, nk - 1));
      a0 = load_a(q + 2);
      ga = load_params(min((q + 3) / GS, ngroups - 1));
      step_body(a1, 1, gb, w);
      w = load_w(min(q + 4, nk - 1));
      a1 = load_a(q + 3);
      gb = load_params(min((q + 4) / GS, ngroups - 1));
      step_body(a0, 0, ga, w);
      w = load_w(min(q + 5, nk - 1));
      a0 = load_a(min(q + 4, nk - 1));
      ga = load_params(min((q + 5) / GS, ngroups - 1));
      step_body(a1, 1, gb, w);
      w = load_w(min(q + 6, nk - 1));
    }
  }

  // epilogue: the accumulators hold X dW^T for this wavefront's tokens;
  // register r of lane l is C[4*(l/16) + r][l % 16] of its 16x16 tile.  Rows
  // past the end of X or W re-read the last row and are masked here.
  const int tb = t0 + wave * WMT + 4 * (lane >> 4);
  const int oc = o0 + (lane & 15);
  const bool full = (t0 + BM <= N) && (o0 + BN <= OUT);
  double dsum = 0.0;
#pragma unroll
  for (int m = 0; m < MBW; ++m) {
    float sq = 0.0f;
#pragma unroll
    for (int n = 0; n < NBW; ++n) {
      const int o = oc + n * 16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = tb + m * 16 + r;
        const float d = acc[m][n][r];
        if (full || (t < N && o < OUT)) sq = fmaf(d, d, sq);
      }
    }
    dsum += (double)sq;
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) dsum += __shfl_xor(dsum, d, kWave);
  if (lane == 0) red[wave] = dsum;
  __syncthreads();
  if (tid == 0) {
    double tot = 0.0;
#pragma unroll
    for (int w = 0; w < NW; ++w) tot += red[w];
    double* slot = partials + 2 * ((size_t)ai * n_tiles + T);
    if (split == 1) {
      slot[0] = tot;
      slot[1] = 0.0;
    } else {
      slot[h] = tot;
    }
  }
}

// Grid kernel for groups of 128 columns (the 512- and 256-token tiles):
// ping-pong phases, operands staged in LDS by whole-line direct loads.
//
// Loads in the MFMA fragment shape (16 rows x 64 bytes per instruction) touch
// half of 16 cache lines each, and the vector memory path moves them at less
// than half the rate of loads that cover whole 128-byte lines (measured on
// this chip: ~21 against ~46 bytes per clock per compute unit from L2).  So
// activations and raw weights move in chunks of 64 columns (two K steps):
// each direct-to-LDS load covers 8 rows x 128 bytes, 16-byte piece p of row r
// stored at position p ^ (r & 7), which keeps the fragment reads and the
// producers' row-per-lane reads free of bank conflicts.
//
// The eight wavefronts form two groups of four (one wavefront per SIMD in
// each).  Every K step has two phases separated by block barriers.  In each
// phase one group multiplies and the other prepares, so on every SIMD one
// wavefront's MFMAs run beside the other wavefront's VALU and LDS work:
//   * preparing step r: produce the group's 64 rows of dW(r+1) (each
//     wavefront one 8-column piece), with step r's B fragments and, for even
//     r, its A fragments read into registers in batches between the pieces'
//     weight pairs;
//   * multiplying step r: the MFMAs, and between their two halves (on the
//     256-token tile: among the second half's MFMAs) the loads: for even r it
//     first reads step r+1's A fragments and then refills its activation
//     buffer with the next chunk; its weight load; its group's data for a
//     later column group.
// Group 0 prepares step r in phase 2r-1 and multiplies it in phase 2r;
// group 1 prepares it in phase 2r and multiplies it in phase 2r+1.  dW(j) is
// complete after phase 2j-2 and first read in phase 2j-1 (two dW buffers).
//
// Loads, each by the wavefront or group that uses the data:
//   * activations: a wavefront's own 64 rows, one buffer per wavefront,
//     refilled once both steps of its chunk have their fragments in registers;
//   * raw weights: a group's own 64 rows, ring of three chunks, each chunk
//     issued four to five steps before its first use;
//   * per-group parameters and scales: a group's own copy, two column groups
//     in flight (four for groups of 32 columns), each loaded in the multiply
//     phase of step GS*g - 3 for column group g of GS steps.
// The loads are inline assembly, so the compiler does not wait for them
// before every LDS read; at the end of each multiply phase a wavefront waits
// for all of its loads except that phase's own.  Nothing else in the loop
// uses the vector memory counter, which keeps those counts exact.
template <int BM, int BN, int GS>
__global__ void __launch_bounds__(512, 1)
k_grid_pp(const _Float16* __restrict__ X, const _Float16* __restrict__ W,
          const float* __restrict__ s_tab, const float* __restrict__ inv_tab,
          const GroupParams* __restrict__ prm, double* __restrict__ partials, int N, int K,
          int OUT, int n_t_tiles, int n_o_tiles, int n_grid, int unit_base, int split) {
  constexpr int NW = 8;
  constexpr int KC = 32;            // k per MFMA step
  constexpr int KCH = 64;           // k per load chunk
  constexpr int GC = 32 * GS;       // columns per quantization group (GS K steps)
  // group-data slots: a group's data is loaded in the multiply phase of step
  // GS*g - 3 (the latest from which it lands before dW(GS*g) is produced);
  // groups of 32 need four slots for the group it replaces to be finished
  constexpr int NGS = GS == 1 ? 4 : 2;
  constexpr int WMT = BM / NW;      // tokens per wavefront
  constexpr int MBW = WMT / 16;
  constexpr int NBW = BN / 16;
  constexpr int LDW = KC + 8;       // dW row stride (halves)
  constexpr int ALD = WMT / 8;      // activation loads per wavefront and chunk
  static_assert(BN == 128 && MBW >= 1 && ALD >= 1, "tile shape");
  __shared__ __attribute__((aligned(16))) _Float16 wq0[BN * LDW];
  __shared__ __attribute__((aligned(16))) _Float16 wq1[BN * LDW];
  __shared__ __attribute__((aligned(16))) _Float16 abuf[NW][WMT * KCH];  // per wavefront
  __shared__ __attribute__((aligned(16))) _Float16 wraw[3][BN * KCH];    // ring of chunks
  __shared__ __attribute__((aligned(16))) float4 gprm[NGS][2][64];       // [slot][group][row]
  __shared__ __attribute__((aligned(16))) float gscl[NGS][2][256];       // [slot][group] s | 1/s
  __shared__ double red[NW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_tiles = n_t_tiles * n_o_tiles;
  const gidx::Unit un =
      gidx::unit_of_block(blockIdx.x, unit_base, split, n_grid, n_o_tiles, BM);
  const int ai = un.ai, T = un.T, h = un.h;
  if (T >= n_tiles) return;
  const int t0 = un.t0, o0 = un.o0;
  if (t0 >= N) {
    if (threadIdx.x == 0) partials[2 * ((size_t)ai * n_tiles + T) + h] = 0.0;
    return;
  }
  const int ngroups = K / GC;
  const int nk = K / KC;     // a multiple of 4
  const int nch = K / KCH;   // chunks
  const float nz = opaque_neg_zero();
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int grp = wv >> 2;   // 0: multiplies first; 1: prepares first
  const int pc = wv & 3;     // the wavefront's 8-column piece of a step in production
  const int prow = 64 * grp + lane;

  // whole-line loads: lane l covers row l/8 of the load's 8 rows and stores
  // its 16 bytes at position l%8, i.e. it reads piece (l%8) ^ (row & 7)
  const _Float16* xt = X + (size_t)t0 * K;
  uint32_t pa[ALD];  // byte offsets from xt of this lane's pieces (chunk 0)
#pragma unroll
  for (int i = 0; i < ALD; ++i) pa[i] = gidx::pp_act_offset(t0, N, K, wave, WMT, i, lane);
  const _Float16* wt = W + (size_t)o0 * K;
  uint32_t pw[2];  // this wavefront's two weight loads per chunk: group rows 16pc + 8i ..
#pragma unroll
  for (int i = 0; i < 2; ++i) pw[i] = gidx::pp_w_offset(o0, OUT, K, grp, pc, i, lane);
  // per-group loads of the wavefront's group: wavefront 0 of the group the
  // parameters of its 64 rows, wavefront 1 the scales (lanes 0-31) and the
  // reciprocals (lanes 32-63, reached from the scale table's base: the
  // library places that table a short positive distance after the scales)
  const GroupParams* pgp = prm + (size_t)ai * ngroups * OUT;
  const uint32_t pgo = gidx::pp_param_offset(o0, OUT, grp, lane);
  const float* pgs = s_tab + (size_t)ai * K;
  // lanes 0 .. GC/4-1 the group's scales, the next GC/4 lanes its reciprocals
  // (further lanes repeat them: a load fills 64 x 16 bytes of LDS)
  const uint32_t pso =
      gidx::pp_scale_offset(lane, GC, (uint32_t)((const char*)inv_tab - (const char*)s_tab));

  floatx4 acc[MBW][NBW];
#pragma unroll
  for (int m = 0; m < MBW; ++m)
#pragma unroll
    for (int n = 0; n < NBW; ++n) acc[m][n] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

  // global address = uniform base + per-lane 32-bit byte offset
  auto dma = [&](const void* base, uint32_t off, const void* l) {
    const uint32_t la = (uint32_t)(uintptr_t)l;
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(off), "s"(base), "s"(la)
                 : "memory", "m0");
  };
  // Loads past the last chunk or group re-read the last one (never used)
  // into the slot the unclamped index selects, so the load counts never vary.
  auto dma_a = [&](int ch) {
    const _Float16* base = xt + min(ch, nch - 1) * KCH;
#pragma unroll
    for (int i = 0; i < ALD; ++i) dma(base, pa[i], &abuf[wv][8 * i * KCH]);
  };
  auto dma_w = [&](int ch, int i) {
    dma(wt + min(ch, nch - 1) * KCH, pw[i], &wraw[ch % 3][(64 * grp + 16 * pc + 8 * i) * KCH]);
  };
  auto dma_g = [&](int g) {
    const int src = min(g, ngroups - 1);
    if (pc == 0)
      dma(pgp + (size_t)src * OUT, pgo, &gprm[g % NGS][grp][0]);
    else if (pc == 1)
      dma(pgs + src * GC, pso, &gscl[g % NGS][grp][0]);
  };
  // whether step r's multiply phase loads group data, and how many loads the
  // wavefront issues in that phase (its wait at the phase end keeps them)
  auto g_phase = [&](int r) { return (r + 3) % GS == 0; };
  const bool gw = pc < 2;
  // this wavefront's part of dW(step): piece pc of row prow.  Split in two so
  // that its LDS reads can be issued before other reads and its arithmetic
  // run while those land.
  struct PIn {
    float4 s0, s1, i0, i1, gp;
    uint4 r;
  };
  auto produce_in = [&](int step) {
    PIn p;
    const int gs = (step / GS) % NGS, c = 8 * (step % GS) + 2 * pc;  // scale index / 4
    const float4* sc = (const float4*)&gscl[gs][grp][0];
    p.s0 = sc[c];
    p.s1 = sc[c + 1];
    p.i0 = sc[GC / 4 + c];
    p.i1 = sc[GC / 4 + c + 1];
    const int piece = 4 * (step & 1) + pc;
    p.r = *(const uint4*)(&wraw[(step >> 1) % 3][prow * KCH + 8 * (piece ^ (prow & 7))]);
    p.gp = gprm[gs][grp][lane];  // step, 1/step, -zero, 15 - zero
    return p;
  };
  // weights 2e and 2e+1 of the piece, as a packed pair of dW halves
  auto produce_pair = [&](const PIn& p, int e) -> uint32_t {
    const float sv[8] = {p.s0.x, p.s0.y, p.s0.z, p.s0.w, p.s1.x, p.s1.y, p.s1.z, p.s1.w};
    const float iv[8] = {p.i0.x, p.i0.y, p.i0.z, p.i0.w, p.i1.x, p.i1.y, p.i1.z, p.i1.w};
    const uint32_t w[4] = {p.r.x, p.r.y, p.r.z, p.r.w};
    const float4 gp = p.gp;
    const float fa = mul_f16_f32<false>(w[e], sv[2 * e], nz);
    const float fb = mul_f16_f32<true>(w[e], sv[2 * e + 1], nz);
    const float ca = med3(rintf(fa * gp.y), gp.z, gp.w) * gp.x;
    const float cb = med3(rintf(fb * gp.y), gp.z, gp.w) * gp.x;
    const uint32_t wq2 = mul_f32_to_f16x2(ca, iv[2 * e], cb, iv[2 * e + 1], nz);
    return sub_f16x2(wq2, w[e]);
  };
  auto store_piece = [&](const uint32_t (&o)[4], _Float16* dst) {
    *(uint4*)(&dst[prow * LDW + 8 * pc]) = make_uint4(o[0], o[1], o[2], o[3]);
  };
  auto produce = [&](int step, _Float16* dst) {
    const PIn p = produce_in(step);
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = produce_pair(p, e);
    store_piece(o, dst);
  };

  // operands of the next multiply phase: A of both steps of a chunk, B of one step
  half8 a0[MBW], a1[MBW], bv[NBW];
  auto read_a = [&](half8 (&av)[MBW], int s, int m0, int m1) {
#pragma unroll
    for (int m = m0; m < m1; ++m) {
      const int r = 16 * m + (lane & 15);
      const int piece = 4 * s + (lane >> 4);
      av[m] = *(const half8*)(&abuf[wv][r * KCH + 8 * (piece ^ (r & 7))]);
    }
  };
  auto read_b = [&](const _Float16* src, int n0, int n1) {
#pragma unroll
    for (int n = n0; n < n1; ++n)
      bv[n] = *(const half8*)(&src[(n * 16 + (lane & 15)) * LDW + 8 * (lane >> 4)]);
  };
  auto mfma_rows = [&](const half8 (&av)[MBW], int m0, int m1) {
#pragma unroll
    for (int m = m0; m < m1; ++m)
#pragma unroll
      for (int n = 0; n < NBW; ++n)
        acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[m], bv[n], acc[m][n], 0, 0, 0);
  };
  // multiply phase of step r (s = r % 2) on A fragments av.  The multiplying
  // wavefront also issues the loads: for s == 0 it first reads step r+1's A
  // fragments, then refills its activation buffer with chunk r/2 + 1; its
  // weight load for chunk (r+5)/2; for r % 4 == 1 its group's data for column
  // group (r+3)/4.  On the 512-token tile the loads go out in one burst between
  // the two halves of the MFMAs; on the 256-token tile, whose multiply phase is
  // half as long, one load follows each pair of MFMAs of the second half (each
  // placement measured the faster for its tile).
  // The multiplying wavefront runs at raised priority, so that on its SIMD
  // the other wavefront's VALU work fills the gaps between MFMAs rather than
  // delaying them.
  auto multiply = [&](const half8 (&av)[MBW], int r, int s) {
    __builtin_amdgcn_s_setprio(1);
    if (s == 0) read_a(a1, 1, 0, MBW);
    __builtin_amdgcn_sched_barrier(0);
    mfma_rows(av, 0, MBW / 2);
    __builtin_amdgcn_sched_barrier(0);
    if (s == 0) __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): A(r+1) read before the refill
    if (s == 0 && MBW == 2) {
      static_assert(MBW != 2 || NBW / 2 == ALD, "one activation load per MFMA pair");
      const _Float16* base = xt + min(r / 2 + 1, nch - 1) * KCH;
#pragma unroll
      for (int n = 0; n < NBW; n += 2) {
        __builtin_amdgcn_sched_barrier(0);
        dma(base, pa[n / 2], &abuf[wv][8 * (n / 2) * KCH]);
        __builtin_amdgcn_sched_barrier(0);
        acc[1][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[1], bv[n], acc[1][n], 0, 0, 0);
        acc[1][n + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[1], bv[n + 1], acc[1][n + 1], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      dma_w((r + 5) >> 1, (r + 1) & 1);
      if (g_phase(r)) dma_g((r + 3) / GS);
    } else {
      if (s == 0) dma_a(r / 2 + 1);
      dma_w((r + 5) >> 1, (r + 1) & 1);
      if (g_phase(r)) dma_g((r + 3) / GS);
      __builtin_amdgcn_sched_barrier(0);
      mfma_rows(av, MBW / 2, MBW);
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
  };
  // preparation of step r: this wavefront's part of dW(r+1) into `nxt`, the B
  // fragments of step r (dW(r) in `cur`) and for s == 0 its A fragments.  The
  // fragment reads go out in small batches between the four weight pairs, so
  // that the wavefront's arithmetic is not held up behind a queue of reads
  // (issuing them all first, then the arithmetic, measured 2-3 % slower).
  auto prepare = [&](int r, int s, const _Float16* cur, _Float16* nxt) {
    static_assert(NBW == 8, "read batches");
    const PIn p = produce_in(r + 1);
    uint32_t o[4];
    __builtin_amdgcn_sched_barrier(0);
    o[0] = produce_pair(p, 0);
    __builtin_amdgcn_sched_barrier(0);
    read_b(cur, 0, 3);
    __builtin_amdgcn_sched_barrier(0);
    o[1] = produce_pair(p, 1);
    __builtin_amdgcn_sched_barrier(0);
    read_b(cur, 3, 6);
    __builtin_amdgcn_sched_barrier(0);
    o[2] = produce_pair(p, 2);
    __builtin_amdgcn_sched_barrier(0);
    read_b(cur, 6, 8);
    if (s == 0) read_a(a0, 0, 0, MBW / 2);
    __builtin_amdgcn_sched_barrier(0);
    o[3] = produce_pair(p, 3);
    __builtin_amdgcn_sched_barrier(0);
    if (s == 0) read_a(a0, 0, MBW / 2, MBW);
    store_piece(o, nxt);
  };
  // after a multiply phase: all loads but that phase's own (for s == 0 the
  // activation chunk and a weight load, else a weight load; possibly the group
  // data) have landed.  For groups of 128 the group-data phases keep one load
  // (the group data then waits for nothing, the weight load with it); for
  // smaller groups, whose phases load group data far more often, the count is
  // exact.
  auto end_phase = [&](int wait_keep) {
    __builtin_amdgcn_sched_barrier(0);
    if (wait_keep == 1) __builtin_amdgcn_s_waitcnt(0x0f71);
    if (wait_keep == 2) __builtin_amdgcn_s_waitcnt(0x0f72);
    if (wait_keep == 1 + ALD) __builtin_amdgcn_s_waitcnt(0x0f70 | (1 + ALD));
    if (wait_keep == 2 + ALD) __builtin_amdgcn_s_waitcnt(0x0f70 | (2 + ALD));
    __syncthreads();
  };
  auto keep = [&](int r, int s) {
    const int own = s == 0 ? 1 + ALD : 1;
    return own + (GS < 4 && gw && g_phase(r) ? 1 : 0);
  };

  // prologue: the group data the loop does not load (groups 0 .. ceil(3/GS)-1),
  // activation chunk 0, weight chunks 0..2 of the group's rows; all of dW(0)
#pragma unroll
  for (int g = 0; g < (3 + GS - 1) / GS; ++g) dma_g(g);
  dma_a(0);
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    dma_w(c, 0);
    dma_w(c, 1);
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  __syncthreads();
  produce(0, wq0);
  __syncthreads();
  // The two groups run separate loops (a wave-uniform branch), so the
  // fragment registers written by a preparation are the ones the next
  // multiply phase reads; both loops pass the same barriers.
  if (grp == 0) {
    prepare(0, 0, wq0, wq1);  // phase -1
    end_phase(0);
    for (int k = 0; k < nk; k += 2) {
      multiply(a0, k, 0);           // phase 2k: step k
      end_phase(keep(k, 0));
      prepare(k + 1, 1, wq1, wq0);  // phase 2k+1
      end_phase(0);
      multiply(a1, k + 1, 1);       // phase 2k+2: step k+1
      end_phase(keep(k + 1, 1));
      prepare(k + 2, 0, wq0, wq1);  // phase 2k+3
      end_phase(0);
    }
  } else {
    end_phase(0);  // phase -1
    for (int k = 0; k < nk; k += 2) {
      prepare(k, 0, wq0, wq1);      // phase 2k
      end_phase(0);
      multiply(a0, k, 0);           // phase 2k+1: step k
      end_phase(keep(k, 0));
      prepare(k + 1, 1, wq1, wq0);  // phase 2k+2
      end_phase(0);
      multiply(a1, k + 1, 1);       // phase 2k+3: step k+1
      end_phase(keep(k + 1, 1));
    }
  }
  // the last loads (re-reads, never used) land before the block ends
  __builtin_amdgcn_s_waitcnt(0x0f70);

  const int tb = t0 + wave * WMT + 4 * (lane >> 4);
  const int oc = o0 + (lane & 15);
  const bool full = (t0 + BM <= N) && (o0 + BN <= OUT);
  double dsum = 0.0;
#pragma unroll
  for (int m = 0; m < MBW; ++m) {
    float sq = 0.0f;
#pragma unroll
    for (int n = 0; n < NBW; ++n) {
      const int o = oc + n * 16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = tb + m * 16 + r;
        const float d = acc[m][n][r];
        if (full || (t < N && o < OUT)) sq = fmaf(d, d, sq);
      }
    }
    dsum += (double)sq;
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) dsum += __shfl_xor(dsum, d, kWave);
  if (lane == 0) red[wave] = dsum;
  __syncthreads();
  if (tid == 0) {
    double tot = 0.0;
#pragma unroll
    for (int w = 0; w < NW; ++w) tot += red[w];
    double* slot = partials + 2 * ((size_t)ai * n_tiles + T);
    if (split == 1) {
      slot[0] = tot;
      slot[1] = 0.0;
    } else {
      slot[h] = tot;
    }
  }
}

int grid_tile_m(int64_t n_tokens, int64_t out_features, int n_grid) {
  // Largest token tile whose block count still fills the chip a few times
  // over; larger tiles spread the weight producer over more tokens and read
  // less from L2 per MFMA.
  const int64_t o_tiles = (out_features + kGridBN - 1) / kGridBN;
  for (int bm : {512, 256}) {
    const int64_t blocks = (n_tokens + bm - 1) / bm * o_tiles * n_grid;
    if (blocks >= 2 * 256) return bm;
  }
  return 128;
}

// The 8-wavefront tiles (512 and 256 tokens) run the ping-pong kernel, the
// 4-wavefront 128-token tile runs k_grid.  The ping-pong kernel reaches the
// reciprocal table from the scale table's base: search_plan places it right
// after that table on the next 256-byte boundary, a positive distance of at
// most 4 * 64 * 2^20 bytes (n_grid <= 64, in_features <= 2^20), which fits
// the kernel's 32-bit lane offsets.
template <int BM, int NW, int GS>
static void launch_one(unsigned blocks, int unit_base, int split, hipStream_t stream,
                       const _Float16* X, const _Float16* W, const float* s_tab,
                       const float* inv_tab, const GroupParams* prm, double* partials, int N,
                       int K, int OUT, int nt, int no, int n_grid) {
  if constexpr (NW == 8)
    hipLaunchKernelGGL((k_grid_pp<BM, kGridBN, GS>), dim3(blocks), dim3(NW * 64), 0, stream, X, W,
                       s_tab, inv_tab, prm, partials, N, K, OUT, nt, no, n_grid, unit_base, split);
  else
    hipLaunchKernelGGL((k_grid<BM, kGridBN, NW, GS>), dim3(blocks), dim3(NW * 64), 0, stream, X,
                       W, s_tab, inv_tab, prm, partials, N, K, OUT, nt, no, n_grid, unit_base,
                       split);
}

// Blocks of the whole-tile kernel that run at once on the current device
// (compute units x resident blocks per unit), cached per device.
template <int BM, int GS>
static int64_t resident_blocks() {
  static std::mutex mu;
  static std::map<int, int64_t> cache;  // key: device
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int cus = 0, per_cu = 0;
  hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_grid_pp<BM, kGridBN, GS>, 512, 0);
  if (e != hipSuccess) return 0;
  const int64_t r = (int64_t)cus * per_cu;
  cache[dev] = r;
  return r;
}

template <int BM, int HBM, int HNW, int GS>
static void launch_split(int64_t units, hipStream_t stream, const _Float16* X,
                         const _Float16* W, const float* s_tab, const float* inv_tab,
                         const GroupParams* prm, double* partials, int N, int K, int OUT, int nt,
                         int no, int n_grid) {
  const int64_t slots = resident_blocks<BM, GS>();
  int64_t whole = units;
  if (slots > 0) {
    const int64_t rest = units % slots;
    if (units > slots && rest > 0 && rest % 8 == 0 && 2 * rest <= slots) whole = units - rest;
  }
  launch_one<BM, 8, GS>((unsigned)whole, 0, 1, stream, X, W, s_tab, inv_tab, prm, partials, N, K,
                        OUT, nt, no, n_grid);
  if (whole < units)  // whole and units are multiples of 8
    launch_one<HBM, HNW, GS>((unsigned)(2 * (units - whole)), (int)whole, 2, stream, X, W, s_tab,
                             inv_tab, prm, partials, N, K, OUT, nt, no, n_grid);
}

template <int GS>
static void launch_tiles(int tile_m, int64_t units, hipStream_t stream, const _Float16* X,
                         const _Float16* W, const float* s_tab, const float* inv_tab,
                         const GroupParams* prm, double* partials, int N, int K, int OUT, int nt,
                         int no, int n_grid) {
  switch (tile_m) {
    case 512:
      launch_split<512, 256, 8, GS>(units, stream, X, W, s_tab, inv_tab, prm, partials, N, K, OUT,
                                    nt, no, n_grid);
      break;
    case 256:
      launch_split<256, 128, 4, GS>(units, stream, X, W, s_tab, inv_tab, prm, partials, N, K, OUT,
                                    nt, no, n_grid);
      break;
    default:
      launch_one<128, 4, GS>((unsigned)units, 0, 1, stream, X, W, s_tab, inv_tab, prm, partials,
                             N, K, OUT, nt, no, n_grid);
      break;
  }
}

void launch_grid(int tile_m, int group, const void* X, const void* W, const float* s_tab,
                 const float* inv_tab, const GroupParams* prm, double* partials, int64_t N,
                 int64_t K, int64_t OUT, int64_t nt, int64_t no, int n_grid, hipStream_t stream) {
  const int64_t units = (nt * no + 7) / 8 * 8 * n_grid;
  const _Float16* Xh = (const _Float16*)X;
  const _Float16* Wh = (const _Float16*)W;
  if (group == 32)
    launch_tiles<1>(tile_m, units, stream, Xh, Wh, s_tab, inv_tab, prm, partials, (int)N, (int)K,
                    (int)OUT, (int)nt, (int)no, n_grid);
  else if (group == 64)
    launch_tiles<2>(tile_m, units, stream, Xh, Wh, s_tab, inv_tab, prm, partials, (int)N, (int)K,
                    (int)OUT, (int)nt, (int)no, n_grid);
  else
    launch_tiles<4>(tile_m, units, stream, Xh, Wh, s_tab, inv_tab, prm, partials, (int)N, (int)K,
                    (int)OUT, (int)nt, (int)no, n_grid);
}

}  // namespace awq
