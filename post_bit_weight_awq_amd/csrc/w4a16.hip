// Inference with the packed weights: y = x Wdq^T for fp16 activations and the
// 4-bit codes of awq_pack, Wdq[o, k] = (q[o, k] - z[o, g]) * step[o, g] with
// g = k / 128 (dev.to "AWQ: How Activation-Aware Quantization Saves 4-bit
// LLMs", "What do you actually deploy": W4A16 with groups of 128, where decode
// streams a quarter of the fp16 weight bytes; esaholic.com "What is AWQ
// Quantization?", INT4 codes in INT32 containers and W4A16 GEMM kernels;
// "AWQ > Salient Weight Preservation", step-size equation).
//
// HBM-bound at decode sizes: 0.5 byte of codes + 4/128 byte of step and zero
// per weight, read once.  A block (the MFMA kernel, k_w4a16, for more than 4
// tokens) owns 16 token rows and TILES 16-row output tiles (two, or four when
// that still gives the chip enough blocks); its 4 (or, on small grids, 8)
// wavefronts split the groups of 128 columns evenly and their partial outputs
// are added in LDS at the end (fixed order, no atomics).  The row tiles share
// each group's activation fragments (the activations are re-read per block,
// so more tiles cut that traffic); a wavefront reads a group's activations as
// whole cache lines and turns them into fragments through LDS, and requests
// the next group's codes, activations, steps and zeros before this group's
// arithmetic.
//   * Lane l holds output row o0 + 16 u + l % 16 of tile u and the 32-column
//     slice l / 16 of the current group: one 16-byte load of 32 codes.  Each of
//     its four words feeds one v_mfma_f32_16x16x32_f16 as the B operand; lane
//     l's A operand is the matching 8 activations of token t0 + l % 16.
//   * Codes become exact fp16 integers by bit placement: (nibble | 0x6400)
//     is the fp16 value 1024 + nibble, and one packed fp16 subtraction of 1024
//     leaves the code itself.  Two bit-select steps put them in column order.
//   * Per group, the MFMAs give A = sum_k x q and, with an all-ones B, the
//     activation sum S = sum_k x, both accumulated in fp32 from exact fp16
//     products; the group adds step * (A - z S) to the output.  The zero
//     point enters as one multiply per group, so it may be any stored fp16
//     value.
#include <map>
#include <mutex>
#include <utility>

#include "awq_device.h"
#include "awq_internal.h"

namespace awq {


__device__ __forceinline__ uint32_t lo_lo(uint32_t a, uint32_t b) {
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t hi_hi(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xffff0000u);
}

// kW4Tiles 16-row output tiles per wavefront (sharing the activations);
// kW4Slices wavefronts per block, each a share of the groups
template <int kW4Tiles, int kW4Slices>
__global__ void __launch_bounds__(kW4Slices * 64)
k_w4a16(const _Float16* __restrict__ X, int M, int K, int OUT, const uint4* __restrict__ qw,
        const _Float16* __restrict__ step16, const _Float16* __restrict__ zero16,
        float* __restrict__ Y) {
  constexpr int kW4Rows = 16 * kW4Tiles;  // output rows per block
  __shared__ float red[kW4Slices][kW4Rows * 16];
  // each wavefront's copy of one group's activations, 16 tokens x 256 bytes,
  // rows padded by 16 bytes so the fragment reads spread over the banks
  constexpr int kXRow = 17;  // uint4 per row
  __shared__ uint4 xs[kW4Slices][16 * kXRow];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int o0 = blockIdx.x * kW4Rows, t0 = blockIdx.y * 16;
  const int r16 = lane & 15, j4 = lane >> 4;
  const int ng = K >> 7;
  const int g0 = (int)((int64_t)wave * ng / kW4Slices);
  const int g1 = (int)((int64_t)(wave + 1) * ng / kW4Slices);
  // activation loads cover whole lines: load i of lane l reads the 16-byte
  // piece l % 16 of token 4 i + l / 16 of the group (4 tokens x 256 bytes per
  // load); tokens past the end read token 0 and count as zero
  const _Float16* xp[4];
  bool xok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + 4 * i + j4;
    xok[i] = t < M;
    xp[i] = X + (size_t)(xok[i] ? t : 0) * K + 8 * r16;
  }
  const uint4* qrow[kW4Tiles];
  const _Float16* srow[kW4Tiles];
  const _Float16* zrow[kW4Tiles];
#pragma unroll
  for (int u = 0; u < kW4Tiles; ++u) {
    const int orow = min(o0 + 16 * u + r16, OUT - 1);  // rows past the end re-read the last row
    qrow[u] = qw + (size_t)orow * (K >> 5) + j4;  // group g at qrow[u][4 g]
    srow[u] = step16 + (size_t)orow * ng;
    zrow[u] = zero16 + (size_t)orow * ng;
  }
  constexpr uint32_t kBias = 0x64006400u;  // fp16 1024 in both halves
  half8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (_Float16)1.0f;
  floatx4 y[kW4Tiles];
#pragma unroll
  for (int u = 0; u < kW4Tiles; ++u) y[u] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  floatx4 sum_x = {0.0f, 0.0f, 0.0f, 0.0f};
  // one group's operands; the next group's are requested before this group's
  // arithmetic (groups past the wavefront's range re-read its last group)
  struct Ops {
    uint4 q[kW4Tiles];
    uint4 xr[4];
    _Float16 st[kW4Tiles], zr[kW4Tiles];
  };
  auto load = [&](Ops& o, int g) {
    g = min(g, g1 - 1);
#pragma unroll
    for (int u = 0; u < kW4Tiles; ++u) {
      o.st[u] = srow[u][g];
      o.zr[u] = zrow[u][g];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o.xr[i] = xok[i] ? *(const uint4*)(xp[i] + 128 * g) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < kW4Tiles; ++u) o.q[u] = qrow[u][4 * g];
  };
  auto compute = [&](const Ops& o) {
    // the group's activations through the wavefront's LDS copy into fragment
    // order: lane l takes token l % 16, columns 32 (l / 16) + 8 j .. + 7.  A
    // wavefront's LDS operations run in order; the empty asm statements keep
    // the compiler from moving these accesses across one another.
    uint4* xw = xs[wave];
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < 4; ++i) xw[(4 * i + j4) * kXRow + r16] = o.xr[i];
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    uint4 xv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) xv[j] = xw[r16 * kXRow + 4 * j4 + j];
    asm volatile("" ::: "memory");
#pragma unroll
    for (int u = 0; u < kW4Tiles; ++u) {
      const uint32_t w[4] = {o.q[u].x, o.q[u].y, o.q[u].z, o.q[u].w};
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
        if (u == 0) as = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, ones, as, 0, 0, 0);
      }
      // the activation sums are the same for every row tile
      if (u == 0) sum_x = as;
      const float st = (float)o.st[u], zf = (float)o.zr[u];
      // register r of lane l: token t0 + 4 (l / 16) + r, output row o0 + 16 u + l % 16
#pragma unroll
      for (int r = 0; r < 4; ++r) y[u][r] = fmaf(st, fmaf(-zf, sum_x[r], aq[r]), y[u][r]);
    }
  };
  if (g0 < g1) {
    Ops a, b;
    load(a, g0);
    int g = g0;
    for (;;) {
      load(b, g + 1);
      compute(a);
      if (++g >= g1) break;
      load(a, g + 1);
      compute(b);
      if (++g >= g1) break;
    }
  }
#pragma unroll
  for (int u = 0; u < kW4Tiles; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][(16 * u + (lane & 15)) * 16 + 4 * (lane >> 4) + r] = y[u][r];
  __syncthreads();
  for (int e = threadIdx.x; e < kW4Rows * 16; e += kW4Slices * 64) {
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < kW4Slices; ++w) s += red[w][e];
    const int o = o0 + e / 16, t = t0 + e % 16;
    if (t < M && o < OUT) Y[(size_t)t * OUT + o] = s;
  }
}

// ---------------------------------------------------------------------------
// Up to MT (1, 2 or 4) tokens: a streaming product without MFMA.  Each block
// first copies the activations into LDS, each group of 8 reordered as
// (x0, x4), (x1, x5), (x2, x6), (x3, x7) to match the code pairs the bit
// placement yields, together with the sum of every 32-column slice.  Then
// each wavefront takes whole output rows, two at a time: lane l reads the
// 32-code slices l, l + 64, ... of both rows with all their 16-byte loads in
// flight, forms sum_k x q over each slice with v_dot2_f32_f16 (exact fp16
// products, binary32 sums), adds step * (that - zero * slice sum), and the
// wavefront adds its lanes at the end of the row pair.
constexpr int kGemvThreads = 512;

// SL: 16-byte loads per lane per row (K <= 64 * SL * 32); RW rows per pass.
template <int MT, int SL, int RW>
__global__ void __launch_bounds__(kGemvThreads)
k_w4a16_gemv(const _Float16* __restrict__ X, int M, int K, int OUT, const uint4* __restrict__ qw,
             const _Float16* __restrict__ step16, const _Float16* __restrict__ zero16,
             float* __restrict__ Y) {
  extern __shared__ uint4 lds[];  // MT x (K / 8) reordered activation octets, then slice sums
  const int n8 = K >> 3, ns = K >> 5, ng = K >> 7;
  float* xsum = (float*)(lds + MT * n8);  // [MT][ns]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int waves = gridDim.x * (kGemvThreads / 64);
  // a thread's staging loads are all requested before the first is stored
  // (one round trip instead of one per load)
  constexpr int kStage = 4;
  for (int e0 = tid; e0 < MT * n8; e0 += kStage * kGemvThreads) {
    uint4 v[kStage];
#pragma unroll
    for (int u = 0; u < kStage; ++u) {
      const int e = e0 + u * kGemvThreads;
      const int t = e / n8, c = e - t * n8;
      v[u] = make_uint4(0, 0, 0, 0);
      if (e < MT * n8 && t < M) v[u] = *(const uint4*)(X + (size_t)t * K + 8 * c);
    }
#pragma unroll
    for (int u = 0; u < kStage; ++u) {
      const int e = e0 + u * kGemvThreads;
      if (e < MT * n8)
        lds[e] = make_uint4(lo_lo(v[u].x, v[u].z), hi_hi(v[u].x, v[u].z), lo_lo(v[u].y, v[u].w),
                            hi_hi(v[u].y, v[u].w));
    }
  }
  __syncthreads();
  for (int e = tid; e < MT * ns; e += kGemvThreads) {
    const int t = e / ns, c = e - t * ns;
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 v = lds[t * n8 + 4 * c + j];
      s += f16_lo(v.x) + f16_hi(v.x) + f16_lo(v.y) + f16_hi(v.y) + f16_lo(v.z) + f16_hi(v.z) +
           f16_lo(v.w) + f16_hi(v.w);
    }
    xsum[e] = s;
  }
  __syncthreads();
  constexpr uint32_t kBias = 0x64006400u;
  typedef _Float16 half2v __attribute__((ext_vector_type(2)));
  for (int ob = blockIdx.x * (kGemvThreads / 64) + wave; ob < OUT; ob += RW * waves) {
    int orow[RW];
#pragma unroll
    for (int r = 0; r < RW; ++r) orow[r] = min(ob + r * waves, OUT - 1);  // past the end: repeat
    // The pass's steps and zeros, then its codes in the order the arithmetic
    // takes them, are all requested before any is used.  Steps and zeros stay
    // in registers of their own (each converted where it is used, so nothing
    // waits for them early), and each slice's arithmetic waits only for its
    // own codes: it starts while later codes still stream in.  Slices past the
    // row's end re-read its last slice and count with step 0, so loads and
    // arithmetic are straight-line code (branches here made the compiler wait
    // for every load before the first product, or sink loads into them).
    uint4 cw[RW][SL];
    _Float16 stp[RW][SL], zrp[RW][SL];
#pragma unroll
    for (int i = 0; i < SL; ++i) {
      const int c = min(lane + 64 * i, ns - 1);
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        stp[r][i] = step16[(size_t)orow[r] * ng + (c >> 2)];
        zrp[r][i] = zero16[(size_t)orow[r] * ng + (c >> 2)];
      }
    }
#pragma unroll
    for (int i = 0; i < SL; ++i) {
      const int c = min(lane + 64 * i, ns - 1);
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        __builtin_amdgcn_sched_barrier(0);
        cw[r][i] = qw[(size_t)orow[r] * ns + c];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    float y[RW][MT];
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int t = 0; t < MT; ++t) y[r][t] = 0.0f;
#pragma unroll
    for (int i = 0; i < SL; ++i) {
      // a slice past the row's end takes step 0: its finite contribution is +0
      const bool live = lane + 64 * i < ns;
      const int c = min(lane + 64 * i, ns - 1);
      {
        float xs[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) xs[t] = xsum[t * ns + c];
#pragma unroll
        for (int r = 0; r < RW; ++r) {
          const float st = live ? (float)stp[r][i] : 0.0f;
          const float zr = (float)zrp[r][i];
          const uint32_t w[4] = {cw[r][i].x, cw[r][i].y, cw[r][i].z, cw[r][i].w};
          float d[MT];
#pragma unroll
          for (int t = 0; t < MT; ++t) d[t] = 0.0f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            uint32_t p[4];
#pragma unroll
            for (int h = 0; h < 4; ++h) p[h] = sub_f16x2(((w[j] >> (4 * h)) & 0x000F000Fu) | kBias, kBias);
#pragma unroll
            for (int t = 0; t < MT; ++t) {
              const uint4 xq = lds[t * n8 + 4 * c + j];
              const uint32_t xp[4] = {xq.x, xq.y, xq.z, xq.w};
#pragma unroll
              for (int h = 0; h < 4; ++h)
                d[t] = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, p[h]),
                                              __builtin_bit_cast(half2v, xp[h]), d[t], false);
            }
          }
#pragma unroll
          for (int t = 0; t < MT; ++t) y[r][t] = fmaf(st, fmaf(-zr, xs[t], d[t]), y[r][t]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) y[r][t] += __shfl_xor(y[r][t], d, 64);
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        if (ob + r * waves < OUT) {
#pragma unroll
          for (int t = 0; t < MT; ++t)
            if (t < M) Y[(size_t)t * OUT + ob + r * waves] = y[r][t];
        }
      }
    }
  }
}

// Blocks of k_w4a16_gemv<MT, SL, RW> resident per compute unit on the current
// device, from the runtime's occupancy query (cached per device and kernel).
template <int MT, int SL, int RW>
static int gemv_blocks_per_cu(int dev, size_t lds) {
  static std::mutex mu;
  static std::map<std::pair<int, size_t>, int> cache;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_pair(dev, lds);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_w4a16_gemv<MT, SL, RW>,
                                                   kGemvThreads, lds) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  cache[key] = per_cu;
  return per_cu;
}

static int device_cus(int* dev_out) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    cus = 256;
  *dev_out = dev;
  return cus;
}

static size_t gemv_lds(int MT, int K) { return (size_t)MT * (K / 8) * 16 + (size_t)MT * (K / 32) * 4; }

// Rows the RW-row kernel covers in one round of resident blocks.
template <int MT, int SL, int RW>
static int64_t gemv_round_rows(int K) {
  int dev = 0;
  const int cus = device_cus(&dev);
  return (int64_t)gemv_blocks_per_cu<MT, SL, RW>(dev, gemv_lds(MT, K)) * cus *
         (kGemvThreads / 64) * RW;
}

template <int MT, int SL, int RW>
static void launch_gemv(const _Float16* X, int M, int K, int OUT, const uint4* qw,
                        const _Float16* st, const _Float16* zr, float* Y, hipStream_t stream) {
  const size_t lds = gemv_lds(MT, K);
  int dev = 0;
  const int cus = device_cus(&dev);
  const int rows_per_block = RW * (kGemvThreads / 64);
  const int want = (OUT + rows_per_block - 1) / rows_per_block;
  const int resident = gemv_blocks_per_cu<MT, SL, RW>(dev, lds) * cus;
  const int blocks = want < resident ? want : resident;
  hipLaunchKernelGGL((k_w4a16_gemv<MT, SL, RW>), dim3(blocks), dim3(kGemvThreads), lds, stream, X,
                     M, K, OUT, qw, st, zr, Y);
}

// SL = 16-byte code loads per lane per row, the smallest of 2 to 8 that
// covers the row (K <= 64 * SL * 32); RW rows per wavefront and pass, the
// fewest (1, 2, 3 or 4; at most 3 for SL > 4, whose registers allow no more)
// with which the resident blocks hold every row in one pass, else the most.
template <int MT, int SL>
static void launch_gemv_rw(const _Float16* X, int M, int K, int OUT, const uint4* qw,
                           const _Float16* st, const _Float16* zr, float* Y, hipStream_t stream) {
  if (OUT <= gemv_round_rows<MT, SL, 1>(K))
    launch_gemv<MT, SL, 1>(X, M, K, OUT, qw, st, zr, Y, stream);
  else if (OUT <= gemv_round_rows<MT, SL, 2>(K))
    launch_gemv<MT, SL, 2>(X, M, K, OUT, qw, st, zr, Y, stream);
  else if (OUT <= gemv_round_rows<MT, SL, 3>(K) || SL > 4)
    launch_gemv<MT, SL, 3>(X, M, K, OUT, qw, st, zr, Y, stream);
  else
    launch_gemv<MT, SL, 4>(X, M, K, OUT, qw, st, zr, Y, stream);
}

template <int MT>
static void launch_gemv_k(const _Float16* X, int M, int K, int OUT, const uint4* qw,
                          const _Float16* st, const _Float16* zr, float* Y, hipStream_t stream) {
  const int sl = (K / 32 + 63) / 64;
  if (sl <= 2)
    launch_gemv_rw<MT, 2>(X, M, K, OUT, qw, st, zr, Y, stream);
  else if (sl <= 3)
    launch_gemv_rw<MT, 3>(X, M, K, OUT, qw, st, zr, Y, stream);
  else if (sl <= 4)
    launch_gemv_rw<MT, 4>(X, M, K, OUT, qw, st, zr, Y, stream);
  else if (sl <= 5)
    launch_gemv_rw<MT, 5>(X, M, K, OUT, qw, st, zr, Y, stream);
  else if (sl <= 6)
    launch_gemv_rw<MT, 6>(X, M, K, OUT, qw, st, zr, Y, stream);
  else if (sl <= 7)
    launch_gemv_rw<MT, 7>(X, M, K, OUT, qw, st, zr, Y, stream);
  else
    launch_gemv_rw<MT, 8>(X, M, K, OUT, qw, st, zr, Y, stream);
}

hipError_t launch_w4a16(const void* X, int64_t M, int64_t K, int64_t OUT, const int32_t* qweight,
                        const void* step16, const void* zero16, float* Y, hipStream_t stream) {
  const _Float16* Xh = (const _Float16*)X;
  const uint4* qw = (const uint4*)qweight;
  const _Float16* st = (const _Float16*)step16;
  const _Float16* zr = (const _Float16*)zero16;
  // the streaming kernel keeps a row's codes in registers (K <= 16384) and its
  // MT staged token rows (1, 2, or 4 for 3 and 4 tokens) with their slice sums
  // in at most 64 KiB of LDS
  const int mt = M == 1 ? 1 : M == 2 ? 2 : 4;
  const bool gemv_fits = K <= 64 * 8 * 32 && M <= 4 && gemv_lds(mt, (int)K) <= 65536;
  if (gemv_fits) {
    if (M == 1)
      launch_gemv_k<1>(Xh, (int)M, (int)K, (int)OUT, qw, st, zr, Y, stream);
    else if (M == 2)
      launch_gemv_k<2>(Xh, (int)M, (int)K, (int)OUT, qw, st, zr, Y, stream);
    else
      launch_gemv_k<4>(Xh, (int)M, (int)K, (int)OUT, qw, st, zr, Y, stream);
    return hipGetLastError();
  }
  // four row tiles per block halve the activation re-reads again, but only
  // pay while the grid still covers most of the chip's 256 compute units
  // (13B block at 16 tokens: 26.3 and 47.2 us for qkv and gate/up against 29.8
  // and 53.0 with two tiles; 25.0 and 53.2 against 17.1 and 35.5 for the
  // 5120-row layers, whose 80 blocks leave most units idle)
  const int64_t t_tiles = (M + 15) / 16;
  const int64_t blocks4 = (OUT + 63) / 64 * t_tiles;
  if (blocks4 >= 192) {
    // eight wavefronts while the four-tile grid is under 1.5 blocks per unit
    // (qkv, 240 blocks: 23.6 against 24.6 us), four above (gate/up, 432
    // blocks: 39.5 against 42.6)
    const dim3 grid((unsigned)((OUT + 63) / 64), (unsigned)t_tiles);
    if (blocks4 < 384)
      hipLaunchKernelGGL((k_w4a16<4, 8>), grid, dim3(8 * 64), 0, stream, Xh, (int)M, (int)K,
                         (int)OUT, qw, st, zr, Y);
    else
      hipLaunchKernelGGL((k_w4a16<4, 4>), grid, dim3(4 * 64), 0, stream, Xh, (int)M, (int)K,
                         (int)OUT, qw, st, zr, Y);
  } else {
    // A grid this small holds few loads in flight, so its blocks take eight
    // wavefronts, each a shorter chain of groups (5120-row layers: 14.9 and
    // 31.0 us against 16.8 and 36.6 with four; sixteen measured no better,
    // and eight on the four-tile grid were slower on gate/up).  One tile per
    // block, twice the blocks, was slower still: 22.1 and 50.2 us, the
    // activation re-reads doubling.
    const dim3 grid((unsigned)((OUT + 31) / 32), (unsigned)t_tiles);
    hipLaunchKernelGGL((k_w4a16<2, 8>), grid, dim3(8 * 64), 0, stream, Xh, (int)M, (int)K,
                       (int)OUT, qw, st, zr, Y);
  }
  return hipGetLastError();
}

}  // namespace awq
