// Host-side interface between the C ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace awq {

struct GroupParams;
constexpr int kGridBN = 128;  // output features per grid-kernel tile

struct StatsPlan {
  int64_t col_blocks;
  int64_t row_chunks;
  int64_t rows_per_chunk;
  size_t workspace_bytes;
};
StatsPlan stats_plan(int64_t n_tokens, int64_t in_features);
hipError_t launch_act_stats(const void* X, int64_t n_tokens, int64_t in_features, float* sal,
                            void* workspace, hipStream_t stream);
// Allocation-free statistics: bytes of partials a shape needs (0 when one
// launch reads all of X), the fixed per-GPU scratch that holds them, and its
// device address on the current GPU.
constexpr size_t kStatsScratchBytes = (size_t)8 << 20;
size_t stats_scratch_need(int64_t n_tokens, int64_t in_features);
hipError_t scratch_address(void** out);

// Quantizer settings: group of 32, 64 or 128 columns, 3- or 4-bit codes,
// zero point (asymmetric) or symmetric.
struct QuantSpec {
  int group = 128;
  int w_bit = 4;
  bool zero_point = true;
};

// Grid-stage kernels: the fused producer-and-contraction kernels (the weight
// error rebuilt per token tile), or, for layers of many token tiles, the
// weight error of every grid point produced once by the preparation stage and
// a plain contraction (search_gemm.hip).
enum GridKernel { kGridFused = 0, kGridGemm = 1 };
// 256-token tiles from which the contraction path runs.  Producing the weight
// error costs a fixed 2 bytes per weight and grid point; measured on 4096- to
// 13824-wide layers, the fused kernels win up to 1024 tokens when the tokens
// fill their 512-token tiles (512 and 1024 tokens: 7-32 %), the contraction
// from 1152 tokens on (2-20 %)
constexpr int64_t kGemmMinTokenTiles = 5;

struct SearchPlan {
  int64_t tile_m, tile_n;        // tokens x outputs per tile
  int64_t n_t_tiles, n_o_tiles;  // tile counts
  int kernel;                    // GridKernel
  int64_t grid_blocks;           // blocks of the grid-kernel launch
  QuantSpec quant;
  size_t off_partials, off_s, off_inv_s;
  size_t off_params;             // fused: parameter records; contraction: weight error
  size_t bytes;
};
SearchPlan search_plan(int64_t n_tokens, int64_t in_features, int64_t out_features, int n_grid,
                       const QuantSpec& qs);
hipError_t launch_search(const void* X, const void* W, const float* sal, int64_t n_tokens,
                         int64_t in_features, int64_t out_features, int n_grid, float sal_floor,
                         double* losses, int32_t* best_idx, float* s_best, void* workspace,
                         const SearchPlan& plan, int stage_mask, hipStream_t stream);

int grid_tile_m(int64_t n_tokens, int64_t out_features, int n_grid);
void launch_grid_gemm(const void* X, const void* dW, double* partials, int64_t N, int64_t K,
                      int64_t OUT, int64_t nt, int64_t no, int n_grid, hipStream_t stream);
int64_t grid_gemm_blocks(int64_t nt, int64_t no, int n_grid);
void launch_grid(int tile_m, int group, const void* X, const void* W, const float* s_tab,
                 const float* inv_tab, const GroupParams* prm, double* partials, int64_t N,
                 int64_t K, int64_t OUT, int64_t nt, int64_t no, int n_grid, hipStream_t stream);
// largest grid the grid kernel is launched with (blocks of 256 threads in x)
constexpr int64_t kMaxGridBlocks = (int64_t)1 << 23;

hipError_t launch_w4a16(const void* X, int64_t M, int64_t K, int64_t OUT, const int32_t* qweight,
                        const void* step16, const void* zero16, float* Y, hipStream_t stream);
// largest token count of one W4A16 launch (16 tokens per block row of the grid)
constexpr int64_t kMaxW4Tokens = (int64_t)65535 * 16;

hipError_t launch_fold(const void* src, const float* s, int64_t rows, int64_t cols, void* dst,
                       hipStream_t stream);

hipError_t launch_select_top(const float* sal, int64_t n, int64_t n_keep, float* out,
                             hipStream_t stream);

hipError_t launch_pack(const void* W, const float* s, int64_t in_features, int64_t out_features,
                       const QuantSpec& qs, int32_t* qweight, void* step16, void* zero16,
                       hipStream_t stream);

}  // namespace awq
