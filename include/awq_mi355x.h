/*
 * awq_mi355x.h -- C ABI of the MI355X (gfx950) AWQ per-layer search library.
 *
 * The library computes, for one linear layer at a time, the data-parallel core
 * of activation-aware weight quantization (AWQ):
 *
 *   1. activation saliency     sal_k = mean_t |X[t,k]|
 *   2. per-channel scales      s_i,k = max(sal_k, floor) ^ alpha_i, alpha_i = i / n_grid
 *   3. group quantization      of W diag(s_i): asymmetric INT4, groups of 128 along
 *                              in_features, step = (max - min) / 15,
 *                              zero = rint(-min / step), q = clamp(rint(w/step) + zero, 0, 15)
 *   4. dequantize and unscale  Wq_i = fp16(((q - zero) * step) * (1 / s_i))
 *   5. loss and choice         L_i = mean over tokens and outputs of (X Wq_i^T - X W^T)^2,
 *                              i* = first index of the minimum finite L_i; the codes of
 *                              W diag(s_i*) are then packed eight nibbles per int32 with
 *                              fp16 step and zero point per group.
 *
 * Sources, by page and section:
 *   - dev.to "AWQ: How Activation-Aware Quantization Saves 4-bit LLMs":
 *     channel_importance listing (step 1), search_scale listing (steps 2-5),
 *     "What do you actually deploy" (zero point, group 128, 4 bit).
 *   - mbrenndoerfer.com "AWQ > Salient Weight Preservation": step-size equation
 *     (step 3) and the scaling identity (why step 4 divides by s).
 *   - mbrenndoerfer.com "AWQ > Summary": saliency is the average absolute
 *     activation; one alpha per layer from a grid search.
 *   - esaholic.com "What is AWQ Quantization?", pipeline step "INT4 Weight
 *     Packing & Export": codes are packed into INT32 containers.
 *
 * Conventions for every call:
 *   - All tensors are dense, row-major, and live in device memory of the GPU
 *     that is current on the calling thread.  The caller owns every buffer;
 *     the library never allocates or frees device memory and keeps no device
 *     state between calls.  Scratch memory is a caller-provided workspace whose
 *     size the matching *_workspace_size call returns; the one exception,
 *     awq_act_stats_noalloc, uses a fixed array that is part of the library's
 *     device code (one copy per GPU).
 *   - Device pointers must be 16-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only enqueue
 *     work and return; results are valid once the stream has reached them.
 *     Calls on different streams with disjoint buffers may run concurrently.
 *   - Every argument is validated on the host before anything is enqueued; a
 *     failed check enqueues nothing and returns a negative awq_status.  A launch
 *     failure returns AWQ_ERR_HIP.  awq_last_error() then describes the failure
 *     (a thread-local string, valid until the thread's next call).
 */
#ifndef AWQ_MI355X_H
#define AWQ_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum awq_status {
  AWQ_OK = 0,
  AWQ_ERR_INVALID_ARG = -1, /* null pointer, bad size, misalignment       */
  AWQ_ERR_UNSUPPORTED = -2, /* configuration outside what is implemented  */
  AWQ_ERR_WORKSPACE = -3,   /* workspace smaller than the queried size    */
  AWQ_ERR_HIP = -4,         /* the HIP runtime reported an error          */
  AWQ_ERR_NONFINITE = -5    /* no grid point gave a finite loss: never
                               returned by a call (the search runs
                               asynchronously); it names the outcome that
                               best_idx_out = -1 reports after the stream
                               sync, as the search_scale listing keeps no
                               scale when no loss beats infinity          */
} awq_status;

/* Quantization settings (the quant_config of the dev.to page's "What do you
 * actually deploy" section, plus the search_scale listing's grid size and
 * saliency floor).  The method's setting is {4, 128, 20, 1e-4f, 1}.  Also
 * implemented, as ablations: w_bit = 3 (codes still one per nibble), group
 * sizes 64 and 32 (the dev.to page: finer groups trade scale storage for
 * accuracy), and zero_point = 0, the symmetric round-to-nearest of the dev.to
 * page's "Why does naive 4-bit quantization wreck LLM accuracy?":
 * step = max|w| / 2^(w_bit-1), codes clamped to the signed range and stored
 * with the fixed zero 2^(w_bit-1).  Other values give AWQ_ERR_UNSUPPORTED.
 * n_grid may be 1..64; sal_floor must be finite and > 0.  in_features must be
 * a multiple of 128 for every group size. */
typedef struct awq_config {
  int32_t w_bit;      /* bits per code: 4 (or 3)                           */
  int32_t group_size; /* weights per step/zero along in_features: 128 (or 64, 32) */
  int32_t n_grid;     /* grid points alpha_i = i / n_grid: default 20      */
  float sal_floor;    /* saliency clamp before the power: default 1e-4f    */
  int32_t zero_point; /* 1: asymmetric with a zero point; 0: symmetric     */
} awq_config;

/* Fills *cfg with the defaults {4, 128, 20, 1e-4f, 1}. */
void awq_default_config(awq_config* cfg);

/* Thread-local description of the last failed call on this thread ("" if none). */
const char* awq_last_error(void);

/* Library version string. */
const char* awq_version(void);

/* ------------------------------------------------------------------------
 * Step 1: activation statistics.
 * sal_out[k] = fp32( (sum_t |X[t,k]|) / n_tokens ), the sum exact (fp16
 * magnitudes are summed as integers in units of 2^-24), the quotient taken in
 * binary64 and rounded to binary32.
 *   X:        [n_tokens, in_features] fp16, read only
 *   sal_out:  [in_features] fp32, written
 *   n_tokens >= 1, in_features >= 8 and a multiple of 8.
 * Non-finite inputs follow IEEE sums of the magnitudes: a channel with a NaN
 * gets NaN, else a channel with an infinity gets +inf.
 * The call takes a caller workspace, unlike a plain (X, n_tokens,
 * in_features, sal_out, stream) form, on purpose: the column sums of a large
 * X are split over many blocks, and the workspace holds their exact per-row-
 * chunk partials (64-bit integers) so the total is exact and bit-for-bit
 * deterministic with no atomics and no memory held by the library.  Size:
 * between 8 * in_features and 8 * in_features * (1 + n_tokens / 64) bytes
 * (none is used when n_tokens <= 8192 and n_tokens * in_features <= 2^22: one
 * launch then reads all of X).  Its contents on entry do not matter.
 * Source: dev.to page, channel_importance listing; Summary page,
 * "Salient weight identification".
 * ---------------------------------------------------------------------- */
size_t awq_act_stats_workspace_size(int64_t n_tokens, int64_t in_features);
int awq_act_stats(const void* X, int64_t n_tokens, int64_t in_features, float* sal_out,
                  void* workspace, size_t workspace_bytes, void* stream);

/* The same statistics, bit for bit, without a workspace and without
 * allocating anything: for callers that cannot allocate device memory (code
 * recorded under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  The caller still passes X and sal_out.  The partial
 * sums go to a fixed 8 MiB scratch array that the library holds on each GPU
 * it runs on until the process ends (its address is looked up on the first
 * call on a device).  Shapes whose partials exceed it are rejected on the
 * host with AWQ_ERR_WORKSPACE before anything is enqueued: shapes with
 * n_tokens <= 8192 and n_tokens * in_features <= 2^22 need none, and the
 * rest need (row chunks) x in_features x 8 bytes, e.g. 3.4 MiB for
 * 4096 x 13824.  Every call on one GPU shares that GPU's array (each call
 * writes all it reads, so nothing carries over), so calls that overlap on
 * one GPU (different streams, or threads) race: serialize them. */
int awq_act_stats_noalloc(const void* X, int64_t n_tokens, int64_t in_features, float* sal_out,
                          void* stream);

/* ------------------------------------------------------------------------
 * Steps 2-5: the alpha-grid search of one layer, all grid points in one pass.
 *   X:            [n_tokens, in_features] fp16
 *   W:            [out_features, in_features] fp16 (fused layers: rows concatenated)
 *   sal:          [in_features] fp32 (from awq_act_stats or any source)
 *   losses_out:   [n_grid] float64: L_i, the mean squared output error
 *   best_idx_out: [1] int32: i*, or -1 when no L_i is finite (the outcome
 *                 AWQ_ERR_NONFINITE names; a caller reads it after the stream
 *                 has reached the call, since the call itself only enqueues)
 *   s_best_out:   [in_features] fp32: s_i* (all NaN when i* = -1)
 *   A NaN or infinite sal_k gives s = 1 at alpha = 0 and NaN or inf above it
 *   (the floor keeps a NaN), so every grid point above 0 has a NaN loss.
 *   in_features must be a multiple of 128; n_tokens, out_features >= 1.
 * The workspace (size from awq_search_workspace_size) holds the scale table,
 * the per-tile partial sums and either the per-group quantizer parameters
 * (layers of at most four 256-token tiles: a fused kernel quantizes,
 * dequantizes and contracts per tile of 512, 256 or 128 tokens x 128 outputs)
 * or, for more tokens, the fp16 weight error of every grid point,
 * 2 * n_grid * out_features * in_features bytes (produced once, then
 * contracted on tiles of 256 tokens x 256 outputs); awq_search_plan describes
 * the tiling and where the partials and scales are.  The squared output error is formed as
 * (X (Wq - W)^T)^2 with the weight error rounded once to fp16 (the same
 * quantity as (X Wq^T - X W^T)^2 up to that rounding), so no reference output
 * is stored.
 * Source: dev.to page, search_scale listing; Salient Weight Preservation page,
 * step-size equation.
 * ---------------------------------------------------------------------- */
typedef struct awq_search_plan {
  int64_t tile_tokens;     /* tokens per output tile                               */
  int64_t tile_out;        /* output features per output tile                      */
  int64_t n_token_tiles;   /* ceil(n_tokens / tile_tokens)                         */
  int64_t n_out_tiles;     /* ceil(out_features / tile_out)                        */
  size_t partials_offset;  /* double [n_grid][n_token_tiles][n_out_tiles][2]: the
                              sum of squared differences over a tile (not
                              averaged) is the sum of its two entries            */
  size_t scales_offset;    /* float [n_grid][in_features]: s_i                     */
  size_t workspace_bytes;  /* total workspace size                                 */
} awq_search_plan;

int awq_search_plan_query(int64_t n_tokens, int64_t in_features, int64_t out_features,
                          const awq_config* cfg, awq_search_plan* plan);
size_t awq_search_workspace_size(int64_t n_tokens, int64_t in_features, int64_t out_features,
                                 const awq_config* cfg);
int awq_search_layer(const void* X, const void* W, const float* sal, int64_t n_tokens,
                     int64_t in_features, int64_t out_features, const awq_config* cfg,
                     double* losses_out, int32_t* best_idx_out, float* s_best_out,
                     void* workspace, size_t workspace_bytes, void* stream);

/* The same search split into its three stages, for callers that time or
 * overlap them: stage_mask is an OR of the AWQ_STAGE_* bits, and
 * awq_search_layer(...) equals awq_search_layer_stages(AWQ_STAGE_ALL, ...).
 * A stage reads what the earlier stages left in the workspace, so the stages of
 * one search must run in order, on one workspace, with the same arguments.
 *   AWQ_STAGE_PREPARE: scale table and, for every grid point, the per-group
 *                      quantizer parameters or (more than four 256-token
 *                      tiles) the fp16 weight error (no reference output is
 *                      formed)
 *   AWQ_STAGE_GRID:    the MFMA contraction and squared errors of all grid
 *                      points (fused with the quantize-dequantize work on
 *                      layers of at most four token tiles)
 *   AWQ_STAGE_SELECT:  losses, argmin and s_best */
#define AWQ_STAGE_PREPARE 1
#define AWQ_STAGE_GRID 2
#define AWQ_STAGE_SELECT 4
#define AWQ_STAGE_ALL 7
int awq_search_layer_stages(int stage_mask, const void* X, const void* W, const float* sal,
                            int64_t n_tokens, int64_t in_features, int64_t out_features,
                            const awq_config* cfg, double* losses_out, int32_t* best_idx_out,
                            float* s_best_out, void* workspace, size_t workspace_bytes,
                            void* stream);

/* ------------------------------------------------------------------------
 * Packing: quantize W diag(s) (exact IEEE division for every code) and pack.
 *   W:            [out_features, in_features] fp16
 *   s:            [in_features] fp32, any positive scales (normally s_best_out)
 *   qweight_out:  [out_features, in_features / 8] int32; nibble j (bits 4j..4j+3)
 *                 of word w holds the code of column 8w + j
 *   step_out:     [out_features, in_features / group_size] fp16
 *   zero_out:     [out_features, in_features / group_size] fp16 (integer values)
 * A group whose values are all equal takes step = 1.  Codes follow cfg's
 * bit width and zero-point setting (3-bit codes take one nibble each);
 * in_features must be a multiple of 128.
 * Source: esaholic.com page, "INT4 Weight Packing & Export"; dev.to page,
 * quant_config; modelrefs.com page, memory example (one 16-bit scale per 128).
 * ---------------------------------------------------------------------- */
int awq_pack(const void* W, const float* s, int64_t in_features, int64_t out_features,
             const awq_config* cfg, int32_t* qweight_out, void* step_out, void* zero_out,
             void* stream);

/* ------------------------------------------------------------------------
 * Inference with the packed weights (W4A16): for every token t and output o
 *   Y[t, o] = sum_k X[t, k] * (q[o, k] - zero[o, k/128]) * step[o, k/128]
 * with q the 4-bit codes of awq_pack's qweight (nibble j of word w = column
 * 8w + j) and step/zero its fp16 group values.  The activations are what the
 * layer receives after the 1/s fold (x / s); fp16 products are exact and are
 * accumulated in binary32, the group's step and zero applied once per group
 * as step * (sum x q - zero * sum x).
 *   X:       [n_tokens, in_features] fp16, read only, 16-byte aligned
 *   qweight: [out_features, in_features/8] int32, 16-byte aligned
 *   step16, zero16: [out_features, in_features/128] fp16, 2-byte aligned
 *   Y:       [n_tokens, out_features] fp32, written, 4-byte aligned
 *   in_features a positive multiple of 128; 1 <= n_tokens <= 1048560.
 * Built for decode: up to 4 tokens stream each row's codes once without the
 * matrix units; more tokens run blocks of 16 tokens x 32 or 64 output rows
 * on them.  Either way the weights stream from HBM once when n_tokens <= 16
 * (HBM-bound at 0.53 byte per weight); larger n_tokens re-read them once per
 * 16 tokens.
 * Errors: AWQ_ERR_INVALID_ARG for NULL or misaligned pointers and sizes out
 * of range (nothing is enqueued); AWQ_ERR_HIP for a launch failure.
 * Source: dev.to page, "What do you actually deploy" (4-bit weights, 16-bit
 * activations, group size 128; decode moves a quarter of the weight bytes);
 * esaholic.com page, INT4 in INT32 containers and W4A16 GEMM kernels.
 * ---------------------------------------------------------------------- */
int awq_w4a16_matmul(const void* X, int64_t n_tokens, int64_t in_features, int64_t out_features,
                     const int32_t* qweight, const void* step16, const void* zero16, float* Y,
                     void* stream);

/* ------------------------------------------------------------------------
 * Folding 1/s into whatever produces the layer's input channels:
 *   dst[j, c] = fp16( fp32(src[j, c]) / s[j] )   (IEEE binary32 division)
 * for a [rows, cols] fp16 array whose row j feeds input channel j: a norm's
 * gain or bias (cols = 1), or a preceding linear's weight ([rows = its
 * out_features, cols = its in_features]) and bias (cols = 1).  Overflow gives
 * an infinity, as the division and rounding do.
 *   src, dst: fp16, 2-byte aligned; dst may be src (in place) but must not
 *             otherwise overlap it
 *   s:        [rows] fp32 (the chosen s_best), 4-byte aligned
 * Errors: AWQ_ERR_INVALID_ARG for NULL, misaligned or overlapping pointers
 * and sizes out of range (nothing is enqueued); AWQ_ERR_HIP for a launch
 * failure.
 * Source: mbrenndoerfer.com "AWQ > Salient Weight Preservation" (the
 * preceding normalization's per-channel scale absorbs 1/s_j); "AWQ > Summary",
 * "Per-channel scaling" (the inverse is fused into preceding layers).
 * ---------------------------------------------------------------------- */
int awq_fold_inverse_scale(const void* src, const float* s, int64_t rows, int64_t cols, void* dst,
                           void* stream);

/* ------------------------------------------------------------------------
 * Saliency ablations.
 * Weight-magnitude saliency needs no entry of its own: awq_act_stats on W
 * ([out_features, in_features] in place of X) gives mean_o |W[o, k]|.
 * Top-n selection: sal_out[k] = sal[k] for the n_keep largest saliencies
 * (equal values: lower k first) and 1.0f for every other k, so that only the
 * kept channels are scaled (s = 1^alpha = 1 elsewhere) when sal_out is
 * passed to awq_search_layer.
 *   sal, sal_out: [n] fp32, 4-byte aligned; sal_out may be sal (in place)
 *                 but must not otherwise overlap it; sal must hold no NaN
 *   0 <= n_keep <= n <= 2^20
 * Errors: AWQ_ERR_INVALID_ARG (nothing is enqueued); AWQ_ERR_HIP.
 * Source: dev.to page, "How does AWQ decide which weights to protect?"
 * (activation versus weight magnitude; protecting about 1% of channels);
 * esaholic.com page (the top 1% channels are scaled).
 * ---------------------------------------------------------------------- */
int awq_select_top_channels(const float* sal, int64_t n, int64_t n_keep, float* sal_out,
                            void* stream);

#ifdef __cplusplus
}
#endif

#endif /* AWQ_MI355X_H */
