// C ABI of the AWQ search library: argument validation, workspace planning and
// kernel launches.  All checks run on the host before anything is enqueued.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/awq_mi355x.h"
#include "awq_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return AWQ_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Largest dimensions accepted: they keep every index inside int64 and the
// launch grids inside their limits.
constexpr int64_t kMaxTokens = (int64_t)1 << 24;  // exact 64-bit saliency sums
constexpr int64_t kMaxFeatures = (int64_t)1 << 20;
constexpr int64_t kMaxWeights = (int64_t)1 << 34;  // one work-item per 8 weights < 2^32

int check_config(const awq_config* cfg) {
  if (!cfg) return fail(AWQ_ERR_INVALID_ARG, "cfg is NULL");
  if (cfg->w_bit != 4 && cfg->w_bit != 3)
    return fail(AWQ_ERR_UNSUPPORTED, "w_bit=%d: 3 and 4 are implemented", cfg->w_bit);
  if (cfg->group_size != 128 && cfg->group_size != 64 && cfg->group_size != 32)
    return fail(AWQ_ERR_UNSUPPORTED, "group_size=%d: 32, 64 and 128 are implemented",
                cfg->group_size);
  if (cfg->zero_point != 1 && cfg->zero_point != 0)
    return fail(AWQ_ERR_UNSUPPORTED, "zero_point=%d: 1 (asymmetric) or 0 (symmetric)",
                cfg->zero_point);
  if (cfg->n_grid < 1 || cfg->n_grid > 64)
    return fail(AWQ_ERR_INVALID_ARG, "n_grid=%d outside 1..64", cfg->n_grid);
  if (!(cfg->sal_floor > 0.0f) || !(cfg->sal_floor < 3.4e38f))
    return fail(AWQ_ERR_INVALID_ARG, "sal_floor must be finite and > 0");
  return AWQ_OK;
}

int check_dims(int64_t n_tokens, int64_t in_features, int64_t out_features, bool need_tokens,
               bool need_out, int64_t in_multiple) {
  if (need_tokens && (n_tokens < 1 || n_tokens > kMaxTokens))
    return fail(AWQ_ERR_INVALID_ARG, "n_tokens=%lld outside 1..%lld", (long long)n_tokens,
                (long long)kMaxTokens);
  if (in_features < in_multiple || in_features > kMaxFeatures || in_features % in_multiple)
    return fail(AWQ_ERR_INVALID_ARG, "in_features=%lld must be a positive multiple of %lld (max %lld)",
                (long long)in_features, (long long)in_multiple, (long long)kMaxFeatures);
  if (need_out && (out_features < 1 || out_features > kMaxFeatures))
    return fail(AWQ_ERR_INVALID_ARG, "out_features=%lld outside 1..%lld", (long long)out_features,
                (long long)kMaxFeatures);
  if (need_out && out_features * in_features > kMaxWeights)
    return fail(AWQ_ERR_INVALID_ARG, "out_features*in_features=%lld above %lld",
                (long long)(out_features * in_features), (long long)kMaxWeights);
  return AWQ_OK;
}

int check_ptr(const void* p, const char* name) {
  if (!p) return fail(AWQ_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(AWQ_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return AWQ_OK;
}

awq::QuantSpec quant_spec(const awq_config* cfg) {
  awq::QuantSpec q;
  q.group = cfg->group_size;
  q.w_bit = cfg->w_bit;
  q.zero_point = cfg->zero_point != 0;
  return q;
}

int hip_result(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(AWQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

void awq_default_config(awq_config* cfg) {
  if (!cfg) return;
  cfg->w_bit = 4;
  cfg->group_size = 128;
  cfg->n_grid = 20;
  cfg->sal_floor = 1e-4f;
  cfg->zero_point = 1;
}

const char* awq_last_error(void) { return g_err; }

const char* awq_version(void) { return "awq_mi355x 0.1 gfx950"; }

size_t awq_act_stats_workspace_size(int64_t n_tokens, int64_t in_features) {
  if (check_dims(n_tokens, in_features, 1, true, false, 8) != AWQ_OK) return 0;
  return awq::stats_plan(n_tokens, in_features).workspace_bytes;
}

int awq_act_stats(const void* X, int64_t n_tokens, int64_t in_features, float* sal_out,
                  void* workspace, size_t workspace_bytes, void* stream) {
  int rc;
  if ((rc = check_dims(n_tokens, in_features, 1, true, false, 8))) return rc;
  if ((rc = check_ptr(X, "X")) || (rc = check_ptr(sal_out, "sal_out")) ||
      (rc = check_ptr(workspace, "workspace")))
    return rc;
  const size_t need = awq::stats_plan(n_tokens, in_features).workspace_bytes;
  if (workspace_bytes < need)
    return fail(AWQ_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, need);
  return hip_result(awq::launch_act_stats(X, n_tokens, in_features, sal_out, workspace,
                                          (hipStream_t)stream),
                    "awq_act_stats launch");
}

int awq_act_stats_noalloc(const void* X, int64_t n_tokens, int64_t in_features, float* sal_out,
                          void* stream) {
  int rc;
  if ((rc = check_dims(n_tokens, in_features, 1, true, false, 8))) return rc;
  if ((rc = check_ptr(X, "X")) || (rc = check_ptr(sal_out, "sal_out"))) return rc;
  const size_t need = awq::stats_scratch_need(n_tokens, in_features);
  if (need > awq::kStatsScratchBytes)
    return fail(AWQ_ERR_WORKSPACE,
                "n_tokens=%lld x in_features=%lld needs %zu bytes of partial sums, above the "
                "%zu-byte scratch of awq_act_stats_noalloc (awq_act_stats takes a workspace)",
                (long long)n_tokens, (long long)in_features, need, awq::kStatsScratchBytes);
  void* ws = nullptr;
  if ((rc = hip_result(awq::scratch_address(&ws), "awq_act_stats_noalloc scratch address")))
    return rc;
  return hip_result(awq::launch_act_stats(X, n_tokens, in_features, sal_out, ws,
                                          (hipStream_t)stream),
                    "awq_act_stats_noalloc launch");
}

int awq_search_plan_query(int64_t n_tokens, int64_t in_features, int64_t out_features,
                          const awq_config* cfg, awq_search_plan* plan) {
  int rc;
  if ((rc = check_config(cfg))) return rc;
  if ((rc = check_dims(n_tokens, in_features, out_features, true, true, 128))) return rc;
  if (!plan) return fail(AWQ_ERR_INVALID_ARG, "plan is NULL");
  const awq::SearchPlan p = awq::search_plan(n_tokens, in_features, out_features, cfg->n_grid,
                                                 quant_spec(cfg));
  if (p.grid_blocks > awq::kMaxGridBlocks)
    return fail(AWQ_ERR_INVALID_ARG, "layer too large for one search launch (%lld tiles)",
                (long long)(p.n_t_tiles * p.n_o_tiles));
  plan->tile_tokens = p.tile_m;
  plan->tile_out = p.tile_n;
  plan->n_token_tiles = p.n_t_tiles;
  plan->n_out_tiles = p.n_o_tiles;
  plan->partials_offset = p.off_partials;
  plan->scales_offset = p.off_s;
  plan->workspace_bytes = p.bytes;
  return ok();
}

size_t awq_search_workspace_size(int64_t n_tokens, int64_t in_features, int64_t out_features,
                                 const awq_config* cfg) {
  awq_search_plan plan;
  if (awq_search_plan_query(n_tokens, in_features, out_features, cfg, &plan) != AWQ_OK) return 0;
  return plan.workspace_bytes;
}

int awq_search_layer(const void* X, const void* W, const float* sal, int64_t n_tokens,
                     int64_t in_features, int64_t out_features, const awq_config* cfg,
                     double* losses_out, int32_t* best_idx_out, float* s_best_out,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return awq_search_layer_stages(AWQ_STAGE_ALL, X, W, sal, n_tokens, in_features, out_features,
                                 cfg, losses_out, best_idx_out, s_best_out, workspace,
                                 workspace_bytes, stream);
}

int awq_search_layer_stages(int stage_mask, const void* X, const void* W, const float* sal,
                            int64_t n_tokens, int64_t in_features, int64_t out_features,
                            const awq_config* cfg, double* losses_out, int32_t* best_idx_out,
                            float* s_best_out, void* workspace, size_t workspace_bytes,
                            void* stream) {
  int rc;
  if (stage_mask < 1 || stage_mask > AWQ_STAGE_ALL)
    return fail(AWQ_ERR_INVALID_ARG, "stage_mask=%d: must be a non-empty OR of AWQ_STAGE_*",
                stage_mask);
  if ((rc = check_config(cfg))) return rc;
  if ((rc = check_dims(n_tokens, in_features, out_features, true, true, 128))) return rc;
  if ((rc = check_ptr(X, "X")) || (rc = check_ptr(W, "W")) || (rc = check_ptr(sal, "sal")) ||
      (rc = check_ptr(losses_out, "losses_out")) ||
      (rc = check_ptr(s_best_out, "s_best_out")) || (rc = check_ptr(workspace, "workspace")))
    return rc;
  if (!best_idx_out) return fail(AWQ_ERR_INVALID_ARG, "best_idx_out is NULL");
  const awq::SearchPlan p = awq::search_plan(n_tokens, in_features, out_features, cfg->n_grid,
                                                 quant_spec(cfg));
  if (p.grid_blocks > awq::kMaxGridBlocks)
    return fail(AWQ_ERR_INVALID_ARG, "layer too large for one search launch (%lld tiles)",
                (long long)(p.n_t_tiles * p.n_o_tiles));
  if (workspace_bytes < p.bytes)
    return fail(AWQ_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, p.bytes);
  return hip_result(awq::launch_search(X, W, sal, n_tokens, in_features, out_features,
                                       cfg->n_grid, cfg->sal_floor, losses_out, best_idx_out,
                                       s_best_out, workspace, p, stage_mask, (hipStream_t)stream),
                    "awq_search_layer launch");
}

int awq_pack(const void* W, const float* s, int64_t in_features, int64_t out_features,
             const awq_config* cfg, int32_t* qweight_out, void* step_out, void* zero_out,
             void* stream) {
  int rc;
  if ((rc = check_config(cfg))) return rc;
  if ((rc = check_dims(1, in_features, out_features, false, true, 128))) return rc;
  if ((rc = check_ptr(W, "W")) || (rc = check_ptr(s, "s")) ||
      (rc = check_ptr(qweight_out, "qweight_out")))
    return rc;
  if (!step_out || !zero_out) return fail(AWQ_ERR_INVALID_ARG, "step_out/zero_out is NULL");
  if (((uintptr_t)step_out & 1u) || ((uintptr_t)zero_out & 1u))
    return fail(AWQ_ERR_INVALID_ARG, "step_out/zero_out must be 2-byte aligned");
  return hip_result(awq::launch_pack(W, s, in_features, out_features, quant_spec(cfg), qweight_out,
                                     step_out, zero_out, (hipStream_t)stream),
                    "awq_pack launch");
}

int awq_w4a16_matmul(const void* X, int64_t n_tokens, int64_t in_features, int64_t out_features,
                     const int32_t* qweight, const void* step16, const void* zero16, float* Y,
                     void* stream) {
  int rc;
  if ((rc = check_dims(1, in_features, out_features, false, true, 128))) return rc;
  if (n_tokens < 1 || n_tokens > awq::kMaxW4Tokens)
    return fail(AWQ_ERR_INVALID_ARG, "n_tokens=%lld outside 1..%lld", (long long)n_tokens,
                (long long)awq::kMaxW4Tokens);
  if ((rc = check_ptr(X, "X")) || (rc = check_ptr(qweight, "qweight"))) return rc;
  if (!step16 || !zero16 || !Y) return fail(AWQ_ERR_INVALID_ARG, "step16/zero16/Y is NULL");
  if (((uintptr_t)step16 & 1u) || ((uintptr_t)zero16 & 1u) || ((uintptr_t)Y & 3u))
    return fail(AWQ_ERR_INVALID_ARG, "step16/zero16 must be 2-byte and Y 4-byte aligned");
  return hip_result(awq::launch_w4a16(X, n_tokens, in_features, out_features, qweight, step16,
                                      zero16, Y, (hipStream_t)stream),
                    "awq_w4a16_matmul launch");
}

int awq_fold_inverse_scale(const void* src, const float* s, int64_t rows, int64_t cols, void* dst,
                           void* stream) {
  if (!src || !s || !dst) return fail(AWQ_ERR_INVALID_ARG, "src/s/dst is NULL");
  if (rows < 1 || rows > kMaxFeatures || cols < 1 || cols > kMaxFeatures || rows * cols > kMaxWeights)
    return fail(AWQ_ERR_INVALID_ARG, "rows=%lld cols=%lld out of range", (long long)rows,
                (long long)cols);
  if (((uintptr_t)src & 1u) || ((uintptr_t)dst & 1u) || ((uintptr_t)s & 3u))
    return fail(AWQ_ERR_INVALID_ARG, "src/dst must be 2-byte and s 4-byte aligned");
  const char* a = (const char*)src;
  const char* b = (const char*)dst;
  const int64_t bytes = rows * cols * 2;
  if (a != b && a < b + bytes && b < a + bytes)
    return fail(AWQ_ERR_INVALID_ARG, "src and dst overlap without being the same array");
  return hip_result(awq::launch_fold(src, s, rows, cols, dst, (hipStream_t)stream),
                    "awq_fold_inverse_scale launch");
}

int awq_select_top_channels(const float* sal, int64_t n, int64_t n_keep, float* sal_out,
                            void* stream) {
  if (!sal || !sal_out) return fail(AWQ_ERR_INVALID_ARG, "sal/sal_out is NULL");
  if (n < 1 || n > kMaxFeatures)
    return fail(AWQ_ERR_INVALID_ARG, "n=%lld outside 1..%lld", (long long)n, (long long)kMaxFeatures);
  if (n_keep < 0 || n_keep > n)
    return fail(AWQ_ERR_INVALID_ARG, "n_keep=%lld outside 0..n", (long long)n_keep);
  if (((uintptr_t)sal & 3u) || ((uintptr_t)sal_out & 3u))
    return fail(AWQ_ERR_INVALID_ARG, "sal/sal_out must be 4-byte aligned");
  if (sal != sal_out && sal < sal_out + n && sal_out < sal + n)
    return fail(AWQ_ERR_INVALID_ARG, "sal and sal_out overlap without being the same array");
  return hip_result(awq::launch_select_top(sal, n, n_keep, sal_out, (hipStream_t)stream),
                    "awq_select_top_channels launch");
}

}  // extern "C"
