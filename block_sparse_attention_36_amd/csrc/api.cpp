// C ABI of libbsa: host-side validation, sizing, and kernel launch orchestration.
// Every entry point validates its arguments with plain host code before any HIP
// call, so a rejected call launches nothing.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/bsa.h"
#include "launch.h"

namespace {

thread_local char g_err[512] = "";

bsa_status fail(bsa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

bsa_status ok() {
  g_err[0] = '\0';
  return BSA_OK;
}

// Shape validation shared by every entry point.  On success fills `sh`.
bsa_status check_problem(const bsa_problem* p, bsa::Shape& sh) {
  if (!p) return fail(BSA_ERR_INVALID_ARGUMENT, "problem is NULL");
  if (p->seq_len < 0) return fail(BSA_ERR_INVALID_ARGUMENT, "seq_len %lld < 0", (long long)p->seq_len);
  if (p->num_q_heads < 1 || p->num_kv_heads < 1)
    return fail(BSA_ERR_INVALID_ARGUMENT, "head counts must be >= 1 (got %d, %d)", p->num_q_heads,
                p->num_kv_heads);
  if (p->num_q_heads % p->num_kv_heads)
    return fail(BSA_ERR_INVALID_ARGUMENT, "num_q_heads %d is not a multiple of num_kv_heads %d",
                p->num_q_heads, p->num_kv_heads);
  if (p->head_dim < 1 || p->block_size < 1)
    return fail(BSA_ERR_INVALID_ARGUMENT, "head_dim and block_size must be >= 1");
  if (p->dtype != BSA_BF16 && p->dtype != BSA_FP8_E4M3)
    return fail(BSA_ERR_INVALID_ARGUMENT, "unknown dtype %d", p->dtype);
  if (p->granularity != BSA_SEL_PER_QHEAD && p->granularity != BSA_SEL_PER_GROUP)
    return fail(BSA_ERR_INVALID_ARGUMENT, "unknown granularity %d", p->granularity);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(BSA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", p->head_dim);
  if (p->block_size != 64 && p->block_size != 128)
    return fail(BSA_ERR_UNSUPPORTED, "block_size %d not supported (64 or 128)", p->block_size);
  const int G = p->num_q_heads / p->num_kv_heads;
  if (p->granularity == BSA_SEL_PER_GROUP && G > 2048 / p->head_dim)
    return fail(BSA_ERR_UNSUPPORTED, "per-group selection supports at most %d heads per group",
                2048 / p->head_dim);
  const int64_t nb = (p->seq_len + p->block_size - 1) / p->block_size;
  const int64_t U = p->granularity == BSA_SEL_PER_GROUP ? p->num_kv_heads : p->num_q_heads;
  if (nb > 65535 * 32 || U * nb > (int64_t)1 << 30 || U > 65535)
    return fail(BSA_ERR_UNSUPPORTED, "problem too large (%lld blocks, %lld units)", (long long)nb,
                (long long)U);
  sh.S = p->seq_len;
  sh.Hq = p->num_q_heads;
  sh.Hkv = p->num_kv_heads;
  sh.D = p->head_dim;
  sh.B = p->block_size;
  sh.nb = (int)nb;
  sh.fp8 = p->dtype == BSA_FP8_E4M3;
  sh.per_group = p->granularity == BSA_SEL_PER_GROUP;
  return BSA_OK;
}

bsa_status check_params(const bsa_select_params* s) {
  if (!s) return fail(BSA_ERR_INVALID_ARGUMENT, "params is NULL");
  if (s->top_k < 0) return fail(BSA_ERR_INVALID_ARGUMENT, "top_k %d < 0", s->top_k);
  if (s->force_sink != 0 && s->force_sink != 1)
    return fail(BSA_ERR_INVALID_ARGUMENT, "force_sink must be 0 or 1");
  if (s->gate != BSA_GATE_NONE && s->gate != BSA_GATE_TOP12_GAP && s->gate != BSA_GATE_SIGMA_CUT)
    return fail(BSA_ERR_INVALID_ARGUMENT, "unknown gate %d", s->gate);
  if (s->gate != BSA_GATE_NONE) {
    if (!(s->gate_threshold > 0.f && s->gate_threshold <= 1.f))
      return fail(BSA_ERR_INVALID_ARGUMENT, "gate_threshold must be in (0, 1]");
    if (s->gate_factor < 1) return fail(BSA_ERR_INVALID_ARGUMENT, "gate_factor must be >= 1");
    if ((int64_t)s->top_k * s->gate_factor > 0x7FFFFFFF)
      return fail(BSA_ERR_INVALID_ARGUMENT, "top_k * gate_factor overflows");
  }
  if (!(s->score_temperature > 0.f) || !std::isfinite(s->score_temperature))
    return fail(BSA_ERR_INVALID_ARGUMENT, "score_temperature must be finite and > 0");
  if (!(s->mass_threshold >= 0.f && s->mass_threshold <= 1.f))
    return fail(BSA_ERR_INVALID_ARGUMENT, "mass_threshold must be in [0, 1]");
  if (!(s->rescue_fraction >= 0.0 && s->rescue_fraction <= 1.0))
    return fail(BSA_ERR_INVALID_ARGUMENT, "rescue_fraction must be in [0, 1]");
  if (s->reserved != 0) return fail(BSA_ERR_INVALID_ARGUMENT, "reserved must be 0");
  return BSA_OK;
}

int64_t capacity_bound(const bsa::Shape& sh, const bsa_select_params* s) {
  int64_t per_unit = 0;
  const int64_t keff =
      (int64_t)s->top_k * (s->gate != BSA_GATE_NONE ? (int64_t)s->gate_factor : 1);
  for (int64_t i = 0; i < sh.nb; ++i) {
    const int64_t nforced = (s->force_sink && i > 0) ? 2 : 1;
    const int64_t nc = i + 1 - nforced;
    int64_t kept = nforced;
    if (s->mass_threshold > 0.f) {
      kept += nc;
    } else {
      if (s->top_k > 0) kept += keff < nc ? keff : nc;
      if (s->rescue_fraction > 0.0 && nc > 0) {
        int64_t nr = (int64_t)std::ceil(s->rescue_fraction * (double)nc);
        kept += nr < nc ? nr : nc;
      }
    }
    per_unit += kept < i + 1 ? kept : i + 1;
  }
  return per_unit * sh.U();
}

// The largest kept set any row can have under the parameters: the padded
// list's width.
int64_t padded_width(const bsa::Shape& sh, const bsa_select_params* s) {
  int64_t width = 0;
  const int64_t keff =
      (int64_t)s->top_k * (s->gate != BSA_GATE_NONE ? (int64_t)s->gate_factor : 1);
  for (int64_t i = 0; i < sh.nb; ++i) {
    const int64_t nforced = (s->force_sink && i > 0) ? 2 : 1;
    const int64_t nc = i + 1 - nforced;
    int64_t kept = nforced;
    if (s->mass_threshold > 0.f) {
      kept += nc;
    } else {
      if (s->top_k > 0) kept += keff < nc ? keff : nc;
      if (s->rescue_fraction > 0.0 && nc > 0) {
        int64_t nr = (int64_t)std::ceil(s->rescue_fraction * (double)nc);
        kept += nr < nc ? nr : nc;
      }
    }
    kept = kept < i + 1 ? kept : i + 1;
    width = kept > width ? kept : width;
  }
  return width;
}

bsa::SelectConfig select_config(const bsa_select_params* params) {
  bsa::SelectConfig cfg;
  cfg.top_k = params->top_k;
  cfg.force_sink = params->force_sink;
  cfg.gate = params->gate == BSA_GATE_TOP12_GAP ? 1 : params->gate == BSA_GATE_SIGMA_CUT ? 2 : 0;
  cfg.gate_factor = params->gate_factor;
  cfg.gate_threshold = params->gate_threshold;
  cfg.temperature = params->score_temperature;
  cfg.mass_threshold = params->mass_threshold;
  cfg.rescue_fraction = params->rescue_fraction;
  return cfg;
}

// Rows too long for the register form of the select kernel keep each row in LDS
// (scores, plus bounds and probabilities when the rescue and mass branches are
// on); rows needing more than one CU's LDS are not supported.
bsa_status check_select_form(const bsa::Shape& sh, const bsa_select_params* params) {
  const size_t need = bsa::select_lds_bytes(sh, select_config(params));
  if (need > bsa::select_lds_limit())
    return fail(BSA_ERR_UNSUPPORTED,
                "rows of %d blocks need %zu bytes of LDS per selection row with these branches "
                "(at most %zu)", sh.nb, need, bsa::select_lds_limit());
  return BSA_OK;
}

bool misaligned(const void* p) { return ((uintptr_t)p & 15) != 0; }

bsa_status device_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(BSA_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int bsa_abi_version(void) { return BSA_ABI_VERSION; }

const char* bsa_status_string(int status) {
  switch (status) {
    case BSA_OK: return "ok";
    case BSA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case BSA_ERR_UNSUPPORTED: return "unsupported";
    case BSA_ERR_CAPACITY: return "CSR capacity too small";
    case BSA_ERR_WORKSPACE: return "workspace too small";
    case BSA_ERR_DEVICE: return "device error";
    default: return "unknown status";
  }
}

const char* bsa_last_error(void) { return g_err; }

int64_t bsa_num_blocks(const bsa_problem* problem) {
  bsa::Shape sh;
  if (check_problem(problem, sh) != BSA_OK) return -1;
  return sh.nb;
}

int64_t bsa_num_select_rows(const bsa_problem* problem) {
  bsa::Shape sh;
  if (check_problem(problem, sh) != BSA_OK) return -1;
  return (int64_t)sh.U() * sh.nb;
}

bsa_status bsa_pool(const bsa_problem* problem, const void* q, const void* k,
                    const float* q_scale, const float* k_scale, float* q_centroid,
                    float* q_norm, float* k_centroid, float* k_radius, void* hip_stream) {
  bsa::Shape sh;
  bsa_status st = check_problem(problem, sh);
  if (st != BSA_OK) return st;
  if (sh.S == 0) return ok();
  if (!q || !k || !q_centroid || !k_centroid)
    return fail(BSA_ERR_INVALID_ARGUMENT, "q, k, q_centroid and k_centroid are required");
  if (sh.fp8 && (!q_scale || !k_scale))
    return fail(BSA_ERR_INVALID_ARGUMENT, "FP8 inputs need q_scale and k_scale");
  if (misaligned(q) || misaligned(k) || misaligned(q_centroid) || misaligned(k_centroid))
    return fail(BSA_ERR_INVALID_ARGUMENT,
                "q, k, q_centroid and k_centroid must be 16-byte aligned");
  return device_status(bsa::launch_pool(sh, q, k, sh.fp8 ? q_scale : nullptr,
                                        sh.fp8 ? k_scale : nullptr, q_centroid, q_norm,
                                        k_centroid, k_radius, (hipStream_t)hip_stream),
                       "bsa_pool launch");
}

int64_t bsa_csr_capacity_bound(const bsa_problem* problem, const bsa_select_params* params) {
  bsa::Shape sh;
  if (check_problem(problem, sh) != BSA_OK || check_params(params) != BSA_OK) return -1;
  return capacity_bound(sh, params);
}

size_t bsa_score_select_workspace_size(const bsa_problem* problem, const bsa_select_params* params,
                                       int export_scores) {
  bsa::Shape sh;
  if (check_problem(problem, sh) != BSA_OK || check_params(params) != BSA_OK) return 0;
  return bsa::select_workspace_layout(sh, export_scores != 0, params->gate == BSA_GATE_SIGMA_CUT)
      .total;
}

namespace {

// Everything bsa_score_select checks except the workspace; fills sh and the
// workspace bytes the call needs.
bsa_status check_score_select(const bsa_problem* problem, const bsa_select_params* params,
                              const float* q_centroid, const float* q_norm,
                              const float* k_centroid, const float* k_radius,
                              const int32_t* row_ptr, const int32_t* col_idx,
                              int64_t col_capacity, const float* scores_out, bsa::Shape& sh,
                              size_t& need) {
  bsa_status st = check_problem(problem, sh);
  if (st != BSA_OK) return st;
  st = check_params(params);
  if (st != BSA_OK) return st;
  st = check_select_form(sh, params);
  if (st != BSA_OK) return st;
  need = 0;
  if (sh.S == 0) return BSA_OK;
  if (!q_centroid || !k_centroid || !row_ptr || !col_idx)
    return fail(BSA_ERR_INVALID_ARGUMENT, "q_centroid, k_centroid, row_ptr and col_idx are required");
  if (((uintptr_t)q_centroid | (uintptr_t)k_centroid | (uintptr_t)row_ptr) & 15)
    return fail(BSA_ERR_INVALID_ARGUMENT, "q_centroid, k_centroid and row_ptr must be 16-byte aligned");
  const bool rescue = params->rescue_fraction > 0.0;
  if (rescue && (!q_norm || !k_radius))
    return fail(BSA_ERR_INVALID_ARGUMENT, "the rescue branch needs q_norm and k_radius");
  const int64_t bound = capacity_bound(sh, params);
  if (bound > 0x7FFFFFFF)
    return fail(BSA_ERR_UNSUPPORTED, "kept-block bound %lld exceeds int32 CSR", (long long)bound);
  if (col_capacity < bound)
    return fail(BSA_ERR_CAPACITY, "col_capacity %lld < bound %lld", (long long)col_capacity,
                (long long)bound);
  need = bsa::select_workspace_layout(sh, scores_out != nullptr, params->gate == BSA_GATE_SIGMA_CUT)
             .total;
  return BSA_OK;
}

bsa_status launch_checked_score_select(const bsa::Shape& sh, const bsa_select_params* params,
                                       const float* q_centroid, const float* q_norm,
                                       const float* k_centroid, const float* k_radius,
                                       int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                                       float* scores_out, float* bound_out, uint8_t* gate_out,
                                       void* workspace, void* hip_stream, const char* what) {
  const bool rescue = params->rescue_fraction > 0.0;
  const bsa::SelectConfig cfg = select_config(params);
  return device_status(
      bsa::launch_score_select(sh, cfg, q_centroid, rescue ? q_norm : nullptr, k_centroid,
                               rescue ? k_radius : nullptr, row_ptr, col_idx, col_capacity,
                               scores_out, rescue ? bound_out : nullptr, gate_out, workspace,
                               (hipStream_t)hip_stream),
      what);
}

}  // namespace

bsa_status bsa_score_select(const bsa_problem* problem, const bsa_select_params* params,
                            const float* q_centroid, const float* q_norm,
                            const float* k_centroid, const float* k_radius, int32_t* row_ptr,
                            int32_t* col_idx, int64_t col_capacity, float* scores_out,
                            float* bound_out, uint8_t* gate_out, void* workspace,
                            size_t workspace_bytes, void* hip_stream) {
  bsa::Shape sh;
  size_t need = 0;
  bsa_status st = check_score_select(problem, params, q_centroid, q_norm, k_centroid, k_radius,
                                     row_ptr, col_idx, col_capacity, scores_out, sh, need);
  if (st != BSA_OK) return st;
  if (sh.S == 0) return ok();
  if ((uintptr_t)workspace & 15)
    return fail(BSA_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  if (!workspace || workspace_bytes < need)
    return fail(BSA_ERR_WORKSPACE, "workspace of %zu bytes < %zu required", workspace_bytes, need);
  return launch_checked_score_select(sh, params, q_centroid, q_norm, k_centroid, k_radius,
                                     row_ptr, col_idx, col_capacity, scores_out, bound_out,
                                     gate_out, workspace, hip_stream, "bsa_score_select launch");
}

bsa_status bsa_score_select_noalloc(const bsa_problem* problem, const bsa_select_params* params,
                                    const float* q_centroid, const float* q_norm,
                                    const float* k_centroid, const float* k_radius,
                                    int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                                    float* scores_out, float* bound_out, uint8_t* gate_out,
                                    void* hip_stream) {
  bsa::Shape sh;
  size_t need = 0;
  bsa_status st = check_score_select(problem, params, q_centroid, q_norm, k_centroid, k_radius,
                                     row_ptr, col_idx, col_capacity, scores_out, sh, need);
  if (st != BSA_OK) return st;
  if (sh.S == 0) return ok();
  if (need > bsa::select_scratch_bytes())
    return fail(BSA_ERR_WORKSPACE,
                "this selection needs %zu bytes of scratch; the allocation-free entry point "
                "holds %zu (with scores_out given the score matrix stays out of it)",
                need, bsa::select_scratch_bytes());
  void* scratch = nullptr;
  const hipError_t e = bsa::select_scratch(&scratch);
  if (e != hipSuccess) return device_status(e, "bsa_score_select_noalloc scratch lookup");
  return launch_checked_score_select(sh, params, q_centroid, q_norm, k_centroid, k_radius,
                                     row_ptr, col_idx, col_capacity, scores_out, bound_out,
                                     gate_out, scratch, hip_stream,
                                     "bsa_score_select_noalloc launch");
}

bsa_status bsa_pool_key_bounds(const bsa_problem* problem, const void* k, const float* k_scale,
                               float* k_min, float* k_max, void* hip_stream) {
  bsa::Shape sh;
  bsa_status st = check_problem(problem, sh);
  if (st != BSA_OK) return st;
  if (sh.S == 0) return ok();
  if (!k || !k_min || !k_max)
    return fail(BSA_ERR_INVALID_ARGUMENT, "k, k_min and k_max are required");
  if (sh.fp8 && !k_scale) return fail(BSA_ERR_INVALID_ARGUMENT, "FP8 keys need k_scale");
  if (misaligned(k) || misaligned(k_min) || misaligned(k_max))
    return fail(BSA_ERR_INVALID_ARGUMENT, "k, k_min and k_max must be 16-byte aligned");
  return device_status(bsa::launch_key_bounds(sh, k, sh.fp8 ? k_scale : nullptr, k_min, k_max,
                                              (hipStream_t)hip_stream),
                       "bsa_pool_key_bounds launch");
}

size_t bsa_quest_scores_workspace_size(const bsa_problem* problem) {
  bsa::Shape sh;
  if (check_problem(problem, sh) != BSA_OK) return 0;
  return bsa::quest_workspace_bytes(sh);
}

bsa_status bsa_quest_scores(const bsa_problem* problem, const void* q, const float* q_scale,
                            const float* k_min, const float* k_max, float* scores,
                            void* workspace, size_t workspace_bytes, void* hip_stream) {
  bsa::Shape sh;
  bsa_status st = check_problem(problem, sh);
  if (st != BSA_OK) return st;
  if (sh.S == 0) return ok();
  if (!q || !k_min || !k_max || !scores)
    return fail(BSA_ERR_INVALID_ARGUMENT, "q, k_min, k_max and scores are required");
  if (sh.fp8 && !q_scale) return fail(BSA_ERR_INVALID_ARGUMENT, "FP8 queries need q_scale");
  if (misaligned(q) || misaligned(k_min) || misaligned(k_max) || misaligned(workspace))
    return fail(BSA_ERR_INVALID_ARGUMENT, "q, k_min, k_max and workspace must be 16-byte aligned");
  const size_t need = bsa::quest_workspace_bytes(sh);
  if (!workspace || workspace_bytes < need)
    return fail(BSA_ERR_WORKSPACE, "workspace of %zu bytes < %zu required", workspace_bytes, need);
  return device_status(bsa::launch_quest_scores(sh, q, sh.fp8 ? q_scale : nullptr, k_min, k_max,
                                                scores, workspace, (hipStream_t)hip_stream),
                       "bsa_quest_scores launch");
}

size_t bsa_select_scores_workspace_size(const bsa_problem* problem,
                                        const bsa_select_params* params) {
  bsa::Shape sh;
  if (check_problem(problem, sh) != BSA_OK || check_params(params) != BSA_OK) return 0;
  return bsa::select_workspace_layout(sh, true, params->gate == BSA_GATE_SIGMA_CUT).total;
}

bsa_status bsa_select_scores(const bsa_problem* problem, const bsa_select_params* params,
                             const float* scores, int32_t* row_ptr, int32_t* col_idx,
                             int64_t col_capacity, uint8_t* gate_out, void* workspace,
                             size_t workspace_bytes, void* hip_stream) {
  bsa::Shape sh;
  bsa_status st = check_problem(problem, sh);
  if (st != BSA_OK) return st;
  st = check_params(params);
  if (st != BSA_OK) return st;
  st = check_select_form(sh, params);
  if (st != BSA_OK) return st;
  if (params->rescue_fraction > 0.0)
    return fail(BSA_ERR_INVALID_ARGUMENT,
                "the rescue branch needs centroid scores and radii (use bsa_score_select)");
  if (sh.S == 0) return ok();
  if (!scores || !row_ptr || !col_idx)
    return fail(BSA_ERR_INVALID_ARGUMENT, "scores, row_ptr and col_idx are required");
  if (misaligned(row_ptr) || misaligned(workspace))
    return fail(BSA_ERR_INVALID_ARGUMENT, "row_ptr and workspace must be 16-byte aligned");
  const int64_t bound = capacity_bound(sh, params);
  if (bound > 0x7FFFFFFF)
    return fail(BSA_ERR_UNSUPPORTED, "kept-block bound %lld exceeds int32 CSR", (long long)bound);
  if (col_capacity < bound)
    return fail(BSA_ERR_CAPACITY, "col_capacity %lld < bound %lld", (long long)col_capacity,
                (long long)bound);
  const size_t need =
      bsa::select_workspace_layout(sh, true, params->gate == BSA_GATE_SIGMA_CUT).total;
  if (!workspace || workspace_bytes < need)
    return fail(BSA_ERR_WORKSPACE, "workspace of %zu bytes < %zu required", workspace_bytes, need);
  const bsa::SelectConfig cfg = select_config(params);
  return device_status(
      bsa::launch_score_select(sh, cfg, nullptr, nullptr, nullptr, nullptr, row_ptr, col_idx,
                               col_capacity, nullptr, nullptr, gate_out, workspace,
                               (hipStream_t)hip_stream, scores),
      "bsa_select_scores launch");
}

int64_t bsa_select_overflow_offset(const bsa_problem* problem, const bsa_select_params* params,
                                   int scores_given_or_exported) {
  bsa::Shape sh;
  if (check_problem(problem, sh) != BSA_OK || check_params(params) != BSA_OK) return -1;
  return (int64_t)bsa::select_workspace_layout(sh, scores_given_or_exported != 0,
                                               params->gate == BSA_GATE_SIGMA_CUT)
      .overflow_off;
}

int64_t bsa_padded_width(const bsa_problem* problem, const bsa_select_params* params) {
  bsa::Shape sh;
  if (check_problem(problem, sh) != BSA_OK || check_params(params) != BSA_OK) return -1;
  return padded_width(sh, params);
}

size_t bsa_score_select_padded_workspace_size(const bsa_problem* problem,
                                              const bsa_select_params* params,
                                              int scores_given_or_exported) {
  bsa::Shape sh;
  if (check_problem(problem, sh) != BSA_OK || check_params(params) != BSA_OK) return 0;
  return bsa::select_workspace_layout(sh, scores_given_or_exported != 0,
                                      params->gate == BSA_GATE_SIGMA_CUT)
      .total;
}

bsa_status bsa_score_select_padded(const bsa_problem* problem, const bsa_select_params* params,
                                   const float* q_centroid, const float* q_norm,
                                   const float* k_centroid, const float* k_radius,
                                   const float* scores_in, int32_t* kv_idx, int64_t width,
                                   float* scores_out, float* bound_out, uint8_t* gate_out,
                                   void* workspace, size_t workspace_bytes, void* hip_stream) {
  bsa::Shape sh;
  bsa_status st = check_problem(problem, sh);
  if (st != BSA_OK) return st;
  st = check_params(params);
  if (st != BSA_OK) return st;
  st = check_select_form(sh, params);
  if (st != BSA_OK) return st;
  const bool rescue = params->rescue_fraction > 0.0;
  if (scores_in && (rescue || scores_out || bound_out))
    return fail(BSA_ERR_INVALID_ARGUMENT,
                "with given scores there is no rescue branch and nothing to export");
  if (sh.S == 0) return ok();
  if (!kv_idx) return fail(BSA_ERR_INVALID_ARGUMENT, "kv_idx is required");
  if (!scores_in && (!q_centroid || !k_centroid))
    return fail(BSA_ERR_INVALID_ARGUMENT, "q_centroid and k_centroid are required");
  if (misaligned(q_centroid) || misaligned(k_centroid) || misaligned(workspace))
    return fail(BSA_ERR_INVALID_ARGUMENT,
                "q_centroid, k_centroid and workspace must be 16-byte aligned");
  if (rescue && (!q_norm || !k_radius))
    return fail(BSA_ERR_INVALID_ARGUMENT, "the rescue branch needs q_norm and k_radius");
  const int64_t need_w = padded_width(sh, params);
  if (width < need_w)
    return fail(BSA_ERR_CAPACITY, "width %lld < %lld kept blocks a row can have",
                (long long)width, (long long)need_w);
  if ((int64_t)sh.U() * sh.nb * width > 0x7FFFFFFF)
    return fail(BSA_ERR_UNSUPPORTED, "padded list of %lld entries exceeds int32 indexing",
                (long long)((int64_t)sh.U() * sh.nb * width));
  const size_t need = bsa::select_workspace_layout(sh, scores_in || scores_out,
                                                   params->gate == BSA_GATE_SIGMA_CUT)
                          .total;
  if (!workspace || workspace_bytes < need)
    return fail(BSA_ERR_WORKSPACE, "workspace of %zu bytes < %zu required", workspace_bytes, need);
  const bsa::SelectConfig cfg = select_config(params);
  return device_status(
      bsa::launch_score_select(sh, cfg, q_centroid, rescue ? q_norm : nullptr, k_centroid,
                               rescue ? k_radius : nullptr, nullptr, kv_idx, 0, scores_out,
                               rescue ? bound_out : nullptr, gate_out, workspace,
                               (hipStream_t)hip_stream, scores_in, (int)width),
      "bsa_score_select_padded launch");
}

bsa_status bsa_attention_fwd_padded(const bsa_problem* problem, const void* q, const void* k,
                                    const void* v, const float* q_scale, const float* k_scale,
                                    const float* v_scale, const int32_t* kv_idx, int64_t width,
                                    float softmax_scale, void* out, float* lse, void* hip_stream) {
  bsa::Shape sh;
  bsa_status st = check_problem(problem, sh);
  if (st != BSA_OK) return st;
  if (sh.S == 0) return ok();
  if (!q || !k || !v || !kv_idx || !out)
    return fail(BSA_ERR_INVALID_ARGUMENT, "q, k, v, kv_idx and out are required");
  if (sh.fp8 && (!q_scale || !k_scale || !v_scale))
    return fail(BSA_ERR_INVALID_ARGUMENT, "FP8 inputs need q_scale, k_scale and v_scale");
  if (!std::isfinite(softmax_scale) || softmax_scale <= 0.f)
    return fail(BSA_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and > 0");
  if (width < 1 || width > sh.nb)
    return fail(BSA_ERR_INVALID_ARGUMENT, "width %lld outside [1, %d]", (long long)width, sh.nb);
  if ((int64_t)sh.U() * sh.nb * width > 0x7FFFFFFF)
    return fail(BSA_ERR_UNSUPPORTED, "padded list exceeds int32 indexing");
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(out))
    return fail(BSA_ERR_INVALID_ARGUMENT, "q, k, v and out must be 16-byte aligned");
  return device_status(bsa::launch_attention(sh, q, k, v, q_scale, k_scale, v_scale, nullptr,
                                             kv_idx, softmax_scale, out, lse,
                                             (hipStream_t)hip_stream, (int)width),
                       "bsa_attention_fwd_padded launch");
}

bsa_status bsa_attention_fwd(const bsa_problem* problem, const void* q, const void* k,
                             const void* v, const float* q_scale, const float* k_scale,
                             const float* v_scale, const int32_t* row_ptr,
                             const int32_t* col_idx, float softmax_scale, void* out, float* lse,
                             void* hip_stream) {
  bsa::Shape sh;
  bsa_status st = check_problem(problem, sh);
  if (st != BSA_OK) return st;
  if (sh.S == 0) return ok();
  if (!q || !k || !v || !row_ptr || !col_idx || !out)
    return fail(BSA_ERR_INVALID_ARGUMENT, "q, k, v, row_ptr, col_idx and out are required");
  if (sh.fp8 && (!q_scale || !k_scale || !v_scale))
    return fail(BSA_ERR_INVALID_ARGUMENT, "FP8 inputs need q_scale, k_scale and v_scale");
  if (!std::isfinite(softmax_scale) || softmax_scale <= 0.f)
    return fail(BSA_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and > 0");
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(out))
    return fail(BSA_ERR_INVALID_ARGUMENT, "q, k, v and out must be 16-byte aligned");
  return device_status(bsa::launch_attention(sh, q, k, v, q_scale, k_scale, v_scale, row_ptr,
                                             col_idx, softmax_scale, out, lse,
                                             (hipStream_t)hip_stream),
                       "bsa_attention_fwd launch");
}

bsa_status bsa_expand_e4m3(const bsa_problem* problem, const void* v, void* v_bf16,
                           void* hip_stream) {
  bsa::Shape sh;
  bsa_status st = check_problem(problem, sh);
  if (st != BSA_OK) return st;
  if (!sh.fp8) return fail(BSA_ERR_INVALID_ARGUMENT, "only E4M3 problems have codes to expand");
  if (sh.S == 0) return ok();
  if (!v || !v_bf16) return fail(BSA_ERR_INVALID_ARGUMENT, "v and v_bf16 are required");
  if (misaligned(v) || misaligned(v_bf16))
    return fail(BSA_ERR_INVALID_ARGUMENT, "v and v_bf16 must be 16-byte aligned");
  return device_status(bsa::launch_expand_e4m3(sh, v, v_bf16, (hipStream_t)hip_stream),
                       "bsa_expand_e4m3 launch");
}

bsa_status bsa_attention_fwd_expanded_v(const bsa_problem* problem, const void* q, const void* k,
                                        const void* v_bf16, const float* q_scale,
                                        const float* k_scale, const float* v_scale,
                                        const int32_t* row_ptr, const int32_t* col_idx,
                                        float softmax_scale, void* out, float* lse,
                                        void* hip_stream) {
  bsa::Shape sh;
  bsa_status st = check_problem(problem, sh);
  if (st != BSA_OK) return st;
  if (!sh.fp8)
    return fail(BSA_ERR_INVALID_ARGUMENT,
                "bsa_attention_fwd_expanded_v is for E4M3 problems; use bsa_attention_fwd");
  if (sh.S == 0) return ok();
  if (!q || !k || !v_bf16 || !row_ptr || !col_idx || !out)
    return fail(BSA_ERR_INVALID_ARGUMENT, "q, k, v_bf16, row_ptr, col_idx and out are required");
  if (!q_scale || !k_scale || !v_scale)
    return fail(BSA_ERR_INVALID_ARGUMENT, "FP8 inputs need q_scale, k_scale and v_scale");
  if (!std::isfinite(softmax_scale) || softmax_scale <= 0.f)
    return fail(BSA_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and > 0");
  if (misaligned(q) || misaligned(k) || misaligned(v_bf16) || misaligned(out))
    return fail(BSA_ERR_INVALID_ARGUMENT, "q, k, v_bf16 and out must be 16-byte aligned");
  return device_status(bsa::launch_attention(sh, q, k, v_bf16, q_scale, k_scale, v_scale, row_ptr,
                                             col_idx, softmax_scale, out, lse,
                                             (hipStream_t)hip_stream, 0, true),
                       "bsa_attention_fwd_expanded_v launch");
}

size_t bsa_prepared_v_bytes(const bsa_problem* problem) {
  bsa::Shape sh;
  if (check_problem(problem, sh) != BSA_OK || sh.D != 128 || sh.B != 128) return 0;
  return (size_t)sh.nb * sh.Hkv * sh.D * sh.B * 2;
}

bsa_status bsa_prepare_v(const bsa_problem* problem, const void* v, void* v_prepared,
                         void* hip_stream) {
  bsa::Shape sh;
  bsa_status st = check_problem(problem, sh);
  if (st != BSA_OK) return st;
  if (sh.D != 128 || sh.B != 128)
    return fail(BSA_ERR_UNSUPPORTED, "prepared V tiles need head_dim = block_size = 128");
  if (sh.S == 0) return ok();
  if (!v || !v_prepared) return fail(BSA_ERR_INVALID_ARGUMENT, "v and v_prepared are required");
  if (misaligned(v) || misaligned(v_prepared))
    return fail(BSA_ERR_INVALID_ARGUMENT, "v and v_prepared must be 16-byte aligned");
  return device_status(bsa::launch_prepare_v(sh, v, v_prepared, (hipStream_t)hip_stream),
                       "bsa_prepare_v launch");
}

bsa_status bsa_attention_fwd_prepared_v(const bsa_problem* problem, const void* q, const void* k,
                                        const void* v_prepared, const float* q_scale,
                                        const float* k_scale, const float* v_scale,
                                        const int32_t* row_ptr, const int32_t* col_idx,
                                        float softmax_scale, void* out, float* lse,
                                        void* hip_stream) {
  bsa::Shape sh;
  bsa_status st = check_problem(problem, sh);
  if (st != BSA_OK) return st;
  if (sh.D != 128 || sh.B != 128)
    return fail(BSA_ERR_UNSUPPORTED, "prepared V tiles need head_dim = block_size = 128");
  if (sh.S == 0) return ok();
  if (!q || !k || !v_prepared || !row_ptr || !col_idx || !out)
    return fail(BSA_ERR_INVALID_ARGUMENT,
                "q, k, v_prepared, row_ptr, col_idx and out are required");
  if (sh.fp8 && (!q_scale || !k_scale || !v_scale))
    return fail(BSA_ERR_INVALID_ARGUMENT, "FP8 inputs need q_scale, k_scale and v_scale");
  if (!std::isfinite(softmax_scale) || softmax_scale <= 0.f)
    return fail(BSA_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and > 0");
  if (misaligned(q) || misaligned(k) || misaligned(v_prepared) || misaligned(out))
    return fail(BSA_ERR_INVALID_ARGUMENT, "q, k, v_prepared and out must be 16-byte aligned");
  return device_status(bsa::launch_attention(sh, q, k, v_prepared, q_scale, k_scale, v_scale,
                                             row_ptr, col_idx, softmax_scale, out, lse,
                                             (hipStream_t)hip_stream, 0, sh.fp8 != 0, true),
                       "bsa_attention_fwd_prepared_v launch");
}

}  // extern "C"
