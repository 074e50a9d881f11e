// Internal host-side interface between the C ABI (api.cpp) and the kernels.
// Every launcher assumes its arguments were validated by api.cpp and only
// enqueues work on the given stream; it returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bsa {

struct Shape {
  int64_t S;
  int Hq, Hkv, D, B, nb, fp8, per_group;
  int G() const { return Hq / Hkv; }
  int U() const { return per_group ? Hkv : Hq; }
};

hipError_t launch_pool(const Shape& sh, const void* q, const void* k, const float* q_scale,
                       const float* k_scale, float* q_centroid, float* q_norm, float* k_centroid,
                       float* k_radius, hipStream_t stream);

struct SelectConfig {
  int top_k, force_sink, gate, gate_factor;  // gate: 0 none, 1 top-1/top-2 gap, 2 sigma cut
  float gate_threshold, temperature, mass_threshold;
  double rescue_fraction;
};

// Workspace carve-up used by launch_score_select (byte offsets, 256-aligned).
struct SelectWorkspace {
  size_t scores_off, mask_off, counts_off, overflow_off;
  size_t run_sum_off, run_off_off;  // per-64-row count sums and their scanned offsets
  size_t sigma_off, mask_x_off, counts_x_off, keys_off, fire_off;  // sigma gate only
  size_t total;
};
SelectWorkspace select_workspace_layout(const Shape& sh, bool export_scores, bool sigma_gate);

// Dynamic LDS the select kernel's LDS form needs for these rows (0 when the
// register form runs), and the most one workgroup may have; above the limit the
// selection is not supported.
size_t select_lds_bytes(const Shape& sh, const SelectConfig& cfg);
size_t select_lds_limit();

// The allocation-free selection's scratch: its size, and its address on the
// current device (looked up on the first call per device).
size_t select_scratch_bytes();
hipError_t select_scratch(void** ptr);

// scores_in != nullptr: selection on the given scores [U, nb, nb] (no centroid
// scores are computed; q_centroid and k_centroid are unused).  width > 0: the
// output is the padded list col_idx[rows][width] (row_ptr unused), else CSR.
hipError_t launch_score_select(const Shape& sh, const SelectConfig& cfg, const float* q_centroid,
                               const float* q_norm, const float* k_centroid,
                               const float* k_radius, int32_t* row_ptr, int32_t* col_idx,
                               int64_t col_capacity, float* scores_out, float* bound_out,
                               uint8_t* gate_out, void* workspace, hipStream_t stream,
                               const float* scores_in = nullptr, int width = 0);

hipError_t launch_key_bounds(const Shape& sh, const void* k, const float* k_scale, float* k_min,
                             float* k_max, hipStream_t stream);

size_t quest_workspace_bytes(const Shape& sh);
hipError_t launch_quest_scores(const Shape& sh, const void* q, const float* q_scale,
                               const float* k_min, const float* k_max, float* scores,
                               void* workspace, hipStream_t stream);

// width > 0: col_idx is the padded list [rows][width] (valid entries first, then
// -1) and row_ptr is unused; else CSR.
hipError_t launch_attention(const Shape& sh, const void* q, const void* k, const void* v,
                            const float* q_scale, const float* k_scale, const float* v_scale,
                            const int32_t* row_ptr, const int32_t* col_idx, float softmax_scale,
                            void* out, float* lse, hipStream_t stream, int width = 0,
                            bool v16 = false, bool vt = false);

// V [S, Hkv, D] (bf16, or E4M3 codes expanded exactly) -> transposed bf16 tiles
// [nb, Hkv, D, B] with each 16-key group in the probabilities' order; keys past S
// are zero.  D = B = 128 only.
hipError_t launch_prepare_v(const Shape& sh, const void* v, void* vt, hipStream_t stream);

// E4M3 V codes [S, Hkv, D] -> their exact bf16 values in the same layout.
hipError_t launch_expand_e4m3(const Shape& sh, const void* codes, void* out, hipStream_t stream);

}  // namespace bsa
