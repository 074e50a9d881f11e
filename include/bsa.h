/*
 * bsa.h -- C ABI of the block-sparse attention prefill library (libbsa.so).
 *
 * Three calls make one prefill layer:
 *
 *   bsa_pool           mean-pooled query and key block centroids, query-centroid
 *                      norms and key-block radii;
 *   bsa_score_select   centroid block scores, then per selection row the kept key
 *                      blocks (top-k with an optional uncertainty gate, a
 *                      cumulative-mass base branch and a radius rescue branch,
 *                      unioned with the forced blocks), emitted as CSR;
 *   bsa_attention_fwd  online-softmax attention of every query block over its kept
 *                      key blocks only, with the causal mask on the diagonal block.
 *
 * The Quest backbone replaces the first two calls by three:
 *
 *   bsa_pool_key_bounds  coordinate-wise minimum and maximum of every key block;
 *   bsa_quest_scores     per query row the largest q.k over each block's box, and
 *                        per query tile the maximum over its rows;
 *   bsa_select_scores    the selection rules of bsa_score_select on given scores.
 *
 * Either selection can instead emit a uniform-width, sentinel-padded list
 * (bsa_score_select_padded) that bsa_attention_fwd_padded consumes.
 *
 * Sources (the method these calls compute):
 *   - "Uncertainty-gated selection for block-sparse attention" (gist.science),
 *     technical summary, Methodology steps 1-2 (block scores from mean-pooled
 *     keys, per-tile top-k into a kv_idx list) and step 5 (expansion to top rho*k),
 *     lay summary "The Solution" (a near tie of the best two doubles the budget).
 *   - "RBS-Attention" (iaonda.com), third and fourth paragraphs: a base branch of
 *     centroid relevance and a rescue branch using a dynamic key-block radius,
 *     independent thresholds, masks fused, sparse FlashAttention downstream.
 *   - "MiniMax presenta MSA" (iaonda.com), "What is MSA and how does it work": a
 *     light index branch picks top-k KV blocks per GQA group; the main branch runs
 *     attention over those blocks only.
 *
 * Conventions shared by every call
 *   Layout: Q is [S, Hq, D], K and V are [S, Hkv, D], token-major and contiguous,
 *   batch 1.  Blocks are B consecutive tokens; nb = ceil(S / B) and the last block
 *   may be ragged (S - (nb-1)*B tokens).  Query head h reads kv head h / (Hq/Hkv).
 *   A selection unit is a query head (BSA_SEL_PER_QHEAD, U = Hq) or a GQA group
 *   (BSA_SEL_PER_GROUP, U = Hkv); a selection row is (unit u, query block i) and
 *   rows are numbered u*nb + i.
 *   FP8 inputs are OCP E4M3 codes (one byte each) with float32 scales [H, nb]:
 *   value = decode(code) * scale[head][block].  BF16 inputs take no scales.
 *   Supported now: head_dim in {64, 128}, block_size in {64, 128}.
 *
 *   Memory: every pointer argument is device memory allocated and owned by the
 *   caller (16-byte aligned); the library never allocates or frees device memory
 *   and never synchronises.  Host structs are read during the call only.
 *
 *   Streams: hip_stream is a hipStream_t passed as void* (NULL = null stream).
 *   After host-side validation each call enqueues its kernels on that stream and
 *   returns; results are ready when the stream reaches that point.  A call makes
 *   no allocation, copy, memset or synchronisation, so a sequence of calls may be
 *   captured into a HIP graph once each has run eagerly on that device (the first
 *   call per device raises kernel LDS limits and, for bsa_score_select_noalloc,
 *   looks up its scratch address).
 *
 *   Errors: arguments are validated on the host before anything is launched; a
 *   failing call launches nothing and returns a non-zero bsa_status, with a
 *   message available from bsa_last_error() (thread-local).  BSA_ERR_DEVICE means
 *   a launch failed (hipGetLastError); faults during execution surface at the
 *   caller's next synchronisation.  seq_len == 0 is valid and launches nothing.
 *   Calls are reentrant; concurrent calls on different streams do not interact.
 */
#ifndef BSA_H
#define BSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BSA_ABI_VERSION 5

typedef enum {
  BSA_OK = 0,
  BSA_ERR_INVALID_ARGUMENT = 1, /* null required pointer, bad shape or parameter */
  BSA_ERR_UNSUPPORTED = 2,      /* valid but not implemented (e.g. head_dim 96)  */
  BSA_ERR_CAPACITY = 3,         /* col_capacity below bsa_csr_capacity_bound      */
  BSA_ERR_WORKSPACE = 4,        /* workspace smaller than required               */
  BSA_ERR_DEVICE = 5            /* a kernel launch failed                        */
} bsa_status;

typedef enum { BSA_BF16 = 0, BSA_FP8_E4M3 = 1 } bsa_dtype;
typedef enum { BSA_SEL_PER_QHEAD = 0, BSA_SEL_PER_GROUP = 1 } bsa_granularity;
typedef enum { BSA_GATE_NONE = 0, BSA_GATE_TOP12_GAP = 1, BSA_GATE_SIGMA_CUT = 2 } bsa_gate;

/* Shape of one prefill layer. */
typedef struct {
  int64_t seq_len;      /* S >= 0                                              */
  int32_t num_q_heads;  /* Hq >= 1                                             */
  int32_t num_kv_heads; /* Hkv >= 1, Hq % Hkv == 0                             */
  int32_t head_dim;     /* D                                                   */
  int32_t block_size;   /* B                                                   */
  int32_t dtype;        /* bsa_dtype of Q, K, V                                */
  int32_t granularity;  /* bsa_granularity of the selection rows               */
} bsa_problem;

/* Selection rule.  Candidates of row (u, i) are C_i = {0..i} minus the forced
 * blocks (the diagonal i, and block 0 when force_sink != 0); every branch ranks
 * C_i by descending score with the lowest block index first on ties, and the
 * kept set is the union of the forced blocks and every enabled branch. */
typedef struct {
  int32_t top_k;            /* k >= 0; 0 switches the top-k branch off          */
  int32_t force_sink;       /* 0/1: also force block 0                          */
  int32_t gate;             /* bsa_gate; applies to the top-k branch            */
  float gate_threshold;     /* in (0, 1]: theta for BSA_GATE_TOP12_GAP, the     */
                            /* percentile level q for BSA_GATE_SIGMA_CUT        */
  int32_t gate_factor;      /* rho >= 1: a fired row keeps rho*k                */
  float score_temperature;  /* tau > 0 in softmax(tau * s) (gate and mass)     */
  float mass_threshold;     /* mu in [0, 1]; 0 switches the base branch off    */
  int32_t reserved;         /* must be 0                                        */
  double rescue_fraction;   /* phi in [0, 1]; 0 switches the rescue branch off */
} bsa_select_params;

int bsa_abi_version(void);
const char* bsa_status_string(int status);
/* Detail of this thread's last failing call ("" if none). */
const char* bsa_last_error(void);

/* nb = ceil(S / B), or -1 if the problem is invalid. */
int64_t bsa_num_blocks(const bsa_problem* problem);
/* U * nb selection rows, or -1 if the problem is invalid. */
int64_t bsa_num_select_rows(const bsa_problem* problem);

/*
 * bsa_pool -- block centroids ("Uncertainty-gated selection ...", Methodology
 * step 1: keys grouped into blocks and scored by mean pooling; RBS-Attention,
 * third paragraph: centroid relevance and a per-(prompt, layer, head) radius).
 *
 *   q, k         [S, Hq, D] / [S, Hkv, D] bf16, or E4M3 codes with q_scale [Hq, nb]
 *                and k_scale [Hkv, nb] (required for FP8, ignored for BF16).
 *   q_centroid   out [U, nb, D] f32: mean of the block's query rows; for per-group
 *                rows the mean over the group's heads and the block's rows.
 *   q_norm       out [U, nb] f32, ||q_centroid||_2 (nullable).
 *   k_centroid   out [Hkv, nb, D] f32: mean of the block's key rows.
 *   k_radius     out [Hkv, nb] f32: max over the block's keys of ||k - k_centroid||_2
 *                (nullable; only the rescue branch needs it).
 */
bsa_status bsa_pool(const bsa_problem* problem, const void* q, const void* k,
                    const float* q_scale, const float* k_scale, float* q_centroid,
                    float* q_norm, float* k_centroid, float* k_radius, void* hip_stream);

/* Upper bound on the total kept blocks over all rows (the col_idx length needed),
 * computed from the parameters alone; -1 if the arguments are invalid. */
int64_t bsa_csr_capacity_bound(const bsa_problem* problem, const bsa_select_params* params);

/* Device workspace bytes bsa_score_select needs (0 on invalid arguments). */
size_t bsa_score_select_workspace_size(const bsa_problem* problem,
                                       const bsa_select_params* params, int export_scores);

/*
 * bsa_score_select -- block scores and kept-block lists.
 *
 * Score s[u][i][j] = q_centroid[u][i] . k_centroid[kv(u)][j] for j <= i
 * ("Uncertainty-gated selection ...", Methodology step 1, the mean-pooling
 * inner product).  Per row (u, i), with p = softmax(tau * s) over C_i:
 *   top-k  : the first k of C_i; when gate == BSA_GATE_TOP12_GAP, |C_i| >= 2 and
 *            p(0) - p(1) < theta, the first rho*k instead (same page, "The
 *            Solution" and Methodology step 5);
 *            when gate == BSA_GATE_SIGMA_CUT the decision is per query block
 *            (tile) over the whole call, taken as one layer (same page,
 *            Methodology steps 3-5): a row with a cut (|C_i| > k) has
 *            sigma = (s(k-1) - s(k)) / (s(0) - s(k)) over its candidate scores
 *            sorted descending (0 when s(0) = s(k)); tile i's signal is the mean
 *            of sigma over the U units; with T tiles that have a cut, tile i
 *            fires when at most floor(q * T) of them (q = gate_threshold, the
 *            product in double) have a mean <= its own; every row of a fired
 *            tile keeps the first rho*k;
 *   base   : the shortest prefix of C_i whose mass reaches mu (RBS-Attention base
 *            branch under its own threshold);
 *   rescue : the first ceil(phi * |C_i|) of C_i ranked by the bound
 *            b = s + q_norm[u][i] * k_radius[kv(u)][j] (RBS-Attention rescue branch);
 *   kept   = forced U top-k U base U rescue, emitted ascending (diagonal last).
 * Threshold decisions are taken in float32.
 *
 *   q_norm, k_radius  required when phi > 0, else nullable.
 *   row_ptr      out int32 [U*nb + 1], exclusive prefix of the row lengths.
 *   col_idx      out int32 [col_capacity]; col_capacity must be at least
 *                bsa_csr_capacity_bound(), else BSA_ERR_CAPACITY.
 *   scores_out   out f32 [U, nb, nb] (nullable): the scores the decisions used,
 *                written for j <= i (other entries untouched).
 *   bound_out    out f32 [U, nb, nb] (nullable): the rescue bounds, j <= i.
 *   gate_out     out uint8 [U*nb] (nullable): 1 where the gate fired (for the
 *                sigma gate: every row of a fired tile).
 *   workspace    device scratch of at least
 *                bsa_score_select_workspace_size(problem, params, scores_out != NULL)
 *                bytes, else BSA_ERR_WORKSPACE.
 * Rows longer than the select kernel's register form (4096 blocks; 8192 with
 * the mass and rescue branches off) are kept in LDS, up to 160 KiB per row with
 * the enabled branches (about 13600 blocks with mass and rescue, 20400 with one
 * of them, 40900 with neither); longer rows return BSA_ERR_UNSUPPORTED.  The same
 * limit applies to bsa_select_scores and bsa_score_select_padded.
 */
bsa_status bsa_score_select(const bsa_problem* problem, const bsa_select_params* params,
                            const float* q_centroid, const float* q_norm,
                            const float* k_centroid, const float* k_radius, int32_t* row_ptr,
                            int32_t* col_idx, int64_t col_capacity, float* scores_out,
                            float* bound_out, uint8_t* gate_out, void* workspace,
                            size_t workspace_bytes, void* hip_stream);

/*
 * bsa_score_select_noalloc -- bsa_score_select without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  It computes exactly what
 * bsa_score_select computes, with the same kernels and the same arguments
 * otherwise, but keeps its scratch (the score matrix when scores_out is NULL,
 * the kept-block masks and counts, the per-64-row count sums and offsets, the
 * sigma gate's tile buffers, the overflow word) in one fixed array of 64 MiB
 * that the library holds on each GPU it runs on until the process ends.  It
 * calls no allocating routine.
 *
 *   Limit: a selection needing more than 64 MiB of scratch (that is
 *   bsa_score_select_workspace_size(problem, params, scores_out != NULL)) returns
 *   BSA_ERR_WORKSPACE before anything is launched; passing scores_out moves the
 *   U*nb*nb score matrix out of the scratch.
 *   Sharing: every call on one GPU uses that GPU's single array, which keeps the
 *   last call's contents; calls that overlap on one GPU (two streams, two host
 *   threads) race and must be serialised by the caller.  Nothing in the array
 *   needs to start zeroed.  The overflow word of this call lives in the array and
 *   is not exposed.
 */
bsa_status bsa_score_select_noalloc(const bsa_problem* problem, const bsa_select_params* params,
                                    const float* q_centroid, const float* q_norm,
                                    const float* k_centroid, const float* k_radius,
                                    int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                                    float* scores_out, float* bound_out, uint8_t* gate_out,
                                    void* hip_stream);

/*
 * Where the selection calls report a kept set that did not fit their output.
 * Returns the byte offset, inside the workspace of bsa_score_select /
 * bsa_select_scores / bsa_score_select_padded (sized with the same arguments;
 * scores_given_or_exported as for the workspace size), of an int32 that each
 * such call sets when its stream reaches the end of the call: 0 when every
 * row's kept set was written in full, 1 when some row's kept blocks exceeded
 * col_capacity (CSR: the row offsets are then clamped to col_capacity) or width
 * (padded list: the row is cut at width).  With col_capacity and width at least
 * the bounds the calls require this cannot happen for any input; the word
 * exists so that a violation is visible instead of a silently shortened list.
 * -1 on invalid arguments.  Reading it is the caller's business (after its own
 * synchronisation); the library never reads it back.
 */
int64_t bsa_select_overflow_offset(const bsa_problem* problem, const bsa_select_params* params,
                                   int scores_given_or_exported);

/*
 * bsa_pool_key_bounds -- the Quest backbone's key-block summary ("Uncertainty-gated
 * selection ...", Methodology step 1: per-coordinate upper bounds from K-min/K-max).
 *
 *   k            [S, Hkv, D] bf16, or E4M3 codes with k_scale [Hkv, nb].
 *   k_min, k_max out [Hkv, nb, D] f32: the coordinate-wise minimum / maximum over
 *                the block's keys (dequantised values; a ragged last block over
 *                the rows it has).
 */
bsa_status bsa_pool_key_bounds(const bsa_problem* problem, const void* k, const float* k_scale,
                               float* k_min, float* k_max, void* hip_stream);

/* Device workspace bytes bsa_quest_scores needs (0 on an invalid problem). */
size_t bsa_quest_scores_workspace_size(const bsa_problem* problem);

/*
 * bsa_quest_scores -- Quest tile scores (same page, Methodology steps 1-2: the
 * per-coordinate upper bound as the block score of a query row; a tile's score is
 * the maximum over its rows).
 *
 *   scores[u][i][j] = max over the query rows t of block i, and over the heads of
 *   unit u, of  sum_d max(q[t][h][d] * k_min[g][j][d], q[t][h][d] * k_max[g][j][d])
 *   for j <= i (g the unit's kv head; other entries untouched).  For E4M3 queries
 *   q is code * q_scale[h][i]; q_scale must be >= 0.
 *
 *   q            [S, Hq, D] bf16, or E4M3 codes with q_scale [Hq, nb].
 *   k_min, k_max as bsa_pool_key_bounds writes them.
 *   scores       out f32 [U, nb, nb].
 *   workspace    at least bsa_quest_scores_workspace_size() bytes, else
 *                BSA_ERR_WORKSPACE (bounds repacked for the matrix cores).
 * The bound is computed on the bf16 matrix cores with fp32 accumulation: exact
 * products for bf16 inputs; bounds of E4M3 keys enter as a bf16 head plus tail
 * (relative representation error <= 2^-18).
 */
bsa_status bsa_quest_scores(const bsa_problem* problem, const void* q, const float* q_scale,
                            const float* k_min, const float* k_max, float* scores,
                            void* workspace, size_t workspace_bytes, void* hip_stream);

/* Device workspace bytes bsa_select_scores needs (0 on invalid arguments). */
size_t bsa_select_scores_workspace_size(const bsa_problem* problem,
                                        const bsa_select_params* params);

/*
 * bsa_select_scores -- bsa_score_select's selection rules (top-k, both gates, the
 * mass branch, forced blocks, CSR) on caller-provided scores [U, nb, nb] (entries
 * j <= i read), e.g. from bsa_quest_scores ("Uncertainty-gated selection ...",
 * technical summary: the router sits on top of any scoring backbone).  The
 * rescue branch is defined on centroid scores and radii, so rescue_fraction must
 * be 0 (BSA_ERR_INVALID_ARGUMENT otherwise).  row_ptr, col_idx, col_capacity,
 * gate_out as in bsa_score_select; workspace of at least
 * bsa_select_scores_workspace_size() bytes.
 */
bsa_status bsa_select_scores(const bsa_problem* problem, const bsa_select_params* params,
                             const float* scores, int32_t* row_ptr, int32_t* col_idx,
                             int64_t col_capacity, uint8_t* gate_out, void* workspace,
                             size_t workspace_bytes, void* hip_stream);

/* Slots per row of the padded list: the largest kept set any row can have under
 * the parameters (forced blocks plus rho*k or k by top-k, ceil(phi*|C|) by
 * rescue, every candidate with the mass branch); -1 on invalid arguments. */
int64_t bsa_padded_width(const bsa_problem* problem, const bsa_select_params* params);

/* Workspace bytes of bsa_score_select_padded (scores_given_or_exported: 1 when
 * scores_in or scores_out will be non-NULL); 0 on invalid arguments. */
size_t bsa_score_select_padded_workspace_size(const bsa_problem* problem,
                                              const bsa_select_params* params,
                                              int scores_given_or_exported);

/*
 * bsa_score_select_padded -- the selection of bsa_score_select (centroid scores)
 * or, with scores_in != NULL, of bsa_select_scores (given scores), written as a
 * uniform list instead of CSR ("Uncertainty-gated selection ...", technical
 * summary, Methodology step 5: one uniform dispatch shape, rows whose gate did
 * not fire padded with sentinels).
 *
 *   kv_idx       out int32 [U*nb, width]: row r holds its kept blocks ascending
 *                from kv_idx[r*width], then -1 to the end of the row.
 *   width        at least bsa_padded_width(), else BSA_ERR_CAPACITY; U*nb*width
 *                must fit int32 (BSA_ERR_UNSUPPORTED).
 *   scores_in    NULL: centroid scores from q_centroid/k_centroid (as
 *                bsa_score_select, exports allowed).  Otherwise the scores to
 *                select on; then rescue_fraction must be 0 and scores_out,
 *                bound_out NULL.
 *   gate_out, workspace as in bsa_score_select (workspace of at least
 *                bsa_score_select_padded_workspace_size() bytes).
 */
bsa_status bsa_score_select_padded(const bsa_problem* problem, const bsa_select_params* params,
                                   const float* q_centroid, const float* q_norm,
                                   const float* k_centroid, const float* k_radius,
                                   const float* scores_in, int32_t* kv_idx, int64_t width,
                                   float* scores_out, float* bound_out, uint8_t* gate_out,
                                   void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * bsa_attention_fwd_padded -- bsa_attention_fwd on a padded list: row (u, i) is
 * kv_idx[(u*nb + i)*width ...], its valid entries first (unique, in any order)
 * and -1 after them; the sentinels cost nothing.  width in [1, nb].
 */
bsa_status bsa_attention_fwd_padded(const bsa_problem* problem, const void* q, const void* k,
                                    const void* v, const float* q_scale, const float* k_scale,
                                    const float* v_scale, const int32_t* kv_idx, int64_t width,
                                    float softmax_scale, void* out, float* lse, void* hip_stream);

/*
 * bsa_attention_fwd -- attention over the kept blocks (RBS-Attention, third
 * paragraph: the fused mask drives sparse FlashAttention; MSA article: the main
 * branch attends only over the preselected blocks).
 *
 * For query head h and token t in block i, with row (u(h), i) of the CSR:
 *   O[t][h] = sum_s softmax_s(l_s) v_s over keys s <= t whose block is listed,
 *   l_s = softmax_scale * q_t . k_s (FP8: times q_scale[h][i] * k_scale[g][j],
 *   and v_s times v_scale[g][j]); lse[h][t] = log sum_s exp(l_s) (natural log).
 *
 *   row_ptr, col_idx  CSR as bsa_score_select writes it; each row's entries must
 *                     be unique.  Entries outside [0, i] are ignored.  A token
 *                     with no allowed key gets O = 0 and lse = -inf.
 *   out               out bf16 [S, Hq, D].
 *   lse               out f32 [Hq, S] (nullable).
 */
bsa_status bsa_attention_fwd(const bsa_problem* problem, const void* q, const void* k,
                             const void* v, const float* q_scale, const float* k_scale,
                             const float* v_scale, const int32_t* row_ptr,
                             const int32_t* col_idx, float softmax_scale, void* out,
                             float* lse, void* hip_stream);

/*
 * bsa_expand_e4m3 -- the V codes of an E4M3 problem as bf16 values, for
 * bsa_attention_fwd_expanded_v.  Every E4M3 value is exactly a bf16 value, so
 * this is a lossless change of format; v_scale is not applied (it stays a
 * separate argument of the attention call).
 *
 *   v        E4M3 codes [S, Hkv, D] (16-byte aligned).
 *   v_bf16   out bf16 [S, Hkv, D] (16-byte aligned, 2*S*Hkv*D bytes, owned by the
 *            caller).
 * BSA_ERR_INVALID_ARGUMENT for a BF16 problem (no codes) or missing pointers.
 */
bsa_status bsa_expand_e4m3(const bsa_problem* problem, const void* v, void* v_bf16,
                           void* hip_stream);

/*
 * bsa_attention_fwd_expanded_v -- bsa_attention_fwd for an E4M3 problem whose V
 * is given as its exact bf16 expansion (bsa_expand_e4m3); q, k and every scale
 * as for bsa_attention_fwd, the results equal its results bit for bit (same
 * passages).  The V tiles then go straight into LDS in the form the P V products
 * read, instead of being expanded there block by block.
 * BSA_ERR_INVALID_ARGUMENT for a BF16 problem (call bsa_attention_fwd).
 */
bsa_status bsa_attention_fwd_expanded_v(const bsa_problem* problem, const void* q, const void* k,
                                        const void* v_bf16, const float* q_scale,
                                        const float* k_scale, const float* v_scale,
                                        const int32_t* row_ptr, const int32_t* col_idx,
                                        float softmax_scale, void* out, float* lse,
                                        void* hip_stream);

/*
 * V in the form the P V products read, for bsa_attention_fwd_prepared_v (head_dim
 * = block_size = 128 only).  Layout: bf16 [nb, Hkv, 128, 128], block j of kv head
 * g a contiguous tile whose row d holds dimension d of the block's 128 keys, each
 * group of 16 keys stored in the order 0-3, 8-11, 4-7, 12-15 (the order in which
 * the probabilities of a 16-key step meet V in the bf16 matrix-core product);
 * keys past seq_len are zero.  E4M3 codes are expanded exactly (v_scale is not
 * applied; it stays an argument of the attention call).
 *
 * bsa_prepared_v_bytes: the size of that buffer (0 on invalid or unsupported
 * problems).
 * bsa_prepare_v:
 *   v            [S, Hkv, D] bf16 or E4M3 codes (16-byte aligned).
 *   v_prepared   out, bsa_prepared_v_bytes() bytes (16-byte aligned, owned by the
 *                caller).
 * BSA_ERR_UNSUPPORTED unless head_dim = block_size = 128.
 */
size_t bsa_prepared_v_bytes(const bsa_problem* problem);
bsa_status bsa_prepare_v(const bsa_problem* problem, const void* v, void* v_prepared,
                         void* hip_stream);

/*
 * bsa_attention_fwd_prepared_v -- bsa_attention_fwd (same passages, same
 * arguments) with V given as bsa_prepare_v wrote it; the results equal
 * bsa_attention_fwd's bit for bit.  Each V operand of the P V products is then
 * one 16-byte LDS read instead of two transposing 8-byte reads.
 * BSA_ERR_UNSUPPORTED unless head_dim = block_size = 128.
 */
bsa_status bsa_attention_fwd_prepared_v(const bsa_problem* problem, const void* q, const void* k,
                                        const void* v_prepared, const float* q_scale,
                                        const float* k_scale, const float* v_scale,
                                        const int32_t* row_ptr, const int32_t* col_idx,
                                        float softmax_scale, void* out, float* lse,
                                        void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* BSA_H */
