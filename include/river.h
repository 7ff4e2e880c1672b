/*
 * river.h -- C interface of the per-token exit-and-KV-fill library for
 * AMD MI355X (gfx950).
 *
 * The step has three calls on the hot path and one off it:
 *
 *   river_route      which tokens exit at this layer
 *   river_compact    stable split of the batch into continuing and exiting
 *                    tokens, plus the exit scatter of hidden states
 *   river_exit_projection  final RMSNorm of the exited rows, scattered to
 *                    their original positions (the LM head's input)
 *   river_kv_fill    K/V of every skipped layer written into each exited
 *                    token's own cache slot
 *   river_kv_fill_layer  the same through the layer's full K/V path (input
 *                    RMSNorm, K/V bias, rotary embedding of K)
 *   river_decode_step  one generation step: route, compact and fill at
 *                    every checkpoint, graph-capturable
 *   river_ridge_fit  the closed-form ridge maps the fill applies
 *   river_router_fit training of a checkpoint's router (BCE + Adam) on
 *                    calibration states (offline)
 *
 * Sources (web pages; cited by title and section):
 *   River-LLM -- "River-LLM: Large Language Model Seamless Exit Based on
 *     KV Share" (paper summary page): sections 前置知识, 核心方法,
 *     方法步骤详情, 技术新颖性.
 *   TIDE -- "TIDE: Token-Informed Depth Execution for Per-Token Early Exit
 *     in LLM Inference" (reading notes): 系统架构, 模块3, 模块4, 关键公式.
 *   RidgeFill -- news article "RidgeFill: 免训练后层缓存填充": method
 *     paragraph under 思路源头 and the closed-form ridge regression box.
 *
 * Conventions for every call:
 *   - Every pointer argument is a DEVICE pointer unless stated otherwise.
 *     The caller owns all memory and keeps it alive until the stream has
 *     run the enqueued work. The library allocates nothing; scratch memory
 *     comes in through a caller-owned workspace (size from
 *     river_workspace_size).
 *   - Calls enqueue kernels on stream `s` and return without waiting,
 *     except river_ridge_fit, which waits so that it can report a failed
 *     factorization.
 *   - Element types: RIVER_F32 (IEEE fp32) or RIVER_BF16 (bfloat16).
 *     Arithmetic accumulates in fp32.
 *   - Row-major matrices with a leading dimension `ld` in elements. Every
 *     base pointer must be 16-byte aligned and ld * element size must be a
 *     multiple of 16 bytes; d must be a multiple of 8.
 *   - Argument errors are reported synchronously as a status code and a
 *     message (river_last_error, thread-local); nothing is enqueued then.
 *     No C++ exception crosses this interface. A failed kernel launch gives
 *     RIVER_ERR_HIP.
 *   - n = 0 (or m_max = 0) is a valid empty call.
 *   - Calls are stateless and may run concurrently on different streams
 *     when their outputs and workspaces do not overlap.
 */
#ifndef RIVER_H
#define RIVER_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RIVER_OK = 0,
  RIVER_ERR_ARG = 1,          /* a size, pointer or threshold is invalid     */
  RIVER_ERR_DTYPE = 2,        /* an element type is not supported here       */
  RIVER_ERR_ALIGN = 3,        /* a pointer or leading dimension is misaligned */
  RIVER_ERR_UNSUPPORTED = 4,  /* a valid shape the library does not handle   */
  RIVER_ERR_WORKSPACE = 5,    /* workspace missing or too small              */
  RIVER_ERR_NOT_SPD = 6,      /* X^T X + lambda I is not positive definite   */
  RIVER_ERR_HIP = 7           /* a HIP runtime call or kernel launch failed  */
} river_status;

typedef enum { RIVER_F32 = 0, RIVER_BF16 = 1 } river_dtype;

/* How per-token decisions become the mask (River-LLM 方法步骤详情 step 3
 * takes the minimum over the batch; the same page's analysis and TIDE's
 * per-token router motivate independent decisions). */
typedef enum { RIVER_RULE_TOKEN = 0, RIVER_RULE_BATCH_MIN = 1 } river_rule;

/* Operation ids for river_workspace_size. */
typedef enum {
  RIVER_OP_ROUTE = 0, RIVER_OP_COMPACT = 1, RIVER_OP_KV_FILL = 2, RIVER_OP_RIDGE_FIT = 3,
  RIVER_OP_KV_FILL_LAYER = 4, RIVER_OP_DECODE_STEP = 5, RIVER_OP_ROUTER_FIT = 6,
  RIVER_OP_KV_FOLD = 7
} river_op;

/*
 * Group-quantized int4 weights of one projection for n_layers consecutive
 * layers (River-LLM 前置知识 PTQ: W4A16, 4-bit weights with 16-bit
 * activations). For layer l, output row o and input channel k:
 *
 *   w[l][o][k] = (q_k - zero[l][o][k / group]) * scale[l][o][k / group]
 *
 * where q_k is the 4-bit value of byte q[l][o][k / 2], low nibble when k is
 * even and high nibble when k is odd. Layers are contiguous:
 *   q     : uint8 [n_layers][n_out][d / 2]
 *   scale : sz_dtype [n_layers][n_out][d / group]
 *   zero  : sz_dtype [n_layers][n_out][d / group]   (a real-valued zero point)
 * n_out = n_kv_heads * head_dim; group must divide d.
 */
typedef struct {
  const uint8_t* q;
  const void* scale;
  const void* zero;
  river_dtype sz_dtype;
  int group;
} river_w4;

/*
 * river_route -- exit decision for n tokens at one layer.
 *
 * River-LLM 前置知识 and 方法步骤详情 step 3: the state-transition
 * similarity cos_i = <h_prev_i, h_cur_i> / (|h_prev_i| |h_cur_i|) between a
 * block's input and output. TIDE 关键公式 formula 3: the router
 * prob_i = sigmoid(w_up . SiLU(W_down . RMSNorm(h_cur_i))), with
 * RMSNorm(x) = gamma * x / sqrt(mean(x^2) + eps) over the d features and no
 * biases. TIDE formula 4 and River-LLM step 3: strict thresholds.
 *
 *   e_i    = (cos_i > tau) AND (prob_i > theta)        (NaN compares false)
 *   mask_i = e_i                          for RIVER_RULE_TOKEN
 *   mask_i = AND_j e_j for every i        for RIVER_RULE_BATCH_MIN
 *   *all_exit_out = AND_j e_j (0 when n = 0)
 *
 * h_prev, h_cur : dt [n][d] with leading dims ld_prev, ld_cur.
 * gamma         : dt [d], or NULL for all ones.
 * w_down        : dt [b][d], or NULL to switch the router off (prob = 1 and
 *                 only the cosine test applies).
 * w_up          : dt [b] (ignored when w_down is NULL).
 * tau, theta    : thresholds; -INFINITY disables a test, +INFINITY forbids
 *                 exit; NaN thresholds are rejected.
 * cos_out, prob_out : fp32 [n], may be NULL.
 * mask_out      : uint8 [n], required; 1 = exit.
 * all_exit_out  : int32 [1], may be NULL.
 * A zero-norm row has cos = 0. cos is clamped to [-1, 1].
 * Requirements: n >= 0, d >= 8 and d % 8 == 0, b in [1, 512] when the
 * router is on.
 */
river_status river_route(int n, int d, river_dtype dt,
                         const void* h_prev, int64_t ld_prev,
                         const void* h_cur, int64_t ld_cur,
                         const void* gamma, float eps,
                         const void* w_down, const void* w_up, int b,
                         float tau, float theta, river_rule rule,
                         float* cos_out, float* prob_out, uint8_t* mask_out,
                         int32_t* all_exit_out, hipStream_t s);

/*
 * river_compact -- stable split by mask, row gather and exit scatter.
 *
 * TIDE 模块4: "Batch Compact" separates continuing from exiting tokens and
 * "Exit Scatter" copies the exited tokens' hidden states back to their
 * original positions in an output buffer.
 *
 *   cont_idx[0..n_cont)  = ascending i with mask[i] == 0
 *   exit_idx[0..n_exit)  = ascending i with mask[i] != 0
 *   counts[0] = n_cont, counts[1] = n_exit
 *   h_cont[j]        = h[cont_idx[j]]            (if h_cont != NULL)
 *   row_ids_cont[j]  = row_ids[cont_idx[j]]      (if row_ids_cont != NULL)
 *   out[row_ids[i]]  = h[i] for every exiting i  (if out != NULL)
 *
 * mask    : uint8 [n].
 * h       : dt [n][d], leading dim ld_h (may be NULL when h_cont and out
 *           are both NULL).
 * row_ids : int32 [n], or NULL for the identity 0..n-1.
 * cont_idx, exit_idx : int32 [n] each; entries past the counts are left
 *           untouched. counts : int32 [2].
 * out     : dt [n_out_rows][d], leading dim ld_out. A row id outside
 *           [0, n_out_rows) is skipped (not written).
 * workspace : river_workspace_size(RIVER_OP_COMPACT, n, ...) bytes.
 * The result is unique and deterministic.
 */
river_status river_compact(int n, int d, river_dtype dt, const uint8_t* mask,
                           const void* h, int64_t ld_h, const int32_t* row_ids,
                           int32_t* cont_idx, int32_t* exit_idx, int32_t* counts,
                           void* h_cont, int64_t ld_cont, int32_t* row_ids_cont,
                           void* out, int64_t ld_out, int64_t n_out_rows,
                           void* workspace, size_t ws_bytes, hipStream_t s);

/*
 * river_exit_projection -- final RMSNorm of the exited rows, scattered to
 * their original rows of the output.
 *
 * TIDE 模块4: "Exit Projection" fuses an RMSNorm with the scatter of the
 * exited tokens; TIDE 模块3: an exited token's logits are the LM head
 * applied to the RMSNorm of its hidden state, so each row written here is
 * the LM head's input for that token.
 *
 * For t = 0..m-1, with r = row_idx[t] (or t) and dst = row_ids[r] (or r):
 *   out[dst][j] = gamma[j] * h[r][j] / sqrt(mean_k(h[r][k]^2) + eps)
 * rounded to dt (round to nearest even for bf16); the sum of squares and
 * the scaling are fp32.
 *
 * m        : min(*m_dev, m_max) when m_dev is not NULL (a device int32,
 *            e.g. counts+1 from river_compact), else m_max.
 * h        : dt [n_rows][d], leading dim ld_h.
 * row_idx  : int32 [m_max] rows of h (e.g. exit_idx), or NULL for 0..m-1
 *            (then m_max <= n_rows). A row outside [0, n_rows) is skipped.
 * row_ids  : int32 [n_rows] output row of each row of h, or NULL for the
 *            identity. A destination outside [0, n_out_rows) is skipped.
 * gamma    : dt [d], or NULL for all ones. eps: finite, >= 0. A zero row
 *            with eps = 0 gives NaN (0 times an infinite reciprocal RMS).
 * out      : dt [n_out_rows][d], leading dim ld_out; must not overlap h.
 *            Destinations of the projected rows must be distinct. Rows
 *            that receive nothing are left unchanged.
 * No workspace. Every d that is a multiple of 8 is handled.
 */
river_status river_exit_projection(int m_max, const int32_t* m_dev, int d, river_dtype dt,
                                   const void* h, int64_t ld_h, int n_rows,
                                   const int32_t* row_idx, const int32_t* row_ids,
                                   const void* gamma, float eps,
                                   void* out, int64_t ld_out, int64_t n_out_rows,
                                   hipStream_t s);

/*
 * river_kv_fill -- K/V of every skipped layer for each exited token.
 *
 * River-LLM 方法步骤详情 step 1 and 技术新颖性: the exit path writes the
 * K/V of each skipped layer at the backbone's own address (same position
 * index, head split and dimension layout), so the cache stays complete.
 * RidgeFill 思路源头: the skipped layer's input is predicted from the exit
 * state by a fitted linear map, then that layer's own projection writes the
 * cache. With no map (identity) this is River-LLM's "State Propagation".
 *
 * For layer l = 0..n_layers-1 and t = 0..m-1, with r = row_idx[t] (or t):
 *   x_hat = maps[l] . h[r]          (x_hat_j = sum_k maps[l][j][k] h[r][k];
 *                                    x_hat = h[r] when maps is NULL)
 *   K = Wk[l] . x_hat,  V = Wv[l] . x_hat      (n_out = n_kv_heads*head_dim)
 *   k_cache[l][slot[r]][hh][dd] = K[hh*head_dim + dd], likewise V.
 *
 * m        : rows to fill = min(*m_dev, m_max) when m_dev is not NULL (a
 *            device int32, e.g. counts+1 from river_compact, so no host
 *            synchronisation is needed), else m_max.
 * h        : dt [n_rows][d], leading dim ld_h.
 * row_idx  : int32 [m_max] rows of h (e.g. exit_idx), or NULL for 0..m-1.
 *            Entries outside [0, n_rows) are skipped.
 * slot     : int32 [n_rows], the cache slot of each row of h. Slots of the
 *            filled rows must be distinct; a slot outside [0, n_slots) is
 *            skipped.
 * maps     : dt [n_layers][d][d] (output-major), or NULL for the identity.
 * wk, wv   : host pointers to int4 descriptors of n_layers layers.
 * k_cache, v_cache : dt [n_layers][n_slots][n_kv_heads][head_dim]; the
 *            first layer is the first skipped layer.
 * workspace: with maps, at least river_workspace_size(RIVER_OP_KV_FILL,
 *            m_max, d, 0, 0, 1) bytes; the layers are processed in as few
 *            chunks as the given size allows. Without maps none is needed.
 *            river_workspace_size(RIVER_OP_KV_FILL, m_max, d,
 *            n_kv_heads * head_dim, 0, n_layers) bytes also hold, for
 *            m_max <= 64 (and up to 256 when the projection has few
 *            tiles: at most 128 of 64 rows x 256 outputs x layers), the
 *            fp32 partial sums of a projection whose reduction over d is
 *            split into parts (so that a few rows still occupy every CU;
 *            the parts are added in a fixed order, so a result does not
 *            depend on which thread finishes first), and for m_max >= 2048
 *            rows given on the host (m_dev NULL) with at least half a
 *            256 x 256 tile per CU the weights dequantised to bf16 (the
 *            values the int4 path forms in
 *            registers), which a 256 x 256 bf16 GEMM then projects. With
 *            less, the projection dequantises in registers, unsplit. With
 *            maps and a workspace for fewer layers than n_layers, a chunk
 *            at such row counts takes as many x_hat layers as leave room
 *            for its dequantised weights (when one layer does).
 *            With maps, bf16, d % 128 == 0 and m_max >= 4 * n_out rows
 *            given on the host (m_dev NULL), the fill instead forms per
 *            layer F = deq([Wk; Wv]) . maps[l] (2 n_out x d, bf16) and
 *            projects the rows through it, K|V = F . h[r]: the same values
 *            up to rounding, in 2 n_out d^2 instead of 2 m d^2 flops for
 *            the maps; it needs 2 x (2 n_out d) + d^2 bf16 per layer of the
 *            chunk (the dequantised weights, the transposed map and F),
 *            which the size above holds at such row counts.
 * Only the filled slots are written; every other byte is left unchanged.
 * Paths: bf16 with d % 256 == 0, n_out % 64 == 0, group % 64 == 0, the
 * same group and scale/zero dtype for wk and wv, an even number of groups
 * per row when scale/zero are bf16, and operand spans under 2^31 bytes runs
 * on MFMA; every other shape (and fp32) runs a generic kernel with fp32
 * arithmetic, one workgroup per (row, layer), which needs d <= 8192
 * (RIVER_ERR_UNSUPPORTED otherwise). n_layers <= 65535 per call.
 */
river_status river_kv_fill(int m_max, const int32_t* m_dev, int d, river_dtype dt,
                           const void* h, int64_t ld_h, int n_rows,
                           const int32_t* row_idx, const int32_t* slot,
                           int n_layers, const void* maps,
                           const river_w4* wk, const river_w4* wv,
                           int n_kv_heads, int head_dim,
                           void* k_cache, void* v_cache, int64_t n_slots,
                           void* workspace, size_t ws_bytes, hipStream_t s);

/*
 * river_kv_fold -- the skipped layers' maps folded into their K/V weights.
 *
 * RidgeFill 思路源头: a skipped layer's K and V come from its own
 * projection applied to the input the fitted map predicts. Both steps are
 * linear in the exit state, so per layer they compose into one matrix,
 * formed once per fitted map (off the per-step path, like the fit):
 *   F[l] = deq([Wk[l]; Wv[l]]) . maps[l]     (2 n_out x d, n_out =
 *                                             n_kv_heads * head_dim)
 *   F[l][o][k] = sum_j deq(W[l])[o][j] maps[l][j][k], rows 0..n_out-1 from
 *   Wk, n_out..2 n_out-1 from Wv; fp32 accumulation, rounded to bf16.
 * Without maps (NULL) F[l] is the dequantised weights themselves.
 *
 * maps     : bf16 [n_layers][d][d] (output-major, as river_kv_fill takes
 *            them), or NULL.
 * wk, wv   : host pointers to int4 descriptors of n_layers layers.
 * F        : bf16 [n_layers][2 n_out][d], written; caller-owned.
 * workspace: with maps, river_workspace_size(RIVER_OP_KV_FOLD, 0, d, n_out,
 *            0, L) bytes process L layers per pass (at least one);
 *            without maps none is needed.
 * Shapes: d % 256 == 0, n_out % 64 == 0, group % 64 == 0 and the same for
 * wk and wv (RIVER_ERR_UNSUPPORTED otherwise). Asynchronous on s.
 */
river_status river_kv_fold(int d, int n_layers, const void* maps,
                           const river_w4* wk, const river_w4* wv,
                           int n_kv_heads, int head_dim, void* F,
                           void* workspace, size_t ws_bytes, hipStream_t s);

/*
 * river_kv_fill_folded -- river_kv_fill through folded products.
 *
 * River-LLM 方法步骤详情 step 1 and 技术新颖性 (the skipped layers' K/V at
 * each exited token's own slot), RidgeFill 思路源头 (the map, then the
 * layer's projection), with the two composed by river_kv_fold:
 *   [K | V] = F[l] . h[r]  ->  k_cache[l][slot[r]], v_cache[l][slot[r]]
 * for l = 0..n_layers-1 and t = 0..m-1, r = row_idx[t] (or t). The same
 * K and V as river_kv_fill with the maps and weights F was folded from, up
 * to rounding (one bf16 rounding of F in place of one of x_hat).
 *
 * Arguments as river_kv_fill's, bf16 only (h, F, caches); F: bf16
 * [n_layers][2 n_out][d] from river_kv_fold. No workspace. Needs d % 256
 * == 0 and n_out % 64 == 0, with h's and F's byte spans under 2^31
 * (RIVER_ERR_UNSUPPORTED otherwise). Rows and slots outside their ranges
 * are skipped; only the filled slots are written.
 */
river_status river_kv_fill_folded(int m_max, const int32_t* m_dev, int d,
                                  const void* h, int64_t ld_h, int n_rows,
                                  const int32_t* row_idx, const int32_t* slot,
                                  int n_layers, const void* F,
                                  int n_kv_heads, int head_dim,
                                  void* k_cache, void* v_cache, int64_t n_slots,
                                  hipStream_t s);

/*
 * The rest of a skipped layer's K/V path, for river_kv_fill_layer. Each
 * part is switched off by a NULL pointer.
 *
 * RidgeFill 思路源头: the predicted input of a skipped layer goes through
 * that layer's own projection, which writes the cache as it normally would.
 * For the Llama-family models River-LLM evaluates that path is the layer's
 * input RMSNorm, the K and V projections, and the rotary position embedding
 * of K; GPT-2-style layers add K and V biases.
 */
typedef struct {
  const void* norm_gamma;   /* dt [n_layers][d]: input RMSNorm weight        */
  float norm_eps;           /* finite, >= 0                                 */
  const void* k_bias;       /* dt [n_layers][n_kv_heads * head_dim]         */
  const void* v_bias;       /* dt [n_layers][n_kv_heads * head_dim]         */
  const int32_t* pos;       /* int32 [n_rows]: rotary position of each row  */
  const float* rope_cos;    /* fp32 [n_pos][head_dim / 2]                   */
  const float* rope_sin;    /* fp32 [n_pos][head_dim / 2]                   */
  int64_t n_pos;
} river_layer;

/*
 * river_kv_fill_layer -- river_kv_fill through the layer's full K/V path.
 *
 * For layer l and row r (as in river_kv_fill, x_hat = maps[l] . h[r]):
 *   x_n = gamma[l] * x_hat / sqrt(mean(x_hat^2) + eps)    (if norm_gamma)
 *   K = Wk[l] . x_n + k_bias[l],  V = Wv[l] . x_n + v_bias[l]
 *   if pos: within each head, element i < head_dim/2 is paired with
 *     i + head_dim/2 and the pair turned by the angle of row pos[r]:
 *     K'[i]  = K[i] cos[p][i] - K[i + hd/2] sin[p][i]
 *     K'[i + hd/2] = K[i] sin[p][i] + K[i + hd/2] cos[p][i]
 * A row whose position is outside [0, n_pos) is skipped (nothing written).
 * layer may be NULL (then this is river_kv_fill). head_dim must be even
 * with rotation. workspace: with maps or norm_gamma, at least
 * river_workspace_size(RIVER_OP_KV_FILL_LAYER, m_max, d, 0, 0, 1) bytes;
 * the layers are processed in as few chunks as the size allows. The MFMA
 * path takes the shapes river_kv_fill's does, and head_dim % 32 == 0 with
 * rotation; every other shape runs the generic kernel (d and n_out with
 * 2 (d + n_out) + 4 floats of LDS <= 64 KB).
 */
river_status river_kv_fill_layer(int m_max, const int32_t* m_dev, int d, river_dtype dt,
                                 const void* h, int64_t ld_h, int n_rows,
                                 const int32_t* row_idx, const int32_t* slot,
                                 int n_layers, const void* maps,
                                 const river_w4* wk, const river_w4* wv,
                                 const river_layer* layer, int n_kv_heads, int head_dim,
                                 void* k_cache, void* v_cache, int64_t n_slots,
                                 void* workspace, size_t ws_bytes, hipStream_t s);

/*
 * One exit checkpoint of river_decode_step: the check after block `layer`.
 */
typedef struct {
  int layer;              /* e: blocks 1..e ran; 1 <= e < n_layers, increasing  */
  const void* h_prev;     /* dt [n][ld]: h^(e-1), the block's input              */
  const void* h_cur;      /* dt [n][ld]: h^(e), its output (the exit state)      */
  float tau, theta;       /* thresholds as in river_route                        */
  const void* w_down;     /* dt [b][d] router, or NULL (cosine test only)        */
  const void* w_up;       /* dt [b]                                              */
  const void* maps;       /* dt [n_layers - e][d][d] (blocks e+1..L), or NULL    */
  const void* folded;     /* bf16 [n_layers - e][2 n_out][d]: river_kv_fold of   */
                          /* the maps of blocks e+1..L (used in place of maps),  */
                          /* or NULL                                             */
} river_checkpoint;

/*
 * river_decode_step -- one generation step of the token-level exit loop.
 *
 * River-LLM 方法步骤详情 step 3: after each checked block the state-transition
 * similarity decides whether a token leaves the backbone for the exit path,
 * which writes the K/V of every remaining block at the token's slot (step 1,
 * 技术新颖性). TIDE formula 3 and 4: the decision may also need the router.
 *
 * For checkpoints c = 0..n_ck-1 in order, over the tokens still running:
 *   decision_i = river_route's decision on (h_prev, h_cur) of row i
 *   rule TOKEN: token i exits at c if decision_i;
 *   rule BATCH_MIN: every running token exits at c if all of them decide so
 *   an exiting token i gets exit_layer[i] = e and blocks e+1..L filled as
 *   river_kv_fill does from row i of h_cur (with the checkpoint's maps),
 *   at slot[i] of cache layers e..L-1.
 * Tokens that never exit get exit_layer[i] = n_layers. Rows of exited tokens
 * in the states of later checkpoints are read but do not matter.
 *
 * wk, wv : host pointers to int4 descriptors of blocks 1..n_layers.
 * k_cache, v_cache : dt [n_layers][n_slots][n_kv_heads][head_dim]; cache
 *          layer j - 1 holds block j.
 * gamma, eps, b : the routers' RMSNorm weight (NULL: ones) and width.
 * exit_layer : int32 [n], written.
 * workspace : river_workspace_size(RIVER_OP_DECODE_STEP, n, d, 0, 0,
 *          n_layers) bytes fill every checkpoint in one pass; with maps at
 *          least the size for n_layers = 2 is needed. Passing d_out =
 *          n_kv_heads * head_dim adds room for the split reduction that
 *          river_kv_fill describes (n <= 256).
 * The call enqueues an ordered sequence of kernels on s and returns: no
 * host synchronisation, allocation or runtime memset, so it may be captured
 * into a HIP graph once and the graph replayed for every step. The fill's
 * shape rules are river_kv_fill's. With n <= 1024 and the routers off at
 * every checkpoint (at most 32), or on at every checkpoint (at most 16, bf16,
 * d % 256 == 0, d <= 8192, b <= 128), two launches decide all checkpoints
 * (instead of a route and a compaction per checkpoint); on the fill's MFMA
 * path one projection then fills the exits of every checkpoint without
 * maps (all of them, or at least two), and each checkpoint with maps
 * fills its own. A checkpoint with folded products (river_checkpoint.folded,
 * bf16 only) fills as river_kv_fill_folded does, with no workspace for it.
 */
river_status river_decode_step(int n, int d, river_dtype dt, int64_t ld, int n_ck,
                               const river_checkpoint* ck, int n_layers, const void* gamma,
                               float eps, int b, river_rule rule,
                               const river_w4* wk, const river_w4* wv,
                               int n_kv_heads, int head_dim, const int32_t* slot,
                               void* k_cache, void* v_cache, int64_t n_slots,
                               int32_t* exit_layer, void* workspace, size_t ws_bytes,
                               hipStream_t s);

/*
 * river_decode_step_static -- river_decode_step with no workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation). It
 * allocates nothing: its scratch is a static device array of 64 MiB
 * (67,108,864 bytes) that the library holds on each GPU it runs on until
 * the process ends; the array's device address is looked up once per
 * device, on the first call with that device current.
 *
 * Arguments, results and the rest of the contract are river_decode_step's.
 * The call uses min(64 MiB, river_workspace_size(RIVER_OP_DECODE_STEP, n,
 * d, n_kv_heads * head_dim, 0, n_layers)) bytes of the scratch, so its
 * result equals river_decode_step's with a workspace of that size. It
 * returns RIVER_ERR_WORKSPACE, with the sizes in river_last_error, when
 * even the least workspace river_decode_step takes (the fixed part, plus
 * one layer of x_hat with maps) exceeds 64 MiB.
 *
 * Every call on one GPU shares that GPU's scratch, which keeps the last
 * call's contents (the step writes every byte it reads before reading it):
 * calls that overlap on one GPU, on any streams or threads, race; the
 * caller orders them (one stream, or events).
 */
river_status river_decode_step_static(int n, int d, river_dtype dt, int64_t ld, int n_ck,
                                      const river_checkpoint* ck, int n_layers, const void* gamma,
                                      float eps, int b, river_rule rule, const river_w4* wk,
                                      const river_w4* wv, int n_kv_heads, int head_dim,
                                      const int32_t* slot, void* k_cache, void* v_cache,
                                      int64_t n_slots, int32_t* exit_layer, hipStream_t s);

/*
 * river_ridge_fit -- closed-form ridge maps (RidgeFill, ridge box):
 *
 *   W_t = (X^T X + lambda I)^-1 X^T Y_t     for t = 0..n_targets-1
 *
 * computed as an fp32 Cholesky factorization of G = X^T X + lambda I (Gram
 * matrices accumulated in fp32), no intercept, lambda not scaled by n.
 * X : xdt [n][d_in]; Y : ydt [n_targets][n][d_out]; xdt == ydt.
 * W : wdt [n_targets][d_out][d_in], output-major, i.e. W[t] = W_t^T, the
 *     layout river_kv_fill takes as maps.
 * Waits for completion; returns RIVER_ERR_NOT_SPD when a pivot of the
 * factorization is not positive (W is then unspecified).
 * Requirements: d_in % 64 == 0 and d_out % 64 == 0 for bf16, n % 64 == 0
 * for bf16; lambda >= 0.
 */
river_status river_ridge_fit(int n, int d_in, int d_out, int n_targets,
                             const void* X, river_dtype xdt,
                             const void* Y, river_dtype ydt, float lambda,
                             void* W, river_dtype wdt,
                             void* workspace, size_t ws_bytes, hipStream_t s);

/*
 * river_router_fit -- train one checkpoint's router on calibration states.
 *
 * TIDE 模块1 (offline calibration): the router of formula 3,
 *   p = sigmoid(w_up . SiLU(W_down . RMSNorm(h))),
 * is trained with binary cross-entropy and Adam (lr 1e-3 on the page) for
 * a number of epochs (100 on the page). The labels are 1 for tokens whose
 * cosine to their final-layer state exceeds 0.98 (formula 1): river_route
 * with h_prev = final states, h_cur = checkpoint states, tau = 0.98 and the
 * router off writes exactly these labels as its mask.
 *
 * Per epoch e the tokens are taken in the order order[e][0..n) (NULL: 0..n-1)
 * in mini-batches of `batch` (the last one possibly shorter); each batch's
 * loss is the mean BCE over its tokens, and one Adam step follows:
 *   m = beta1 m + (1 - beta1) g,  v = beta2 v + (1 - beta2) g^2,
 *   w -= lr (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + adam_eps),
 * t counting steps from 1 over the whole fit. The RMSNorm weight gamma is
 * fixed (NULL: ones); only W_down and w_up are trained.
 *
 * h       : dt [n][d] checkpoint states, leading dim ld_h.
 * labels  : uint8 [n], 0 or non-zero.
 * w_down  : fp32 [b][d], the initial weights in, the trained ones out.
 * w_up    : fp32 [b], likewise.
 * loss_out: fp32 [epochs], the mean training loss of each epoch (the sum of
 *           its batches' per-token losses over n), or NULL.
 * workspace: river_workspace_size(RIVER_OP_ROUTER_FIT, n, d, b, batch,
 *           epochs) bytes.
 * Arithmetic is fp32 with reductions in a fixed order: a fit is
 * deterministic. The call enqueues two kernels per batch and returns.
 * Requirements: d % 8 == 0, b in [1, 512], batch in [1, 1000], epochs >= 1,
 * finite lr > 0, beta1 and beta2 in [0, 1), adam_eps > 0.
 */
river_status river_router_fit(int n, int d, river_dtype dt, const void* h, int64_t ld_h,
                              const uint8_t* labels, const void* gamma, float eps, int b,
                              float* w_down, float* w_up, int epochs, int batch,
                              const int32_t* order, float lr, float beta1, float beta2,
                              float adam_eps, float* loss_out, void* workspace, size_t ws_bytes,
                              hipStream_t s);

/* Workspace bytes for an operation (arguments that do not apply are
 * ignored): ROUTE -> 0; COMPACT (n); KV_FILL (n = m_max, d, n_layers; 0
 * layers gives 0, the identity case; optional d_out = n_kv_heads *
 * head_dim); KV_FILL_LAYER (n = m_max, d,
 * n_layers; the bytes for n_layers layers, needed with maps or a norm);
 * DECODE_STEP (n, d, n_layers: the blocks of the model; optional d_out as
 * for KV_FILL); ROUTER_FIT (n, d,
 * d_out = b, n_targets = batch, n_layers = epochs);
 * RIDGE_FIT (n, d = d_in, d_out,
 * n_targets, and n_layers carries the dtype: RIVER_F32 or RIVER_BF16). */
size_t river_workspace_size(int op, int n, int d, int d_out, int n_targets, int n_layers);

/* Message of the last failed call on this thread ("" when none). */
const char* river_last_error(void);

/* Library version string. */
const char* river_version(void);

/* Test hook: force the compaction path (0 = automatic; 1 = single wave
 * ballot, n <= 64; 2 = one workgroup scan; 3 = multi-workgroup scan; 1-3
 * then copy rows in a second launch; 4 = one fused launch, each workgroup
 * counting the exits before its 16 (n <= 16384) or 64 tokens itself, the
 * automatic choice for n <= 65536). Process-wide; the paths give
 * bitwise-identical results. */
river_status river_debug_set_compact_path(int path);

/* Test hook: force the tiles of the fill's GEMMs (0 = automatic: 256 x 256
 * from 1024 rows (2048 for the projection) when that gives enough tiles to
 * occupy the compute units, else 128 x 128; with the row count on the
 * device only for the map GEMM and only at two 256 x 256 tiles per CU
 * for the row bound;
 * 1 = 128 x 128 for the map GEMM and the int4 projection; 2 = 256 x 256
 * for the map GEMM and, with room in the workspace and more than 64 rows,
 * the projection on dequantised weights; 1 and 2 also keep the map GEMM
 * from splitting its reduction at small row counts; 3 = as 2, with the
 * 256 x 256 tiles on the 8-wave kernel even where d % 128 == 0 would take
 * the 4-wave one). Process-wide. The 128 and 256 tiles group the reduction
 * over d into MFMA steps differently, so their results agree to fp32
 * rounding, not bit for bit; the two 256 x 256 kernels (paths 2 and 3 at
 * d % 128 == 0) run the same MFMAs in the same order and agree bit for
 * bit. */
river_status river_debug_set_gemm_path(int path);

/* Test hook: 1 forces river_decode_step onto its per-checkpoint launches
 * (route, compact, fill per checkpoint) where it would take the two
 * decision launches for all checkpoints (n <= 1024, and the routers off at
 * every checkpoint with at most 32 checkpoints, or on at every checkpoint
 * with at most 16 and bf16 states of d % 256 == 0, d <= 8192, b <= 128);
 * 0 = automatic. Process-wide. The decisions are
 * bit-identical; the caches too when both paths split the projection's
 * reduction into the same parts (otherwise they agree to rounding). */
river_status river_debug_set_decode_path(int path);

/* Test hook: how river_kv_fill runs a plain fill with maps on its MFMA path
 * (bf16, d % 128 == 0, the row count given on the host): 0 = automatic
 * (through the product F = deq([Wk; Wv]) . maps per layer from m_max >=
 * 4 n_out rows on, when the workspace holds one layer of dequantised
 * weights, transposed map and F), 1 = never, 2 = whenever the workspace
 * holds it. Process-wide; the two ways agree to rounding. */
river_status river_debug_set_fill_fuse(int mode);

/* Launches river_kv_fill can time (river_debug_time_kernels). */
typedef enum {
  RIVER_TIMED_FILL_PROJECTION = 0, /* the bf16 projection into the cache: through the
                                      product F, or on dequantised weights           */
  RIVER_TIMED_FILL_PRODUCT = 1     /* the GEMM F = deq([Wk; Wv]) . maps               */
} river_timed_kernel;

/* Measurement hook: with on != 0, river_kv_fill records a pair of HIP events
 * on its stream right before and after each launch named in
 * river_timed_kernel (of the current device, up to 1024 pairs not yet read;
 * none on a stream under graph capture). Process-wide; on = 0 stops new
 * records. Timing adds an event record before and after the launch and no
 * other work. */
river_status river_debug_time_kernels(int on);

/* Reads and clears the records of one river_timed_kernel: waits for each
 * record's end event, then *total_ms = the sum of the elapsed times and
 * *launches = their number (0 and 0.0 when none). Records whose end was
 * never recorded (a launch that failed) are dropped uncounted.
 * RIVER_ERR_ARG for an unknown kind or a null pointer, RIVER_ERR_HIP when
 * waiting for an event fails. */
river_status river_debug_kernel_times(int kind, double* total_ms, int* launches);

/* Test hook, host only (enqueues nothing): the plan river_kv_fill takes for
 * a plain bf16 fill with maps on its MFMA path (d % 256 == 0, n_out =
 * n_kv_heads * head_dim with n_out % 64 == 0) given ws_bytes of workspace:
 * *chunk = layers per chunk (x_hat of that many layers held at once; at
 * large row counts after the room of the chunk's dequantised weights, when
 * at least one layer fits beside them), *path = the projection's
 * path for the first chunk (3 = through the product F = deq(W) . maps,
 * *chunk then its layers per chunk; 0 = int4 dequantised in registers, 1 = split
 * reduction over d in *parts parts, 2 = bf16 GEMM on weights dequantised
 * into the workspace), *parts = the split's parts (1 otherwise).
 * dev_count != 0: the row count lives on the device. The gemm-path hook
 * applies. RIVER_ERR_WORKSPACE when not even one layer of x_hat fits. */
river_status river_debug_kv_fill_plan(int m_max, int dev_count, int d, int n_out, int n_layers,
                                      size_t ws_bytes, int* chunk, int* path, int* parts);

#ifdef __cplusplus
}
#endif

#endif /* RIVER_H */
