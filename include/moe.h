/*
 * libmoe — forward pass of a fine-grained MoE FFN layer on MI355X (gfx950).
 *
 * The layer (as the pages state it):
 *   router      l = W_r x (+ b)            "大模型工程（一）：Transformer 到 MoE", section
 *                                           "MoE 数学：路由、容量与平衡详解" (g(x) = W_g x, no bias)
 *   scores      s = sigmoid(l) or softmax(l)  "FusionLLM：融合 MLA、GDN 与 MoE 的高效混合架构大模型训练框架",
 *                                           section "混合专家（MoE）" (sigmoid gating); MoEBlock listing (softmax)
 *   selection   group-limited top-k, weights renormalised over the k picks
 *   experts     SwiGLU  W2 (silu(W1 x) * (W3 x))   or  ReLU^2  W2 (max(W1 x, 0))^2
 *   shared      S always-on experts added with weight 1
 *   combine     out[t] = sum_j w_j FFN_{e_j}(x_t) + sum_s FFN^sh_s(x_t)
 *
 * Conventions of every call:
 *   - Tensor pointers are DEVICE pointers, row-major, owned by the caller; the library
 *     keeps no pointer after a call returns, allocates no device memory and never
 *     synchronises.  Work is enqueued on `stream` (NULL = the default stream).
 *   - Weights use the nn.Linear layout [out, in], stacked over experts on dim 0.
 *   - Arguments are validated on the host before anything is enqueued; a call that
 *     returns an error has enqueued nothing.  Asynchronous device faults surface at the
 *     caller's next synchronisation.  No C++ exception crosses this interface.
 *   - act_dtype applies to x, the router weight, the intermediates and the output
 *     (MOE_F32 or MOE_BF16); weight_dtype applies to the expert weights (MOE_F32 with
 *     MOE_F32 activations; MOE_BF16 or MOE_FP8_E4M3 with MOE_BF16 activations).
 *   - Limits: 1 <= E <= 64, 1 <= k <= E, E % G == 0, 1 <= Gk <= G, k <= Gk*E/G,
 *     n_g in {1, 2} and n_g <= E/G; dim and inter_dim multiples of 8 (bf16 weights), of
 *     16 (e4m3 weights, and fp32); with fp8_act dim a multiple of 128 and inter_dim of 64;
 *     moe_backward needs multiples of 64.  Multiples of 64 take the tiled MFMA kernels,
 *     other sizes a kernel built for the tails (moe_gemm_kernel_path tells which);
 *     num_tokens >= 0 (0 is a no-op); pointers 16-byte aligned; sizes whose element
 *     offsets exceed 2^31 - 1 (T*k*max(dim, inter_dim), T*S*inter_dim, E*dim*inter_dim,
 *     S*inter_dim*dim) are MOE_ERR_UNSUPPORTED.
 *     Violations return MOE_ERR_INVALID_ARG (bad values) or MOE_ERR_UNSUPPORTED
 *     (valid but not implemented).
 *   - Calls are re-entrant; calls that share output or workspace buffers on the same
 *     stream are ordered by the stream, on different streams they race.
 */
#ifndef LIBMOE_MOE_H
#define LIBMOE_MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,  /* null required pointer, out-of-range or inconsistent value */
  MOE_ERR_UNSUPPORTED = 2,  /* valid request outside what the library implements      */
  MOE_ERR_WORKSPACE = 3,    /* workspace pointer null or smaller than required          */
  MOE_ERR_HIP = 4,          /* a HIP launch or runtime call failed (see moe_last_hip_error) */
  MOE_ERR_INTERNAL = 5      /* unexpected internal failure                              */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2 } moe_dtype;
typedef enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_score_fn;
typedef enum { MOE_ACT_SWIGLU = 0, MOE_ACT_RELU2 = 1 } moe_act;
typedef enum { MOE_STAGE_UP = 0, MOE_STAGE_DOWN = 1 } moe_stage;
typedef enum { MOE_EXPERTS_ROUTED = 0, MOE_EXPERTS_SHARED = 1 } moe_expert_set;

typedef struct {
  int32_t num_tokens;        /* T                                                        */
  int32_t dim;               /* d                                                        */
  int32_t num_experts;       /* E routed experts                                         */
  int32_t top_k;             /* k experts per token                                      */
  int32_t num_groups;        /* G contiguous groups of E/G experts (1 = no group limit)  */
  int32_t topk_groups;       /* Gk groups kept per token                                 */
  int32_t group_score_topn;  /* n_g: a group's score is the sum of its n_g best scores   */
  int32_t num_shared;        /* S always-on shared experts (0 allowed)                   */
  int32_t inter_dim;         /* I, inter dim of every routed and shared expert           */
  moe_score_fn score_fn;     /* sigmoid or softmax over the E logits                     */
  int32_t renormalize;       /* 1: w = s / sum(selected s); 0: w = s                     */
  float route_scale;         /* multiplies every routing weight (1.0f)                   */
  moe_act act;               /* SwiGLU (gate, up, down) or ReLU^2 (gate, down)           */
  moe_dtype act_dtype;       /* MOE_F32 or MOE_BF16                                      */
  moe_dtype weight_dtype;    /* MOE_F32, MOE_BF16 or MOE_FP8_E4M3                        */
  float capacity_factor;     /* c > 0: each expert takes at most floor(c*T*k/E) rows per
                                batch, in token order, and drops the rest (the dropped slots
                                contribute nothing); c <= 0: unlimited (no dropping).
                                Source: expert capacity c|T|k/E and token dropping, section
                                "MoE 数学：路由、容量与平衡详解" of "大模型工程（一）"   */
  int32_t fp8_act;           /* 1: the up projections multiply e4m3 activations (each token
                                row quantised with scale max|x|/448, moe_quantize_rows) by the
                                e4m3 weights, fp32 accumulation; needs act_dtype MOE_BF16,
                                weight_dtype MOE_FP8_E4M3 and dim a multiple of 128
                                (MOE_ERR_UNSUPPORTED otherwise).  0: bf16 activations.
                                Source: FP8 E4M3 products with FP32 accumulation, section
                                "生产现实：前沿实验室真正交付的内容" of "大模型工程（一）"  */
  int32_t pre_norm;          /* 1: the layer reads RMSNorm(x) = x / sqrt(mean_c x_c^2 + eps)
                                * norm_gamma (per token, no mean subtraction): the router and
                                the experts take the normalised rows, stored in act_dtype
                                (moe_rmsnorm_route).  0: x as given.
                                Source: the pre-norm decoder-layer sketch and item 2 (RMSNorm)
                                of section "变了什么，为什么变" of "大模型工程（一）"       */
  float norm_eps;            /* eps of the RMSNorm, finite, >= 0 (1e-6 for bf16: section
                                "常见陷阱", item 3); with eps = 0 an all-zero row is 0/0    */
  int32_t residual;          /* 1: moe_forward adds x (the unnormalised input) to its output,
                                h + moe(rms_norm(h)) of the same sketch.  0: no residual    */
} moe_config;

/* Expert weights.  [out, in] per expert, stacked on dim 0.  e4m3 weights carry one fp32
 * scale per output channel (per row): W[n, :] = scale[n] * e4m3(code[n, :]). */
typedef struct {
  const void* router;        /* [E, d] act_dtype                                           */
  const float* logit_bias;   /* [E] added to the logits before scoring, or NULL            */
  const void* w_gate;        /* [E, I, d]                                                  */
  const void* w_up;          /* [E, I, d]; NULL for MOE_ACT_RELU2                          */
  const void* w_down;        /* [E, d, I]                                                  */
  const float* s_gate;       /* [E, I]  e4m3 scales, else NULL                             */
  const float* s_up;         /* [E, I]                                                     */
  const float* s_down;       /* [E, d]                                                     */
  const void* sh_gate;       /* [S, I, d]  (NULL when S = 0)                               */
  const void* sh_up;         /* [S, I, d]                                                  */
  const void* sh_down;       /* [S, d, I]                                                  */
  const float* sh_s_gate;    /* [S, I]                                                     */
  const float* sh_s_up;      /* [S, I]                                                     */
  const float* sh_s_down;    /* [S, d]                                                     */
  const float* select_bias;  /* [E] selection-only expert bias, or NULL (see moe_route)     */
  const float* norm_gamma;   /* [d] fp32 RMSNorm gain; required when cfg->pre_norm, else
                                ignored                                                      */
} moe_weights;

/* Bytes of device workspace moe_forward needs for this config (host only, no HIP call).
 * moe_permute, moe_load_stats and moe_grouped_gemm need at most the same amount. */
moe_status moe_workspace_size(const moe_config* cfg, size_t* bytes);

/* Router, scoring and group-limited top-k for T tokens.
 *   l[t,e] = sum_c x[t,c] router[e,c] (+ logit_bias[e]), fp32 accumulation;
 *   s = sigmoid(l) or softmax over e;
 *   selection keys: s, or with a selection bias the scores of l + select_bias (sigmoid,
 *   or softmax over e, of the biased logits);
 *   groups g = experts [g*E/G, (g+1)*E/G); group score = sum of its n_g largest keys;
 *   keep the Gk best groups (ties: lower group index), then the k best experts of the
 *   kept groups by key (ties: lower expert index), slot order key-descending;
 *   w_j = route_scale * s_j / sum_i s_i (or route_scale * s_j without renormalisation),
 *   always from the unbiased scores s.
 * x [T, d] act_dtype; router [E, d] act_dtype; logit_bias, select_bias [E] fp32 or NULL;
 * scores [T, E] fp32 (optional, NULL = not written; the unbiased s); topk_idx [T, k]
 * int32; topk_w [T, k] fp32.
 * Source: the MoEBlock listing and section "MoE 数学：路由、容量与平衡详解" of
 * "大模型工程（一）：Transformer 到 MoE" (the selection-only bias b_e: its sections
 * "负载均衡" and "MoE 数学"); group-limited sigmoid gating in section "混合专家（MoE）" of
 * the FusionLLM training-framework page. */
moe_status moe_route(const moe_config* cfg, const void* x, const void* router,
                     const float* logit_bias, const float* select_bias, float* scores,
                     int32_t* topk_idx, float* topk_w, hipStream_t stream);

/* The pre-norm step in one launch: x_norm = RMSNorm(x) per token, with
 *   inv_rms[t] = 1 / sqrt(sum_c x[t,c]^2 / d + cfg->norm_eps) (fp32, fixed summation order),
 *   x_norm[t,c] = act_dtype(x[t,c] * inv_rms[t] * gamma[c]) (fp32 products, one rounding),
 * then moe_route on x_norm: the router multiplies exactly the stored x_norm values, so the
 * results equal those of moe_route called on x_norm.  cfg->pre_norm is not consulted.
 * x, x_norm [T, d] act_dtype (x_norm written; must not alias x); gamma [d] fp32; the other
 * arguments as in moe_route.  All pointers 16-byte aligned.
 * Source: RMSNorm before the MoE in the decoder-layer sketch and item 2 of section
 * "变了什么，为什么变" of "大模型工程（一）：Transformer 到 MoE"; routing as in moe_route. */
moe_status moe_rmsnorm_route(const moe_config* cfg, const void* x, const float* gamma,
                             const void* router, const float* logit_bias,
                             const float* select_bias, void* x_norm, float* scores,
                             int32_t* topk_idx, float* topk_w, hipStream_t stream);

/* The selection step of moe_route alone, on given fp32 scores [T, E] and optional
 * selection keys [T, E] (NULL: the scores are the keys).  Every value must be finite and
 * >= 0, as sigmoid and softmax values are.  Same outputs and tie rules.
 * Source: top-k over the gate scores with the selected weights renormalised (the MoEBlock
 * listing and section "MoE 数学：路由、容量与平衡详解" of "大模型工程（一）：Transformer 到
 * MoE"); the group limit of section "混合专家（MoE）" of the FusionLLM training-framework
 * page ("组限制路由", groups ranked by the sum of their n_g best scores). */
moe_status moe_select(const moe_config* cfg, const float* scores, const float* keys,
                      int32_t* topk_idx, float* topk_w, hipStream_t stream);

/* Load statistics of one batch and the Switch auxiliary-loss value:
 *   f[e] = (number of (t, j) with topk_idx[t, j] = e) / (T*k)   (routed, before capacity)
 *   p[e] = (1/T) sum_t scores[t, e] / sum_e' scores[t, e']     (mean routing probability)
 *   loss[0] = alpha * E * sum_e f[e] p[e]
 * scores [T, E] fp32 (the unbiased scores, as moe_route writes them), topk_idx [T, k];
 * f, p [E] and loss [1] fp32.  Sums are taken in a fixed order (deterministic).  ws: at
 * least moe_workspace_size bytes (per-chunk partial sums).
 * Source: the auxiliary loss alpha E sum f_e p_e and its terms, sections "负载均衡" and
 * "MoE 数学：路由、容量与平衡详解" of "大模型工程（一）：Transformer 到 MoE". */
moe_status moe_load_stats(const moe_config* cfg, const float* scores, const int32_t* topk_idx,
                          float alpha, float* f, float* p, float* loss, void* ws,
                          size_t ws_bytes, hipStream_t stream);

/* Expert-sorted permutation of the T*k (token, slot) pairs: rows ordered by
 * (expert ascending, token ascending); deterministic.  With cfg->capacity_factor > 0 each
 * expert keeps only its first floor(c*T*k/E) slots in that order (computed in double
 * from the fp32 factor) and the others are dropped.
 *   counts[e]      number of rows of expert e (slots kept)               [E]
 *   offsets[e]     exclusive prefix sum of counts (offsets[E] = rows)    [E+1]
 *   perm_token[p]  token of permuted row p                               [T*k]
 *   slot_pos[t*k+j] permuted row of slot j of token t, -1 when dropped   [T*k]
 *   perm_weight[p] topk_w of permuted row p (optional: both topk_w and perm_weight
 *                  NULL, or both set)                                    [T*k]
 * All int32/fp32 device buffers.  ws: at least moe_workspace_size bytes.  Every row of
 * topk_idx should hold k distinct experts in [0, E) (as moe_route produces).  An id
 * outside [0, E) (e.g. -1 padding) is skipped: it gets no row, is not counted, and its
 * slot_pos is -1, so moe_combine skips it.  Duplicates within a row give an unspecified
 * permutation.
 * Source: token routing to experts and per-expert batching ("MoE 数学" section and the
 * expert-parallel paragraph of "大模型工程（一）"; "批处理策略" of "开源混合架构大模型技术解析"). */
moe_status moe_permute(const moe_config* cfg, const int32_t* topk_idx, const float* topk_w,
                       int32_t* counts, int32_t* offsets, int32_t* perm_token,
                       int32_t* slot_pos, float* perm_weight, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/* Per-row e4m3 quantisation of bf16 rows a [rows, cols] (cols a multiple of 8):
 *   scale[r] = max_c |a[r, c]| / 448                    (fp32 division)
 *   q[r, c]  = e4m3(clamp(a[r, c] / scale[r], +-448))   (fp32 division, nearest even)
 * A row of zeros gets scale 0 and codes 0.  q [rows, cols] uint8 (8-byte aligned),
 * scale [rows] fp32.  Needs cfg->act_dtype MOE_BF16.
 * Source: FP8 E4M3 with FP32 accumulation, section "生产现实：前沿实验室真正交付的内容" of
 * "大模型工程（一）：Transformer 到 MoE"; the per-token scale is this library's reading. */
moe_status moe_quantize_rows(const moe_config* cfg, const void* a, int32_t rows, int32_t cols,
                             uint8_t* q, float* scale, hipStream_t stream);

/* One stage of the expert FFNs as a grouped GEMM over expert segments.
 *   set = MOE_EXPERTS_ROUTED: segment e is rows [offsets[e], offsets[e+1]) of a row space
 *         of `rows` rows (offsets: device [E+1], from moe_permute); routed weights.
 *   set = MOE_EXPERTS_SHARED: one segment of `rows` rows; the S shared experts act as one
 *         expert of inter dim S*I (offsets ignored).
 *   A row r of the row space is a[row_index[r]] when row_index is given (a gather, e.g.
 *   perm_token over x), else a[r].
 *   stage UP:   a rows have d elements (act_dtype); out[r] = act(a_r W_gate^T, a_r W_up^T),
 *               [rows, I] (routed) or [rows, S*I] (shared), act_dtype;
 *               SwiGLU: silu(g) * u; ReLU^2: max(g, 0)^2.
 *   stage DOWN: a rows have I (routed) or S*I (shared) elements; out[r] =
 *               row_weight[r] * (a_r W_down^T) (row_weight NULL = 1), [rows, d], act_dtype;
 *               for the shared set the S experts' outputs are summed.
 * e4m3 weights are multiplied by their per-output-channel scales.  fp32 accumulation.
 * With cfg->fp8_act the UP stage takes a = e4m3 codes (moe_quantize_rows) and row_weight
 * = the per-row scales of a (indexed like a, i.e. through row_index); it is required.
 * ws / ws_bytes: reserved, may be NULL / 0.
 * Source: grouped GEMM after routing and the fused Linear+ReLU^2 kernel, section
 * "融合内核" of the FusionLLM training-framework page; SwiGLU in item 3 of section
 * "变了什么，为什么变" of "大模型工程（一）". */
moe_status moe_grouped_gemm(const moe_config* cfg, moe_stage stage, moe_expert_set set,
                            const void* a, const int32_t* row_index, const int32_t* offsets,
                            int32_t rows, const moe_weights* w, const float* row_weight,
                            void* out, void* ws, size_t ws_bytes, hipStream_t stream);

/* Kernel family that moe_grouped_gemm (and moe_forward) runs for one stage and expert set
 * of `rows` rows (host only, no HIP call):
 *   MOE_GEMM_PATH_TILED   MFMA kernel on LDS-staged 64-wide K-slices (dim and inter_dim
 *                         multiples of 64; the fast path of the prefill shapes);
 *   MOE_GEMM_PATH_DECODE  weight-streaming kernel for few rows per expert;
 *   MOE_GEMM_PATH_TAIL    MFMA kernel on directly loaded operands, for a K or N that is a
 *                         multiple of 8 (bf16) or 16 (e4m3) but not of 64;
 *   MOE_GEMM_PATH_F32     fp32 activations and weights;
 *   MOE_GEMM_PATH_FP8_ACT e4m3 x e4m3 up projection (cfg->fp8_act).
 * The choice depends only on cfg, stage, set and rows.  MOE_ERR_INVALID_ARG / _UNSUPPORTED
 * as moe_grouped_gemm for the config.  Source: the grouped GEMM after routing, section
 * "融合内核" of the FusionLLM training-framework page. */
typedef enum {
  MOE_GEMM_PATH_TILED = 0,
  MOE_GEMM_PATH_DECODE = 1,
  MOE_GEMM_PATH_TAIL = 2,
  MOE_GEMM_PATH_F32 = 3,
  MOE_GEMM_PATH_FP8_ACT = 4
} moe_gemm_path;
moe_status moe_gemm_kernel_path(const moe_config* cfg, moe_stage stage, moe_expert_set set,
                                int32_t rows, int32_t* path);

/* out[t] = sum_{j<k} y_perm[slot_pos[t*k+j]] + y_shared[t], summed in that fixed order in
 * fp32, rounded to act_dtype; slots with slot_pos < 0 (dropped) are skipped.
 * y_perm [T*k, d], y_shared [T, d] or NULL, out [T, d].
 * Source: the weighted merge of the selected experts' outputs (MoEBlock listing;
 * "四、工作原理" of "开源混合架构大模型技术解析") plus the always-on shared experts. */
moe_status moe_combine(const moe_config* cfg, const void* y_perm, const int32_t* slot_pos,
                       const void* y_shared, void* out, hipStream_t stream);

/* The whole layer: route -> permute -> UP/DOWN grouped GEMMs (routed and shared) ->
 * combine.  x [T, d] and out [T, d] act_dtype; ws at least moe_workspace_size bytes
 * (16-byte aligned).  The per-stage tensors (topk_idx, topk_w, counts, offsets,
 * perm_token, slot_pos, intermediates) live in ws.  With cfg->pre_norm the routing is
 * moe_rmsnorm_route (w->norm_gamma) and the experts read the normalised rows (kept in ws);
 * with cfg->residual, out[t] also adds x[t], after the expert outputs (fp32 sum).
 * With shared experts and more rows than the one-launch decode path takes, the shared
 * GEMMs run on a second stream that the library keeps per (device, caller stream)
 * (default priority, created on first use with its events, kept until the process ends):
 * it waits for everything queued on `stream` before the call, and `stream` waits for it
 * before the combine, so the call is ordered on `stream` as a whole, also under graph
 * capture.  Calls on different caller streams never share a side stream; after 32 caller
 * streams on one device, further ones run the shared GEMMs on `stream` itself.  Stage
 * events (moe_forward_ex) switch the second stream off. */
moe_status moe_forward(const moe_config* cfg, const moe_weights* w, const void* x,
                       void* out, void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_forward for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same layer with no
 * workspace argument and no allocation of any kind.  Its workspace is a 64 MiB array that
 * the library holds on every device it runs on until the process ends (moe_workspace_size
 * at most 64 MiB, e.g. T <= 1024 tokens at d = 2048, E = 64, k = 6, S = 4, I = 1536; a
 * larger config returns MOE_ERR_WORKSPACE before anything is enqueued).  Every launch,
 * shared experts included, runs on `stream` (no side stream).  Every call on a device
 * shares that device's array: calls that overlap on one device (on different streams, or
 * from different threads without ordering) race; calls ordered on one stream do not.
 * Nothing in the array needs to start at zero: each byte a kernel reads was written
 * earlier in the same call.  Arguments, results and errors as moe_forward. */
moe_status moe_forward_noalloc(const moe_config* cfg, const moe_weights* w, const void* x,
                               void* out, hipStream_t stream);

/* Options of moe_forward_ex. */
typedef struct {
  /* Events recorded on `stream` at the stage boundaries of the forward (NULL entries are
   * skipped): [0] before routing, [1] after routing, [2] after the permutation, [3] after
   * the routed up projection, [4] after the shared up projection, [5] after the routed
   * down projection, [6] after the shared down projection, [7] after the combine.  When
   * routed and shared experts run in one launch (few rows per expert), [3] and [4] (and
   * [5] and [6]) are recorded back to back after that launch.  Caller-owned events. */
  hipEvent_t stage_events[8];
  /* Device buffer [2E + 1] fp32, or NULL: when given, the forward also writes the load
   * statistics of moe_load_stats for its routing (f, then p, then the loss) with
   * aux_alpha as alpha; they are computed between events [1] and [2]. */
  float* load_stats;
  float aux_alpha;
} moe_forward_opts;

/* moe_forward with options (opts may be NULL, which is moe_forward). */
moe_status moe_forward_ex(const moe_config* cfg, const moe_weights* w, const void* x,
                          void* out, void* ws, size_t ws_bytes, hipStream_t stream,
                          const moe_forward_opts* opts);

/* ---------------------------------------------------------------------------------- */
/* Backward pass.                                                                      */

/* Gradients written by moe_backward: dx in the activation dtype, every other one fp32 in
 * the layout of its parameter.  All device pointers; NULL entries (other than dx) are not
 * computed. */
typedef struct {
  void* dx;             /* [T, d] act_dtype: dL/dx (includes dout when cfg->residual)     */
  float* d_router;      /* [E, d]                                                         */
  float* d_logit_bias;  /* [E]   (the gradient of an added logit bias)                    */
  float* d_w_gate;      /* [E, I, d]                                                      */
  float* d_w_up;        /* [E, I, d]  (SwiGLU only)                                       */
  float* d_w_down;      /* [E, d, I]                                                      */
  float* d_sh_gate;     /* [S, I, d]                                                      */
  float* d_sh_up;       /* [S, I, d]  (SwiGLU only)                                       */
  float* d_sh_down;     /* [S, d, I]                                                      */
} moe_grads;

/* Bytes of device workspace moe_backward needs (host only). */
moe_status moe_backward_workspace_size(const moe_config* cfg, size_t* bytes);

/* Gradients of L = sum(dout * out) for the forward that moe_forward computed from the same
 * cfg, weights and x into fwd_ws (its routing, permutation, h and y are read from there, so
 * the forward must have been enqueued before on the same stream and fwd_ws left unchanged).
 * The selection is held fixed (its derivative is zero); every other step is differentiated:
 *   expert FFNs: dy = w dout, dW2 = dy^T h, dh = dy W2, SwiGLU da = dh b silu'(a),
 *     db = dh silu(a) (ReLU^2: da = dh 2 max(a, 0)), dW1 = da^T x, dW3 = db^T x,
 *     dx += da W1 + db W3 (a, b recomputed); shared experts alike with weight 1;
 *   routing weights: dw_j = dout . y_hat_j; renormalised weights w_j = c s_j / sum_i s_i
 *     give ds = (c / S)(dw - sum_j dw_j s_j / S) on the selected scores (dropped slots have
 *     dw = 0 but keep their place in S); sigmoid ds s (1 - s), or softmax through all E
 *     logits; d_router = dl^T x, d_logit_bias = sum_t dl, dx += dl W_r;
 *   residual: dx += dout.
 * The shared experts' chain runs on the side stream of moe_forward (same rules).
 * Supported: act_dtype and weight_dtype MOE_BF16, dim and inter_dim multiples of 64, no
 * pre_norm, no fp8_act, route_scale != 0 (else MOE_ERR_UNSUPPORTED / MOE_ERR_INVALID_ARG).
 * dout [T, d] bf16.  Weight gradients
 * accumulate in fp32 over the tokens in a fixed order; the result is deterministic.
 * Source: the chain rule through the forward of moe_forward; the router gradient through
 * the logits follows item 4 of section "常见陷阱" of "大模型工程（一）：Transformer 到 MoE". */
moe_status moe_backward(const moe_config* cfg, const moe_weights* w, const void* x,
                        const void* dout, const void* fwd_ws, size_t fwd_ws_bytes,
                        const moe_grads* grads, void* ws, size_t ws_bytes, hipStream_t stream);

/* Static description of a status code. */
const char* moe_status_string(moe_status status);

/* The hipError_t of the last MOE_ERR_HIP returned on the calling thread (0 if none). */
int32_t moe_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* LIBMOE_MOE_H */
