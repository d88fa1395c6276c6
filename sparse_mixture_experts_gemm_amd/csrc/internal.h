// Host-side declarations shared between the C ABI (api.cpp) and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// Routing parameters passed by value to the route / select kernels.
struct RouteParams {
  int T, d, E, k, G, Gk, n_g;
  int score_fn;       // moe_score_fn
  int renormalize;
  float route_scale;
  const float* select_bias;   // [E] selection-only bias or null
  // pre-norm: route RMSNorm(x) (gain norm_gamma [d] fp32, eps norm_eps) and write it to
  // x_norm [T, d] (activation dtype); norm_gamma null: route x as given
  const float* norm_gamma;
  float norm_eps;
  void* x_norm;
};

// Segments of a grouped GEMM.  Routed: segment e = rows [offsets[e], offsets[e+1]).
// Shared: one segment of `rows` rows.
struct GemmParams {
  const void* a;            // activations (bf16 or fp32), row length K_a
  const int32_t* row_index; // gather map for A rows (row space -> a row), or null
  const int32_t* offsets;   // [nseg+1] device, or null for a single segment of `rows` rows
  int nseg;
  int rows;                 // rows of the row space (bounds)
  int d, I, S;              // model dim, expert inter dim, shared count
  int N;                    // output columns (UP: I_eff; DOWN: d)
  int K;                    // contraction length (UP: d; DOWN: I_eff)
  int kblock;               // K is split in blocks of kblock with separate weight slabs
  // weights for this call (already offset for routed/shared)
  const void* w_gate;       // UP: [nseg][N][K] (shared: [S*I][d] contiguous)
  const void* w_up;         // UP SwiGLU
  const void* w_down;       // DOWN: routed [nseg][d][I]; shared [S][d][I]
  const float* s_gate;      // e4m3 scales
  const float* s_up;
  const float* s_down;
  const float* row_weight;  // DOWN: per-row multiplier or null
  void* out;                // [rows][N]  (UP backward: [rows][2N] SwiGLU, [rows][N] ReLU^2)
  const void* dact;         // UP backward: gradient of the activation output h, [rows][N]
  // DOWN stage on weights stored [K][N] per segment (launch_down_trb): B(n, k) is
  // w_down[seg][k][n] for k < trb_split, then w_up[seg][k - trb_split][n]
  int trb_split;
};

enum class Stage { Up = 0, Down = 1 };

hipError_t launch_route(const RouteParams& p, int act_dtype, const void* x, const void* router,
                        const float* bias, float* scores, int32_t* idx, float* w,
                        hipStream_t s);
// Small batches of bf16 tokens (no pre-norm): the router's logits as four partial sums
// spread over many workgroups (into part, split_route_part_bytes), then one wave per token
// sums them, scores and selects.  Bit for bit launch_route.
constexpr int kSplitRouteTokens = 256;
bool split_route_applies(const RouteParams& p, int act_dtype);
size_t split_route_part_bytes(int T, int E);
hipError_t launch_route_split(const RouteParams& p, const void* x, const void* router,
                              const float* bias, float* part, float* scores, int32_t* idx,
                              float* w, hipStream_t s);
hipError_t launch_select(const RouteParams& p, const float* scores, const float* keys,
                         int32_t* idx, float* w, hipStream_t s);

// Load statistics: per-chunk partial sums in ws (stats_ws_bytes), then one reduction.
size_t stats_ws_bytes(int T, int E);
hipError_t launch_load_stats(int T, int E, int k, const float* scores, const int32_t* idx,
                             float alpha, float* f, float* p, float* loss, void* ws,
                             hipStream_t s);

// capacity: rows an expert may keep (INT_MAX: unlimited); dropped slots get slot_pos -1.
size_t permute_ws_bytes(int T, int E);
hipError_t launch_permute(int T, int E, int k, int capacity, const int32_t* idx,
                          const float* topk_w, int32_t* counts, int32_t* offsets,
                          int32_t* perm_token, int32_t* slot_pos, float* perm_weight, void* ws,
                          hipStream_t s);

// Per-row e4m3 quantisation of bf16 rows [rows, cols] (cols a multiple of 8): codes
// [rows, cols] and one fp32 scale per row.
hipError_t launch_quant_rows(int rows, int cols, const void* a, uint8_t* q, float* scale,
                             hipStream_t s);

// fp8_act: UP stage on e4m3 activations (a = codes, row_weight = per-a-row scales) with
// e4m3 weights.
hipError_t launch_grouped_gemm(const GemmParams& p, Stage stage, int act, int act_dtype,
                               int weight_dtype, int num_cus, hipStream_t s, bool fp8_act = false);

// UP stage recomputed for the backward pass (bf16 weights and activations): the epilogue
// reads dh = p.dact [rows][N] and writes the gradients of the two pre-activations a = A W1^T
// and b = A W3^T: SwiGLU out[r] = [da (N) | db (N)], ReLU^2 out[r] = da.
hipError_t launch_up_backward(const GemmParams& p, int act, int num_cus, hipStream_t s);

// DOWN-stage grouped GEMM whose weights are stored [K][N] (row k of N contiguous outputs)
// instead of [N][K]: out[r] = row_weight[r] * sum_k a[r][k] B(n, k), with B as described at
// GemmParams::trb_split (bf16 only).  The data gradients of the backward pass use it on the
// forward weights as they are.
hipError_t launch_down_trb(const GemmParams& p, int num_cus, hipStream_t s);

// Grouped GEMM for K, kblock or N off the 64-element grid (multiples of 8; bf16
// activations, bf16 or e4m3 weights): operands straight from global memory, 64 x 64 tiles.
bool tail_gemm_applies(const GemmParams& p);
hipError_t launch_tail_gemm(const GemmParams& p, Stage stage, int act, int weight_dtype,
                            int num_cus, hipStream_t s);

// Weight-streaming variant of the grouped GEMM for few rows per segment.  `second`, when
// given, is a second segment set (e.g. the shared experts) run in the same launch.
bool decode_gemm_applies(const GemmParams& p, int act_dtype);
hipError_t launch_decode_gemm(const GemmParams& p, Stage stage, int act, int weight_dtype,
                              hipStream_t s, const GemmParams* second = nullptr);

// residual [T, d] or null: added last (the unnormalised input of a pre-norm layer)
hipError_t launch_combine(int T, int d, int k, int act_dtype, const void* y_perm,
                          const int32_t* slot_pos, const void* y_shared, const void* residual,
                          void* out, hipStream_t s);

}  // namespace moe
