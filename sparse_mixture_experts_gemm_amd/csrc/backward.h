// Host-side declarations of the backward-pass launchers (backward.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "internal.h"

namespace moe {

// Weight-gradient GEMM on token-major rows: out(seg, m, n) = sum over the segment's rows p
// of A(p, m) B(p, n) (see backward.hip for the layouts).
struct WgradParams {
  const uint16_t* a;        // A(p, m) = a[p * lda + a_col + m]
  int lda, a_col;
  const uint16_t* b;        // B(p, n) = b[p * ldb + b_col + n]
  int ldb, b_col;
  const int32_t* offsets;   // [nseg + 1] row ranges of the segments, or null: rows [0, rows)
  int rows;
  int M, N;
  int nsplit;               // column-block size of the output layout (N: plain [M][N])
  float* out;               // fp32 [nseg][M][N] (in nsplit blocks)
};

// out[b * obs + c * ld + r] = in[b][r][c] (bf16, R and C multiples of 64).
hipError_t launch_transpose_mat(const void* in, void* out, int batch, int R, int C, long long obs,
                                int ld, hipStream_t s);

// out[p] = scale[p] * in[index[p]] for p < *valid_rows (a device count <= max_rows; bf16 rows
// of C columns; scale may be null).  Rows past the count are neither read nor written.
hipError_t launch_gather_rows(const void* in, const int32_t* index, const float* scale,
                              const int32_t* valid_rows, int max_rows, int C, void* out,
                              hipStream_t s);

// dw[t*k + j] = dout[t] . y[slot_pos[t*k + j]] / topk_w[t*k + j] (0 for dropped slots).
hipError_t launch_routing_weight_grad(int T, int k, int d, const void* dout, const void* y,
                                      const int32_t* slot_pos, const float* topk_w, float* dw,
                                      hipStream_t s);

// Logit gradients dl [T, E] from the scores [T, E], the selection and dw.
hipError_t launch_router_grad(const RouteParams& p, const float* scores, const int32_t* idx,
                              const float* dw, float* dl, hipStream_t s);

// d_router [E, d] = dl^T x and d_bias [E] = column sums of dl (either may be null).
size_t router_wgrad_ws_bytes(int T, int d, int E);
hipError_t launch_router_wgrad(int T, int d, int E, const void* x, const float* dl, float* d_router,
                               float* d_bias, void* ws, hipStream_t s);

// dx = dl W_r + scattered dx_perm rows + dx_shared (+ residual), bf16.
hipError_t launch_dx_combine(int T, int d, int E, int k, const float* dl, const void* wr,
                             const void* dx_perm, const int32_t* slot_pos, const void* dx_shared,
                             const void* residual, void* dx, hipStream_t s);

hipError_t launch_wgrad(const WgradParams& p, int nseg, int num_cus, hipStream_t s);

}  // namespace moe
