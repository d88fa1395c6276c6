// Expert-sorted permutation of the (token, slot) pairs.
//
// Tokens are routed to experts and batched per expert before the expert FFNs run
// ("大模型工程（一）：Transformer 到 MoE", sections "MoE 数学：路由、容量与平衡详解" and the
// expert-parallel paragraph; "开源混合架构大模型技术解析", "批处理策略").  The order is
// fixed: expert ascending, then token ascending, so the result does not depend on
// scheduling.  Three launches:
//   1. histogram: one workgroup per chunk of kChunk tokens counts its slots per expert
//      in LDS and writes the chunk's row of a [chunks][E] table;
//   2. scan: one workgroup turns the table into counts, offsets (exclusive scan over
//      experts) and each chunk's starting row per expert (scan over chunks);
//   3. scatter: one wave per chunk walks its tokens 64 at a time (lane = token); each lane
//      sets its bit in a 64-bit LDS mask per expert it picked, and the rank of a slot
//      among earlier tokens of the same expert is a popcount of the lower bits.
#include "common.h"
#include "internal.h"

namespace moe {

namespace {

constexpr int kChunk = 256;   // tokens per histogram / scatter workgroup

__global__ __launch_bounds__(256) void hist_kernel(int T, int E, int k,
                                                   const int32_t* __restrict__ idx,
                                                   int32_t* __restrict__ chunk_hist) {
  __shared__ int h[64];
  if (threadIdx.x < 64) h[threadIdx.x] = 0;
  __syncthreads();
  const int t = blockIdx.x * kChunk + threadIdx.x;
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[(size_t)t * k + j];
      if ((unsigned)e < (unsigned)E) atomicAdd(&h[e], 1);   // out-of-range ids are skipped
    }
  }
  __syncthreads();
  if (threadIdx.x < E) chunk_hist[(size_t)blockIdx.x * E + threadIdx.x] = h[threadIdx.x];
}

__global__ __launch_bounds__(64) void scan_kernel(int nchunks, int E,
                                                  const int32_t* __restrict__ chunk_hist,
                                                  int32_t* __restrict__ chunk_base,
                                                  int32_t* __restrict__ counts,
                                                  int32_t* __restrict__ offsets) {
  const int e = threadIdx.x;
  int total = 0;
  if (e < E) {
    for (int c = 0; c < nchunks; ++c) total += chunk_hist[(size_t)c * E + e];
  }
  // exclusive scan over experts (wave-wide inclusive scan, then shift)
  int incl = total;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int v = __shfl_up(incl, o, 64);
    if (e >= o) incl += v;
  }
  const int excl = incl - total;
  if (e < E) {
    counts[e] = total;
    offsets[e] = excl;
    int run = excl;
    for (int c = 0; c < nchunks; ++c) {
      chunk_base[(size_t)c * E + e] = run;
      run += chunk_hist[(size_t)c * E + e];
    }
  }
  if (e == E - 1) offsets[E] = incl;
}

__global__ __launch_bounds__(64) void scatter_kernel(int T, int E, int k,
                                                     const int32_t* __restrict__ idx,
                                                     const float* __restrict__ topk_w,
                                                     const int32_t* __restrict__ chunk_base,
                                                     int32_t* __restrict__ perm_token,
                                                     int32_t* __restrict__ slot_pos,
                                                     float* __restrict__ perm_weight) {
  __shared__ int run[64];
  __shared__ unsigned long long mask[64];
  const int lane = threadIdx.x;
  if (lane < E) run[lane] = chunk_base[(size_t)blockIdx.x * E + lane];
  const int tbeg = blockIdx.x * kChunk;
  const int tend = min(T, tbeg + kChunk);
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int t0 = tbeg; t0 < tend; t0 += 64) {
    mask[lane] = 0ull;
    __syncthreads();
    const int t = t0 + lane;
    const bool ok = t < tend;
    if (ok) {
      for (int j = 0; j < k; ++j) {
        const int e = idx[(size_t)t * k + j];
        if ((unsigned)e < (unsigned)E) atomicOr(&mask[e], 1ull << lane);
      }
    }
    __syncthreads();
    if (ok) {
      for (int j = 0; j < k; ++j) {
        const int e = idx[(size_t)t * k + j];
        if ((unsigned)e >= (unsigned)E) continue;
        const int pos = run[e] + __popcll(mask[e] & below);
        perm_token[pos] = t;
        slot_pos[(size_t)t * k + j] = pos;
        if (perm_weight != nullptr) perm_weight[pos] = topk_w[(size_t)t * k + j];
      }
    }
    __syncthreads();
    if (lane < E) run[lane] += __popcll(mask[lane]);
    __syncthreads();
  }
}

}  // namespace

size_t permute_ws_bytes(int T, int E) {
  const size_t nchunks = (size_t)(T + kChunk - 1) / kChunk;
  return 2 * nchunks * (size_t)E * sizeof(int32_t);
}

hipError_t launch_permute(int T, int E, int k, const int32_t* idx, const float* topk_w,
                          int32_t* counts, int32_t* offsets, int32_t* perm_token,
                          int32_t* slot_pos, float* perm_weight, void* ws, hipStream_t s) {
  const int nchunks = (T + kChunk - 1) / kChunk;
  int32_t* chunk_hist = static_cast<int32_t*>(ws);
  int32_t* chunk_base = chunk_hist + (size_t)nchunks * E;
  if (nchunks > 0) {
    hipLaunchKernelGGL(hist_kernel, dim3(nchunks), dim3(256), 0, s, T, E, k, idx, chunk_hist);
  }
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(64), 0, s, nchunks, E, chunk_hist, chunk_base,
                     counts, offsets);
  if (nchunks > 0) {
    hipLaunchKernelGGL(scatter_kernel, dim3(nchunks), dim3(64), 0, s, T, E, k, idx, topk_w,
                       chunk_base, perm_token, slot_pos, perm_weight);
  }
  return hipGetLastError();
}

}  // namespace moe
