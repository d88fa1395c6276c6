// Expert-sorted permutation of the (token, slot) pairs.
//
// Tokens are routed to experts and batched per expert before the expert FFNs run
// ("大模型工程（一）：Transformer 到 MoE", sections "MoE 数学：路由、容量与平衡详解" and the
// expert-parallel paragraph; "开源混合架构大模型技术解析", "批处理策略").  The order is
// fixed: expert ascending, then token ascending, so the result does not depend on
// scheduling.  Two launches:
//   1. histogram: one workgroup per chunk of tokens (at most 64 chunks) counts its slots per expert
//      in LDS and writes the chunk's row of a [chunks][E] table;
//   2. scatter: one wave per chunk first reads the whole table (lane = expert): the column
//      sums are the counts, their exclusive scan the offsets, and the sum over earlier
//      chunks the chunk's starting row per expert.  It then walks its tokens 64 at a time
//      (lane = token); each lane sets its bit in a 64-bit LDS mask per expert it picked, and
//      the rank of a slot among earlier tokens of the same expert is a popcount of the
//      lower bits.  Chunk 0 also writes counts and offsets.
// With an expert capacity ("MoE 数学：路由、容量与平衡详解" of "大模型工程（一）": tokens beyond an
// expert's capacity are dropped), a slot whose rank inside its expert reaches the
// capacity gets slot_pos -1 and no row; counts and offsets count the kept rows.
// Up to kFusedMaxTokens tokens (and kFusedMaxSlots pairs), one workgroup of 16 waves (of 4
// waves up to kSmallSlots pairs) does both steps in a single launch from an LDS copy of
// topk_idx (each wave owns a contiguous run of tokens; the scan runs between two barriers).
#include "common.h"
#include "internal.h"
#include "permute_core.h"

namespace moe {

namespace {

// Tokens per histogram / scatter workgroup: a multiple of 64 chosen so that there are at
// most 64 chunks (the scatter reads one column of the chunk table per lane).
constexpr int kMaxChunks = 64;
inline int chunk_tokens(int T) {
  const int per = (T + kMaxChunks - 1) / kMaxChunks;
  return per <= 64 ? 64 : (per + 63) & ~63;
}

__global__ __launch_bounds__(256) void hist_kernel(int T, int E, int k, int chunk,
                                                   const int32_t* __restrict__ idx,
                                                   int32_t* __restrict__ chunk_hist) {
  __shared__ int h[64];
  if (threadIdx.x < 64) h[threadIdx.x] = 0;
  __syncthreads();
  const int cbeg = blockIdx.x * chunk;
  const int cend = min(T, cbeg + chunk);
  for (int i = cbeg * k + threadIdx.x; i < cend * k; i += 256) {
    const int e = idx[i];
    if ((unsigned)e < (unsigned)E) atomicAdd(&h[e], 1);   // out-of-range ids are skipped
  }
  __syncthreads();
  if ((int)threadIdx.x < E) chunk_hist[(size_t)blockIdx.x * E + threadIdx.x] = h[threadIdx.x];
}

__global__ __launch_bounds__(64) void scatter_kernel(int T, int E, int k, int capacity,
                                                     int nchunks, int chunk,
                                                     const int32_t* __restrict__ idx,
                                                     const float* __restrict__ topk_w,
                                                     const int32_t* __restrict__ chunk_hist,
                                                     int32_t* __restrict__ counts,
                                                     int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ perm_token,
                                                     int32_t* __restrict__ slot_pos,
                                                     float* __restrict__ perm_weight) {
  __shared__ int run[64];        // rank inside its expert of the chunk's next slot
  __shared__ int koff[64];       // first permuted row of each expert
  __shared__ unsigned long long mask[64];
  const int lane = threadIdx.x;
  {
    // column sums (slots per expert), the kept rows min(sum, capacity), their exclusive
    // scan (offsets) and the number of this expert's slots in earlier chunks
    int total = 0, before = 0;
    if (lane < E) {
#pragma unroll 8
      for (int c = 0; c < nchunks; ++c) {
        const int v = chunk_hist[(size_t)c * E + lane];
        total += v;
        before += c < (int)blockIdx.x ? v : 0;
      }
    }
    const int kept = min(total, capacity);
    int incl = kept;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    if (lane < E) {
      run[lane] = before;
      koff[lane] = incl - kept;
    }
    if (blockIdx.x == 0) {
      if (lane < E) {
        counts[lane] = kept;
        offsets[lane] = incl - kept;
      }
      if (lane == E - 1) offsets[E] = incl;
    }
  }
  const int tbeg = blockIdx.x * chunk;
  const int tend = min(T, tbeg + chunk);
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
        if ((unsigned)e >= (unsigned)E) {   // skipped id: no row, like a dropped slot
          slot_pos[(size_t)t * k + j] = -1;
          continue;
        }
        const int rank = run[e] + __popcll(mask[e] & below);
        if (rank < capacity) {
          const int pos = koff[e] + rank;
          perm_token[pos] = t;
          slot_pos[(size_t)t * k + j] = pos;
          if (perm_weight != nullptr) perm_weight[pos] = topk_w[(size_t)t * k + j];
        } else {
          slot_pos[(size_t)t * k + j] = -1;
        }
      }
    }
    __syncthreads();
    if (lane < E) run[lane] += __popcll(mask[lane]);
    __syncthreads();
  }
}

constexpr int kFusedMaxTokens = 1024;   // above this, one workgroup is slower than two launches
constexpr int kFusedMaxSlots = 28672;   // T * k staged in LDS (112 KB)
// Small batches (T * k <= kSmallSlots): a workgroup of 4 waves and 8 KB of staged ids.  It
// fits a CU beside the shared experts' GEMM that runs on the second stream meanwhile; the
// 16-wave, 112 KB workgroup has to wait until one of that GEMM's workgroups leaves a CU.
constexpr int kSmallSlots = 2048;

// One workgroup of W waves.  The whole topk_idx array is first copied into LDS with every
// load in flight at once; histogram, scan and scatter then read it from LDS.  Each wave
// owns a contiguous run of tokens.
template <int W, int MAXSLOTS>
__global__ __launch_bounds__(W * 64) void permute_fused_kernel(int T, int E, int k, int capacity,
                                                               const int32_t* __restrict__ idx,
                                                               const float* __restrict__ topk_w,
                                                               int32_t* __restrict__ counts,
                                                               int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ perm_token,
                                                               int32_t* __restrict__ slot_pos,
                                                               float* __restrict__ perm_weight) {
  __shared__ __align__(16) int sidx[MAXSLOTS];
  __shared__ PermuteLds<W> pl;
  const int nslot = T * k;
  // stage topk_idx (16-byte loads where the array allows, then the tail)
  const int n4 = ((reinterpret_cast<uintptr_t>(idx) & 15) == 0) ? nslot / 4 : 0;
  for (int i = threadIdx.x; i < n4; i += W * 64)
    reinterpret_cast<int4*>(sidx)[i] = reinterpret_cast<const int4*>(idx)[i];
  for (int i = 4 * n4 + threadIdx.x; i < nslot; i += W * 64) sidx[i] = idx[i];
  __syncthreads();
  permute_lds<W>(T, E, k, capacity, sidx, topk_w, pl, counts, offsets, perm_token, slot_pos,
                 perm_weight);
}

}  // namespace

size_t permute_ws_bytes(int T, int E) {
  const size_t chunk = (size_t)chunk_tokens(T);
  const size_t nchunks = ((size_t)T + chunk - 1) / chunk;
  return nchunks * (size_t)E * sizeof(int32_t);
}

hipError_t launch_permute(int T, int E, int k, int capacity, const int32_t* idx,
                          const float* topk_w, int32_t* counts, int32_t* offsets,
                          int32_t* perm_token, int32_t* slot_pos, float* perm_weight, void* ws,
                          hipStream_t s) {
  if ((long long)T * k <= kSmallSlots && k <= 8) {
    hipLaunchKernelGGL((permute_fused_kernel<4, kSmallSlots>), dim3(1), dim3(256), 0, s, T, E, k,
                       capacity, idx, topk_w, counts, offsets, perm_token, slot_pos,
                       perm_weight);
    return hipGetLastError();
  }
  if (T <= kFusedMaxTokens && (long long)T * k <= kFusedMaxSlots && k <= 8) {
    hipLaunchKernelGGL((permute_fused_kernel<16, kFusedMaxSlots>), dim3(1), dim3(1024), 0, s, T,
                       E, k, capacity, idx, topk_w, counts, offsets, perm_token, slot_pos,
                       perm_weight);
    return hipGetLastError();
  }
  const int chunk = chunk_tokens(T);
  const int nchunks = (T + chunk - 1) / chunk;
  int32_t* chunk_hist = static_cast<int32_t*>(ws);
  hipLaunchKernelGGL(hist_kernel, dim3(nchunks), dim3(256), 0, s, T, E, k, chunk, idx, chunk_hist);
  hipLaunchKernelGGL(scatter_kernel, dim3(nchunks), dim3(64), 0, s, T, E, k, capacity, nchunks,
                     chunk, idx, topk_w, chunk_hist, counts, offsets, perm_token, slot_pos,
                     perm_weight);
  return hipGetLastError();
}

}  // namespace moe
