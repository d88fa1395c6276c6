// Single-workgroup permutation of (token, slot) pairs whose expert ids are already in LDS,
// used by the small-batch permutation of permute.hip.  Order: expert ascending, then token
// ascending.
#pragma once
#include "common.h"

namespace moe {

// LDS of a workgroup of W waves (W * 64 threads)
template <int W>
struct PermuteLds {
  int hist[W][64];
  int run[W][64];                // rank inside its expert of the wave's next slot
  int koff[64];                  // first permuted row of each expert
  unsigned long long mask[W][64];
};

__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

// sidx: [T * k] expert ids in LDS; wsrc: [T * k] routing weights (LDS or global) or null.
// Each expert keeps its first `capacity` slots (token order); the others get slot_pos -1.
// Every thread of the workgroup (W waves) must call it.  k <= 8, E <= 64.
template <int W>
__device__ __forceinline__ void permute_lds(int T, int E, int k, int capacity, const int* sidx,
                                            const float* wsrc, PermuteLds<W>& pl,
                                            int32_t* __restrict__ counts,
                                            int32_t* __restrict__ offsets,
                                            int32_t* __restrict__ perm_token,
                                            int32_t* __restrict__ slot_pos,
                                            float* __restrict__ perm_weight) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // tokens per wave: a multiple of 64 so that every scatter step is a full wave of tokens
  const int per = (((T + W - 1) / W) + 63) & ~63;
  const int tbeg = min(T, wave * per);
  const int tend = min(T, tbeg + per);

  pl.hist[wave][lane] = 0;
  wave_lds_sync();
  for (int i = tbeg * k + lane; i < tend * k; i += 64) {
    const int e = sidx[i];
    if ((unsigned)e < (unsigned)E) atomicAdd(&pl.hist[wave][e], 1);   // out-of-range ids are skipped
  }
  __syncthreads();
  if (wave == 0) {
    const int e = lane;
    int total = 0;
    for (int w = 0; w < W; ++w) total += (e < E) ? pl.hist[w][e] : 0;
    const int kept = min(total, capacity);
    int incl = kept;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int v = __shfl_up(incl, o, 64);
      if (e >= o) incl += v;
    }
    if (e < E) {
      counts[e] = kept;
      offsets[e] = incl - kept;
      pl.koff[e] = incl - kept;
      int rank = 0;
      for (int w = 0; w < W; ++w) {
        pl.run[w][e] = rank;
        rank += pl.hist[w][e];
      }
    }
    if (e == E - 1) offsets[E] = incl;
  }
  __syncthreads();

  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int t0 = tbeg; t0 < tend; t0 += 64) {
    const int t = t0 + lane;
    const bool ok = t < tend;
    float wv[8];
    if (perm_weight != nullptr && ok) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < k) wv[j] = wsrc[(size_t)t * k + j];
    }
    pl.mask[wave][lane] = 0ull;
    wave_lds_sync();
    if (ok) {
      for (int j = 0; j < k; ++j) {
        const int e = sidx[t * k + j];
        if ((unsigned)e < (unsigned)E) atomicOr(&pl.mask[wave][e], 1ull << lane);
      }
    }
    wave_lds_sync();
    if (ok) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j >= k) break;
        const int e = sidx[t * k + j];
        if ((unsigned)e >= (unsigned)E) {   // skipped id: no row, like a dropped slot
          slot_pos[(size_t)t * k + j] = -1;
          continue;
        }
        const int rank = pl.run[wave][e] + __popcll(pl.mask[wave][e] & below);
        if (rank < capacity) {
          const int pos = pl.koff[e] + rank;
          perm_token[pos] = t;
          slot_pos[(size_t)t * k + j] = pos;
          if (perm_weight != nullptr) perm_weight[pos] = wv[j];
        } else {
          slot_pos[(size_t)t * k + j] = -1;
        }
      }
    }
    wave_lds_sync();
    if (lane < E) pl.run[wave][lane] += __popcll(pl.mask[wave][lane]);
    wave_lds_sync();
  }
}

}  // namespace moe
