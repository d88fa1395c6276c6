// Load statistics of one batch and the Switch auxiliary-loss value.
//
// f_e is the fraction of the T*k routed (token, slot) assignments that went to expert e,
// p_e the mean over tokens of expert e's routing probability (its score divided by the
// token's sum over all experts), and the loss alpha * E * sum_e f_e p_e ("大模型工程（一）：
// Transformer 到 MoE", section "负载均衡"; minimal at f_e = p_e = 1/E, section "MoE 数学：
// 路由、容量与平衡详解").
//
// Two launches: workgroups of 4 waves each take 64 tokens (lane = expert; a wave adds its
// tokens' normalised scores in token order, the 4 waves are added in wave order, slot
// counts are integer LDS atomics), then one wave adds the chunk partials in chunk order.
// Every sum has a fixed order, so the result is the same on every run.
#include "common.h"
#include "internal.h"

namespace moe {

namespace {

constexpr int kStatsChunk = 64;   // tokens per partial workgroup

__global__ __launch_bounds__(256) void stats_partial_kernel(int T, int E, int k,
                                                            const float* __restrict__ scores,
                                                            const int32_t* __restrict__ idx,
                                                            float* __restrict__ part_p,
                                                            int32_t* __restrict__ part_c) {
  __shared__ float wsum[4][64];
  __shared__ int cnt[64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  if (threadIdx.x < 64) cnt[threadIdx.x] = 0;
  __syncthreads();
  const bool valid = lane < E;
  const int t0 = blockIdx.x * kStatsChunk;
  float acc = 0.0f;
  for (int i = wave; i < kStatsChunk; i += 4) {
    const int t = t0 + i;
    if (t >= T) break;                          // uniform per wave
    const float s = valid ? scores[(size_t)t * E + lane] : 0.0f;
    const float rs = wave_sum_f(s);
    acc += rs > 0.0f ? s / rs : 0.0f;
    if (lane < k) {
      const int e = idx[(size_t)t * k + lane];
      if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);
    }
  }
  wsum[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    part_p[(size_t)blockIdx.x * 64 + lane] = ((wsum[0][lane] + wsum[1][lane]) + wsum[2][lane]) + wsum[3][lane];
    part_c[(size_t)blockIdx.x * 64 + lane] = cnt[lane];
  }
}

__global__ __launch_bounds__(64) void stats_final_kernel(int T, int E, int k, int nchunks,
                                                         float alpha,
                                                         const float* __restrict__ part_p,
                                                         const int32_t* __restrict__ part_c,
                                                         float* f, float* p, float* loss) {
  const int lane = threadIdx.x;
  const bool valid = lane < E;
  float ps = 0.0f;
  long long c = 0;
  for (int b = 0; b < nchunks; ++b) {
    ps += part_p[(size_t)b * 64 + lane];
    c += part_c[(size_t)b * 64 + lane];
  }
  const float fe = valid ? (float)((double)c / ((double)T * (double)k)) : 0.0f;
  const float pe = valid ? ps / (float)T : 0.0f;
  const float sfp = wave_sum_f(fe * pe);
  if (valid) {
    f[lane] = fe;
    p[lane] = pe;
  }
  if (lane == 0) loss[0] = alpha * (float)E * sfp;
}

}  // namespace

size_t stats_ws_bytes(int T, int E) {
  (void)E;
  const size_t nchunks = ((size_t)T + kStatsChunk - 1) / kStatsChunk;
  return nchunks * 64 * (sizeof(float) + sizeof(int32_t));
}

hipError_t launch_load_stats(int T, int E, int k, const float* scores, const int32_t* idx,
                             float alpha, float* f, float* p, float* loss, void* ws,
                             hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int nchunks = (T + kStatsChunk - 1) / kStatsChunk;
  float* part_p = static_cast<float*>(ws);
  int32_t* part_c = reinterpret_cast<int32_t*>(part_p + (size_t)nchunks * 64);
  hipLaunchKernelGGL(stats_partial_kernel, dim3(nchunks), dim3(256), 0, s, T, E, k, scores, idx,
                     part_p, part_c);
  hipLaunchKernelGGL(stats_final_kernel, dim3(1), dim3(64), 0, s, T, E, k, nchunks, alpha,
                     part_p, part_c, f, p, loss);
  return hipGetLastError();
}

}  // namespace moe
