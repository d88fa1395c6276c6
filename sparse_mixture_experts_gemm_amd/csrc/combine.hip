// Weighted scatter-combine back to token order.
//
// out[t] = sum_j y[slot_pos[t*k+j]] + y_shared[t] (+ x[t]): the merge of the selected
// experts' outputs ("大模型工程（一）：Transformer 到 MoE", MoEBlock listing; "开源混合架构大模型技术解析",
// "四、工作原理") plus the always-on shared experts and, for a pre-norm layer, the residual
// input (the decoder-layer sketch of "变了什么，为什么变").  The routing weight is already in
// y (applied by the down-projection epilogue).  The k gathers happen in slot order, then the
// shared row, then the residual, in fp32, so the result is the same on every run.
//
// One workgroup per token row; each thread moves 16 bytes (8 bf16 or 4 fp32) per row read.
#include "common.h"
#include "internal.h"

namespace moe {

namespace {

__device__ __forceinline__ void add_bf16x8(float (&acc)[8], const uint16_t* src) {
  const uint4 v = *reinterpret_cast<const uint4*>(src);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[2 * i] += bf16_bits_to_f32(w[i] & 0xffffu);
    acc[2 * i + 1] += bf16_bits_to_f32(w[i] >> 16);
  }
}

__global__ __launch_bounds__(256) void combine_bf16_kernel(int d, int k,
                                                           const uint16_t* __restrict__ y,
                                                           const int32_t* __restrict__ slot_pos,
                                                           const uint16_t* __restrict__ ysh,
                                                           const uint16_t* __restrict__ res,
                                                           uint16_t* __restrict__ out) {
  const int t = blockIdx.x;
  for (int c = threadIdx.x * 8; c < d; c += blockDim.x * 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const int p = slot_pos[(size_t)t * k + j];
      if (p < 0) continue;   // dropped by the expert capacity
      add_bf16x8(acc, y + (size_t)p * d + c);
    }
    if (ysh != nullptr) add_bf16x8(acc, ysh + (size_t)t * d + c);
    if (res != nullptr) add_bf16x8(acc, res + (size_t)t * d + c);
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    *reinterpret_cast<uint4*>(out + (size_t)t * d + c) = o;
  }
}

__global__ __launch_bounds__(256) void combine_f32_kernel(int d, int k, const float* __restrict__ y,
                                                          const int32_t* __restrict__ slot_pos,
                                                          const float* __restrict__ ysh,
                                                          const float* __restrict__ res,
                                                          float* __restrict__ out) {
  const int t = blockIdx.x;
  for (int c = threadIdx.x * 4; c < d; c += blockDim.x * 4) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
      const int p = slot_pos[(size_t)t * k + j];
      if (p < 0) continue;   // dropped by the expert capacity
      const float4 v = *reinterpret_cast<const float4*>(y + (size_t)p * d + c);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    if (ysh != nullptr) {
      const float4 v = *reinterpret_cast<const float4*>(ysh + (size_t)t * d + c);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    if (res != nullptr) {
      const float4 v = *reinterpret_cast<const float4*>(res + (size_t)t * d + c);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    *reinterpret_cast<float4*>(out + (size_t)t * d + c) = acc;
  }
}

}  // namespace

hipError_t launch_combine(int T, int d, int k, int act_dtype, const void* y_perm,
                          const int32_t* slot_pos, const void* y_shared, const void* residual,
                          void* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (act_dtype == MOE_BF16) {
    hipLaunchKernelGGL(combine_bf16_kernel, dim3(T), dim3(256), 0, s, d, k,
                       static_cast<const uint16_t*>(y_perm), slot_pos,
                       static_cast<const uint16_t*>(y_shared),
                       static_cast<const uint16_t*>(residual), static_cast<uint16_t*>(out));
  } else {
    hipLaunchKernelGGL(combine_f32_kernel, dim3(T), dim3(256), 0, s, d, k,
                       static_cast<const float*>(y_perm), slot_pos,
                       static_cast<const float*>(y_shared), static_cast<const float*>(residual),
                       static_cast<float*>(out));
  }
  return hipGetLastError();
}

}  // namespace moe
