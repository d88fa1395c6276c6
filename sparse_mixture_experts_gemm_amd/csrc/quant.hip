// Per-row e4m3 quantisation of bf16 activations for the e4m3 x e4m3 up projections.
//
// FP8 E4M3 products with FP32 accumulation ("大模型工程（一）：Transformer 到 MoE", section
// "生产现实：前沿实验室真正交付的内容", FP8 item); each token row gets its own scale:
//   scale = max|a_row| / 448            (fp32 division)
//   q     = e4m3(clamp(a / scale, +-448))  (fp32 division, round to nearest even)
// A row of zeros has scale 0 and codes 0.  One wave per row; every lane converts 8
// consecutive values per step (16-byte loads, 8-byte stores).
#include "common.h"
#include "internal.h"

namespace moe {

namespace {

// |v| <= 448 to the nearest e4m3 code (ties to even), with the sign of v.
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  const float a = fabsf(v);
  uint32_t code;
  if (a < 0.015625f) {                               // below 2^-6: multiples of 2^-9
    code = (uint32_t)rintf(a * 512.0f);              // exact scaling; 8 is the smallest normal
  } else {
    const uint32_t bits = __float_as_uint(a);
    int ex = (int)(bits >> 23) - 127;
    uint32_t keep = (bits >> 20) & 7u;
    const uint32_t rem = bits & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) ++keep;
    if (keep == 8u) {
      keep = 0u;
      ++ex;
    }
    code = ((uint32_t)(ex + 7) << 3) | keep;
  }
  return (code != 0u && v < 0.0f) ? (code | 0x80u) : code;
}

__global__ __launch_bounds__(256) void quant_rows_kernel(int rows, int cols,
                                                         const uint16_t* __restrict__ a,
                                                         uint8_t* __restrict__ q,
                                                         float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;                           // whole wave
  const uint16_t* src = a + (size_t)row * cols;
  float amax = 0.0f;
  for (int c = lane * 8; c < cols; c += 512) {
    const uint4 v = *reinterpret_cast<const uint4*>(src + c);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      amax = fmaxf(amax, fabsf(bf16_bits_to_f32(w[i] & 0xffffu)));
      amax = fmaxf(amax, fabsf(bf16_bits_to_f32(w[i] >> 16)));
    }
  }
  amax = wave_max_f(amax);
  const float sc = amax / 448.0f;
  if (lane == 0) scale[row] = sc;
  uint8_t* dst = q + (size_t)row * cols;
  for (int c = lane * 8; c < cols; c += 512) {
    uint2 out = make_uint2(0u, 0u);
    if (sc > 0.0f) {
      const uint4 v = *reinterpret_cast<const uint4*>(src + c);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      uint32_t b[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float lo = fminf(fmaxf(bf16_bits_to_f32(w[i] & 0xffffu) / sc, -448.0f), 448.0f);
        const float hi = fminf(fmaxf(bf16_bits_to_f32(w[i] >> 16) / sc, -448.0f), 448.0f);
        b[2 * i] = e4m3_rne(lo);
        b[2 * i + 1] = e4m3_rne(hi);
      }
      out.x = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
      out.y = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
    }
    *reinterpret_cast<uint2*>(dst + c) = out;
  }
}

}  // namespace

hipError_t launch_quant_rows(int rows, int cols, const void* a, uint8_t* q, float* scale,
                             hipStream_t s) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_rows_kernel, dim3((rows + 3) / 4), dim3(256), 0, s, rows, cols,
                     static_cast<const uint16_t*>(a), q, scale);
  return hipGetLastError();
}

}  // namespace moe
