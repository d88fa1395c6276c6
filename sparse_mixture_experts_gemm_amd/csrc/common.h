// Device-side helpers shared by the libmoe kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// fp32 -> bf16 bits, round to nearest even (NaN -> canonical quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Four e4m3 codes (one per byte) -> four bf16 values packed in two uint32.
// e4m3 (bias 7) placed in the fp32 exponent/mantissa fields and multiplied by 2^120
// gives the exact value for normals and subnormals alike; three mantissa bits fit
// bf16 exactly, so the truncation to the upper half is exact.  NaN codes are not
// produced by the quantiser and are not special-cased.
__device__ __forceinline__ void e4m3x4_to_bf16x4(uint32_t q, uint32_t& lo, uint32_t& hi) {
  const float two120 = 1.329227995784916e36f;  // 2^120
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t c = (q >> (8 * i)) & 0xffu;
    float mag = __uint_as_float((c & 0x7fu) << 20) * two120;
    v[i] = __uint_as_float(__float_as_uint(mag) | ((c & 0x80u) << 24));
  }
  lo = (__float_as_uint(v[0]) >> 16) | (__float_as_uint(v[1]) & 0xffff0000u);
  hi = (__float_as_uint(v[2]) >> 16) | (__float_as_uint(v[3]) & 0xffff0000u);
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + expf(-z)); }

template <typename T>
__device__ __forceinline__ T wave_shfl(T v, int src) {
  return __shfl(v, src, kWave);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    uint64_t w = __shfl_xor(v, o, kWave);
    v = w > v ? w : v;
  }
  return v;
}

__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Butterfly sum: the same association on every call, so results are reproducible.
__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// DPP reductions (gfx9 encodings): quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E,
// row_half_mirror = 0x141, row_mirror = 0x140, row_bcast:15 = 0x142, row_bcast:31 = 0x143.
__device__ __forceinline__ uint32_t dpp_max_step(uint32_t x, int ctrl_sel) {
  int y;
  switch (ctrl_sel) {
    case 0: y = __builtin_amdgcn_update_dpp((int)x, (int)x, 0xB1, 0xF, 0xF, false); break;
    case 1: y = __builtin_amdgcn_update_dpp((int)x, (int)x, 0x4E, 0xF, 0xF, false); break;
    case 2: y = __builtin_amdgcn_update_dpp((int)x, (int)x, 0x141, 0xF, 0xF, false); break;
    case 3: y = __builtin_amdgcn_update_dpp((int)x, (int)x, 0x140, 0xF, 0xF, false); break;
    case 4: y = __builtin_amdgcn_update_dpp((int)x, (int)x, 0x142, 0xA, 0xF, false); break;
    default: y = __builtin_amdgcn_update_dpp((int)x, (int)x, 0x143, 0xC, 0xF, false); break;
  }
  return x > (uint32_t)y ? x : (uint32_t)y;
}

// Max of an unsigned value over each aligned group of 8 lanes (every lane gets its group's).
__device__ __forceinline__ uint32_t group8_max_u32(uint32_t x) {
  x = dpp_max_step(x, 0);
  x = dpp_max_step(x, 1);
  return dpp_max_step(x, 2);
}

// Max of an unsigned value over the whole wave (uniform result).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
#pragma unroll
  for (int i = 0; i < 6; ++i) x = dpp_max_step(x, i);
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// 16 bytes per lane from global memory into LDS at lds_base + 16 * lane (the LDS base is
// taken from M0; no VGPR is written).  The caller waits with vmcnt before reading the LDS.
// An LDS-DMA load that reads M0 needs one wait state after the scalar write of M0 (a gfx9
// hazard that the compiler cannot see inside inline assembly): the s_nop provides it.  M0
// is restored afterwards.
__device__ __forceinline__ void lds_dma16(uint32_t lds_base, const void* src) {
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "s"(lds_base), "v"(src)
      : "memory");
}

// As lds_dma16, reading from base + off: `base` is the same for every lane of the wave (it
// is passed in scalar registers), `off` is this lane's byte offset (below 4 GB).
__device__ __forceinline__ void lds_dma16_off(uint32_t lds_base, const void* base, uint32_t off) {
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "s"(lds_base), "v"(off), "s"(base)
      : "memory");
}

// A pointer that the caller knows to be the same in every lane, made visibly uniform (the
// first lane's value) so that it can live in scalar registers.
__device__ __forceinline__ const unsigned char* uniform_ptr(const void* p) {
  const unsigned long long v = reinterpret_cast<unsigned long long>(p);
  const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)v);
  const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)(v >> 32));
  return reinterpret_cast<const unsigned char*>(((unsigned long long)hi << 32) | lo);
}

// Logical workgroup -> XCD-contiguous order.  Workgroups are dispatched round-robin over
// the 8 XCDs (workgroup b runs on XCD b % 8), so map workgroup b to a slot such that each
// XCD walks a contiguous range of logical tiles and its L2 sees their shared operands.
constexpr int kNumXcd = 8;

}  // namespace moe
