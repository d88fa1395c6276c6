// Tile-walk, LDS-layout and memory helpers shared by the grouped-GEMM kernels (gfx950).
#pragma once
#include "common.h"
#include "internal.h"

namespace moe {

namespace {

constexpr int kGroupM = 8;   // m-tiles walked together per n-tile inside a large segment

// Builds, in LDS, the first tile index of every segment and its row range.  Run by
// wave 0; nseg <= 64.
__device__ void build_schedule(const GemmParams& p, int BM, int NT, int* s_tile0, int* s_row0,
                               int* s_rows) {
  const int lane = threadIdx.x;
  if (lane < 64) {
    int row0 = 0, rows = 0, tiles = 0;
    if (lane < p.nseg) {
      if (p.offsets != nullptr) {
        row0 = p.offsets[lane];
        rows = p.offsets[lane + 1] - row0;
      } else {
        row0 = 0;
        rows = p.rows;
      }
      tiles = ((rows + BM - 1) / BM) * NT;
    }
    int incl = tiles;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    if (lane < p.nseg) {
      s_tile0[lane + 1] = incl;
      s_row0[lane] = row0;
      s_rows[lane] = rows;
    }
    if (lane == 0) s_tile0[0] = 0;
  }
}

struct TileCoord {
  int seg, m_tile, n_tile, row0, rows;
};

__device__ __forceinline__ TileCoord decode_tile(int L, int nseg, int BM, int NT,
                                                 const int* s_tile0, const int* s_row0,
                                                 const int* s_rows) {
  int lo = 0, hi = nseg - 1;  // last segment with s_tile0[seg] <= L
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (s_tile0[mid] <= L) lo = mid; else hi = mid - 1;
  }
  TileCoord c;
  c.seg = lo;
  c.row0 = s_row0[lo];
  c.rows = s_rows[lo];
  const int u = L - s_tile0[lo];
  const int mt = (c.rows + BM - 1) / BM;
  const int grp = u / (kGroupM * NT);
  const int first_m = grp * kGroupM;
  const int gm = min(kGroupM, mt - first_m);
  const int r = u - grp * kGroupM * NT;
  c.m_tile = first_m + r % gm;
  c.n_tile = r / gm;
  return c;
}

// LDS swizzles and the weight-row staging order of a 32-row MFMA block (see gemm.hip).
__device__ __forceinline__ int swz8(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz4(int r) { return (r >> 1) & 3; }
__device__ __forceinline__ int perm32(int r) { return ((r >> 2) & 1) * 16 + (r >> 3) * 4 + (r & 3); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 encoding: vmcnt[3:0] | expcnt[6:4] = 7 | lgkmcnt[11:8] = 15 | vmcnt[5:4] << 14
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8 widen_e4m3x8(uint2 q) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.x, 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.x, 1.0f, true);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.y, 1.0f, false);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.y, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// 16 consecutive fp32 values (scaled by the per-feature factors when given) -> 16 bf16 at
// dst (32-byte aligned), as two 16-byte stores.
__device__ __forceinline__ void store16_bf16(void* dst, const float (&v)[16]) {
  uint4 lo, hi;
  lo.x = pack_bf16x2(v[0], v[1]);   lo.y = pack_bf16x2(v[2], v[3]);
  lo.z = pack_bf16x2(v[4], v[5]);   lo.w = pack_bf16x2(v[6], v[7]);
  hi.x = pack_bf16x2(v[8], v[9]);   hi.y = pack_bf16x2(v[10], v[11]);
  hi.z = pack_bf16x2(v[12], v[13]); hi.w = pack_bf16x2(v[14], v[15]);
  uint4* d = static_cast<uint4*>(dst);
  d[0] = lo;
  d[1] = hi;
}

__device__ __forceinline__ void load16_f32(const float* src, float (&v)[16]) {
  const float4* s4 = reinterpret_cast<const float4*>(src);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 t = s4[q];
    v[4 * q] = t.x; v[4 * q + 1] = t.y; v[4 * q + 2] = t.z; v[4 * q + 3] = t.w;
  }
}

}  // namespace

}  // namespace moe
