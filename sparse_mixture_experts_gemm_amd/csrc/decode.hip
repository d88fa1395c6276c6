// Expert FFN stages for few rows per expert (decode-shaped batches).
//
// With a handful of tokens per expert the layer is bound by reading the weights of every
// touched expert once from HBM: at decode time the weights are streamed once per step
// ("大模型工程（一）：Transformer 到 MoE", worked example "实战示例", the decode bound of
// bytes / bandwidth).  These kernels are built for that bound: every workgroup owns one
// (expert, column slice) pair, each wave streams its 16 weight rows straight from HBM into
// registers (64 bytes per lane per 128-wide K step, double-buffered, no LDS), and the few
// activation rows are read from L2 as MFMA operands (v_mfma_f32_16x16x32_bf16, 16 rows per
// row chunk, up to four chunks per pass).  Experts with no rows exit before touching their
// weights, so untouched experts cost nothing.
//
// K order: in step q, MFMA s takes K elements [128 q + 32 s, +32); lane (column n, group g)
// supplies elements 128 q + 32 s + 8 g .. + 8 of its row, so each of the four 16-byte loads
// of a step reads 64 contiguous bytes per row across the four lanes of that row.  The
// activation operand uses the same order.
#include "common.h"
#include "internal.h"

#include <utility>

namespace moe {

namespace {

constexpr int kRowsPerChunk = 16;
constexpr int kChunks = 4;            // rows per pass = 64
constexpr int kStepK = 128;           // K elements per step

constexpr int kLdsMaxK = 2048;        // activation rows staged in LDS up to this K

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void widen16(uint4 q, bf16x8& lo, bf16x8& hi) {
  bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.x, 1.0f, false);
  bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.x, 1.0f, true);
  bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.y, 1.0f, false);
  bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.y, 1.0f, true);
  bf16x2_t e = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.z, 1.0f, false);
  bf16x2_t f = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.z, 1.0f, true);
  bf16x2_t g = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.w, 1.0f, false);
  bf16x2_t h = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.w, 1.0f, true);
  lo = bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  hi = bf16x8{e[0], e[1], f[0], f[1], g[0], g[1], h[0], h[1]};
}

// One weight-row fragment of a 128-wide K step: for MFMA s, 8 K values of this lane's row
// at element offset 32 s (64 bytes apart for bf16, 32 bytes for e4m3).
template <bool FP8>
struct BFrag {
  uint4 raw[FP8 ? 2 : 4];
  __device__ __forceinline__ void load(const unsigned char* p, bool ok) {
    if (FP8) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint2 lo = ok ? *reinterpret_cast<const uint2*>(p + 64 * i) : make_uint2(0, 0);
        const uint2 hi = ok ? *reinterpret_cast<const uint2*>(p + 64 * i + 32) : make_uint2(0, 0);
        raw[i] = make_uint4(lo.x, lo.y, hi.x, hi.y);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        raw[i] = ok ? *reinterpret_cast<const uint4*>(p + 64 * i) : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void get(bf16x8 (&b)[4]) const {
    if (FP8) {
      widen16(raw[0], b[0], b[1]);
      widen16(raw[1], b[2], b[3]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) b[i] = __builtin_bit_cast(bf16x8, raw[i]);
    }
  }
};

// STAGE 0 (UP): a column group owns 8 output columns; its 16 weight rows are those columns
// of W_gate (n < 8) and W_up (n >= 8) for SwiGLU, or 16 columns of W_gate for ReLU^2.
// STAGE 1 (DOWN): a column group owns 16 output columns (rows of W_down).
// ksplit waves share one column group and split its K range; their partial sums meet in
// LDS and are added in wave order, so a narrow problem still has enough waves streaming.
// One launch serves two segment sets (the routed experts and the shared ones): workgroups
// [0, first.nwg) take the first set, the rest the second.
struct DecSet {
  GemmParams p;
  int nslices;   // column slices per segment
  int ksplit;    // waves per column group (1, 2 or 4)
  int nwg;       // workgroups of this set
};

constexpr int kDecWaves = 8;          // waves per workgroup

template <int STAGE, int ACT, bool FP8>
__global__ __launch_bounds__(kDecWaves * 64) void dec_gemm_kernel(DecSet first, DecSet second) {
  constexpr bool SWIGLU = (STAGE == 0) && (ACT == MOE_ACT_SWIGLU);
  constexpr int COLS_PER_WAVE = SWIGLU ? 8 : 16;
  constexpr int ESZ = FP8 ? 1 : 2;
  // One LDS buffer, used either for the activation rows of a segment with at most 16 rows
  // and K <= kLdsMaxK (16 rows x K bf16; 16-byte chunk c of row m stored at chunk
  // c ^ (m & 15) so that the 16 rows of an MFMA operand read fall in distinct banks), or,
  // with K split across waves, for their partial sums.
  __shared__ __align__(16) unsigned char a_lds[kRowsPerChunk * kLdsMaxK * 2];
  f32x4(*red)[kChunks][64] = reinterpret_cast<f32x4(*)[kChunks][64]>(a_lds);
  static_assert(sizeof(f32x4) * kDecWaves * kChunks * 64 <= sizeof(a_lds), "reduction buffer");
  const bool in_first = (int)blockIdx.x < first.nwg;
  const DecSet& ds = in_first ? first : second;
  const GemmParams& p = ds.p;
  const int bid = in_first ? (int)blockIdx.x : (int)blockIdx.x - first.nwg;
  const int nslices = ds.nslices;
  const int KSPLIT = ds.ksplit;
  const int GROUPS = kDecWaves / KSPLIT;      // column groups per workgroup
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int grp = wave / KSPLIT;
  const int kpart = wave % KSPLIT;
  const int seg = bid / nslices;
  const int slice = bid % nslices;
  int row0 = 0, nrows = p.rows;
  if (p.offsets != nullptr) {
    row0 = p.offsets[seg];
    nrows = p.offsets[seg + 1] - row0;
  }
  if (nrows <= 0) return;                     // untouched expert: no weight traffic
  const int N = p.N, K = p.K;
  const int n = lane & 15;                    // weight row of the wave's 16 / output column
  const int g = lane >> 4;                    // 32-element K group
  const int col0 = (slice * GROUPS + grp) * COLS_PER_WAVE;

  // the weight row this lane streams
  int wcol;
  const void* wb;
  if (STAGE == 0) {
    wcol = col0 + (SWIGLU ? (n & 7) : n);
    wb = (SWIGLU && n >= 8) ? p.w_up : p.w_gate;
  } else {
    wcol = col0 + n;
    wb = p.w_down;
  }
  const bool col_ok = wcol < N;
  const unsigned char* wrow = static_cast<const unsigned char*>(wb) +
                              ((size_t)seg * N * K + (size_t)(col_ok ? wcol : 0) * p.kblock) * ESZ;
  auto wptr = [&](int q) {   // step q of this lane's row (the block holding it)
    const int k = q * kStepK;
    const size_t e = (size_t)(k / p.kblock) * N * p.kblock + (k % p.kblock) + g * 8;
    return wrow + e * ESZ;
  };

  const uint16_t* a_base = static_cast<const uint16_t*>(p.a);
  const int nsteps_all = K / kStepK;
  const int q_beg = (nsteps_all * kpart) / KSPLIT;
  const int q_end = (nsteps_all * (kpart + 1)) / KSPLIT;
  const int nblk_k = K / p.kblock;

  const bool a_in_lds = nrows <= kRowsPerChunk && K <= kLdsMaxK && K % 512 == 0 && KSPLIT == 1;
  const uint32_t a_lds_base =
      (uint32_t)(size_t)(__attribute__((address_space(3))) unsigned char*)a_lds;

  for (int r0 = 0; r0 < nrows; r0 += kRowsPerChunk * kChunks) {
    const int nch = min(kChunks, (nrows - r0 + kRowsPerChunk - 1) / kRowsPerChunk);
    const uint16_t* arow[kChunks];
    bool aok[kChunks];
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int r = r0 + c * kRowsPerChunk + n;
      aok[c] = c < nch && r < nrows;
      int src = row0 + (aok[c] ? r : 0);
      if (p.row_index != nullptr) src = p.row_index[src];
      arow[c] = a_base + (size_t)src * K + g * 8;
    }
    if (a_in_lds) {
      // stage the (<= 16) rows: one 1 KB DMA per (row, 512-element block)
      const int blocks = K / 512;
      for (int i = wave; i < nrows * blocks; i += kDecWaves) {
        const int m = i / blocks, blk = i % blocks;
        int srow = row0 + m;
        if (p.row_index != nullptr) srow = p.row_index[srow];
        const uint16_t* src = a_base + (size_t)srow * K + (size_t)(blk * 64 + (lane ^ (m & 15))) * 8;
        lds_dma16((uint32_t)__builtin_amdgcn_readfirstlane((int)(a_lds_base + (uint32_t)(m * K * 2 + blk * 1024))),
                  src);
      }
    }
    f32x4 acc[kChunks], acc_tot[kChunks];
#pragma unroll
    for (int c = 0; c < kChunks; ++c) acc[c] = acc_tot[c] = f32x4{0.f, 0.f, 0.f, 0.f};

    // weights: three steps in flight per lane
    BFrag<FP8> f0, f1, f2;
    if (q_beg < q_end) f0.load(wptr(q_beg), col_ok);
    if (q_beg + 1 < q_end) f1.load(wptr(q_beg + 1), col_ok);
    if (a_in_lds) {
      // every lane's staging DMAs (and the first weight loads) have landed
      __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
      __syncthreads();
    }
    int fold_blk = q_beg * kStepK / p.kblock;   // K block the accumulator currently holds
    for (int q = q_beg; q < q_end; ++q) {
      if (q + 2 < q_end) f2.load(wptr(q + 2), col_ok);
      if (FP8 && STAGE == 1 && (q * kStepK) / p.kblock != fold_blk) {
        // a new K block starts (another shared expert): fold the finished one with its
        // per-channel scale
        const float sc = col_ok ? p.s_down[((size_t)seg * nblk_k + fold_blk) * N + wcol] : 0.f;
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
          acc_tot[c] += sc * acc[c];
          acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        fold_blk = (q * kStepK) / p.kblock;
      }
      bf16x8 b[4];
      f0.get(b);
#pragma unroll
      for (int c = 0; c < kChunks; ++c) {
        if (c < nch) {
          uint4 a[4];
          if (a_in_lds) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              const int ch = q * (kStepK / 8) + 4 * s + g;   // logical 16-byte chunk of row n
              a[s] = *reinterpret_cast<const uint4*>(a_lds + n * K * 2 + ((ch ^ n) << 4));
            }
          } else {
#pragma unroll
            for (int s = 0; s < 4; ++s)
              a[s] = aok[c] ? *reinterpret_cast<const uint4*>(arow[c] + q * kStepK + 32 * s)
                            : make_uint4(0, 0, 0, 0);
          }
#pragma unroll
          for (int s = 0; s < 4; ++s)
            acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[s]), b[s],
                                                             acc[c], 0, 0, 0);
        }
      }
      f0 = f1;
      f1 = f2;
    }
    if (FP8 && STAGE == 1) {
      const float sc = col_ok ? p.s_down[((size_t)seg * nblk_k + fold_blk) * N + wcol] : 0.f;
#pragma unroll
      for (int c = 0; c < kChunks; ++c) acc[c] = acc_tot[c] + sc * acc[c];
    }
    if (KSPLIT > 1) {
      // partial sums of the K parts meet in LDS; part 0 adds them in order
#pragma unroll
      for (int c = 0; c < kChunks; ++c) red[wave][c][lane] = acc[c];
      __syncthreads();
      if (kpart == 0) {
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
          f32x4 t = red[wave][c][lane];
#pragma unroll
          for (int j = 1; j < 4; ++j)
            if (j < KSPLIT) t += red[wave + j][c][lane];
          acc[c] = t;
        }
      }
      __syncthreads();
    }

    // 16x16 result: element i of a lane is row 4*(lane/16) + i of the chunk, column lane%16
    if (kpart != 0) continue;
    if (STAGE == 0) {
      float sg = 1.f, su = 1.f;
      if (FP8) {
        const float s_own = col_ok ? ((SWIGLU && n >= 8) ? p.s_up : p.s_gate)[(size_t)seg * N + wcol] : 0.f;
        sg = s_own;
        su = SWIGLU ? __shfl_xor(s_own, 8, 64) : 1.f;
      }
#pragma unroll
      for (int c = 0; c < kChunks; ++c) {
        if (c >= nch) break;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = acc[c][i];
          const float other = SWIGLU ? __shfl_xor(v, 8, 64) : 0.f;   // up value of this column
          const int r = r0 + c * kRowsPerChunk + 4 * g + i;
          if (SWIGLU) {
            if (n < 8 && col_ok && r < nrows) {
              const float gv = v * sg, uv = other * su;
              const float h = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
              static_cast<uint16_t*>(p.out)[(size_t)(row0 + r) * N + wcol] =
                  (uint16_t)f32_to_bf16_bits(h);
            }
          } else if (col_ok && r < nrows) {
            const float gv = fmaxf(v * sg, 0.f);
            static_cast<uint16_t*>(p.out)[(size_t)(row0 + r) * N + wcol] =
                (uint16_t)f32_to_bf16_bits(gv * gv);
          }
        }
      }
    } else {
#pragma unroll
      for (int c = 0; c < kChunks; ++c) {
        if (c >= nch) break;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = r0 + c * kRowsPerChunk + 4 * g + i;
          if (!col_ok || r >= nrows) continue;
          float v = acc[c][i];
          if (p.row_weight != nullptr) v *= p.row_weight[row0 + r];
          static_cast<uint16_t*>(p.out)[(size_t)(row0 + r) * N + wcol] =
              (uint16_t)f32_to_bf16_bits(v);
        }
      }
    }
  }
}

// Enough waves must stream to cover HBM latency: split K inside the workgroup when the
// (segments x column groups) grid is small.
template <int STAGE, int ACT>
DecSet make_set(const GemmParams& p) {
  constexpr bool SWIGLU = (STAGE == 0) && (ACT == MOE_ACT_SWIGLU);
  const int cols = SWIGLU ? 8 : 16;
  const long long groups = (long long)((p.N + cols - 1) / cols) * p.nseg;
  const int steps = p.K / kStepK;
  DecSet d;
  d.p = p;
  d.ksplit = (groups < 2048 && steps >= 16) ? 4 : (groups < 4096 && steps >= 8) ? 2 : 1;
  const int cols_per_wg = (kDecWaves / d.ksplit) * cols;
  d.nslices = (p.N + cols_per_wg - 1) / cols_per_wg;
  d.nwg = d.nslices * p.nseg;
  return d;
}

template <int STAGE, int ACT, bool FP8>
hipError_t launch_dec(const GemmParams& p, const GemmParams* p2, hipStream_t s) {
  DecSet a = make_set<STAGE, ACT>(p), b{};
  if (p2 != nullptr) {
    b = make_set<STAGE, ACT>(*p2);
    // the set with more work per workgroup goes first so that it starts early
    if (b.p.rows > a.p.rows / (a.p.nseg > 0 ? a.p.nseg : 1)) std::swap(a, b);
  }
  const long long grid = (long long)a.nwg + b.nwg;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((dec_gemm_kernel<STAGE, ACT, FP8>), dim3((unsigned)grid), dim3(kDecWaves * 64), 0,
                     s, a, b);
  return hipGetLastError();
}

}  // namespace

bool decode_gemm_applies(const GemmParams& p, int act_dtype) {
  if (act_dtype != MOE_BF16) return false;
  if (p.K % kStepK != 0 || p.kblock % kStepK != 0 || p.N % 64 != 0) return false;
  // few rows per segment: streaming the weights dominates
  if (p.offsets != nullptr) return (long long)p.rows <= 32LL * p.nseg;
  return p.rows <= 128;
}

hipError_t launch_decode_gemm(const GemmParams& p, Stage stage, int act, int weight_dtype,
                              hipStream_t s, const GemmParams* second) {
  const bool fp8 = weight_dtype == MOE_FP8_E4M3;
  const bool relu2 = act == MOE_ACT_RELU2;
  if (stage == Stage::Up) {
    if (fp8) return relu2 ? launch_dec<0, MOE_ACT_RELU2, true>(p, second, s)
                          : launch_dec<0, MOE_ACT_SWIGLU, true>(p, second, s);
    return relu2 ? launch_dec<0, MOE_ACT_RELU2, false>(p, second, s)
                 : launch_dec<0, MOE_ACT_SWIGLU, false>(p, second, s);
  }
  return fp8 ? launch_dec<1, MOE_ACT_SWIGLU, true>(p, second, s)
             : launch_dec<1, MOE_ACT_SWIGLU, false>(p, second, s);
}

}  // namespace moe
