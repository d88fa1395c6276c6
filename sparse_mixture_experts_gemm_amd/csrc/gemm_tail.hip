// Grouped GEMMs of the expert FFNs for shapes off the 64-element grid: K (dim or inter_dim)
// or N a multiple of 8 but not of 64, bf16 activations, bf16 or e4m3 weights.
//
// Same operation as the MFMA kernels of gemm.hip (grouped GEMM after routing, section
// "融合内核" of the FusionLLM training-framework page; SwiGLU W2 (silu(W1 x) * (W3 x)) of
// "大模型工程（一）：Transformer 到 MoE", section "变了什么，为什么变", item 3, or ReLU^2):
//   UP:   h = act(A W_gate^T, A W_up^T)     A rows gathered through row_index
//   DOWN: y = row_weight * (h W_down^T)
// but built for any multiple of 8 rather than for speed: 64 x 64 output tiles, four waves
// of 32 x 32, v_mfma_f32_16x16x32_bf16 on operands loaded straight from global memory
// (16 bytes per lane, one 8-element K group), every group past the end of its K block,
// every weight row past N and every token row past its segment read as zeros.  K blocks
// (the stacked shared experts of the DOWN stage) are folded one by one, each with its own
// e4m3 channel scales.
#include "common.h"
#include "gemm_core.h"
#include "internal.h"

namespace moe {

namespace {

constexpr int kTailBM = 64, kTailBN = 64;

template <int STAGE, int ACT, bool FP8>
__global__ __launch_bounds__(256) void gg_tail_kernel(GemmParams p) {
  constexpr bool SWIGLU = (STAGE == 0) && (ACT == MOE_ACT_SWIGLU);
  constexpr int NW = SWIGLU ? 2 : 1;                 // weight matrices multiplied
  __shared__ int s_tile0[65], s_row0[64], s_rows[64];
  const int N = p.N, K = p.K, kblock = p.kblock;
  const int nblk = K / kblock;
  const int NT = (N + kTailBN - 1) / kTailBN;
  build_schedule(p, kTailBM, NT, s_tile0, s_row0, s_rows);
  __syncthreads();
  const int total = s_tile0[p.nseg];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wr = wave >> 1, wc = wave & 1;           // 32-row token block, 32-column block
  const int l16 = lane & 15, kg = lane >> 4;         // operand row, 8-element K group
  const uint16_t* a = static_cast<const uint16_t*>(p.a);
  const void* wmat[2] = {STAGE == 1 ? p.w_down : p.w_gate, p.w_up};
  const float* smat[2] = {STAGE == 1 ? p.s_down : p.s_gate, p.s_up};

  for (int L = blockIdx.x; L < total; L += gridDim.x) {
    const TileCoord tc = decode_tile(L, p.nseg, kTailBM, NT, s_tile0, s_row0, s_rows);
    const int m0 = tc.m_tile * kTailBM, n0 = tc.n_tile * kTailBN;
    // the two token rows (i) and two weight rows (j) this lane supplies to the operands
    int arow[2];
    bool rok[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int rr = m0 + wr * 32 + i * 16 + l16;
      rok[i] = rr < tc.rows;
      const int sr = tc.row0 + (rok[i] ? rr : 0);
      arow[i] = p.row_index != nullptr ? p.row_index[sr] : sr;
    }
    int wrow[2];
    bool nok[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      wrow[j] = n0 + wc * 32 + j * 16 + l16;
      nok[j] = wrow[j] < N;
    }

    f32x4 tot[NW][2][2];
#pragma unroll
    for (int q = 0; q < NW; ++q)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 2; ++i) tot[q][j][i] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int blk = 0; blk < nblk; ++blk) {
      f32x4 acc[NW][2][2];
#pragma unroll
      for (int q = 0; q < NW; ++q)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int i = 0; i < 2; ++i) acc[q][j][i] = f32x4{0.f, 0.f, 0.f, 0.f};
      const size_t wbase = ((size_t)tc.seg * nblk + blk) * (size_t)N;   // weight row 0 of the block
      for (int k0 = 0; k0 < kblock; k0 += 32) {
        const int kk = k0 + 8 * kg;
        const bool kok = kk < kblock;
        bf16x8 xa[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          uint4 v = make_uint4(0, 0, 0, 0);
          if (kok && rok[i]) v = *reinterpret_cast<const uint4*>(a + (size_t)arow[i] * K + blk * kblock + kk);
          xa[i] = __builtin_bit_cast(bf16x8, v);
        }
#pragma unroll
        for (int q = 0; q < NW; ++q) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            bf16x8 wv;
            const size_t e = (wbase + wrow[j]) * kblock + kk;
            if (FP8) {
              uint2 c = make_uint2(0, 0);
              if (kok && nok[j]) c = *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(wmat[q]) + e);
              wv = widen_e4m3x8(c);
            } else {
              uint4 v = make_uint4(0, 0, 0, 0);
              if (kok && nok[j]) v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(wmat[q]) + e);
              wv = __builtin_bit_cast(bf16x8, v);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
              acc[q][j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wv, xa[i], acc[q][j][i], 0, 0, 0);
          }
        }
      }
      // fold the block: lane holds features 4 * kg + v of its 16-row weight block
#pragma unroll
      for (int q = 0; q < NW; ++q)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int n = n0 + wc * 32 + j * 16 + 4 * kg + v;
            const float sc = (FP8 && n < N) ? smat[q][wbase + n] : 1.0f;
#pragma unroll
            for (int i = 0; i < 2; ++i) tot[q][j][i][v] = fmaf(sc, acc[q][j][i][v], tot[q][j][i][v]);
          }
    }

    // epilogue: lane (kg, l16) holds, for token row m0 + 32 wr + 16 i + l16, the four
    // consecutive features n0 + 32 wc + 16 j + 4 kg + v
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int rr = m0 + wr * 32 + i * 16 + l16;
      if (rr >= tc.rows) continue;
      const size_t orow = (size_t)(tc.row0 + rr);
      const float rw = (STAGE == 1 && p.row_weight != nullptr) ? p.row_weight[orow] : 1.0f;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int nb = n0 + wc * 32 + j * 16 + 4 * kg;
        if (nb >= N) continue;                         // N % 8 == 0: all four or none
        float y[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float g = tot[0][j][i][v];
          if (STAGE == 1) {
            y[v] = rw * g;
          } else if (SWIGLU) {
            const float u = tot[NW - 1][j][i][v];
            y[v] = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
          } else {
            const float r = fmaxf(g, 0.f);
            y[v] = r * r;
          }
        }
        uint2 o;
        o.x = pack_bf16x2(y[0], y[1]);
        o.y = pack_bf16x2(y[2], y[3]);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + orow * N + nb) = o;
      }
    }
  }
}

template <int STAGE, int ACT, bool FP8>
hipError_t launch_tail(const GemmParams& p, int num_cus, hipStream_t s) {
  hipLaunchKernelGGL((gg_tail_kernel<STAGE, ACT, FP8>), dim3(num_cus * 4), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

bool tail_gemm_applies(const GemmParams& p) {
  return p.K % 64 != 0 || p.kblock % 64 != 0 || p.N % 64 != 0;
}

hipError_t launch_tail_gemm(const GemmParams& p, Stage stage, int act, int weight_dtype,
                            int num_cus, hipStream_t s) {
  if (p.rows == 0) return hipSuccess;
  const bool fp8 = weight_dtype == MOE_FP8_E4M3;
  const bool relu2 = act == MOE_ACT_RELU2;
  if (stage == Stage::Up) {
    if (fp8) return relu2 ? launch_tail<0, MOE_ACT_RELU2, true>(p, num_cus, s)
                          : launch_tail<0, MOE_ACT_SWIGLU, true>(p, num_cus, s);
    return relu2 ? launch_tail<0, MOE_ACT_RELU2, false>(p, num_cus, s)
                 : launch_tail<0, MOE_ACT_SWIGLU, false>(p, num_cus, s);
  }
  return fp8 ? launch_tail<1, MOE_ACT_SWIGLU, true>(p, num_cus, s)
             : launch_tail<1, MOE_ACT_SWIGLU, false>(p, num_cus, s);
}

}  // namespace moe
