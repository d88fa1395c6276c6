// Grouped GEMMs of the expert FFNs.
//
// After routing, every expert multiplies the rows routed to it; FusionLLM runs this as a
// grouped GEMM and fuses Linear+ReLU^2 ("FusionLLM：融合 MLA、GDN 与 MoE 的高效混合架构大模型
// 训练框架", section "融合内核").  The expert is SwiGLU W2 (silu(W1 x) * (W3 x))
// ("大模型工程（一）：Transformer 到 MoE", section "变了什么，为什么变", item 3) or ReLU^2.
//
// Two stages, each one launch over all segments (experts):
//   UP:   h = act(A W_gate^T, A W_up^T)     A rows gathered on load through row_index
//   DOWN: y = row_weight * (h W_down^T)     routing weight applied in the epilogue
// Segments come from the device-side offsets, so the host never waits for the routing.
//
// gfx950 mapping (bf16 / e4m3 weights): persistent workgroups of 4 waves own a BM x BN
// output tile; waves are laid out 2 x 2 and issue v_mfma_f32_32x32x16_bf16 on 64 x 64
// sub-tiles.  A and B K-slices (BK = 64) are staged in LDS, double-buffered, with the 16-byte
// chunks of each 128-byte row XOR-swizzled by (row & 7) so that the MFMA operand reads
// (32 rows, one chunk each) spread over all banks.  For SwiGLU the B tile interleaves
// gate and up rows per 32-column MFMA tile, so the gate and up results of an output
// element land in the same lane and the activation runs in registers.  e4m3 weights are
// staged as bytes and widened to bf16 (exactly) when read from LDS; their per-channel
// scales multiply the fp32 accumulator.  Tiles are walked in XCD-contiguous order:
// workgroup b runs on XCD b % 8, and each XCD takes a contiguous range of (expert,
// n-tile, m-tile) tiles so that tiles sharing an expert's weights share that XCD's L2.
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

__device__ __forceinline__ void store_out(void* out, size_t off, float v, bool bf16) {
  if (bf16) static_cast<uint16_t*>(out)[off] = (uint16_t)f32_to_bf16_bits(v);
  else static_cast<float*>(out)[off] = v;
}

// ------------------------------------------------------------------------------------
// bf16 activations, bf16 or e4m3 weights, MFMA 32x32x16.
template <int STAGE, int ACT, bool FP8>
__global__ __launch_bounds__(256, 2) void gg_mfma_kernel(GemmParams p) {
  constexpr int BM = 128, BN = 128, BK = 64;
  constexpr int WTM = 64, WTN = 64, FM = 2, FN = 2;
  constexpr bool SWIGLU = (STAGE == 0) && (ACT == MOE_ACT_SWIGLU);
  constexpr int BROW = FP8 ? BK : BK * 2;            // bytes per B tile row in LDS
  constexpr int A_BYTES = BM * BK * 2;
  constexpr int B_BYTES = BN * BROW;

  __shared__ __align__(16) unsigned char lds[2 * (A_BYTES + B_BYTES)];
  __shared__ int s_tile0[65], s_row0[64], s_rows[64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const int N = p.N, K = p.K;
  const int hcols_per_tile = SWIGLU ? BN / 2 : BN;
  const int NT = (N + hcols_per_tile - 1) / hcols_per_tile;

  build_schedule(p, BM, NT, s_tile0, s_row0, s_rows);
  __syncthreads();
  const int total = s_tile0[p.nseg];

  const int nwg = gridDim.x;
  const int xcd = blockIdx.x % kNumXcd;
  const int slot = blockIdx.x / kNumXcd;
  const int per_x = (nwg - xcd + kNumXcd - 1) / kNumXcd;
  const int lo = (int)(((long long)xcd * total) / kNumXcd);
  const int hi = (int)(((long long)(xcd + 1) * total) / kNumXcd);

  const uint16_t* a_base = static_cast<const uint16_t*>(p.a);
  const size_t wmat = (size_t)N * K;                  // weights per segment per matrix
  const int nblk_k = K / p.kblock;

  for (int L = lo + slot; L < hi; L += per_x) {
    const TileCoord tc = decode_tile(L, p.nseg, BM, NT, s_tile0, s_row0, s_rows);
    const int m0 = tc.m_tile * BM;

    // ---- per-thread global source pointers for this tile
    // A: 4 chunks of 16 B per thread: row = tid/8 + 32 i, chunk = tid % 8
    const uint16_t* a_src[4];
    bool a_ok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (tid >> 3) + 32 * i;
      const int r = m0 + row;
      a_ok[i] = r < tc.rows;
      int src = tc.row0 + (a_ok[i] ? r : 0);
      if (p.row_index != nullptr) src = a_ok[i] ? p.row_index[src] : 0;
      a_src[i] = a_base + (size_t)src * K + (tid & 7) * 8;
    }
    // B: bf16: 4 chunks of 16 B (row = tid/8 + 32 i); e4m3: 2 chunks (row = tid/4 + 64 i)
    constexpr int BCH = FP8 ? 2 : 4;
    const unsigned char* b_src[BCH];
    bool b_ok[BCH];
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
      const int n = FP8 ? (tid >> 2) + 64 * i : (tid >> 3) + 32 * i;
      const int cbyte = FP8 ? (tid & 3) * 16 : (tid & 7) * 16;
      int wrow;
      const void* wb;
      if (STAGE == 0) {
        if (SWIGLU) {
          const int wc = n / WTN, r = n % WTN;
          const int half = r / (WTN / 2);
          wrow = tc.n_tile * (BN / 2) + wc * (WTN / 2) + (r % (WTN / 2));
          wb = half ? p.w_up : p.w_gate;
        } else {
          wrow = tc.n_tile * BN + n;
          wb = p.w_gate;
        }
      } else {
        wrow = tc.n_tile * BN + n;
        wb = p.w_down;
      }
      b_ok[i] = wrow < N;
      const size_t esz = FP8 ? 1 : 2;
      b_src[i] = static_cast<const unsigned char*>(wb) +
                 ((size_t)tc.seg * wmat + (size_t)(b_ok[i] ? wrow : 0) * p.kblock) * esz + cbyte;
    }

    f32x16 acc[FM][FN];
    f32x16 acc_tot[FM][FN];
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
      for (int b = 0; b < FN; ++b) {
        acc[a][b] = f32x16{};
        if (FP8 && STAGE == 1) acc_tot[a][b] = f32x16{};
      }

    uint4 ra[4];
    uint4 rb[BCH];
    auto gload = [&](int kt) {
      const int k0 = kt * BK;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ra[i] = a_ok[i] ? *reinterpret_cast<const uint4*>(a_src[i] + k0) : make_uint4(0, 0, 0, 0);
      const size_t koff = (size_t)(k0 / p.kblock) * N * p.kblock + (k0 % p.kblock);
#pragma unroll
      for (int i = 0; i < BCH; ++i)
        rb[i] = b_ok[i] ? *reinterpret_cast<const uint4*>(b_src[i] + koff * (FP8 ? 1 : 2))
                        : make_uint4(0, 0, 0, 0);
    };
    auto sstore = [&](int buf) {
      unsigned char* A = lds + buf * (A_BYTES + B_BYTES);
      unsigned char* B = A + A_BYTES;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = (tid >> 3) + 32 * i, c = tid & 7;
        *reinterpret_cast<uint4*>(A + row * 128 + ((c ^ (row & 7)) << 4)) = ra[i];
      }
      if (!FP8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = (tid >> 3) + 32 * i, c = tid & 7;
          *reinterpret_cast<uint4*>(B + row * 128 + ((c ^ (row & 7)) << 4)) = rb[i];
        }
      } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int row = (tid >> 2) + 64 * i, c = (tid & 3) * 2;   // two 8-byte units
          *reinterpret_cast<uint2*>(B + row * 64 + (((c) ^ (row & 7)) << 3)) =
              make_uint2(rb[i].x, rb[i].y);
          *reinterpret_cast<uint2*>(B + row * 64 + (((c + 1) ^ (row & 7)) << 3)) =
              make_uint2(rb[i].z, rb[i].w);
        }
      }
    };

    const int nk = K / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      if (kt + 1 < nk) gload(kt + 1);
      if (FP8 && STAGE == 1 && kt > 0 && ((kt * BK) % p.kblock) == 0) {
        // new K block (another shared expert): fold the finished block with its scales
        const int blk = (kt * BK) / p.kblock - 1;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          const int col = tc.n_tile * BN + wn * WTN + fn * 32 + (lane & 31);
          const float sc = col < N ? p.s_down[((size_t)tc.seg * nblk_k + blk) * N + col] : 0.f;
#pragma unroll
          for (int fm = 0; fm < FM; ++fm) {
            acc_tot[fm][fn] += sc * acc[fm][fn];
            acc[fm][fn] = f32x16{};
          }
        }
      }
      const unsigned char* A = lds + (kt & 1) * (A_BYTES + B_BYTES);
      const unsigned char* B = A + A_BYTES;
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        const int c = ks * 2 + (lane >> 5);
        bf16x8 af[FM], bfr[FN];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
          const int row = wm * WTM + fm * 32 + (lane & 31);
          af[fm] = *reinterpret_cast<const bf16x8*>(A + row * 128 + ((c ^ (row & 7)) << 4));
        }
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          const int row = wn * WTN + fn * 32 + (lane & 31);
          if (!FP8) {
            bfr[fn] = *reinterpret_cast<const bf16x8*>(B + row * 128 + ((c ^ (row & 7)) << 4));
          } else {
            const uint2 q = *reinterpret_cast<const uint2*>(B + row * 64 + ((c ^ (row & 7)) << 3));
            uint4 w;
            e4m3x4_to_bf16x4(q.x, w.x, w.y);
            e4m3x4_to_bf16x4(q.y, w.z, w.w);
            bfr[fn] = __builtin_bit_cast(bf16x8, w);
          }
        }
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
          for (int fn = 0; fn < FN; ++fn)
            acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[fm], bfr[fn], acc[fm][fn], 0, 0, 0);
      }
      if (kt + 1 < nk) sstore((kt + 1) & 1);
      __syncthreads();
    }

    // ---- epilogue.  32x32 MFMA result: element i of a lane is row 8*(i/4) + 4*(lane/32)
    // + i%4, column lane%32 of the 32x32 sub-tile.
    const int col_in = lane & 31;
    if (STAGE == 0) {
      constexpr int FH = SWIGLU ? FN / 2 : FN;
#pragma unroll
      for (int fh = 0; fh < FH; ++fh) {
        const int hcol = SWIGLU ? tc.n_tile * (BN / 2) + wn * (WTN / 2) + fh * 32 + col_in
                                : tc.n_tile * BN + wn * WTN + fh * 32 + col_in;
        if (hcol >= N) continue;
        float sg = 1.f, su = 1.f;
        if (FP8) {
          sg = p.s_gate[(size_t)tc.seg * N + hcol];
          if (SWIGLU) su = p.s_up[(size_t)tc.seg * N + hcol];
        }
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int r = m0 + wm * WTM + fm * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
            if (r >= tc.rows) continue;
            float h;
            if (SWIGLU) {
              const float g = acc[fm][fh][i] * sg;
              const float u = acc[fm][fh + FN / 2][i] * su;
              h = silu_f(g) * u;
            } else {
              const float g = acc[fm][fh][i] * sg;
              const float rr = fmaxf(g, 0.f);
              h = rr * rr;
            }
            store_out(p.out, (size_t)(tc.row0 + r) * N + hcol, h, true);
          }
        }
      }
    } else {
      if (FP8) {
        const int blk = nblk_k - 1;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          const int col = tc.n_tile * BN + wn * WTN + fn * 32 + col_in;
          const float sc = col < N ? p.s_down[((size_t)tc.seg * nblk_k + blk) * N + col] : 0.f;
#pragma unroll
          for (int fm = 0; fm < FM; ++fm) acc[fm][fn] = acc_tot[fm][fn] + sc * acc[fm][fn];
        }
      }
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int col = tc.n_tile * BN + wn * WTN + fn * 32 + col_in;
        if (col >= N) continue;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int r = m0 + wm * WTM + fm * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
            if (r >= tc.rows) continue;
            const float rw = p.row_weight != nullptr ? p.row_weight[tc.row0 + r] : 1.f;
            store_out(p.out, (size_t)(tc.row0 + r) * N + col, rw * acc[fm][fn][i], true);
          }
        }
      }
    }
    __syncthreads();   // LDS of this tile is reused by the next one
  }
}

// ------------------------------------------------------------------------------------
// fp32 activations and weights: plain FMA tiles (small, latency-bound layers).
// 64 x 64 output tile per workgroup, 256 threads, 4 x 4 outputs per thread, K step 16.
template <int STAGE, int ACT>
__global__ __launch_bounds__(256) void gg_f32_kernel(GemmParams p) {
  constexpr int BM = 64, BN = 64, BK = 16;
  constexpr bool SWIGLU = (STAGE == 0) && (ACT == MOE_ACT_SWIGLU);
  __shared__ float As[BK][BM + 4];
  __shared__ float Bg[BK][BN + 4];
  __shared__ float Bu[BK][BN + 4];
  __shared__ int s_tile0[65], s_row0[64], s_rows[64];

  const int tid = threadIdx.x;
  const int N = p.N, K = p.K;
  const int NT = (N + BN - 1) / BN;
  build_schedule(p, BM, NT, s_tile0, s_row0, s_rows);
  __syncthreads();
  const int total = s_tile0[p.nseg];
  const float* a_base = static_cast<const float*>(p.a);
  const size_t wmat = (size_t)N * K;

  for (int L = blockIdx.x; L < total; L += gridDim.x) {
    const TileCoord tc = decode_tile(L, p.nseg, BM, NT, s_tile0, s_row0, s_rows);
    const int m0 = tc.m_tile * BM, n0 = tc.n_tile * BN;
    const int tr = (tid >> 4) * 4, tcn = (tid & 15) * 4;
    float accg[4][4] = {}, accu[4][4] = {};
    // loader: thread loads A[row = tid/4][k = (tid%4)*4 .. +4] and same for B rows
    const int lrow = tid >> 2, lk = (tid & 3) * 4;
    const int ar = m0 + lrow;
    const bool a_ok = ar < tc.rows;
    int asrc = tc.row0 + (a_ok ? ar : 0);
    if (p.row_index != nullptr) asrc = a_ok ? p.row_index[asrc] : 0;
    const int brow = n0 + lrow;
    const bool b_ok = brow < N;
    const float* wg = static_cast<const float*>(STAGE == 0 ? p.w_gate : p.w_down);
    const float* wu = static_cast<const float*>(p.w_up);
    for (int k0 = 0; k0 < K; k0 += BK) {
      const size_t koff = (size_t)(k0 / p.kblock) * N * p.kblock + (k0 % p.kblock);
      float4 av = a_ok ? *reinterpret_cast<const float4*>(a_base + (size_t)asrc * K + k0 + lk)
                       : make_float4(0, 0, 0, 0);
      const size_t wo = tc.seg * wmat + (size_t)(b_ok ? brow : 0) * p.kblock + koff + lk;
      float4 gv = b_ok ? *reinterpret_cast<const float4*>(wg + wo) : make_float4(0, 0, 0, 0);
      float4 uv = make_float4(0, 0, 0, 0);
      if (SWIGLU && b_ok) uv = *reinterpret_cast<const float4*>(wu + wo);
      __syncthreads();
      As[lk + 0][lrow] = av.x; As[lk + 1][lrow] = av.y; As[lk + 2][lrow] = av.z; As[lk + 3][lrow] = av.w;
      Bg[lk + 0][lrow] = gv.x; Bg[lk + 1][lrow] = gv.y; Bg[lk + 2][lrow] = gv.z; Bg[lk + 3][lrow] = gv.w;
      if (SWIGLU) {
        Bu[lk + 0][lrow] = uv.x; Bu[lk + 1][lrow] = uv.y; Bu[lk + 2][lrow] = uv.z; Bu[lk + 3][lrow] = uv.w;
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < BK; ++kk) {
        float a4[4], g4[4], u4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a4[i] = As[kk][tr + i];
          g4[i] = Bg[kk][tcn + i];
          if (SWIGLU) u4[i] = Bu[kk][tcn + i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            accg[i][j] = fmaf(a4[i], g4[j], accg[i][j]);
            if (SWIGLU) accu[i][j] = fmaf(a4[i], u4[j], accu[i][j]);
          }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = m0 + tr + i;
      if (r >= tc.rows) continue;
      const float rw = (STAGE == 1 && p.row_weight != nullptr) ? p.row_weight[tc.row0 + r] : 1.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = n0 + tcn + j;
        if (c >= N) continue;
        float v;
        if (STAGE == 0) {
          if (SWIGLU) v = silu_f(accg[i][j]) * accu[i][j];
          else { const float rr = fmaxf(accg[i][j], 0.f); v = rr * rr; }
        } else {
          v = rw * accg[i][j];
        }
        static_cast<float*>(p.out)[(size_t)(tc.row0 + r) * N + c] = v;
      }
    }
    __syncthreads();
  }
}

template <int STAGE, int ACT, bool FP8>
hipError_t launch_mfma(const GemmParams& p, int num_cus, hipStream_t s) {
  const int grid = num_cus * 2;
  hipLaunchKernelGGL((gg_mfma_kernel<STAGE, ACT, FP8>), dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int STAGE, int ACT>
hipError_t launch_f32(const GemmParams& p, int num_cus, hipStream_t s) {
  const int grid = num_cus * 4;
  hipLaunchKernelGGL((gg_f32_kernel<STAGE, ACT>), dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_gemm(const GemmParams& p, Stage stage, int act, int act_dtype,
                               int weight_dtype, int num_cus, hipStream_t s) {
  if (p.rows == 0) return hipSuccess;
  const bool up = stage == Stage::Up;
  const bool relu2 = act == MOE_ACT_RELU2;
  if (act_dtype == MOE_F32) {
    if (up) return relu2 ? launch_f32<0, MOE_ACT_RELU2>(p, num_cus, s)
                         : launch_f32<0, MOE_ACT_SWIGLU>(p, num_cus, s);
    return launch_f32<1, MOE_ACT_SWIGLU>(p, num_cus, s);
  }
  const bool fp8 = weight_dtype == MOE_FP8_E4M3;
  if (up) {
    if (fp8) return relu2 ? launch_mfma<0, MOE_ACT_RELU2, true>(p, num_cus, s)
                          : launch_mfma<0, MOE_ACT_SWIGLU, true>(p, num_cus, s);
    return relu2 ? launch_mfma<0, MOE_ACT_RELU2, false>(p, num_cus, s)
                 : launch_mfma<0, MOE_ACT_SWIGLU, false>(p, num_cus, s);
  }
  return fp8 ? launch_mfma<1, MOE_ACT_SWIGLU, true>(p, num_cus, s)
             : launch_mfma<1, MOE_ACT_SWIGLU, false>(p, num_cus, s);
}

}  // namespace moe
