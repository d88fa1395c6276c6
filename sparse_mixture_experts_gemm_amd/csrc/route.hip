// Router GEMM, gate scoring and group-limited top-k.
//
// The router is the bias-free linear map g(x) = W_g x followed by a deterministic top-k
// ("大模型工程（一）：Transformer 到 MoE", section "MoE 数学：路由、容量与平衡详解"), with
// sigmoid gating and group-limited routing as in the FusionLLM MoE ("FusionLLM：融合 MLA、
// GDN 与 MoE 的高效混合架构大模型训练框架", section "混合专家（MoE）").
//
// Layout on the chip: one workgroup owns 16 tokens.  Its sixteen waves split the dim
// (K) of the 16 x E logit block between them and run bf16 MFMA 16x16x32 on operands read
// straight from global memory (x rows are read once; the E x d router weight is shared
// by every workgroup and stays in L2).  The partial logits are summed through LDS in a
// fixed order, then each wave scores and selects for one token with lane = expert:
// group maxima by DPP inside aligned groups of 8 lanes (shuffles for other group sizes),
// group rank by comparing against every group's score (readlane), and k rounds of a DPP
// wave max over the score bits, where the lowest lane holding the max wins (ballot), i.e.
// the lower expert index on equal scores.
//
// Pre-norm variant: the layer's MoE reads RMSNorm(x) ("大模型工程（一）：Transformer 到 MoE",
// section "变了什么，为什么变": the decoder-layer sketch and item 2, RMSNorm keeps only the
// root-mean-square scaling).  The same launch computes every token's 1/rms (one wave per
// token, its row held in registers, fixed-order sum of squares), writes the normalised row
// in the activation dtype, and feeds the router GEMM with exactly those values: staged in
// LDS (rows padded by 16 bytes so the MFMA operand reads of 16 rows hit distinct banks)
// when d <= 4096, else recomputed from x by the same expression.
#include "common.h"
#include "internal.h"

namespace moe {

namespace {

constexpr int kRouteTok = 16;   // tokens per workgroup (bf16 path)

// Gate score of one expert lane: sigmoid, or softmax over the wave's valid lanes.
__device__ __forceinline__ float gate_score(float logit, bool valid, const RouteParams& p) {
  if (p.score_fn == MOE_SCORE_SIGMOID) return 1.0f / (1.0f + expf(-logit));
  const float mx = wave_max_f(valid ? logit : -INFINITY);
  const float e = valid ? expf(logit - mx) : 0.0f;
  const float sum = wave_sum_f(e);
  return e / sum;
}

// Selection for token t on per-lane selection keys (>= 0) with weights from the scores s.
__device__ __forceinline__ void select_write(float s, float key, bool valid, int lane,
                                             const RouteParams& p, int t, int32_t* idx,
                                             float* wout) {
  // fp32 bit patterns of non-negative keys order like the keys themselves
  const uint32_t sbits = __float_as_uint(key);
  bool elig = valid;
  if (p.G > 1 && p.Gk < p.G) {
    const int gsz = p.E / p.G;
    const int g = min(lane / gsz, p.G - 1);
    float gs;
    if (gsz == 8) {
      // groups are aligned runs of 8 lanes: DPP max inside the group
      const uint32_t b1 = group8_max_u32(valid ? sbits : 0u);
      gs = __uint_as_float(b1);
      if (p.n_g == 2) {
        // drop the first lane holding the group max, then take the max again
        const uint64_t m = __ballot(valid && sbits == b1);
        const uint32_t gm = (uint32_t)(m >> (8 * g)) & 0xffu;
        const int first = 8 * g + __builtin_ctz(gm | 0x100u);
        const uint32_t b2 = group8_max_u32((valid && lane != first) ? sbits : 0u);
        gs = __uint_as_float(b1) + __uint_as_float(b2);
      }
    } else {
      float b1 = -1.0f, b2 = -1.0f;  // scores are >= 0
      for (int i = 0; i < gsz; ++i) {
        float v = wave_shfl(key, g * gsz + i);
        if (v > b1) {
          b2 = b1;
          b1 = v;
        } else if (v > b2) {
          b2 = v;
        }
      }
      gs = (p.n_g == 2) ? (b1 + b2) : b1;
    }
    int rank = 0;
    for (int h = 0; h < p.G; ++h) {
      const float o = __uint_as_float(
          (uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(gs), h * gsz));
      rank += (o > gs) || (o == gs && h < g);
    }
    elig = valid && rank < p.Gk;
  }

  // k rounds: wave max of (score bits + 1) over eligible lanes; the lowest lane holding the
  // max wins, i.e. the lower expert index on equal scores
  uint32_t kb = elig ? sbits + 1u : 0u;
  float sel = 0.0f;
  int sel_e = 0;
  for (int j = 0; j < p.k; ++j) {
    const uint32_t mx = wave_max_u32(kb);
    const uint64_t m = __ballot(kb == mx);
    const int win = (int)__builtin_ctzll(m);
    const float s_win = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(s), win));
    if (lane == win) kb = 0u;
    if (lane == j) {
      sel = s_win;
      sel_e = win;
    }
  }
  float sum = 0.0f;
  for (int j = 0; j < p.k; ++j) sum += __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(sel), j));
  if (lane < p.k) {
    const float wj = (p.renormalize ? sel / sum : sel) * p.route_scale;
    idx[(size_t)t * p.k + lane] = sel_e;
    wout[(size_t)t * p.k + lane] = wj;
  }
}

// Scores of one expert lane from its logit, then selection for token t.  The selection
// compares the scores of the logits plus the selection-only bias when one is given; the
// weights use the unbiased scores.  `valid` marks lanes < E.
__device__ __forceinline__ void score_select_write(float logit, bool valid, int lane,
                                                   const RouteParams& p, int t, float* scores,
                                                   int32_t* idx, float* wout) {
  const float s = gate_score(logit, valid, p);
  if (scores != nullptr && valid) scores[(size_t)t * p.E + lane] = s;
  float key = s;
  if (p.select_bias != nullptr) key = gate_score(logit + (valid ? p.select_bias[lane] : 0.0f), valid, p);
  select_write(s, key, valid, lane, p, t, idx, wout);
}

// The bf16 router's logit is the sum of 16 partial dot products, partial w over the
// 32-wide K-steps w, w + 16, w + 32, ...  They are summed as four sums of four, always in
// this order, so that a split of the partials over workgroups gives the same bits.
__device__ __forceinline__ float sum4(float a, float b, float c, float d) {
  return ((a + b) + c) + d;
}

// bf16 router: 16 tokens per workgroup; its 16 waves split K in 32-wide MFMA steps
// (wave w takes steps w, w+16, ...), so each wave needs a single round of loads for d = 2048.
constexpr int kRouteWaves = 16;

// Normalised bf16 values of 8 consecutive channels: bf16(x * inv_rms * gamma), fp32 steps.
__device__ __forceinline__ uint4 norm_bf16x8(uint4 v, float inv_rms, const float* g) {
  const float4 g0 = *reinterpret_cast<const float4*>(g);
  const float4 g1 = *reinterpret_cast<const float4*>(g + 4);
  const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = (bf16_bits_to_f32(w[i] & 0xffffu) * inv_rms) * gv[2 * i];
    const float hi = (bf16_bits_to_f32(w[i] >> 16) * inv_rms) * gv[2 * i + 1];
    o[i] = pack_bf16x2(lo, hi);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// 1 / sqrt(mean of squares + eps) from a wave's sum of squares.
__device__ __forceinline__ float inv_rms(float sumsq, int d, float eps) {
  return 1.0f / sqrtf(sumsq / (float)d + eps);
}

// NORM: 0 = route x; 1 = pre-norm, normalised rows staged in LDS (d <= kNormLdsDim);
// 2 = pre-norm, normalised values recomputed where the router reads them (any d).
constexpr int kNormLdsDim = 4096;
constexpr int kNormRowBytes = kNormLdsDim * 2 + 16;
constexpr int kPartBytes = kRouteWaves * kRouteTok * 64 * 4;

// KTAIL: d is not a multiple of 32 (a multiple of 8): one more K-step, whose 8-element
// groups past d read zeros.  With KTAIL false the code is that of a 32-aligned d.
template <int NORM, bool KTAIL>
__global__ __launch_bounds__(1024) void route_bf16_kernel(RouteParams p,
                                                          const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ wr,
                                                          const float* __restrict__ bias,
                                                          float* scores, int32_t* idx,
                                                          float* wout) {
  // the partial logits, and with NORM == 1 before them the 16 normalised rows
  constexpr int kSmem = NORM == 1 ? kRouteTok * kNormRowBytes : kPartBytes;
  static_assert(kRouteTok * kNormRowBytes >= kPartBytes, "partial logits fit the row tile");
  __shared__ __align__(16) unsigned char smem[kSmem];
  auto part = reinterpret_cast<float (*)[kRouteTok][64]>(smem);
  __shared__ float s_inv_rms[kRouteTok];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * kRouteTok;
  if (NORM == 1) {
    // wave w: token t0 + w, its row in registers (8 channels per lane per chunk)
    constexpr int kChunks = kNormLdsDim / 512;
    const int t = t0 + wave;
    if (t < p.T) {
      const uint16_t* xr = x + (size_t)t * p.d;
      uint4 xv[kChunks];
      float ss = 0.0f;
#pragma unroll
      for (int i = 0; i < kChunks; ++i) {
        const int c = (i * 64 + lane) * 8;
        if (c < p.d) {
          xv[i] = *reinterpret_cast<const uint4*>(xr + c);
          const uint32_t w[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float lo = bf16_bits_to_f32(w[q] & 0xffffu), hi = bf16_bits_to_f32(w[q] >> 16);
            ss = fmaf(lo, lo, ss);
            ss = fmaf(hi, hi, ss);
          }
        }
      }
      const float r = inv_rms(wave_sum_f(ss), p.d, p.norm_eps);
      uint16_t* xo = static_cast<uint16_t*>(p.x_norm) + (size_t)t * p.d;
      unsigned char* row = smem + wave * kNormRowBytes;
#pragma unroll
      for (int i = 0; i < kChunks; ++i) {
        const int c = (i * 64 + lane) * 8;
        if (c < p.d) {
          const uint4 v = norm_bf16x8(xv[i], r, p.norm_gamma + c);
          *reinterpret_cast<uint4*>(xo + c) = v;
          *reinterpret_cast<uint4*>(row + c * 2) = v;
        }
      }
    }
    __syncthreads();
  } else if (NORM == 2) {
    // wave w: token t0 + w; lanes stride over the row in 8-channel chunks
    const int t = t0 + wave;
    float r = 0.0f;
    if (t < p.T) {
      const uint16_t* xr = x + (size_t)t * p.d;
      float ss = 0.0f;
      for (int c = lane * 8; c < p.d; c += 64 * 8) {
        const uint4 v = *reinterpret_cast<const uint4*>(xr + c);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float lo = bf16_bits_to_f32(w[q] & 0xffffu), hi = bf16_bits_to_f32(w[q] >> 16);
          ss = fmaf(lo, lo, ss);
          ss = fmaf(hi, hi, ss);
        }
      }
      r = inv_rms(wave_sum_f(ss), p.d, p.norm_eps);
      uint16_t* xo = static_cast<uint16_t*>(p.x_norm) + (size_t)t * p.d;
      for (int c = lane * 8; c < p.d; c += 64 * 8)
        *reinterpret_cast<uint4*>(xo + c) =
            norm_bf16x8(*reinterpret_cast<const uint4*>(xr + c), r, p.norm_gamma + c);
    }
    if (lane == 0) s_inv_rms[wave] = r;
    __syncthreads();
  }
  const int m = lane & 15;        // token row within the block / expert column in a tile
  const int g = lane >> 4;        // 8-element K group
  const int ntiles = (p.E + 15) >> 4;
  const bool row_ok = (t0 + m) < p.T;
  const uint16_t* xrow = x + (size_t)(row_ok ? t0 + m : 0) * p.d;
  // the A operand: x, or its normalised value (0 for rows past T)
  const float row_r = NORM == 2 ? s_inv_rms[m] : 0.0f;
  const unsigned char* lds_row = smem + m * kNormRowBytes;
  auto load_a = [&](int kk) -> uint4 {
    if (!row_ok || (KTAIL && kk >= p.d)) return make_uint4(0, 0, 0, 0);
    if (NORM == 1) return *reinterpret_cast<const uint4*>(lds_row + kk * 2);
    const uint4 v = *reinterpret_cast<const uint4*>(xrow + kk);
    return NORM == 2 ? norm_bf16x8(v, row_r, p.norm_gamma + kk) : v;
  };

  f32x4 acc[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nsteps = KTAIL ? (p.d + 31) >> 5 : p.d >> 5;
  auto load_b = [&](int kk, int n) -> uint4 {
    const int e = n * 16 + m;
    return (n < ntiles && e < p.E && (!KTAIL || kk < p.d))
               ? *reinterpret_cast<const uint4*>(wr + (size_t)e * p.d + kk)
               : make_uint4(0, 0, 0, 0);
  };
  int st = wave;
  for (; st + 3 * kRouteWaves < nsteps; st += 4 * kRouteWaves) {
    uint4 av[4], bv[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int kk = (st + kRouteWaves * u) * 32 + g * 8;
      av[u] = load_a(kk);
#pragma unroll
      for (int n = 0; n < 4; ++n) bv[u][n] = load_b(kk, n);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int n = 0; n < 4; ++n)
        acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[u]),
                                                         __builtin_bit_cast(bf16x8, bv[u][n]),
                                                         acc[n], 0, 0, 0);
  }
  for (; st < nsteps; st += kRouteWaves) {
    const int kk = st * 32 + g * 8;
    const uint4 av = load_a(kk);
#pragma unroll
    for (int n = 0; n < 4; ++n)
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                       __builtin_bit_cast(bf16x8, load_b(kk, n)),
                                                       acc[n], 0, 0, 0);
  }
  // 16x16 MFMA result: lane holds rows 4*(lane/16)+i of column lane%16.
  if (NORM == 1) __syncthreads();   // the partial logits overwrite the staged rows
#pragma unroll
  for (int n = 0; n < 4; ++n) {
#pragma unroll
    for (int i = 0; i < 4; ++i) part[wave][4 * g + i][n * 16 + m] = acc[n][i];
  }
  __syncthreads();
  const int row = wave;            // one token per wave
  const int t = t0 + row;
  if (t >= p.T) return;            // uniform per wave; no barrier follows
  const bool valid = lane < p.E;
  float l = 0.0f;
  if (valid) {
    float q[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      q[j] = sum4(part[4 * j][row][lane], part[4 * j + 1][row][lane], part[4 * j + 2][row][lane],
                  part[4 * j + 3][row][lane]);
    l = sum4(q[0], q[1], q[2], q[3]);
    if (bias != nullptr) l += bias[lane];
  }
  score_select_write(l, valid, lane, p, t, scores, idx, wout);
}

// Small batches (the decode shape): the one-workgroup-per-16-tokens router above reads the
// whole E x d router matrix into each of its few CUs, which bounds it by one CU's load
// rate.  Here the same logits are spread over (16-token block, 16-expert tile, quarter)
// workgroups: wave w of quarter j computes partial 4j + w of the kernel above (the same
// K-steps, MFMA chain and operands) and the workgroup writes the sum of its four, in the
// same order, to part[j][t][e].  route_select_part_kernel finishes the sum, scores and
// selects with one wave per token, so a small batch routes bit for bit like the kernel
// above.  (Selection costs a few hundred instructions per token: one workgroup selecting
// for the whole batch is bound by one CU's issue rate, so it stays spread over CUs.)
template <bool KTAIL>
__global__ __launch_bounds__(256) void route_part_kernel(RouteParams p,
                                                         const uint16_t* __restrict__ x,
                                                         const uint16_t* __restrict__ wr,
                                                         float* __restrict__ part) {
  __shared__ float red[4][16][17];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * kRouteTok;
  const int e0 = blockIdx.y * 16;
  const int quarter = blockIdx.z;
  const int m = lane & 15;
  const int g = lane >> 4;
  const bool row_ok = (t0 + m) < p.T;
  const bool col_ok = (e0 + m) < p.E;
  const uint16_t* xrow = x + (size_t)(row_ok ? t0 + m : 0) * p.d;
  const uint16_t* wrow = wr + (size_t)(col_ok ? e0 + m : 0) * p.d;
  const int nsteps = KTAIL ? (p.d + 31) >> 5 : p.d >> 5;
  auto load = [&](const uint16_t* r, bool ok, int kk) -> uint4 {
    return (ok && (!KTAIL || kk < p.d)) ? *reinterpret_cast<const uint4*>(r + kk)
                                        : make_uint4(0, 0, 0, 0);
  };
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  int st = 4 * quarter + wave;
  for (; st + 3 * kRouteWaves < nsteps; st += 4 * kRouteWaves) {
    uint4 av[4], bv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int kk = (st + kRouteWaves * u) * 32 + g * 8;
      av[u] = load(xrow, row_ok, kk);
      bv[u] = load(wrow, col_ok, kk);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[u]),
                                                    __builtin_bit_cast(bf16x8, bv[u]), acc, 0,
                                                    0, 0);
  }
  for (; st < nsteps; st += kRouteWaves) {
    const int kk = st * 32 + g * 8;
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
        __builtin_bit_cast(bf16x8, load(xrow, row_ok, kk)),
        __builtin_bit_cast(bf16x8, load(wrow, col_ok, kk)), acc, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) red[wave][4 * g + i][m] = acc[i];
  __syncthreads();
  const int r = threadIdx.x >> 4, c = threadIdx.x & 15;
  if (t0 + r < p.T && e0 + c < p.E)
    part[((size_t)quarter * p.T + t0 + r) * p.E + e0 + c] =
        sum4(red[0][r][c], red[1][r][c], red[2][r][c], red[3][r][c]);
}

// One wave per token (lane = expert): the sum of the four quarters of each logit in order,
// the logit bias, then scores and selection as in the kernels above.
__global__ __launch_bounds__(256) void route_select_part_kernel(RouteParams p,
                                                                const float* __restrict__ part,
                                                                const float* __restrict__ bias,
                                                                float* scores, int32_t* idx,
                                                                float* wout) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= p.T) return;  // whole wave
  const bool valid = lane < p.E;
  float l = 0.0f;
  if (valid) {
    const size_t o = (size_t)t * p.E + lane, n = (size_t)p.T * p.E;
    l = sum4(part[o], part[o + n], part[o + 2 * n], part[o + 3 * n]);
    if (bias != nullptr) l += bias[lane];
  }
  score_select_write(l, valid, lane, p, t, scores, idx, wout);
}


// fp32 router: one wave per token, lane = expert, plain fp32 FMA over the dim.  Pre-norm:
// the wave first computes the token's 1/rms and writes the normalised row, and every lane
// recomputes the normalised values it multiplies with the same expression.
template <bool NORM>
__global__ __launch_bounds__(256) void route_f32_kernel(RouteParams p, const float* __restrict__ x,
                                                        const float* __restrict__ wr,
                                                        const float* __restrict__ bias,
                                                        float* scores, int32_t* idx,
                                                        float* wout) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= p.T) return;  // whole wave
  const bool valid = lane < p.E;
  const float* xr = x + (size_t)t * p.d;
  const float* wrow = wr + (size_t)(valid ? lane : 0) * p.d;
  float r = 1.0f;
  if (NORM) {
    float ss = 0.0f;
    for (int c = lane; c < p.d; c += 64) ss = fmaf(xr[c], xr[c], ss);
    r = inv_rms(wave_sum_f(ss), p.d, p.norm_eps);
    float* xo = static_cast<float*>(p.x_norm) + (size_t)t * p.d;
    for (int c = lane; c < p.d; c += 64) xo[c] = (xr[c] * r) * p.norm_gamma[c];
  }
  float l = 0.0f;
  if (valid) {
    for (int c = 0; c < p.d; ++c) l = fmaf(NORM ? (xr[c] * r) * p.norm_gamma[c] : xr[c], wrow[c], l);
    if (bias != nullptr) l += bias[lane];
  }
  score_select_write(l, valid, lane, p, t, scores, idx, wout);
}

__global__ __launch_bounds__(256) void select_kernel(RouteParams p, const float* __restrict__ scores,
                                                     const float* __restrict__ keys,
                                                     int32_t* idx, float* wout) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= p.T) return;
  const bool valid = lane < p.E;
  const float s = valid ? scores[(size_t)t * p.E + lane] : 0.0f;
  const float key = (keys == nullptr) ? s : (valid ? keys[(size_t)t * p.E + lane] : 0.0f);
  select_write(s, key, valid, lane, p, t, idx, wout);
}

}  // namespace

hipError_t launch_route(const RouteParams& p, int act_dtype, const void* x, const void* router,
                        const float* bias, float* scores, int32_t* idx, float* w,
                        hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  const bool norm = p.norm_gamma != nullptr;
  if (act_dtype == MOE_BF16) {
    dim3 grid((p.T + kRouteTok - 1) / kRouteTok);
    const int nm = !norm ? 0 : (p.d <= kNormLdsDim ? 1 : 2);
    auto kern = (p.d & 31) == 0
                    ? (nm == 0 ? route_bf16_kernel<0, false>
                               : nm == 1 ? route_bf16_kernel<1, false> : route_bf16_kernel<2, false>)
                    : (nm == 0 ? route_bf16_kernel<0, true>
                               : nm == 1 ? route_bf16_kernel<1, true> : route_bf16_kernel<2, true>);
    hipLaunchKernelGGL(kern, grid, dim3(64 * kRouteWaves), 0, s, p,
                       static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(router),
                       bias, scores, idx, w);
  } else {
    dim3 grid((p.T + 3) / 4);
    auto kern = norm ? route_f32_kernel<true> : route_f32_kernel<false>;
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, p, static_cast<const float*>(x),
                       static_cast<const float*>(router), bias, scores, idx, w);
  }
  return hipGetLastError();
}

bool split_route_applies(const RouteParams& p, int act_dtype) {
  return act_dtype == MOE_BF16 && p.norm_gamma == nullptr && p.T <= kSplitRouteTokens;
}

size_t split_route_part_bytes(int T, int E) { return (size_t)4 * T * E * sizeof(float); }

hipError_t launch_route_split(const RouteParams& p, const void* x, const void* router,
                              const float* bias, float* part, float* scores, int32_t* idx,
                              float* w, hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  dim3 grid((p.T + kRouteTok - 1) / kRouteTok, (p.E + 15) / 16, 4);
  auto kern = (p.d & 31) == 0 ? route_part_kernel<false> : route_part_kernel<true>;
  hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, p, static_cast<const uint16_t*>(x),
                     static_cast<const uint16_t*>(router), part);
  hipLaunchKernelGGL(route_select_part_kernel, dim3((p.T + 3) / 4), dim3(256), 0, s, p, part,
                     bias, scores, idx, w);
  return hipGetLastError();
}

hipError_t launch_select(const RouteParams& p, const float* scores, const float* keys,
                         int32_t* idx, float* w, hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  dim3 grid((p.T + 3) / 4);
  hipLaunchKernelGGL(select_kernel, grid, dim3(256), 0, s, p, scores, keys, idx, w);
  return hipGetLastError();
}

}  // namespace moe
