// Backward pass of the MoE layer: the kernels besides the grouped GEMMs.
//
// The layer's gradients follow the chain rule through the forward ("大模型工程（一）：Transformer
// 到 MoE": the MoEBlock listing and section "MoE 数学：路由、容量与平衡详解" for the routing,
// section "变了什么，为什么变" item 3 for SwiGLU; section "常见陷阱" item 4: the router
// gradient goes through the logits themselves).  The data gradients (dh = dy W2, dx =
// da W1 + db W3) run on the forward's grouped-GEMM kernel with transposed weight copies;
// the kernels here are the transposes, the routing-weight and router gradients, the final
// combine of dx, and the weight-gradient GEMMs, whose contraction runs over the tokens of
// each expert (K differs per expert).
//
// Layouts: activations bf16 and token-major ([rows][features]), as the forward leaves them
// (the weight gradients read them in place, transposing in LDS); weight gradients fp32 in
// the weights' [out, in] layout.
#include "backward.h"
#include "common.h"

namespace moe {

namespace {

constexpr int kT = 64;   // transpose tile

// out[b * obs + c * ld + r] = in[b * R * C + r * C + c] for r < R, c < C (both multiples of
// 64): 64 x 64 tiles through LDS, 16-byte loads and stores.
__global__ __launch_bounds__(256) void transpose_mat_kernel(const uint16_t* __restrict__ in,
                                                            uint16_t* __restrict__ out, int R,
                                                            int C, long long obs, int ld) {
  __shared__ uint16_t t[kT][kT + 8];
  const int tiles_c = C / kT;
  const int r0 = (blockIdx.x / tiles_c) * kT, c0 = (blockIdx.x % tiles_c) * kT;
  const uint16_t* src = in + (size_t)blockIdx.y * R * C;
  uint16_t* dst = out + (size_t)blockIdx.y * obs;
  const int tid = threadIdx.x;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = h * 32 + tid / 8, c = (tid % 8) * 8;
    const uint4 v = *reinterpret_cast<const uint4*>(src + (size_t)(r0 + r) * C + c0 + c);
    *reinterpret_cast<uint4*>(&t[r][c]) = v;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = h * 32 + tid / 8, r = (tid % 8) * 8;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (uint32_t)t[r + 2 * i][c] | ((uint32_t)t[r + 2 * i + 1][c] << 16);
    *reinterpret_cast<uint4*>(dst + (size_t)(c0 + c) * ld + r0 + r) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// out[p] = scale(p) * in[index[p]] for p < *valid_rows (bf16 rows of C columns; scale in
// fp32, one rounding): a permuted, optionally weighted copy of token rows.  The grid covers
// the largest row count; the device-side count bounds it, because index is only written up
// to there (a capacity drops slots, and the permutation then has fewer rows).  One workgroup
// per row.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint16_t* __restrict__ in,
                                                          const int32_t* __restrict__ index,
                                                          const float* __restrict__ scale,
                                                          const int32_t* __restrict__ valid_rows,
                                                          int C, uint16_t* __restrict__ out) {
  const int p = blockIdx.x;
  if (p >= *valid_rows) return;   // uniform: past the permuted rows
  const uint16_t* src = in + (size_t)index[p] * C;
  const float s = scale != nullptr ? scale[p] : 1.0f;
  for (int c = threadIdx.x * 8; c < C; c += 256 * 8) {
    uint4 v = *reinterpret_cast<const uint4*>(src + c);
    if (scale != nullptr) {
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[i] = pack_bf16x2(s * bf16_bits_to_f32(w[i] & 0xffffu), s * bf16_bits_to_f32(w[i] >> 16));
      v = make_uint4(o[0], o[1], o[2], o[3]);
    }
    *reinterpret_cast<uint4*>(out + (size_t)p * C + c) = v;
  }
}

// Gradient of each routing weight: dw[t, j] = dout[t] . y_hat[p], with y_hat = y[p] / w[t, j]
// the expert's unweighted output (y is the forward's weighted output); 0 for dropped slots.
// A selected expert whose weight is exactly 0 (its score underflowed to 0) gets dw = 0:
// y_hat is then unknown, but dw only reaches the logits multiplied by that score (and the
// score's own gradient by s (1 - s) or the softmax Jacobian, both 0 at s = 0), so 0 is exact.
// One wave per slot, fixed-order sum.
__global__ __launch_bounds__(256) void routing_weight_grad_kernel(
    int Tk, int k, int d, const uint16_t* __restrict__ dout, const uint16_t* __restrict__ y,
    const int32_t* __restrict__ slot_pos, const float* __restrict__ topk_w, float* __restrict__ dw) {
  const int q = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (q >= Tk) return;   // whole wave
  const int p = slot_pos[q];
  if (p < 0) {
    if (lane == 0) dw[q] = 0.0f;
    return;
  }
  const uint16_t* g = dout + (size_t)(q / k) * d;
  const uint16_t* yr = y + (size_t)p * d;
  float acc = 0.0f;
  for (int c = lane * 8; c < d; c += 64 * 8) {
    const uint4 a = *reinterpret_cast<const uint4*>(g + c);
    const uint4 b = *reinterpret_cast<const uint4*>(yr + c);
    const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = fmaf(bf16_bits_to_f32(wa[i] & 0xffffu), bf16_bits_to_f32(wb[i] & 0xffffu), acc);
      acc = fmaf(bf16_bits_to_f32(wa[i] >> 16), bf16_bits_to_f32(wb[i] >> 16), acc);
    }
  }
  acc = wave_sum_f(acc);
  if (lane == 0) {
    const float wq = topk_w[q];
    dw[q] = wq != 0.0f ? acc / wq : 0.0f;
  }
}

// Logit gradients of one token per wave (lane = expert): the routing weights w_j = c s_j /
// sum_i s_i over the selected experts (or c s_j) are differentiated with respect to every
// score, then through sigmoid, or through softmax over all E logits.
__global__ __launch_bounds__(256) void router_grad_kernel(RouteParams p, const float* __restrict__ scores,
                                                          const int32_t* __restrict__ idx,
                                                          const float* __restrict__ dw,
                                                          float* __restrict__ dl) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= p.T) return;   // whole wave
  const bool valid = lane < p.E;
  const float s = valid ? scores[(size_t)t * p.E + lane] : 0.0f;
  float tot = 0.0f, wsum = 0.0f;
  for (int j = 0; j < p.k; ++j) {
    const int e = idx[(size_t)t * p.k + j];
    const float se = __shfl(s, e, 64);
    tot += se;
    wsum += dw[(size_t)t * p.k + j] * se;
  }
  float ds = 0.0f;
  for (int j = 0; j < p.k; ++j) {
    if (idx[(size_t)t * p.k + j] != lane) continue;
    const float g = dw[(size_t)t * p.k + j];
    ds += p.renormalize ? (p.route_scale / tot) * (g - wsum / tot) : p.route_scale * g;
  }
  float g;
  if (p.score_fn == MOE_SCORE_SIGMOID) {
    g = ds * s * (1.0f - s);
  } else {
    const float dot = wave_sum_f(valid ? ds * s : 0.0f);
    g = s * (ds - dot);
  }
  if (valid) dl[(size_t)t * p.E + lane] = g;
}

// Router weight and logit-bias gradients, in two passes with a fixed summation order:
// partials over chunks of 256 tokens, then their sum.  Block (64-column block of d, chunk);
// thread: 4 experts x 4 columns.
constexpr int kRgChunk = 256;

__global__ __launch_bounds__(256) void router_wgrad_partial_kernel(
    int T, int d, int E, const uint16_t* __restrict__ x, const float* __restrict__ dl,
    float* __restrict__ part, float* __restrict__ part_bias) {
  // the chunk is walked in sub-chunks of 64 tokens staged in LDS (dl rows padded to 64
  // experts with zeros, x as 64 columns)
  __shared__ __align__(16) float s_dl[64][64];
  __shared__ __align__(16) uint16_t s_x[64][64];
  const int c0 = blockIdx.x * 64, chunk = blockIdx.y;
  const int tid = threadIdx.x;
  const int eg = tid / 16, cg = tid % 16;
  const int t0 = chunk * kRgChunk, t1 = min(T, t0 + kRgChunk);
  float acc[4][4] = {};
  float accb[4] = {};
  for (int ts = t0; ts < t1; ts += 64) {
    for (int i = tid; i < 64 * 64; i += 256) {
      const int tl = i / 64, e = i % 64;
      s_dl[tl][e] = (ts + tl < t1 && e < E) ? dl[(size_t)(ts + tl) * E + e] : 0.0f;
    }
    for (int i = tid; i < 64 * 8; i += 256) {
      const int tl = i / 8, c = (i % 8) * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (ts + tl < t1) v = *reinterpret_cast<const uint4*>(x + (size_t)(ts + tl) * d + c0 + c);
      *reinterpret_cast<uint4*>(&s_x[tl][c]) = v;
    }
    __syncthreads();
    for (int tl = 0; tl < 64; ++tl) {
      const float4 g4 = *reinterpret_cast<const float4*>(&s_dl[tl][eg * 4]);
      const uint2 xv = *reinterpret_cast<const uint2*>(&s_x[tl][cg * 4]);
      const float g[4] = {g4.x, g4.y, g4.z, g4.w};
      const float xf[4] = {bf16_bits_to_f32(xv.x & 0xffffu), bf16_bits_to_f32(xv.x >> 16),
                           bf16_bits_to_f32(xv.y & 0xffffu), bf16_bits_to_f32(xv.y >> 16)};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        accb[i] += g[i];
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(g[i], xf[j], acc[i][j]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = eg * 4 + i;
    if (e >= E) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) part[((size_t)chunk * E + e) * d + c0 + cg * 4 + j] = acc[i][j];
    if (blockIdx.x == 0 && cg == 0) part_bias[(size_t)chunk * E + e] = accb[i];
  }
}

__global__ __launch_bounds__(256) void router_wgrad_reduce_kernel(
    int nchunks, int n, const float* __restrict__ part, float* __restrict__ out) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.0f;
  for (int c = 0; c < nchunks; ++c) s += part[(size_t)c * n + i];
  out[i] = s;
}

// dx[t] = sum_e dl[t, e] W_r[e] + sum_j dx_perm[slot_pos[t, j]] + dx_shared[t] (+ dout[t]),
// fp32 in that order, rounded to bf16.  Block: 16 tokens x 256 columns; thread: 16 columns
// of one token.
__global__ __launch_bounds__(256) void dx_combine_kernel(
    int T, int d, int E, int k, const float* __restrict__ dl, const uint16_t* __restrict__ wr,
    const uint16_t* __restrict__ dx_perm, const int32_t* __restrict__ slot_pos,
    const uint16_t* __restrict__ dx_shared, const uint16_t* __restrict__ residual,
    uint16_t* __restrict__ dx) {
  __shared__ float s_dl[16][64];
  __shared__ __align__(16) uint16_t s_wr[64][256];
  const int t0 = blockIdx.x * 16, c0 = blockIdx.y * 256;
  const int tid = threadIdx.x;
  for (int i = tid; i < 16 * 64; i += 256) {
    const int tl = i / 64, e = i % 64;
    s_dl[tl][e] = (t0 + tl < T && e < E) ? dl[(size_t)(t0 + tl) * E + e] : 0.0f;
  }
  for (int i = tid; i < 64 * 32; i += 256) {
    const int e = i / 32, c = (i % 32) * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (e < E && c0 + c < d) v = *reinterpret_cast<const uint4*>(wr + (size_t)e * d + c0 + c);
    *reinterpret_cast<uint4*>(&s_wr[e][c]) = v;
  }
  __syncthreads();
  const int tl = tid / 16, cl = (tid % 16) * 16;
  const int t = t0 + tl, c = c0 + cl;
  if (t >= T || c >= d) return;
  float acc[16] = {};
  for (int e = 0; e < E; ++e) {
    const float g = s_dl[tl][e];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = fmaf(g, bf16_bits_to_f32(s_wr[e][cl + i]), acc[i]);
  }
  auto add16 = [&](const uint16_t* src) {
    const uint4 a = *reinterpret_cast<const uint4*>(src), b = *reinterpret_cast<const uint4*>(src + 8);
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      acc[2 * i] += bf16_bits_to_f32(w[i] & 0xffffu);
      acc[2 * i + 1] += bf16_bits_to_f32(w[i] >> 16);
    }
  };
  for (int j = 0; j < k; ++j) {
    const int p = slot_pos[(size_t)t * k + j];
    if (p >= 0) add16(dx_perm + (size_t)p * d + c);
  }
  if (dx_shared != nullptr) add16(dx_shared + (size_t)t * d + c);
  if (residual != nullptr) add16(residual + (size_t)t * d + c);
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
  uint4* dst = reinterpret_cast<uint4*>(dx + (size_t)t * d + c);
  dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
  dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
}

// ------------------------------------------------------------------------------------
// Weight-gradient GEMM with the contraction over each segment's tokens, on token-major data:
//   out(seg, m, n) = sum over rows p of the segment of A(p, m) B(p, n),
//   A(p, m) = a[p * lda + a_col + m], B(p, n) = b[p * ldb + b_col + n]     (bf16 in, fp32 out)
// out(seg, m, n) is stored at out + seg * M * N + (n / nsplit) * M * nsplit + m * nsplit +
// n % nsplit (nsplit = N: the plain [M][N] layout; a smaller nsplit stores column blocks of
// nsplit columns as consecutive [M][nsplit] matrices).
//
// One workgroup per BM x BN output tile (256 x 256 with 8 waves of 128 x 64, or 128 x 128
// with 4 waves of 64 x 64; MFMA 32x32x16), the segment's rows in slices of 64 through a
// two-stage LDS ring filled by global_load_lds_dwordx4, one barrier per slice.  A slice is
// stored as it arrives, [64 rows][BM columns] and [64 rows][BN columns]; the MFMA operands,
// which need 8 consecutive rows (the contraction index) of one column per lane, are read with
// the transposing LDS load ds_read_b64_tr_b16.  Within a group of 16 lanes that load hands
// lane i element i % 4 of the 8-byte pieces addressed by lanes (i % 16) / 4 + 4 r, r = 0..3;
// so lane 16 g + j addresses row r = j / 4 of a 4-row block at column 4 (j % 4) of its
// 16-column group, and two loads (rows 0-3, 4-7) give each lane its 8 rows.  16-byte chunks
// are XOR-swizzled by 4 (row & 3), which puts the four rows read together in different bank
// windows.  Rows past the segment's end and columns past M or N read a zero row.

constexpr int kWgBK = 64;
__device__ const uint16_t kZeroRow[256] = {};   // source of rows and columns out of range

typedef short v4s __attribute__((ext_vector_type(4)));

template <int BM, int BN, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void wgrad_kernel(WgradParams p) {
  constexpr int WN = WAVES / 2, WTM = BM / 2, WTN = BN / WN, FM = WTM / 32, FN = WTN / 32;
  constexpr int AROW = BM * 2, BROW = BN * 2;          // bytes per LDS row
  constexpr int A_BYTES = kWgBK * AROW, ST_BYTES = A_BYTES + kWgBK * BROW;
  constexpr int NDMA = ST_BYTES / 1024 / WAVES;        // 1 KB DMAs per wave per slice
  static_assert(ST_BYTES % (1024 * WAVES) == 0 && A_BYTES % 1024 == 0, "DMA split");
  static_assert(BM >= 128 && BN >= 128 && BM <= 256 && BN <= 256, "swizzle and zero row");
  __shared__ __align__(1024) unsigned char lds[2 * ST_BYTES];
  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  const int seg = blockIdx.x / (tiles_m * tiles_n);
  const int rem = blockIdx.x % (tiles_m * tiles_n);
  const int m0 = (rem / tiles_n) * BM, n0 = (rem % tiles_n) * BN;
  const int r0 = p.offsets != nullptr ? p.offsets[seg] : 0;
  const int nrows = p.offsets != nullptr ? p.offsets[seg + 1] - r0 : p.rows;
  const int nk = (nrows + kWgBK - 1) / kWgBK;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const uint32_t lds_base = (uint32_t)(size_t)(__attribute__((address_space(3))) unsigned char*)lds;

  // DMA q of a slice covers 1 KB of LDS: A rows for q < A_BYTES / 1 KB, then B rows.  This
  // lane's slice row, operand and source column for each of its DMAs (the row moves with
  // the slice; the column is fixed).
  int drow[NDMA];
  bool dis_b[NDMA], dcol_ok[NDMA];
  const uint16_t* dbase[NDMA];
#pragma unroll
  for (int i = 0; i < NDMA; ++i) {
    const int q = wave * NDMA + i;
    const bool isb = q * 1024 >= A_BYTES;
    const int rowb = isb ? BROW : AROW;
    const int off = isb ? q * 1024 - A_BYTES : q * 1024;
    const int row = off / rowb + (lane * 16) / rowb;           // slice row 0..63
    const int pchunk = ((lane * 16) % rowb) / 16;               // physical 16-byte chunk
    const int col = (pchunk ^ ((row & 3) << 2)) * 8;            // logical column in the tile
    const int gcol = (isb ? n0 : m0) + col;
    drow[i] = row;
    dis_b[i] = isb;
    dcol_ok[i] = gcol < (isb ? p.N : p.M);
    dbase[i] = isb ? p.b + p.b_col + gcol : p.a + p.a_col + gcol;
  }
  auto issue = [&](int kt) {
    const uint32_t st = lds_base + (uint32_t)((kt & 1) * ST_BYTES);
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
      const int rr = kt * kWgBK + drow[i];
      const bool ok = rr < nrows && dcol_ok[i];
      const size_t ld = dis_b[i] ? (size_t)p.ldb : (size_t)p.lda;
      const uint16_t* src = ok ? dbase[i] + (size_t)(r0 + rr) * ld : kZeroRow;
      lds_dma16(st + (uint32_t)((wave * NDMA + i) * 1024), src);
    }
  };
  // transposing operand load: 8 rows (k) of column base + (lane % 32) in two halves
  const int g = lane >> 4, jj = lane & 15;
  const int trow = 8 * (g >> 1) + (jj >> 2);                   // + 4 h + 16 ks
  const int tcol = 16 * (g & 1) + 4 * (jj & 3);               // + fragment base column
  auto ld_tr = [&](const unsigned char* base, int rowb, int ks, int colbase) -> bf16x8 {
    v4s v[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = ks * 16 + 4 * h + trow;
      const int col = colbase + tcol;
      const int addr = row * rowb + ((((col >> 3) ^ ((row & 3) << 2)) << 4) | ((col & 7) << 1));
      v[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s*)(base + addr));
    }
    const v4s lo = v[0], hi = v[1];
    return __builtin_bit_cast(bf16x8, (short __attribute__((ext_vector_type(8)))){
        lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int a = 0; a < FM; ++a)
#pragma unroll
    for (int b = 0; b < FN; ++b) acc[a][b] = f32x16{};
  if (nk > 0) {
    issue(0);
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
    __syncthreads();
  }
  for (int kt = 0; kt < nk; ++kt) {
    // slice kt + 1 goes to the stage read in slice kt - 1 (all waves passed the barrier
    // that ended it) and lands while slice kt is multiplied
    if (kt + 1 < nk) issue(kt + 1);
    const unsigned char* As = lds + (kt & 1) * ST_BYTES;
    const unsigned char* Bs = As + A_BYTES;
    // operands of K-step ks + 1 are read while the MFMAs of step ks run
    bf16x8 af[2][FM], bf[2][FN];
    auto load = [&](int ks, bf16x8 (&a)[FM], bf16x8 (&b)[FN]) {
#pragma unroll
      for (int f = 0; f < FM; ++f) a[f] = ld_tr(As, AROW, ks, wm * WTM + f * 32);
#pragma unroll
      for (int f = 0; f < FN; ++f) b[f] = ld_tr(Bs, BROW, ks, wn * WTN + f * 32);
    };
    load(0, af[0], bf[0]);
#pragma unroll
    for (int ks = 0; ks < kWgBK / 16; ++ks) {
      if (ks + 1 < kWgBK / 16) load(ks + 1, af[(ks + 1) & 1], bf[(ks + 1) & 1]);
#pragma unroll
      for (int fa = 0; fa < FM; ++fa)
#pragma unroll
        for (int fb = 0; fb < FN; ++fb)
          acc[fa][fb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks & 1][fa], bf[ks & 1][fb], acc[fa][fb], 0, 0, 0);
      // instruction order for the scheduler: the transposing reads of step ks + 1 (two per
      // operand) spread over the MFMAs of step ks
      constexpr int NDS = 2 * (FM + FN), NMF = FM * FN;
      constexpr int DPM = NDS / NMF, R = NDS - DPM * NMF;   // the first R MFMAs take one more
      static_assert(DPM >= 1, "a read after every MFMA");
      if (ks + 1 < kWgBK / 16) {
#pragma unroll
        for (int i = 0; i < NMF; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (i < R) __builtin_amdgcn_sched_group_barrier(0x100, DPM + 1, 0);
          else __builtin_amdgcn_sched_group_barrier(0x100, DPM, 0);
        }
      } else {
        __builtin_amdgcn_sched_group_barrier(0x008, NMF, 0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));   // slice kt + 1 landed (own DMAs)
    __syncthreads();                                        // ... everyone's; stage kt free
  }
  // element i of lane l: row 8 (i / 4) + 4 (l / 32) + i % 4 of A's block, column l % 32 of B's
  float* out = p.out + (size_t)seg * p.M * p.N;
#pragma unroll
  for (int fa = 0; fa < FM; ++fa)
#pragma unroll
    for (int fb = 0; fb < FN; ++fb) {
      const int n = n0 + wn * WTN + fb * 32 + (lane & 31);
      if (n >= p.N) continue;
      float* col = out + (size_t)(n / p.nsplit) * p.M * p.nsplit + (n % p.nsplit);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = m0 + wm * WTM + fa * 32 + 8 * (i / 4) + 4 * (lane >> 5) + (i % 4);
        if (m < p.M) col[(size_t)m * p.nsplit] = acc[fa][fb][i];
      }
    }
}

}  // namespace

hipError_t launch_transpose_mat(const void* in, void* out, int batch, int R, int C, long long obs,
                                int ld, hipStream_t s) {
  if (batch == 0 || R == 0 || C == 0) return hipSuccess;
  dim3 grid((unsigned)((R / kT) * (C / kT)), (unsigned)batch);
  hipLaunchKernelGGL(transpose_mat_kernel, grid, dim3(256), 0, s,
                     static_cast<const uint16_t*>(in), static_cast<uint16_t*>(out), R, C, obs, ld);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* in, const int32_t* index, const float* scale,
                              const int32_t* valid_rows, int max_rows, int C, void* out,
                              hipStream_t s) {
  if (max_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)max_rows), dim3(256), 0, s,
                     static_cast<const uint16_t*>(in), index, scale, valid_rows, C,
                     static_cast<uint16_t*>(out));
  return hipGetLastError();
}

hipError_t launch_routing_weight_grad(int T, int k, int d, const void* dout, const void* y,
                                      const int32_t* slot_pos, const float* topk_w, float* dw,
                                      hipStream_t s) {
  const int Tk = T * k;
  if (Tk == 0) return hipSuccess;
  hipLaunchKernelGGL(routing_weight_grad_kernel, dim3((Tk + 3) / 4), dim3(256), 0, s, Tk, k, d,
                     static_cast<const uint16_t*>(dout), static_cast<const uint16_t*>(y), slot_pos,
                     topk_w, dw);
  return hipGetLastError();
}

hipError_t launch_router_grad(const RouteParams& p, const float* scores, const int32_t* idx,
                              const float* dw, float* dl, hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  hipLaunchKernelGGL(router_grad_kernel, dim3((p.T + 3) / 4), dim3(256), 0, s, p, scores, idx, dw, dl);
  return hipGetLastError();
}

size_t router_wgrad_ws_bytes(int T, int d, int E) {
  const size_t chunks = ((size_t)T + kRgChunk - 1) / kRgChunk;
  return chunks * (size_t)E * ((size_t)d + 1) * sizeof(float);
}

hipError_t launch_router_wgrad(int T, int d, int E, const void* x, const float* dl, float* d_router,
                               float* d_bias, void* ws, hipStream_t s) {
  const int chunks = (T + kRgChunk - 1) / kRgChunk;
  if (chunks == 0) return hipSuccess;
  float* part = static_cast<float*>(ws);
  float* part_bias = part + (size_t)chunks * E * d;
  hipLaunchKernelGGL(router_wgrad_partial_kernel, dim3((unsigned)(d / 64), (unsigned)chunks), dim3(256),
                     0, s, T, d, E, static_cast<const uint16_t*>(x), dl, part, part_bias);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (d_router != nullptr) {
    const int n = E * d;
    hipLaunchKernelGGL(router_wgrad_reduce_kernel, dim3((n + 255) / 256), dim3(256), 0, s, chunks, n,
                       part, d_router);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (d_bias != nullptr) {
    hipLaunchKernelGGL(router_wgrad_reduce_kernel, dim3((E + 255) / 256), dim3(256), 0, s, chunks, E,
                       part_bias, d_bias);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_dx_combine(int T, int d, int E, int k, const float* dl, const void* wr,
                             const void* dx_perm, const int32_t* slot_pos, const void* dx_shared,
                             const void* residual, void* dx, hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 grid((unsigned)((T + 15) / 16), (unsigned)((d + 255) / 256));
  hipLaunchKernelGGL(dx_combine_kernel, grid, dim3(256), 0, s, T, d, E, k, dl,
                     static_cast<const uint16_t*>(wr), static_cast<const uint16_t*>(dx_perm),
                     slot_pos, static_cast<const uint16_t*>(dx_shared),
                     static_cast<const uint16_t*>(residual), static_cast<uint16_t*>(dx));
  return hipGetLastError();
}

hipError_t launch_wgrad(const WgradParams& p, int nseg, int num_cus, hipStream_t s) {
  auto tiles = [&](int bm, int bn) {
    return (long long)nseg * ((p.M + bm - 1) / bm) * ((p.N + bn - 1) / bn);
  };
  // 256 x 256 tiles (less LDS traffic per MFMA) unless they would leave most CUs idle
  const long long wide = tiles(256, 256);
  if (wide == 0) return hipSuccess;
  if (2 * wide >= num_cus)
    hipLaunchKernelGGL((wgrad_kernel<256, 256, 8>), dim3((unsigned)wide), dim3(8 * 64), 0, s, p);
  else
    hipLaunchKernelGGL((wgrad_kernel<128, 128, 4>), dim3((unsigned)tiles(128, 128)), dim3(4 * 64), 0, s, p);
  return hipGetLastError();
}

}  // namespace moe
