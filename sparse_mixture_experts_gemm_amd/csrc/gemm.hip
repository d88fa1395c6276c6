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
// gfx950 mapping (bf16 / e4m3 weights): one persistent workgroup of 8 waves per CU walks a
// list of BM x BN output tiles; the waves form a 2 x 4 grid over the tile and issue
// v_mfma_f32_32x32x16_bf16 on 32 x 32 sub-tiles.  A and B K-slices (BK = 64) stream into a
// ring of LDS stages through direct global->LDS loads; the 16-byte chunks of every 128-byte
// LDS row are XOR-swizzled so that MFMA operand reads are free of bank conflicts.  The
// weights are the MFMA's first operand and the token rows its second, and the weight rows
// of each 32-row block are staged in a fixed permutation, so that every lane ends with 16
// consecutive output features of one token and writes them with two 16-byte stores.  For
// SwiGLU the B tile interleaves gate and up rows per 32-row MFMA block, so the gate and up
// results of an output element land in the same lane and the activation runs in
// registers.  e4m3 weights are staged as bytes and widened to bf16 (exactly) when read from
// LDS; their per-channel scales multiply the fp32 accumulator.  Tiles are walked in
// XCD-contiguous order: workgroup b runs on XCD b % 8, and each XCD takes a contiguous range
// of (expert, n-tile, m-tile) tiles so that tiles sharing an expert's weights share that
// XCD's L2; the slot-to-tile map rotates by one per step, so that every workgroup alternates
// an expert's full and padded m-tiles and the two stay in step over the same weights.  A
// tile's K-loop is compiled once per count of the wave's 32-row blocks that hold rows of the
// segment, so the padded rows of an expert's last m-tile cost neither LDS reads nor MFMAs.
// Every DMA reads from a base address that is the same over the wave (scalar registers)
// plus a 32-bit offset per lane, which keeps the address registers few.  The
// K-slices of a workgroup's consecutive tiles form one stream, so the loads of the next
// tile are in flight while the current tile's epilogue runs.  Within a slice, scheduling
// directives place the LDS reads of the next K-step between the MFMAs of the current one.
#include "common.h"
#include "gemm_core.h"
#include "internal.h"

#include <type_traits>

namespace moe {

namespace {


// ------------------------------------------------------------------------------------
// bf16 activations, bf16 or e4m3 weights, MFMA 32x32x16.
//
// Workgroup tile BM x BN (B = weight rows), WAVES waves in a 2 x (WAVES/2) layout, wave
// tile WTM x WTN = FM x FN MFMA blocks of 32 x 32.  K advances in slices of BK = 64 through
// an NSTAGE-deep LDS ring filled by global_load_lds_dwordx4 (global -> LDS without VGPR
// staging): one instruction writes 1 KB of LDS, 16 bytes per lane at M0 + 16 * lane.  The
// slices of all the tiles a workgroup owns form one sequence; slice g + NSTAGE - 1 is
// requested while slice g is multiplied, and a partial vmcnt wait (loads retire in order)
// lets the younger slices stay in flight across the barrier.
//
// LDS layout: a bf16 operand row holds 64 K values in 8 chunks of 16 bytes; chunk c of row
// r sits at position c ^ swz(r), swz(r) = (r & 7) ^ ((r >> 3) & 1), so the 8 or 16 lanes
// that the LDS serves per cycle in an MFMA operand read (32 consecutive rows, one chunk)
// hit distinct banks.  Each DMA lane therefore fetches the logical chunk that belongs at
// its physical position.  e4m3 B slices are stored raw (64 bytes per row, 16-byte chunks
// swizzled by (r >> 1) & 3) and widened to bf16 with v_cvt_scalef32_pk_bf16_fp8 (scale 1,
// exact) when the operand is read.
//
// Output layout: D = W_blk * A_blk^T per 32 x 32 block, so element i of lane l is token
// (column) l % 32 and MFMA row 8 * (i / 4) + 4 * (l / 32) + i % 4.  LDS row r of a 32-row
// weight block holds weight row perm32(r) of the block, which makes that element feature
// 16 * (l / 32) + i: a lane's 16 values are consecutive features of one token.

// Tile shapes: 256 x 256 when the problem gives every CU at least two such tiles, else
// 128 x 256.  Eight waves (two per SIMD) per workgroup, so one wave's LDS and barrier waits
// are covered by its partner's MFMAs.
template <int BM, int BN, int WAVES, int NSTAGE, int OCC, int STAGE, int ACT, bool FP8,
          bool A8 = false, bool BWD = false, bool TRB = false, bool KBLK = true>
__global__ __launch_bounds__(WAVES * 64, OCC) void gg_mfma_kernel(GemmParams p) {
  constexpr int NTHR = WAVES * 64;
  // K values per slice: 64 (128-byte bf16 rows), or 128 e4m3 bytes with e4m3 activations
  constexpr int BK = A8 ? 128 : 64;
  constexpr int WM = 2, WN = WAVES / 2;
  constexpr int WTM = BM / WM, WTN = BN / WN, FM = WTM / 32, FN = WTN / 32;
  constexpr bool SWIGLU = (STAGE == 0) && (ACT == MOE_ACT_SWIGLU);
  // A8: e4m3 activations and weights, v_mfma_scale_f32_32x32x64_f8f6f4 (unit scales) on
  // 128-byte LDS rows (two 64-K MFMA steps per slice, the chunks swizzled as for bf16);
  // in each step every lane reads 32 bytes of a row as two 16-byte chunks
  static_assert(!A8 || (FP8 && STAGE == 0), "e4m3 activations: up projection, e4m3 weights");
  // BWD: the UP stage recomputed in the backward pass; the epilogue turns dh into the
  // gradients of the two pre-activations instead of applying the activation
  static_assert(!BWD || (STAGE == 0 && !FP8 && !A8), "backward epilogue: bf16 up projection");
  // TRB: bf16 weights stored [K][N] (the transpose of the usual layout).  A B slice is staged
  // as it lies in memory, [BK rows k][BN columns n] (16-byte chunks XOR-swizzled by
  // 4 (k & 3)), and the MFMA operand, 8 consecutive k of one weight row n per lane, is read
  // with the transposing load ds_read_b64_tr_b16: within a group of 16 lanes it gives lane i
  // element i % 4 of the 8-byte pieces addressed by lanes (i % 16) / 4 + 4 r, so lane 16 g +
  // j addresses row j / 4 of a 4-row block at a column chosen per lane quad; the columns
  // reproduce the perm32 order of the usual staging, so the epilogue is unchanged.
  static_assert(!TRB || (STAGE == 1 && !FP8 && !A8 && BN == 256), "transposed weights: bf16 DOWN");
  constexpr int ESZ_A = A8 ? 1 : 2;                 // bytes per A element
  constexpr int AROW = BK * ESZ_A;                  // bytes per A row in LDS
  constexpr int CPR_A = AROW / 16;                  // 16-byte chunks per A row
  constexpr int BROW = FP8 ? BK : BK * 2;           // bytes per B row in LDS
  constexpr int A_BYTES = BM * AROW, B_BYTES = BN * BROW, ST_BYTES = A_BYTES + B_BYTES;
  constexpr int A_DMA = A_BYTES / 1024, B_DMA = B_BYTES / 1024;   // 1 KB per DMA instruction
  constexpr int NDMA = (A_DMA + B_DMA) / WAVES;                    // per wave per slice
  constexpr int B_RPD = 1024 / BROW;                                // B rows per DMA
  static_assert((A_DMA + B_DMA) % WAVES == 0, "DMA split");
  static_assert(!SWIGLU || FN % 2 == 0, "SwiGLU pairs gate/up MFMA tiles");
  static_assert(NSTAGE >= 2 && NSTAGE <= 4, "ring depth");
  auto swz_a = [](int r) { return swz8(r); };                        // A rows (128 bytes)
  auto swz_b8 = [](int r) { return swz4(r); };                       // 64-byte e4m3 B rows
  static_assert(NDMA * (NSTAGE - 2) < 64, "vmcnt range");
  static_assert(BM <= NTHR, "one thread per tile row when per-row data is staged");
  // forward bf16-activation tiles: per-tile copies of the K-loop for 0 .. FM live row blocks
  // (with e4m3 weights, up projection only, and only for none, half or all of them: more
  // copies spill registers, and the down projections measured no gain)
  constexpr bool SPEC = !A8 && !BWD && !TRB && (!FP8 || STAGE == 0);
  static_assert(!SPEC || FM == 2 || FM == 4, "row-block specialisation");

  __shared__ __align__(1024) unsigned char lds[NSTAGE * ST_BYTES];
  __shared__ int s_tile0[65], s_row0[64], s_rows[64];
  __shared__ int s_arow[2][BM];     // gathered A rows of upcoming tiles, by tile parity
  __shared__ float s_rw[3][BM];     // row weights of upcoming tiles, by tile index mod 3

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int N = p.N, K = p.K;
  const int hcols_per_tile = SWIGLU ? BN / 2 : BN;
  const int NT = (N + hcols_per_tile - 1) / hcols_per_tile;

  build_schedule(p, BM, NT, s_tile0, s_row0, s_rows);
  __syncthreads();
  const int total = s_tile0[p.nseg];

  // this workgroup's tiles inside its XCD's range [lo, hi): at step j the XCD's per_x
  // workgroups take the j-th block of per_x consecutive tiles, slot s the tile
  // (s + j) mod per_x of the block.  The rotation mixes the tiles of different cost: an
  // expert's m-tiles alternate in the tile order (full, then part padding), so a fixed
  // slot would see only one kind with an even per_x.
  const int nwg = gridDim.x;
  const int xcd = blockIdx.x % kNumXcd;
  const int slot = blockIdx.x / kNumXcd;
  const int per_x = (nwg - xcd + kNumXcd - 1) / kNumXcd;
  const int lo = (int)(((long long)xcd * total) / kNumXcd);
  const int hi = (int)(((long long)(xcd + 1) * total) / kNumXcd);
  const int full = (hi - lo) / per_x, rem = (hi - lo) % per_x;
  const int ntiles = full + ((slot + full) % per_x < rem ? 1 : 0);
  if (ntiles == 0) return;   // uniform over the workgroup
  const int nk = K / BK;
  const int nslices = ntiles * nk;

  const unsigned char* a_base = static_cast<const unsigned char*>(p.a);
  const bool gather = p.row_index != nullptr;
  // per-row factor staged with the tile: the routing weight (DOWN) or, for e4m3
  // activations, the scale of the A row (UP; indexed like A, through row_index)
  const bool has_rw = (STAGE == 1 || A8) && p.row_weight != nullptr;
  // Per-row data (gathered A rows, row weights) is staged in LDS by the epilogue two tiles
  // before its use, which needs a tile's slices to span at least NSTAGE - 1 steps; global
  // loads issued in the main loop would make the compiler's waits drain the DMA stream.
  const bool prefetch = (gather || has_rw) && nk >= NSTAGE - 1;
  const int nblk_k = K / p.kblock;
  const uint32_t lds_base = (uint32_t)(size_t)(__attribute__((address_space(3))) unsigned char*)lds;
  const int sw = swz_a(lane & 31);     // swizzle of every A operand row this lane reads

  auto tile_at = [&](int j) {
    return decode_tile(lo + j * per_x + (slot + j) % per_x, p.nseg, BM, NT, s_tile0, s_row0, s_rows);
  };
  // row of the segment's row space that A row r of a tile reads (clamped into the segment;
  // the results of clamped rows are never stored)
  auto seg_row = [&](const TileCoord& tc, int r) {
    int rr = tc.m_tile * BM + r;
    rr = rr < tc.rows ? rr : tc.rows - 1;
    return tc.row0 + rr;
  };

  if (prefetch) {
    for (int j = 0; j < 2 && j < ntiles; ++j) {
      const TileCoord tc = tile_at(j);
      if (tid < BM) {
        const int sr = seg_row(tc, tid);
        if (gather) s_arow[j][tid] = p.row_index[sr];
        if (has_rw) s_rw[j][tid] = p.row_weight[A8 && gather ? p.row_index[sr] : sr];
      }
    }
    __syncthreads();
  }

  // ---- sources of every DMA this lane takes part in, for the tile being loaded
  // (a base address that is the same for the whole wave, held in scalar registers, and this
  // lane's 32-bit byte offset from it: an activation matrix and one segment's weights stay
  // below 4 GB)
  const unsigned char* sbase[NDMA];
  uint32_t soff[NDMA];
  bool is_b[NDMA];
#pragma unroll
  for (int i = 0; i < NDMA; ++i) is_b[i] = wave * NDMA + i >= A_DMA;
  int src_seg = 0;   // segment of the tile being loaded (TRB: offset of the second matrix)
  constexpr int ESZ_B = FP8 ? 1 : 2;

  auto set_sources = [&](int j) __attribute__((always_inline)) {
    const TileCoord tc = tile_at(j);
    if (gather && !prefetch) {
      // short K: the rows of tile j are gathered here, at the cost of draining the loads
      // in flight (buffer j & 1 was last read two tiles ago, before several barriers)
      if (tid < BM) s_arow[j & 1][tid] = p.row_index[seg_row(tc, tid)];
      __syncthreads();
    }
    src_seg = __builtin_amdgcn_readfirstlane(tc.seg);
    const size_t seg_off = (size_t)src_seg * N * K;   // weight elements per segment
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
      const int q = wave * NDMA + i;
      if (TRB && is_b[i]) {
        // two k rows of BN columns per DMA; lane -> (row, physical chunk)
        const int qb = q - A_DMA;
        const int kr = qb * 2 + lane / 32;
        const int lc = (lane % 32) ^ ((kr & 3) << 2);                    // logical chunk
        int n = tc.n_tile * BN + lc * 8;
        n = n < N ? n : 0;
        // byte offset inside a 64-row block of the [K][N] matrix; the block's base
        // (first or second matrix) is chosen per slice
        sbase[i] = nullptr;
        soff[i] = (uint32_t)(((size_t)kr * N + n) * 2);
      } else if (!is_b[i]) {
        const int row = q * (1024 / AROW) + lane / CPR_A;
        const int srow = gather ? s_arow[j & 1][row] : seg_row(tc, row);
        sbase[i] = a_base;
        soff[i] = (uint32_t)((size_t)srow * K * ESZ_A + (size_t)(((lane % CPR_A) ^ swz_a(row)) * 16));
      } else {
        const int qb = q - A_DMA;
        const int n = (FP8 && !A8) ? qb * B_RPD + lane / 4 : qb * B_RPD + lane / 8;   // LDS row
        const int nl = (n & ~31) | perm32(n & 31);                           // weight row
        int wrow;
        const void* wb;
        if (STAGE == 0) {
          if (SWIGLU) {
            const int wc = nl / WTN, r = nl % WTN;
            const int half = r / (WTN / 2);
            wrow = tc.n_tile * (BN / 2) + wc * (WTN / 2) + (r % (WTN / 2));
            wb = half ? p.w_up : p.w_gate;
          } else {
            wrow = tc.n_tile * BN + nl;
            wb = p.w_gate;
          }
        } else {
          wrow = tc.n_tile * BN + nl;
          wb = p.w_down;
        }
        wrow = wrow < N ? wrow : 0;
        // the rows of one DMA lie in one 32-row block, so all its lanes read one matrix
        sbase[i] = uniform_ptr(static_cast<const unsigned char*>(wb) + seg_off * ESZ_B);
        soff[i] = (uint32_t)((size_t)wrow * p.kblock * ESZ_B +
                             (FP8 && !A8 ? ((lane & 3) ^ swz_b8(n)) : ((lane & 7) ^ swz8(n))) * 16);
      }
    }
  };

  // next slice to request: tile ij, k-slice ikt, ring stage ist
  int ij = 0, ikt = 0, ist = 0;
  set_sources(0);
  auto issue_next = [&]() __attribute__((always_inline)) {
    if (ikt == nk) {
      ikt = 0;
      ++ij;
      set_sources(ij);
    }
    const int k0 = ikt * BK;
    const uint32_t st = lds_base + (uint32_t)(ist * ST_BYTES);
    const size_t aoff = (size_t)k0 * ESZ_A;
    const size_t koff = (size_t)(k0 / p.kblock) * N * p.kblock + (k0 % p.kblock);
    const size_t boff = FP8 ? koff : koff * 2;
    // TRB: rows k0 .. of the segment's first matrix, or (k0 >= trb_split) of its second one
    const unsigned char* tbase = nullptr;
    if (TRB) {
      const size_t nb = (size_t)N * 2;
      const int ks = K - p.trb_split;   // rows of the second matrix per segment
      tbase = k0 < p.trb_split
                  ? static_cast<const unsigned char*>(p.w_down) + ((size_t)src_seg * p.trb_split + k0) * nb
                  : static_cast<const unsigned char*>(p.w_up) +
                        ((size_t)src_seg * ks + (k0 - p.trb_split)) * nb;
    }
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
      const int q = wave * NDMA + i;
      const unsigned char* base = (TRB && is_b[i]) ? tbase : sbase[i] + (is_b[i] ? boff : aoff);
      lds_dma16_off((uint32_t)__builtin_amdgcn_readfirstlane((int)(st + (uint32_t)(q * 1024))), base,
                    soff[i]);
    }
    ++ikt;
    ist = ist + 1 == NSTAGE ? 0 : ist + 1;
  };

  // e4m3 DOWN over several weight-scale blocks of K (the stacked shared experts): the
  // finished blocks are folded into a second accumulator set.  KBLK = false: one block
  // (p.kblock == K, checked by the launcher), the scale is applied in the epilogue only.
  constexpr bool FOLD = FP8 && STAGE == 1 && KBLK;
  constexpr int TFM = FOLD ? FM : 1, TFN = FOLD ? FN : 1;

  // prologue: slices 0 .. NSTAGE-2 in flight, slice 0 landed
#pragma unroll
  for (int s = 0; s < NSTAGE - 1; ++s)
    if (s < nslices) issue_next();
  {
    const int younger = min(NSTAGE - 2, nslices - 1);
    if (NSTAGE >= 4 && younger >= 2) wait_vmcnt<(NSTAGE >= 4 ? 2 * NDMA : 0)>();
    else if (NSTAGE >= 3 && younger >= 1) wait_vmcnt<(NSTAGE >= 3 ? NDMA : 0)>();
    else wait_vmcnt<0>();
  }
  __syncthreads();

  const int col_in = lane & 31;    // token column of this lane in a 32 x 32 block
  const int fhalf = lane >> 5;     // which 16 features of a block this lane holds
  TileCoord tc = tile_at(0);
  // rows of the segment left from this wave's first tile row (<= 0: all padding)
  auto rows_of_wave = [&](const TileCoord& t) {
    return __builtin_amdgcn_readfirstlane(t.rows - t.m_tile * BM - wm * WTM);
  };
  int wave_rows = rows_of_wave(tc);
  int j = 0, kt = 0, cst = 0;      // tile, k-slice and ring stage being multiplied
  int j3 = 0;                      // j mod 3
  int g = 0;                       // slice of the workgroup's sequence being multiplied
  // The nk slices of one tile.  NF: how many of the wave's 32-row blocks hold rows of the
  // segment; the others are padding, neither multiplied nor stored.  NF is fixed for the
  // whole tile, so that each specialised copy of the loop keeps its own accumulators and
  // none of them is live where the copies meet.
  auto run_tile = [&](auto nf_tag) __attribute__((always_inline)) {
    constexpr int NF = decltype(nf_tag)::value;
    f32x16 acc[FM][FN];
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
      for (int b = 0; b < FN; ++b) acc[a][b] = f32x16{};
    f32x16 acc_tot[TFM][TFN];
#pragma unroll
    for (int a = 0; a < TFM; ++a)
#pragma unroll
      for (int b = 0; b < TFN; ++b) acc_tot[a][b] = f32x16{};
    for (int islice = 0; islice < nk; ++islice, ++g) {
      if (g + NSTAGE - 1 < nslices) issue_next();
      if (FOLD && kt > 0 && ((kt * BK) % p.kblock) == 0) {
        // the next K block belongs to another shared expert: fold the finished block
        // with its per-channel scales
        const int blk = (kt * BK) / p.kblock - 1;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          const int col = tc.n_tile * BN + wn * WTN + fn * 32 + 16 * fhalf;
          float sc[16];
          if (col < N) load16_f32(p.s_down + ((size_t)tc.seg * nblk_k + blk) * N + col, sc);
          else {
#pragma unroll
            for (int i = 0; i < 16; ++i) sc[i] = 0.f;
          }
#pragma unroll
          for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
            for (int i = 0; i < 16; ++i) acc_tot[fm % TFM][fn % TFN][i] += sc[i] * acc[fm][fn][i];
            acc[fm][fn] = f32x16{};
          }
        }
      }
      const unsigned char* A = lds + cst * ST_BYTES;
      const unsigned char* B = A + A_BYTES;
      // operand fragments of K-step ks + 1 are read from LDS while the MFMAs of step ks run
      bf16x8 af[2][FM], bfr[2][FN];
      auto load_frags = [&](int ks, bf16x8 (&a)[FM], bf16x8 (&b)[FN]) {
        const int c = ks * 2 + (lane >> 5);
#pragma unroll
        for (int fm = 0; fm < NF; ++fm) {
          const int row = wm * WTM + fm * 32 + (lane & 31);
          a[fm] = *reinterpret_cast<const bf16x8*>(A + row * AROW + ((c ^ sw) << 4));
        }
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          const int row = wn * WTN + fn * 32 + (lane & 31);
          if (TRB) {
            typedef short v4s __attribute__((ext_vector_type(4)));
            const int g = lane >> 4, jj = lane & 15, q4 = jj & 3;
            const int col = wn * WTN + fn * 32 + 16 * (q4 & 1) + 8 * (g & 1) + 4 * (q4 >> 1);
            v4s v[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int kr = ks * 16 + 8 * (g >> 1) + 4 * h + (jj >> 2);
              const int addr = kr * (BN * 2) + ((((col >> 3) ^ ((kr & 3) << 2)) << 4) | ((col & 7) << 1));
              v[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (__attribute__((address_space(3))) v4s*)(B + addr));
            }
            b[fn] = __builtin_bit_cast(bf16x8, (short __attribute__((ext_vector_type(8)))){
                v[0][0], v[0][1], v[0][2], v[0][3], v[1][0], v[1][1], v[1][2], v[1][3]});
          } else if (!FP8) {
            b[fn] = *reinterpret_cast<const bf16x8*>(B + row * BROW + ((c ^ sw) << 4));
          } else {
            const uint2 q = *reinterpret_cast<const uint2*>(
                B + row * BROW + ((ks ^ swz4(row)) << 4) + ((lane >> 5) << 3));
            b[fn] = widen_e4m3x8(q);
          }
        }
      };
      // rows past the end of the segment (the padding of an expert's last m-tile) are not
      // multiplied: in the specialised copies only the wave's first NF 32-row blocks are
      // read and multiplied; otherwise a wave whose rows are all padding skips its LDS
      // reads and MFMAs
      if (A8) {
        if (wave_rows > 0) {
          // two 32x32x64 e4m3 MFMA steps per block and slice: in step ks, lane half h holds K
          // bytes [64 ks + 32 h, + 32) of its row in both operands (logical chunks 4 ks + 2 h
          // and 4 ks + 2 h + 1); the operands of step 1 are read while step 0 multiplies
          typedef int v8i __attribute__((ext_vector_type(8)));
          const int h = lane >> 5;
          auto frag8 = [&](const unsigned char* base, int row, int ks) {
            const int z = swz8(row), c0 = 4 * ks + 2 * h;
            const uint4 lo = *reinterpret_cast<const uint4*>(base + row * 128 + ((c0 ^ z) << 4));
            const uint4 hi = *reinterpret_cast<const uint4*>(base + row * 128 + (((c0 + 1) ^ z) << 4));
            return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          };
          // B fragments of both steps and the A fragments of step 0 first; each A fragment of
          // step 1 is read into its register once step 0's MFMAs of that fragment are issued
          v8i a8[FM], b8[2][FN];
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) b8[ks][fn] = frag8(B, wn * WTN + fn * 32 + (lane & 31), ks);
#pragma unroll
          for (int fm = 0; fm < FM; ++fm) a8[fm] = frag8(A, wm * WTM + fm * 32 + (lane & 31), 0);
          __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
              for (int fn = 0; fn < FN; ++fn)
                acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    b8[ks][fn], a8[fm], acc[fm][fn], 0, 0, 0, 127, 0, 127);
              if (ks == 0) a8[fm] = frag8(A, wm * WTM + fm * 32 + (lane & 31), 1);
            }
          }
          // instruction order: the two reads of A fragment fm of step 1 right after step 0's
          // MFMAs of fm
          __builtin_amdgcn_sched_group_barrier(0x100, 4 * FN + 2 * FM, 0);
#pragma unroll
          for (int fm = 0; fm < FM; ++fm) {
            __builtin_amdgcn_sched_group_barrier(0x008, FN, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, FM * FN, 0);
        }
      } else {
        // K-steps [k0, k1) of the slice: the LDS reads of step ks + 1 run behind the MFMAs of
        // step ks, placed one by one between them by scheduling directives (left to itself
        // the compiler issues some of them just before their first use)
        auto mfma_steps = [&](auto k0_tag, auto k1_tag) {
          constexpr int K0 = decltype(k0_tag)::value, K1 = decltype(k1_tag)::value;
          if (K0 == 0) load_frags(0, af[0], bfr[0]);
          __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int ks = K0; ks < K1; ++ks) {
            if (ks + 1 < BK / 16) load_frags(ks + 1, af[(ks + 1) & 1], bfr[(ks + 1) & 1]);
#pragma unroll
            for (int fm = 0; fm < NF; ++fm)
#pragma unroll
              for (int fn = 0; fn < FN; ++fn)
                acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[ks & 1][fn], af[ks & 1][fm],
                                                                      acc[fm][fn], 0, 0, 0);
          }
          constexpr int NDS = NF + (TRB ? 2 : 1) * FN, NMF = NF * FN;
          constexpr int NPAIR = NDS < NMF ? NDS : NMF;
#pragma unroll
          for (int ks = K0; ks < K1; ++ks) {
            if (ks + 1 < BK / 16) {
#pragma unroll
              for (int i = 0; i < NPAIR; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
              }
              if (NMF > NPAIR) __builtin_amdgcn_sched_group_barrier(0x008, NMF - NPAIR, 0);
              if (NDS > NPAIR) __builtin_amdgcn_sched_group_barrier(0x100, NDS - NPAIR, 0);
            } else {
              __builtin_amdgcn_sched_group_barrier(0x008, NMF, 0);
            }
          }
        };
        using I0 = std::integral_constant<int, 0>;
        using IE = std::integral_constant<int, BK / 16>;
        if constexpr (SPEC) {
          if constexpr (NF > 0) mfma_steps(I0{}, IE{});
        } else if (wave_rows > 0) {
          mfma_steps(I0{}, IE{});
        }
      }
      __builtin_amdgcn_s_setprio(0);

      if (kt == nk - 1) {
        // ---- tile j's last slice: the per-row data of tile j + 2, the barrier, then the
        // epilogue of tile j while the next tile's first slices are in flight
        int pf_row = 0;
        float pf_w = 0.f;
        const bool pf = prefetch && j + 2 < ntiles && tid < BM;
        if (pf) {
          const int sr = seg_row(tile_at(j + 2), tid);
          if (gather) pf_row = p.row_index[sr];
          if (has_rw) pf_w = p.row_weight[A8 && gather ? p.row_index[sr] : sr];
        }
        // slice g + 1 and the loads above have landed; no store is in flight
        wait_vmcnt<0>();
        if (pf) {
          if (gather) s_arow[j & 1][tid] = pf_row;   // tile j + 2 has the parity of tile j
          if (has_rw) s_rw[j3 == 0 ? 2 : j3 - 1][tid] = pf_w;   // (j + 2) mod 3
        }
        cst = cst + 1 == NSTAGE ? 0 : cst + 1;
        __syncthreads();
        // The epilogue runs behind the barrier, so its stores complete while the next slice
        // is multiplied; the next slice's wait (a full one on the 2-stage ring) covers them.
        if (has_rw && !prefetch) {
          // short K: this tile's row weights are staged here (buffer j3 was last read by the
          // epilogue three tiles ago)
          if (tid < BM) {
            const int sr = seg_row(tc, tid);
            s_rw[j3][tid] = p.row_weight[A8 && gather ? p.row_index[sr] : sr];
          }
          __syncthreads();
        }
        const int m0 = tc.m_tile * BM;
        // every load of the epilogue is issued before its first store, so that the waits
        // for them do not also wait for stores
        if (STAGE == 0) {
          constexpr int FH = SWIGLU ? FN / 2 : FN;
          float ra[FM];   // e4m3 activations: the scale of each lane's A row
#pragma unroll
          for (int fm = 0; fm < FM; ++fm) ra[fm] = (A8 && has_rw) ? s_rw[j3][wm * WTM + fm * 32 + col_in] : 1.f;
          float sg[FH][16], su[FH][16];
          if (FP8) {
#pragma unroll
            for (int fh = 0; fh < FH; ++fh) {
              const int hcol = SWIGLU ? tc.n_tile * (BN / 2) + wn * (WTN / 2) + fh * 32 + 16 * fhalf
                                      : tc.n_tile * BN + wn * WTN + fh * 32 + 16 * fhalf;
              const int hc = hcol < N ? hcol : 0;
              load16_f32(p.s_gate + (size_t)tc.seg * N + hc, sg[fh]);
              if (SWIGLU) load16_f32(p.s_up + (size_t)tc.seg * N + hc, su[fh]);
            }
          }
#pragma unroll
          for (int fh = 0; fh < FH; ++fh) {
            const int hcol = SWIGLU ? tc.n_tile * (BN / 2) + wn * (WTN / 2) + fh * 32 + 16 * fhalf
                                    : tc.n_tile * BN + wn * WTN + fh * 32 + 16 * fhalf;
            if (hcol >= N) continue;
            if (BWD) {
#pragma unroll
              for (int fm = 0; fm < FM; ++fm) {
                const int r = m0 + wm * WTM + fm * 32 + col_in;
                if (r >= tc.rows) continue;
                const size_t row = (size_t)(tc.row0 + r);
                // dh of these 16 features (bf16)
                const uint4* dsrc = reinterpret_cast<const uint4*>(
                    static_cast<const uint16_t*>(p.dact) + row * N + hcol);
                const uint4 d0 = dsrc[0], d1 = dsrc[1];
                const uint32_t dw[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
                float da[16], db[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                  const float dh = bf16_bits_to_f32((i & 1) ? (dw[i >> 1] >> 16) : (dw[i >> 1] & 0xffffu));
                  const float a = acc[fm][fh][i];
                  if (SWIGLU) {
                    const float b = acc[fm][fh + FN / 2][i];
                    const float sig = 1.0f / (1.0f + __expf(-a));
                    da[i] = dh * b * (sig * (1.0f + a * (1.0f - sig)));   // silu'(a)
                    db[i] = dh * (a * sig);                                // silu(a)
                  } else {
                    da[i] = dh * 2.0f * fmaxf(a, 0.f);
                  }
                }
                uint16_t* o = static_cast<uint16_t*>(p.out) + row * (SWIGLU ? 2 * N : N);
                store16_bf16(o + hcol, da);
                if (SWIGLU) store16_bf16(o + N + hcol, db);
              }
              continue;
            }
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
              const int r = m0 + wm * WTM + fm * 32 + col_in;
              if (r >= tc.rows) continue;
              float h[16];
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                if (SWIGLU) {
                  const float gv = FP8 ? acc[fm][fh][i] * (sg[fh][i] * ra[fm]) : acc[fm][fh][i];
                  const float uv = FP8 ? acc[fm][fh + FN / 2][i] * (su[fh][i] * ra[fm]) : acc[fm][fh + FN / 2][i];
                  h[i] = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
                } else {
                  const float gv = FP8 ? acc[fm][fh][i] * (sg[fh][i] * ra[fm]) : acc[fm][fh][i];
                  const float rr = fmaxf(gv, 0.f);
                  h[i] = rr * rr;
                }
              }
              store16_bf16(static_cast<uint16_t*>(p.out) + (size_t)(tc.row0 + r) * N + hcol, h);
            }
          }
        } else {
          float rw[FM];
#pragma unroll
          for (int fm = 0; fm < FM; ++fm) rw[fm] = has_rw ? s_rw[j3][wm * WTM + fm * 32 + col_in] : 1.f;
          if (FP8) {
            const int blk = nblk_k - 1;
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
              const int col = tc.n_tile * BN + wn * WTN + fn * 32 + 16 * fhalf;
              float sc[16];
              if (col < N) load16_f32(p.s_down + ((size_t)tc.seg * nblk_k + blk) * N + col, sc);
              else {
#pragma unroll
                for (int i = 0; i < 16; ++i) sc[i] = 0.f;
              }
#pragma unroll
              for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                  acc[fm][fn][i] = acc_tot[fm % TFM][fn % TFN][i] + sc[i] * acc[fm][fn][i];
            }
          }
#pragma unroll
          for (int fm = 0; fm < FM; ++fm) {
            const int r = m0 + wm * WTM + fm * 32 + col_in;
            if (r >= tc.rows) continue;
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
              const int col = tc.n_tile * BN + wn * WTN + fn * 32 + 16 * fhalf;
              if (col >= N) continue;
              float y[16];
#pragma unroll
              for (int i = 0; i < 16; ++i) y[i] = rw[fm] * acc[fm][fn][i];
              store16_bf16(static_cast<uint16_t*>(p.out) + (size_t)(tc.row0 + r) * N + col, y);
            }
          }
        }
        ++j;
        j3 = j3 == 2 ? 0 : j3 + 1;
        kt = 0;
        if (j < ntiles) {
          tc = tile_at(j);
          wave_rows = rows_of_wave(tc);
        }
      } else {
        ++kt;
        // slice g + 1 must have landed; younger slices may stay in flight
        const int younger = min(NSTAGE - 2, nslices - 2 - g);
        if (NSTAGE >= 4 && younger >= 2) wait_vmcnt<(NSTAGE >= 4 ? 2 * NDMA : 0)>();
        else if (NSTAGE >= 3 && younger >= 1) wait_vmcnt<(NSTAGE >= 3 ? NDMA : 0)>();
        else wait_vmcnt<0>();
        cst = cst + 1 == NSTAGE ? 0 : cst + 1;
        __syncthreads();
      }
    }
  };
  while (g < nslices) {
    if constexpr (SPEC) {
      const int nf = wave_rows <= 0 ? 0 : min(FM, (wave_rows + 31) / 32);
      if constexpr (FP8) {
        if (nf > FM / 2) run_tile(std::integral_constant<int, FM>{});
        else if (nf > 0) run_tile(std::integral_constant<int, FM / 2>{});
        else run_tile(std::integral_constant<int, 0>{});
      } else {
        if (nf == FM) run_tile(std::integral_constant<int, FM>{});
        else if (nf <= 0) run_tile(std::integral_constant<int, 0>{});
        else if (nf == 1) run_tile(std::integral_constant<int, 1>{});
        else if (nf == 2) run_tile(std::integral_constant<int, (FM > 2 ? 2 : 1)>{});
        else run_tile(std::integral_constant<int, (FM > 3 ? 3 : 1)>{});
      }
    } else {
      run_tile(std::integral_constant<int, FM>{});
    }
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

// Tile configuration per call, from what the host knows of the problem: 256 x 256 tiles
// whenever that still gives every CU at least two tiles (measured faster than 128 x 256
// tiles even for routed segments of ~400 rows, where a third of the last m-tile is
// padding: the larger tile halves the L2 and LDS traffic per MFMA), else 128 x 256.
// Each configuration is (BM, BN, waves, LDS stages, workgroups per CU).
#define MOE_CFG_NARROW_UP 128, 256, 8, 3, 1
#define MOE_CFG_NARROW_DOWN 128, 256, 8, 3, 1
#define MOE_CFG_WIDE 256, 256, 8, 2, 1

// e4m3 activations: 128-byte slices of 128 K values (two MFMA steps), the bf16 ring depths
#define MOE_CFG_NARROW_A8 128, 256, 8, 3, 1
#define MOE_CFG_WIDE_A8 256, 256, 8, 2, 1

template <int BM, int BN, int WAVES, int NSTAGE, int OCC, int STAGE, int ACT, bool FP8,
          bool A8 = false, bool BWD = false, bool TRB = false, bool KBLK = true>
hipError_t launch_cfg(const GemmParams& p, int num_cus, hipStream_t s) {
  hipLaunchKernelGGL((gg_mfma_kernel<BM, BN, WAVES, NSTAGE, OCC, STAGE, ACT, FP8, A8, BWD, TRB, KBLK>),
                     dim3(num_cus * OCC), dim3(WAVES * 64), 0, s, p);
  return hipGetLastError();
}

template <int ACT>
hipError_t launch_mfma_a8(const GemmParams& p, int num_cus, hipStream_t s) {
  const long long bcols = ACT == MOE_ACT_SWIGLU ? 2LL * p.N : p.N;
  const long long wide_tiles = ((p.rows + 255) / 256) * ((bcols + 255) / 256);
  if (wide_tiles >= 2LL * num_cus) return launch_cfg<MOE_CFG_WIDE_A8, 0, ACT, true, true>(p, num_cus, s);
  return launch_cfg<MOE_CFG_NARROW_A8, 0, ACT, true, true>(p, num_cus, s);
}

template <int STAGE, int ACT, bool FP8>
hipError_t launch_mfma(const GemmParams& p, int num_cus, hipStream_t s) {
  const bool swiglu = STAGE == 0 && ACT == MOE_ACT_SWIGLU;
  const long long bcols = swiglu ? 2LL * p.N : p.N;
  const long long wide_tiles = ((p.rows + 255) / 256) * ((bcols + 255) / 256);
  if (wide_tiles >= 2LL * num_cus) {
    if constexpr (FP8 && STAGE == 1) {
      // e4m3 down: 256 x 256 tiles only with one weight-scale block (no second
      // accumulator set)
      if (p.kblock == p.K)
        return launch_cfg<MOE_CFG_WIDE, STAGE, ACT, FP8, false, false, false, false>(p, num_cus, s);
    } else {
      return launch_cfg<MOE_CFG_WIDE, STAGE, ACT, FP8>(p, num_cus, s);
    }
  }
  if constexpr (STAGE == 0) return launch_cfg<MOE_CFG_NARROW_UP, STAGE, ACT, FP8>(p, num_cus, s);
  else return launch_cfg<MOE_CFG_NARROW_DOWN, STAGE, ACT, FP8>(p, num_cus, s);
}

template <int ACT>
hipError_t launch_bwd(const GemmParams& p, int num_cus, hipStream_t s) {
  const long long bcols = ACT == MOE_ACT_SWIGLU ? 2LL * p.N : p.N;
  const long long wide_tiles = ((p.rows + 255) / 256) * ((bcols + 255) / 256);
  if (wide_tiles >= 2LL * num_cus)
    return launch_cfg<MOE_CFG_WIDE, 0, ACT, false, false, true>(p, num_cus, s);
  return launch_cfg<MOE_CFG_NARROW_UP, 0, ACT, false, false, true>(p, num_cus, s);
}

template <int STAGE, int ACT>
hipError_t launch_f32(const GemmParams& p, int num_cus, hipStream_t s) {
  const int grid = num_cus * 4;
  hipLaunchKernelGGL((gg_f32_kernel<STAGE, ACT>), dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_down_trb(const GemmParams& p, int num_cus, hipStream_t s) {
  if (p.rows == 0) return hipSuccess;
  const long long wide_tiles = ((p.rows + 255) / 256) * ((p.N + 255LL) / 256);
  if (wide_tiles >= 2LL * num_cus)
    return launch_cfg<MOE_CFG_WIDE, 1, MOE_ACT_SWIGLU, false, false, false, true>(p, num_cus, s);
  return launch_cfg<MOE_CFG_NARROW_DOWN, 1, MOE_ACT_SWIGLU, false, false, false, true>(p, num_cus, s);
}

hipError_t launch_up_backward(const GemmParams& p, int act, int num_cus, hipStream_t s) {
  if (p.rows == 0) return hipSuccess;
  return act == MOE_ACT_RELU2 ? launch_bwd<MOE_ACT_RELU2>(p, num_cus, s)
                              : launch_bwd<MOE_ACT_SWIGLU>(p, num_cus, s);
}

hipError_t launch_grouped_gemm(const GemmParams& p, Stage stage, int act, int act_dtype,
                               int weight_dtype, int num_cus, hipStream_t s, bool fp8_act) {
  if (p.rows == 0) return hipSuccess;
  if (fp8_act) {
    // e4m3 x e4m3 up projection (the caller checked stage, dtypes and the scales)
    return act == MOE_ACT_RELU2 ? launch_mfma_a8<MOE_ACT_RELU2>(p, num_cus, s)
                                : launch_mfma_a8<MOE_ACT_SWIGLU>(p, num_cus, s);
  }
  const bool up = stage == Stage::Up;
  const bool relu2 = act == MOE_ACT_RELU2;
  if (act_dtype == MOE_F32) {
    if (up) return relu2 ? launch_f32<0, MOE_ACT_RELU2>(p, num_cus, s)
                         : launch_f32<0, MOE_ACT_SWIGLU>(p, num_cus, s);
    return launch_f32<1, MOE_ACT_SWIGLU>(p, num_cus, s);
  }
  const bool fp8 = weight_dtype == MOE_FP8_E4M3;
  if (tail_gemm_applies(p)) return launch_tail_gemm(p, stage, act, weight_dtype, num_cus, s);
  if (decode_gemm_applies(p, act_dtype)) return launch_decode_gemm(p, stage, act, weight_dtype, s);
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
