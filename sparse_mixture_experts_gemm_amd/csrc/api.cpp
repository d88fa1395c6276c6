// libmoe C ABI: argument validation, workspace carve-up and kernel launches.
// Declarations and the meaning of every argument are in include/moe.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "backward.h"
#include "internal.h"
#include "moe.h"

namespace {

thread_local int32_t g_last_hip_error = 0;

moe_status hip_status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  g_last_hip_error = static_cast<int32_t>(e);
  return MOE_ERR_HIP;
}

constexpr int kMaxDevices = 64;
std::atomic<int> g_num_cus[kMaxDevices];

// Compute units of the current device, queried once per device.
moe_status current_cus(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  int v = g_num_cus[dev].load(std::memory_order_relaxed);
  if (v <= 0) {
    e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_status(e);
    if (v <= 0) v = 1;
    g_num_cus[dev].store(v, std::memory_order_relaxed);
  }
  *cus = v;
  return MOE_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A second stream for the shared experts, which do not depend on the routing: their GEMMs
// overlap routing, permutation and the routed GEMMs.  One side stream (default priority,
// non-blocking) with its own fork / join events is kept per (device, caller stream), created
// on first use and kept until the process ends, so calls on different caller streams (or
// under graph capture on one of them) never share a side stream.  Calls on the same caller
// stream share its entry: they are ordered by that stream, and an event re-recorded by a
// later call on it only makes an earlier call's wait more conservative.  Past
// kMaxSideStreams caller streams per device, the shared experts run on the caller's stream.
constexpr int kMaxSideStreams = 32;
constexpr int kSideEvents = 3;   // fork, intermediate join, final join

struct SideEntry {
  hipStream_t caller;
  hipStream_t side;
  hipEvent_t ev[kSideEvents];
};

std::mutex g_side_mu;
SideEntry g_side[kMaxDevices][kMaxSideStreams];
int g_side_n[kMaxDevices];

// *out = the entry of (current device, caller), or null when the table is full.
moe_status side_entry(hipStream_t caller, const SideEntry** out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_side_mu);
  for (int i = 0; i < g_side_n[dev]; ++i) {
    if (g_side[dev][i].caller == caller) {
      *out = &g_side[dev][i];
      return MOE_OK;
    }
  }
  if (g_side_n[dev] == kMaxSideStreams) return MOE_OK;
  SideEntry ent{};
  ent.caller = caller;
  e = hipStreamCreateWithFlags(&ent.side, hipStreamNonBlocking);
  for (int i = 0; e == hipSuccess && i < kSideEvents; ++i)
    e = hipEventCreateWithFlags(&ent.ev[i], hipEventDisableTiming);
  if (e != hipSuccess) {
    for (int i = 0; i < kSideEvents; ++i)
      if (ent.ev[i] != nullptr) (void)hipEventDestroy(ent.ev[i]);
    if (ent.side != nullptr) (void)hipStreamDestroy(ent.side);
    return hip_status(e);
  }
  g_side[dev][g_side_n[dev]] = ent;
  *out = &g_side[dev][g_side_n[dev]++];
  return MOE_OK;
}

moe_status check_config(const moe_config* c) {
  if (c == nullptr) return MOE_ERR_INVALID_ARG;
  if (c->num_tokens < 0 || c->dim <= 0 || c->num_experts <= 0 || c->top_k <= 0 ||
      c->num_groups <= 0 || c->topk_groups <= 0 || c->num_shared < 0 || c->inter_dim <= 0)
    return MOE_ERR_INVALID_ARG;
  const int E = c->num_experts, G = c->num_groups;
  if (c->top_k > E || E % G != 0 || c->topk_groups > G) return MOE_ERR_INVALID_ARG;
  if ((long long)c->top_k > (long long)c->topk_groups * (E / G)) return MOE_ERR_INVALID_ARG;
  if (c->group_score_topn != 1 && c->group_score_topn != 2) return MOE_ERR_INVALID_ARG;
  if (c->group_score_topn > E / G) return MOE_ERR_INVALID_ARG;
  if (c->score_fn != MOE_SCORE_SOFTMAX && c->score_fn != MOE_SCORE_SIGMOID) return MOE_ERR_INVALID_ARG;
  if (c->act != MOE_ACT_SWIGLU && c->act != MOE_ACT_RELU2) return MOE_ERR_INVALID_ARG;
  if (c->renormalize != 0 && c->renormalize != 1) return MOE_ERR_INVALID_ARG;
  if (!std::isfinite(c->capacity_factor)) return MOE_ERR_INVALID_ARG;
  if (c->fp8_act != 0 && c->fp8_act != 1) return MOE_ERR_INVALID_ARG;
  if (c->pre_norm != 0 && c->pre_norm != 1) return MOE_ERR_INVALID_ARG;
  if (c->residual != 0 && c->residual != 1) return MOE_ERR_INVALID_ARG;
  if (!std::isfinite(c->norm_eps) || c->norm_eps < 0.0f) return MOE_ERR_INVALID_ARG;
  if (c->act_dtype != MOE_F32 && c->act_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (c->weight_dtype != MOE_F32 && c->weight_dtype != MOE_BF16 && c->weight_dtype != MOE_FP8_E4M3)
    return MOE_ERR_INVALID_ARG;
  // implemented combinations and shapes
  if (E > 64) return MOE_ERR_UNSUPPORTED;
  if (c->fp8_act && (c->act_dtype != MOE_BF16 || c->weight_dtype != MOE_FP8_E4M3))
    return MOE_ERR_UNSUPPORTED;
  // e4m3 activations: 128-byte K-slices of the up projection, 64-wide output tiles
  if (c->fp8_act && (c->dim % 128 != 0 || c->inter_dim % 64 != 0)) return MOE_ERR_UNSUPPORTED;
  if (c->act_dtype == MOE_F32) {
    if (c->weight_dtype != MOE_F32) return MOE_ERR_UNSUPPORTED;
    if (c->dim % 16 != 0 || c->inter_dim % 16 != 0) return MOE_ERR_UNSUPPORTED;
  } else {
    // 16-byte rows of operands: 8 bf16 values, or 16 e4m3 weights (multiples of 64 take
    // the tiled kernels, other multiples the tail kernel of gemm_tail.hip)
    if (c->weight_dtype == MOE_F32) return MOE_ERR_UNSUPPORTED;
    const int q = c->weight_dtype == MOE_FP8_E4M3 ? 16 : 8;
    if (c->dim % q != 0 || c->inter_dim % q != 0) return MOE_ERR_UNSUPPORTED;
  }
  const long long Tk = (long long)c->num_tokens * c->top_k;
  if (Tk > INT_MAX / 2) return MOE_ERR_UNSUPPORTED;
  if ((long long)c->num_shared * c->inter_dim > INT_MAX / 2) return MOE_ERR_UNSUPPORTED;
  // the kernels index activations and one expert's weights (the stacked shared experts
  // count as one) with 32-bit element offsets, or byte offsets below 4 GB
  const long long widest = c->dim > c->inter_dim ? c->dim : c->inter_dim;
  if (Tk * widest > INT_MAX || (long long)c->num_tokens * c->num_shared * c->inter_dim > INT_MAX ||
      (long long)c->num_experts * c->dim * c->inter_dim > INT_MAX ||
      (long long)c->num_shared * c->inter_dim * c->dim > INT_MAX)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe::RouteParams route_params(const moe_config* c) {
  moe::RouteParams p;
  p.T = c->num_tokens;
  p.d = c->dim;
  p.E = c->num_experts;
  p.k = c->top_k;
  p.G = c->num_groups;
  p.Gk = c->topk_groups;
  p.n_g = c->group_score_topn;
  p.score_fn = c->score_fn;
  p.renormalize = c->renormalize;
  p.route_scale = c->route_scale;
  p.select_bias = nullptr;
  p.norm_gamma = nullptr;
  p.norm_eps = c->norm_eps;
  p.x_norm = nullptr;
  return p;
}

// Rows an expert may keep: floor(c * T * k / E) in double from the fp32 factor, or
// INT_MAX (unlimited) for c <= 0.
int expert_capacity(const moe_config* c) {
  if (!(c->capacity_factor > 0.0f)) return INT_MAX;
  const double cap = std::floor((double)c->capacity_factor * (double)c->num_tokens *
                                (double)c->top_k / (double)c->num_experts);
  return cap >= (double)INT_MAX ? INT_MAX : (int)cap;
}

size_t act_size(const moe_config* c) { return c->act_dtype == MOE_BF16 ? 2 : 4; }

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }

// Workspace of moe_forward, in carve order.
struct Carve {
  size_t topk_idx, topk_w, counts, offsets, perm_token, slot_pos, perm_weight, perm_ws;
  size_t scores, stats_ws, route_part, x_norm, x_q, x_scale;
  size_t h_routed, h_shared, y_routed, y_shared, total;
};

Carve carve(const moe_config* c) {
  const size_t T = (size_t)c->num_tokens, k = (size_t)c->top_k, E = (size_t)c->num_experts;
  const size_t d = (size_t)c->dim, I = (size_t)c->inter_dim, S = (size_t)c->num_shared;
  const size_t as = act_size(c);
  Carve w{};
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o += align_up(bytes); return at; };
  w.topk_idx = take(T * k * 4);
  w.topk_w = take(T * k * 4);
  w.counts = take(E * 4);
  w.offsets = take((E + 1) * 4);
  w.perm_token = take(T * k * 4);
  w.slot_pos = take(T * k * 4);
  w.perm_weight = take(T * k * 4);
  w.perm_ws = take(moe::permute_ws_bytes((int)T, (int)E));
  w.scores = take(T * E * 4);                    // only written when statistics are asked
  w.stats_ws = take(moe::stats_ws_bytes((int)T, (int)E));
  // partial router logits of a small batch
  w.route_part = take(T <= (size_t)moe::kSplitRouteTokens ? moe::split_route_part_bytes((int)T, (int)E) : 0);
  w.x_norm = take(c->pre_norm ? T * d * as : 0); // normalised input of a pre-norm layer
  w.x_q = take(c->fp8_act ? T * d : 0);          // e4m3 activations of the up projections
  w.x_scale = take(c->fp8_act ? T * 4 : 0);
  w.h_routed = take(T * k * I * as);
  w.h_shared = take(T * S * I * as);
  w.y_routed = take(T * k * d * as);
  w.y_shared = take(S > 0 ? T * d * as : 0);
  w.total = o;
  return w;
}

// Workspace of moe_backward, in carve order.
struct BwdCarve {
  size_t sh_w2t;                               // shared W2 transposed to [S I][d] (bf16)
  size_t scores, idx, tw, dw, dl;
  size_t dh_r, dh_s, dab_r, dab_s, dxp_r, dx_s;  // data-gradient intermediates (bf16)
  size_t x_perm, dy_perm;                        // routed rows in permuted order (bf16)
  size_t rg, total;
};

BwdCarve bwd_carve(const moe_config* c) {
  const size_t T = (size_t)c->num_tokens, k = (size_t)c->top_k, E = (size_t)c->num_experts;
  const size_t d = (size_t)c->dim, I = (size_t)c->inter_dim, S = (size_t)c->num_shared;
  const size_t nab = c->act == MOE_ACT_SWIGLU ? 2 : 1;   // pre-activations per inter feature
  BwdCarve b{};
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o += align_up(bytes); return at; };
  b.sh_w2t = take(S * I * d * 2);
  b.scores = take(T * E * 4);
  b.idx = take(T * k * 4);
  b.tw = take(T * k * 4);
  b.dw = take(T * k * 4);
  b.dl = take(T * E * 4);
  b.dh_r = take(T * k * I * 2);
  b.dh_s = take(T * S * I * 2);
  b.dab_r = take(T * k * nab * I * 2);
  b.dab_s = take(T * nab * S * I * 2);
  b.dxp_r = take(T * k * d * 2);
  b.dx_s = take(S > 0 ? T * d * 2 : 0);
  b.x_perm = take(T * k * d * 2);
  b.dy_perm = take(T * k * d * 2);
  b.rg = take(moe::router_wgrad_ws_bytes((int)T, (int)d, (int)E));
  b.total = o;
  return b;
}

moe_status check_backward_config(const moe_config* c) {
  moe_status st = check_config(c);
  if (st != MOE_OK) return st;
  if (!std::isfinite(c->route_scale) || c->route_scale == 0.0f) return MOE_ERR_INVALID_ARG;
  if (c->act_dtype != MOE_BF16 || c->weight_dtype != MOE_BF16 || c->pre_norm || c->fp8_act)
    return MOE_ERR_UNSUPPORTED;
  if (c->dim % 64 != 0 || c->inter_dim % 64 != 0) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status gemm_params(const moe_config* c, moe_stage stage, moe_expert_set set, const void* a,
                       const int32_t* row_index, const int32_t* offsets, int32_t rows,
                       const moe_weights* w, const float* row_weight, void* out,
                       moe::GemmParams* p) {
  if (w == nullptr || a == nullptr || out == nullptr || rows < 0) return MOE_ERR_INVALID_ARG;
  if (stage != MOE_STAGE_UP && stage != MOE_STAGE_DOWN) return MOE_ERR_INVALID_ARG;
  if (set != MOE_EXPERTS_ROUTED && set != MOE_EXPERTS_SHARED) return MOE_ERR_INVALID_ARG;
  const bool routed = set == MOE_EXPERTS_ROUTED;
  const bool fp8 = c->weight_dtype == MOE_FP8_E4M3;
  const bool swiglu = c->act == MOE_ACT_SWIGLU;
  if (routed && offsets == nullptr) return MOE_ERR_INVALID_ARG;
  if (!routed && c->num_shared == 0) return MOE_ERR_INVALID_ARG;
  const int I_eff = routed ? c->inter_dim : c->num_shared * c->inter_dim;
  moe::GemmParams g{};
  g.a = a;
  g.row_index = row_index;
  g.offsets = routed ? offsets : nullptr;
  g.nseg = routed ? c->num_experts : 1;
  g.rows = rows;
  g.d = c->dim;
  g.I = c->inter_dim;
  g.S = c->num_shared;
  g.row_weight = row_weight;
  g.out = out;
  if (stage == MOE_STAGE_UP) {
    g.N = I_eff;
    g.K = c->dim;
    g.kblock = c->dim;
    g.w_gate = routed ? w->w_gate : w->sh_gate;
    g.w_up = routed ? w->w_up : w->sh_up;
    g.s_gate = routed ? w->s_gate : w->sh_s_gate;
    g.s_up = routed ? w->s_up : w->sh_s_up;
    if (g.w_gate == nullptr || (swiglu && g.w_up == nullptr)) return MOE_ERR_INVALID_ARG;
    if (fp8 && (g.s_gate == nullptr || (swiglu && g.s_up == nullptr))) return MOE_ERR_INVALID_ARG;
    if (!aligned16(g.w_gate) || (swiglu && !aligned16(g.w_up))) return MOE_ERR_UNSUPPORTED;
  } else {
    g.N = c->dim;
    g.K = I_eff;
    g.kblock = c->inter_dim;
    g.w_down = routed ? w->w_down : w->sh_down;
    g.s_down = routed ? w->s_down : w->sh_s_down;
    if (g.w_down == nullptr || (fp8 && g.s_down == nullptr)) return MOE_ERR_INVALID_ARG;
    if (!aligned16(g.w_down)) return MOE_ERR_UNSUPPORTED;
  }
  if (!aligned16(a) || !aligned16(out)) return MOE_ERR_UNSUPPORTED;
  *p = g;
  return MOE_OK;
}

// Workspace of moe_forward_noalloc, for callers that cannot allocate device memory: one
// array per device (the code object's own storage, held until the process ends), shared by
// every call on that device.  Host code never passes `scratch` itself to a kernel or a copy:
// in host code the name stands for a host-side shadow, not a device address.  The device
// address is taken once per device with hipGetSymbolAddress (with that device current) and
// kept in g_scratch_ptr.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// *out = the device address of the current device's scratch array.
moe_status device_scratch(void** out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (ptr == nullptr) return MOE_ERR_INTERNAL;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP runtime or launch error";
    case MOE_ERR_INTERNAL: return "internal error";
  }
  return "unknown status";
}

int32_t moe_last_hip_error(void) { return g_last_hip_error; }

moe_status moe_workspace_size(const moe_config* cfg, size_t* bytes) {
  try {
    if (bytes == nullptr) return MOE_ERR_INVALID_ARG;
    moe_status st = check_config(cfg);
    if (st != MOE_OK) return st;
    *bytes = carve(cfg).total;
    return MOE_OK;
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

moe_status moe_route(const moe_config* cfg, const void* x, const void* router,
                     const float* logit_bias, const float* select_bias, float* scores,
                     int32_t* topk_idx, float* topk_w, hipStream_t stream) {
  try {
    moe_status st = check_config(cfg);
    if (st != MOE_OK) return st;
    if (cfg->num_tokens == 0) return MOE_OK;
    if (x == nullptr || router == nullptr || topk_idx == nullptr || topk_w == nullptr)
      return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(router)) return MOE_ERR_UNSUPPORTED;
    moe::RouteParams rp = route_params(cfg);
    rp.select_bias = select_bias;
    return hip_status(moe::launch_route(rp, cfg->act_dtype, x, router, logit_bias, scores,
                                        topk_idx, topk_w, stream));
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

moe_status moe_rmsnorm_route(const moe_config* cfg, const void* x, const float* gamma,
                             const void* router, const float* logit_bias,
                             const float* select_bias, void* x_norm, float* scores,
                             int32_t* topk_idx, float* topk_w, hipStream_t stream) {
  try {
    moe_status st = check_config(cfg);
    if (st != MOE_OK) return st;
    if (cfg->num_tokens == 0) return MOE_OK;
    if (x == nullptr || gamma == nullptr || router == nullptr || x_norm == nullptr ||
        topk_idx == nullptr || topk_w == nullptr)
      return MOE_ERR_INVALID_ARG;
    if (x_norm == x) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(router) || !aligned16(gamma) || !aligned16(x_norm))
      return MOE_ERR_UNSUPPORTED;
    moe::RouteParams rp = route_params(cfg);
    rp.select_bias = select_bias;
    rp.norm_gamma = gamma;
    rp.x_norm = x_norm;
    return hip_status(moe::launch_route(rp, cfg->act_dtype, x, router, logit_bias, scores,
                                        topk_idx, topk_w, stream));
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

moe_status moe_select(const moe_config* cfg, const float* scores, const float* keys,
                      int32_t* topk_idx, float* topk_w, hipStream_t stream) {
  try {
    moe_status st = check_config(cfg);
    if (st != MOE_OK) return st;
    if (cfg->num_tokens == 0) return MOE_OK;
    if (scores == nullptr || topk_idx == nullptr || topk_w == nullptr) return MOE_ERR_INVALID_ARG;
    return hip_status(moe::launch_select(route_params(cfg), scores, keys, topk_idx, topk_w,
                                         stream));
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

moe_status moe_load_stats(const moe_config* cfg, const float* scores, const int32_t* topk_idx,
                          float alpha, float* f, float* p, float* loss, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
  try {
    moe_status st = check_config(cfg);
    if (st != MOE_OK) return st;
    if (cfg->num_tokens == 0) return MOE_OK;
    if (scores == nullptr || topk_idx == nullptr || f == nullptr || p == nullptr ||
        loss == nullptr)
      return MOE_ERR_INVALID_ARG;
    if (!std::isfinite(alpha)) return MOE_ERR_INVALID_ARG;
    const size_t need = moe::stats_ws_bytes(cfg->num_tokens, cfg->num_experts);
    if (ws == nullptr || ws_bytes < need) return MOE_ERR_WORKSPACE;
    return hip_status(moe::launch_load_stats(cfg->num_tokens, cfg->num_experts, cfg->top_k,
                                             scores, topk_idx, alpha, f, p, loss, ws, stream));
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

moe_status moe_permute(const moe_config* cfg, const int32_t* topk_idx, const float* topk_w,
                       int32_t* counts, int32_t* offsets, int32_t* perm_token, int32_t* slot_pos,
                       float* perm_weight, void* ws, size_t ws_bytes, hipStream_t stream) {
  try {
    moe_status st = check_config(cfg);
    if (st != MOE_OK) return st;
    if (counts == nullptr || offsets == nullptr) return MOE_ERR_INVALID_ARG;
    if (cfg->num_tokens > 0 && (topk_idx == nullptr || perm_token == nullptr || slot_pos == nullptr))
      return MOE_ERR_INVALID_ARG;
    if ((topk_w == nullptr) != (perm_weight == nullptr)) return MOE_ERR_INVALID_ARG;
    const size_t need = moe::permute_ws_bytes(cfg->num_tokens, cfg->num_experts);
    if (need > 0 && (ws == nullptr || ws_bytes < need)) return MOE_ERR_WORKSPACE;
    return hip_status(moe::launch_permute(cfg->num_tokens, cfg->num_experts, cfg->top_k,
                                          expert_capacity(cfg), topk_idx, topk_w, counts,
                                          offsets, perm_token, slot_pos, perm_weight, ws,
                                          stream));
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

moe_status moe_grouped_gemm(const moe_config* cfg, moe_stage stage, moe_expert_set set,
                            const void* a, const int32_t* row_index, const int32_t* offsets,
                            int32_t rows, const moe_weights* w, const float* row_weight,
                            void* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  (void)ws;
  (void)ws_bytes;
  try {
    moe_status st = check_config(cfg);
    if (st != MOE_OK) return st;
    if (rows == 0) return MOE_OK;
    const bool a8 = cfg->fp8_act && stage == MOE_STAGE_UP;
    if (a8 && row_weight == nullptr) return MOE_ERR_INVALID_ARG;   // the A-row scales
    moe::GemmParams p;
    st = gemm_params(cfg, stage, set, a, row_index, offsets, rows, w, row_weight, out, &p);
    if (st != MOE_OK) return st;
    int cus = 0;
    st = current_cus(&cus);
    if (st != MOE_OK) return st;
    return hip_status(moe::launch_grouped_gemm(
        p, stage == MOE_STAGE_UP ? moe::Stage::Up : moe::Stage::Down, cfg->act, cfg->act_dtype,
        cfg->weight_dtype, cus, stream, a8));
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

moe_status moe_combine(const moe_config* cfg, const void* y_perm, const int32_t* slot_pos,
                       const void* y_shared, void* out, hipStream_t stream) {
  try {
    moe_status st = check_config(cfg);
    if (st != MOE_OK) return st;
    if (cfg->num_tokens == 0) return MOE_OK;
    if (y_perm == nullptr || slot_pos == nullptr || out == nullptr) return MOE_ERR_INVALID_ARG;
    if (!aligned16(y_perm) || !aligned16(out) || (y_shared != nullptr && !aligned16(y_shared)))
      return MOE_ERR_UNSUPPORTED;
    return hip_status(moe::launch_combine(cfg->num_tokens, cfg->dim, cfg->top_k, cfg->act_dtype,
                                          y_perm, slot_pos, y_shared, nullptr, out, stream));
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

moe_status moe_quantize_rows(const moe_config* cfg, const void* a, int32_t rows, int32_t cols,
                             uint8_t* q, float* scale, hipStream_t stream) {
  try {
    moe_status st = check_config(cfg);
    if (st != MOE_OK) return st;
    if (rows < 0 || cols <= 0) return MOE_ERR_INVALID_ARG;
    if (rows == 0) return MOE_OK;
    if (a == nullptr || q == nullptr || scale == nullptr) return MOE_ERR_INVALID_ARG;
    if (cfg->act_dtype != MOE_BF16 || cols % 8 != 0) return MOE_ERR_UNSUPPORTED;
    if ((long long)rows * cols > INT_MAX) return MOE_ERR_UNSUPPORTED;
    if (!aligned16(a) || (reinterpret_cast<uintptr_t>(q) & 7u) != 0) return MOE_ERR_UNSUPPORTED;
    return hip_status(moe::launch_quant_rows(rows, cols, a, q, scale, stream));
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

// The forward of moe_forward_ex on a given workspace.  allow_side = false keeps every launch
// on `stream` (no side stream or event is created or used).
static moe_status forward_impl(const moe_config* cfg, const moe_weights* w, const void* x,
                               void* out, void* ws, size_t ws_bytes, hipStream_t stream,
                               const moe_forward_opts* opts, bool allow_side) {
  try {
    moe_status st = check_config(cfg);
    if (st != MOE_OK) return st;
    if (w == nullptr) return MOE_ERR_INVALID_ARG;
    if (cfg->num_tokens == 0) return MOE_OK;
    if (x == nullptr || out == nullptr || w->router == nullptr) return MOE_ERR_INVALID_ARG;
    const Carve cv = carve(cfg);
    if (ws == nullptr || ws_bytes < cv.total) return MOE_ERR_WORKSPACE;
    if (!aligned16(ws) || !aligned16(x) || !aligned16(out)) return MOE_ERR_UNSUPPORTED;
    char* base = static_cast<char*>(ws);
    auto at = [&](size_t off) { return static_cast<void*>(base + off); };
    int32_t* idx = static_cast<int32_t*>(at(cv.topk_idx));
    float* tw = static_cast<float*>(at(cv.topk_w));
    int32_t* counts = static_cast<int32_t*>(at(cv.counts));
    int32_t* offsets = static_cast<int32_t*>(at(cv.offsets));
    int32_t* perm_token = static_cast<int32_t*>(at(cv.perm_token));
    int32_t* slot_pos = static_cast<int32_t*>(at(cv.slot_pos));
    float* perm_weight = static_cast<float*>(at(cv.perm_weight));
    const int T = cfg->num_tokens, Tk = cfg->num_tokens * cfg->top_k;
    const bool shared = cfg->num_shared > 0;

    // validate every grouped-GEMM argument before the first launch
    const bool a8 = cfg->fp8_act != 0;
    const bool pre = cfg->pre_norm != 0;
    if (pre && (w->norm_gamma == nullptr)) return MOE_ERR_INVALID_ARG;
    if (pre && !aligned16(w->norm_gamma)) return MOE_ERR_UNSUPPORTED;
    const void* x_in = pre ? at(cv.x_norm) : x;               // the MoE input rows
    const void* x_up = a8 ? at(cv.x_q) : x_in;                // rows of the up projections
    const float* x_up_scale = a8 ? static_cast<const float*>(at(cv.x_scale)) : nullptr;
    moe::GemmParams up_r, up_s{}, dn_r, dn_s{};
    st = gemm_params(cfg, MOE_STAGE_UP, MOE_EXPERTS_ROUTED, x_up, perm_token, offsets, Tk, w,
                     x_up_scale, at(cv.h_routed), &up_r);
    if (st != MOE_OK) return st;
    st = gemm_params(cfg, MOE_STAGE_DOWN, MOE_EXPERTS_ROUTED, at(cv.h_routed), nullptr, offsets,
                     Tk, w, perm_weight, at(cv.y_routed), &dn_r);
    if (st != MOE_OK) return st;
    if (shared) {
      st = gemm_params(cfg, MOE_STAGE_UP, MOE_EXPERTS_SHARED, x_up, nullptr, nullptr, T, w,
                       x_up_scale, at(cv.h_shared), &up_s);
      if (st != MOE_OK) return st;
      st = gemm_params(cfg, MOE_STAGE_DOWN, MOE_EXPERTS_SHARED, at(cv.h_shared), nullptr, nullptr,
                       T, w, nullptr, at(cv.y_shared), &dn_s);
      if (st != MOE_OK) return st;
    }
    if (!aligned16(w->router)) return MOE_ERR_UNSUPPORTED;
    int cus = 0;
    st = current_cus(&cus);
    if (st != MOE_OK) return st;

    hipError_t e = hipSuccess;
    auto mark = [&](int i) {
      if (opts != nullptr && opts->stage_events[i] != nullptr && e == hipSuccess)
        e = hipEventRecord(opts->stage_events[i], stream);
    };
    const bool stats = opts != nullptr && opts->load_stats != nullptr;
    if (stats && !std::isfinite(opts->aux_alpha)) return MOE_ERR_INVALID_ARG;
    bool events = false;
    for (int i = 0; opts != nullptr && i < 8; ++i) events = events || opts->stage_events[i] != nullptr;
    // few rows per expert: weight-streaming GEMMs (bf16 activations only)
    const int adt = cfg->act_dtype;
    const bool decode = !a8 && moe::decode_gemm_applies(up_r, adt) && moe::decode_gemm_applies(dn_r, adt) &&
                        (!shared || (moe::decode_gemm_applies(up_s, adt) &&
                                     moe::decode_gemm_applies(dn_s, adt)));
    // shared experts on a second stream from the start, where they overlap the routing,
    // unless the stages are being timed one by one (then, in decode, the routed and shared
    // experts stream their weights in one launch per stage)
    const SideEntry* side_ent = nullptr;
    if (shared && !events && allow_side) {
      st = side_entry(stream, &side_ent);
      if (st != MOE_OK) return st;
    }
    const bool fork = side_ent != nullptr;
    hipStream_t side = fork ? side_ent->side : nullptr;
    hipEvent_t fork_ev = fork ? side_ent->ev[0] : nullptr;
    hipEvent_t join = fork ? side_ent->ev[2] : nullptr;
    moe::RouteParams rp = route_params(cfg);
    rp.select_bias = w->select_bias;
    if (pre) {
      rp.norm_gamma = w->norm_gamma;
      rp.x_norm = at(cv.x_norm);
    }
    float* scores = stats ? static_cast<float*>(at(cv.scores)) : nullptr;
    // a small batch routes through partial logits spread over many CUs
    const bool split = moe::split_route_applies(rp, cfg->act_dtype);
    float* rpart = static_cast<float*>(at(cv.route_part));
    auto route = [&]() {
      mark(0);
      if (e == hipSuccess)
        e = split ? moe::launch_route_split(rp, x, w->router, w->logit_bias, rpart, scores, idx,
                                            tw, stream)
                  : moe::launch_route(rp, cfg->act_dtype, x, w->router, w->logit_bias, scores,
                                      idx, tw, stream);
      mark(1);
    };
    // the shared experts need only the up-projection input: x, or the normalised rows
    // written by the routing launch of a pre-norm layer (then e4m3-quantised if asked)
    if (pre) route();
    if (a8 && e == hipSuccess)
      e = moe::launch_quant_rows(T, cfg->dim, x_in, static_cast<uint8_t*>(at(cv.x_q)),
                                 static_cast<float*>(at(cv.x_scale)), stream);
    if (fork) {
      if (e == hipSuccess) e = hipEventRecord(fork_ev, stream);
      if (e == hipSuccess) e = hipStreamWaitEvent(side, fork_ev, 0);
      if (e == hipSuccess)
        e = moe::launch_grouped_gemm(up_s, moe::Stage::Up, cfg->act, adt, cfg->weight_dtype, cus,
                                     side, a8);
      if (e == hipSuccess)
        e = moe::launch_grouped_gemm(dn_s, moe::Stage::Down, cfg->act, adt, cfg->weight_dtype,
                                     cus, side);
      // recorded also after an error, so that the wait on it below orders whatever the side
      // stream took before the caller's next work (which may free the workspace)
      const hipError_t re = hipEventRecord(join, side);
      if (e == hipSuccess) e = re;
    }
    if (!pre) route();
    if (e == hipSuccess)
      e = moe::launch_permute(T, cfg->num_experts, cfg->top_k, expert_capacity(cfg), idx, tw,
                              counts, offsets, perm_token, slot_pos, perm_weight,
                              at(cv.perm_ws), stream);
    if (stats && e == hipSuccess) {
      const int E = cfg->num_experts;
      e = moe::launch_load_stats(T, E, cfg->top_k, scores, idx, opts->aux_alpha,
                                 opts->load_stats, opts->load_stats + E,
                                 opts->load_stats + 2 * E, at(cv.stats_ws), stream);
    }
    mark(2);
    if (decode) {
      const bool with_shared = shared && !fork;
      if (e == hipSuccess)
        e = moe::launch_decode_gemm(up_r, moe::Stage::Up, cfg->act, cfg->weight_dtype, stream,
                                    with_shared ? &up_s : nullptr);
      mark(3);
      mark(4);
      if (e == hipSuccess)
        e = moe::launch_decode_gemm(dn_r, moe::Stage::Down, cfg->act, cfg->weight_dtype, stream,
                                    with_shared ? &dn_s : nullptr);
      mark(5);
      mark(6);
    } else if (fork) {
      // routed GEMMs here, shared GEMMs on the side stream since the start of the forward
      if (e == hipSuccess)
        e = moe::launch_grouped_gemm(up_r, moe::Stage::Up, cfg->act, adt, cfg->weight_dtype, cus,
                                     stream, a8);
      if (e == hipSuccess)
        e = moe::launch_grouped_gemm(dn_r, moe::Stage::Down, cfg->act, adt, cfg->weight_dtype,
                                     cus, stream);
    } else {
      if (e == hipSuccess)
        e = moe::launch_grouped_gemm(up_r, moe::Stage::Up, cfg->act, adt, cfg->weight_dtype, cus,
                                     stream, a8);
      mark(3);
      if (shared && e == hipSuccess)
        e = moe::launch_grouped_gemm(up_s, moe::Stage::Up, cfg->act, adt, cfg->weight_dtype, cus,
                                     stream, a8);
      mark(4);
      if (e == hipSuccess)
        e = moe::launch_grouped_gemm(dn_r, moe::Stage::Down, cfg->act, adt, cfg->weight_dtype,
                                     cus, stream);
      mark(5);
      if (shared && e == hipSuccess)
        e = moe::launch_grouped_gemm(dn_s, moe::Stage::Down, cfg->act, adt, cfg->weight_dtype,
                                     cus, stream);
      mark(6);
    }
    if (fork) {
      // also after an error: the side stream's work is ordered before what follows
      const hipError_t we = hipStreamWaitEvent(stream, join, 0);
      if (e == hipSuccess) e = we;
    }
    if (e == hipSuccess)
      e = moe::launch_combine(T, cfg->dim, cfg->top_k, adt, at(cv.y_routed), slot_pos,
                              shared ? at(cv.y_shared) : nullptr, cfg->residual ? x : nullptr,
                              out, stream);
    mark(7);
    return hip_status(e);
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

moe_status moe_backward_workspace_size(const moe_config* cfg, size_t* bytes) {
  try {
    if (bytes == nullptr) return MOE_ERR_INVALID_ARG;
    moe_status st = check_backward_config(cfg);
    if (st != MOE_OK) return st;
    *bytes = bwd_carve(cfg).total;
    return MOE_OK;
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

moe_status moe_backward(const moe_config* cfg, const moe_weights* w, const void* x,
                        const void* dout, const void* fwd_ws, size_t fwd_ws_bytes,
                        const moe_grads* grads, void* ws, size_t ws_bytes, hipStream_t stream) {
  try {
    moe_status st = check_backward_config(cfg);
    if (st != MOE_OK) return st;
    if (cfg->num_tokens == 0) return MOE_OK;
    if (w == nullptr || x == nullptr || dout == nullptr || grads == nullptr || grads->dx == nullptr ||
        w->router == nullptr || w->w_gate == nullptr || w->w_down == nullptr)
      return MOE_ERR_INVALID_ARG;
    const bool swiglu = cfg->act == MOE_ACT_SWIGLU;
    const bool shared = cfg->num_shared > 0;
    if (swiglu && w->w_up == nullptr) return MOE_ERR_INVALID_ARG;
    if (shared && (w->sh_gate == nullptr || w->sh_down == nullptr || (swiglu && w->sh_up == nullptr)))
      return MOE_ERR_INVALID_ARG;
    const Carve cv = carve(cfg);
    if (fwd_ws == nullptr || fwd_ws_bytes < cv.total) return MOE_ERR_WORKSPACE;
    const BwdCarve bc = bwd_carve(cfg);
    if (ws == nullptr || ws_bytes < bc.total) return MOE_ERR_WORKSPACE;
    const void* ptrs[] = {x, dout, fwd_ws, ws, grads->dx, w->router, w->w_gate, w->w_up, w->w_down,
                          w->sh_gate, w->sh_up, w->sh_down};
    for (const void* q : ptrs)
      if (q != nullptr && !aligned16(q)) return MOE_ERR_UNSUPPORTED;
    int cus = 0;
    st = current_cus(&cus);
    if (st != MOE_OK) return st;

    const int T = cfg->num_tokens, k = cfg->top_k, E = cfg->num_experts, Tk = T * k;
    const int d = cfg->dim, I = cfg->inter_dim, S = cfg->num_shared, SI = S * I;
    const int nab = swiglu ? 2 : 1;
    const char* fb = static_cast<const char*>(fwd_ws);
    auto fat = [&](size_t off) { return static_cast<const void*>(fb + off); };
    char* wb = static_cast<char*>(ws);
    auto at = [&](size_t off) { return static_cast<void*>(wb + off); };
    const int32_t* idx = static_cast<const int32_t*>(fat(cv.topk_idx));
    const float* topk_w = static_cast<const float*>(fat(cv.topk_w));
    const int32_t* offsets = static_cast<const int32_t*>(fat(cv.offsets));
    const int32_t* perm_token = static_cast<const int32_t*>(fat(cv.perm_token));
    const int32_t* slot_pos = static_cast<const int32_t*>(fat(cv.slot_pos));
    const float* perm_weight = static_cast<const float*>(fat(cv.perm_weight));
    const void* h_r = fat(cv.h_routed);
    const void* h_s = fat(cv.h_shared);
    const void* y_r = fat(cv.y_routed);
    uint16_t* sh_w2t = static_cast<uint16_t*>(at(bc.sh_w2t));
    float* dw = static_cast<float*>(at(bc.dw));
    float* dl = static_cast<float*>(at(bc.dl));
    const moe_weights wt_fwd = *w;

    hipError_t e = hipSuccess;
    auto ok = [&]() { return e == hipSuccess; };
    // weight gradients: contractions over each expert's rows, read token-major
    auto wg = [&](const void* a, int lda, int a_col, const void* b, int ldb, int b_col,
                  const int32_t* offs, int nseg, int rows, int M, int N, int nsplit, float* out,
                  hipStream_t s) {
      moe::WgradParams wp{static_cast<const uint16_t*>(a), lda, a_col, static_cast<const uint16_t*>(b),
                          ldb, b_col, offs, rows, M, N, nsplit, out};
      if (ok()) e = moe::launch_wgrad(wp, nseg, cus, s);
    };
    // The shared experts' chain (steps 1-4 and 7 below for them) runs on a second stream:
    // its GEMMs overlap the routed ones, and its weight gradients, bound by the MFMAs,
    // share the CUs with the routed weight gradients, bound by their fp32 stores.  The main
    // stream waits for its dx rows before the combine and for all of it at the end.
    const SideEntry* side_ent = nullptr;
    if (shared) {
      st = side_entry(stream, &side_ent);
      if (st != MOE_OK) return st;
    }
    // without a side stream of its own (table full) the chain runs on the caller's stream
    const bool fork = side_ent != nullptr;
    hipStream_t side = fork ? side_ent->side : stream;
    hipEvent_t fork_ev = fork ? side_ent->ev[0] : nullptr;
    hipEvent_t dxs_ev = fork ? side_ent->ev[1] : nullptr;
    hipEvent_t join = fork ? side_ent->ev[2] : nullptr;
    if (shared) {
      if (fork) {
        e = hipEventRecord(fork_ev, stream);
        if (ok()) e = hipStreamWaitEvent(side, fork_ev, 0);
      }
      // 1. the shared W2 stacked [S][d][I] is not one [d][S I] matrix: a transposed copy
      //    [S I][d] for its data gradient (the routed and the other weights are read as
      //    stored)
      if (ok()) e = moe::launch_transpose_mat(w->sh_down, sh_w2t, S, d, I, (long long)I * d, d, side);
      // 2. dh = dout W2
      moe::GemmParams gs{};
      gs.a = dout; gs.nseg = 1; gs.rows = T; gs.d = d; gs.I = I; gs.S = S; gs.N = SI; gs.K = d;
      gs.kblock = d; gs.w_down = sh_w2t; gs.out = at(bc.dh_s);
      if (ok()) e = moe::launch_grouped_gemm(gs, moe::Stage::Down, cfg->act, MOE_BF16, MOE_BF16, cus, side);
      // 3. up projection recomputed, activation backward in the epilogue
      moe::GemmParams us{};
      us.a = x; us.nseg = 1; us.rows = T; us.d = d; us.I = I; us.S = S; us.N = SI; us.K = d;
      us.kblock = d; us.w_gate = w->sh_gate; us.w_up = w->sh_up; us.out = at(bc.dab_s);
      us.dact = at(bc.dh_s);
      if (ok()) e = moe::launch_up_backward(us, cfg->act, cus, side);
      // 4. dx rows: [da | db] [W1 ; W3]
      moe::GemmParams dxs{};
      dxs.a = at(bc.dab_s); dxs.nseg = 1; dxs.rows = T; dxs.d = d; dxs.I = I; dxs.S = S; dxs.N = d;
      dxs.K = nab * SI; dxs.kblock = nab * SI; dxs.w_down = w->sh_gate; dxs.w_up = w->sh_up;
      dxs.trb_split = SI; dxs.out = at(bc.dx_s);
      if (ok()) e = moe::launch_down_trb(dxs, cus, side);
      if (fork && ok()) e = hipEventRecord(dxs_ev, side);
      // 7. weight gradients
      if (grads->d_sh_down != nullptr)
        wg(dout, d, 0, h_s, SI, 0, nullptr, 1, T, d, SI, I, grads->d_sh_down, side);
      if (grads->d_sh_gate != nullptr)
        wg(at(bc.dab_s), nab * SI, 0, x, d, 0, nullptr, 1, T, SI, d, d, grads->d_sh_gate, side);
      if (swiglu && grads->d_sh_up != nullptr)
        wg(at(bc.dab_s), 2 * SI, SI, x, d, 0, nullptr, 1, T, SI, d, d, grads->d_sh_up, side);
      if (fork && ok()) e = hipEventRecord(join, side);
    }
    // 2. dh = (w dout) W2 (routed rows gathered from dout; W2 [E][d][I] is [K][N])
    moe::GemmParams g{};
    g.a = dout; g.row_index = perm_token; g.offsets = offsets; g.nseg = E; g.rows = Tk;
    g.d = d; g.I = I; g.S = S; g.N = I; g.K = d; g.kblock = d; g.w_down = w->w_down;
    g.trb_split = d; g.row_weight = perm_weight; g.out = at(bc.dh_r);
    if (ok()) e = moe::launch_down_trb(g, cus, stream);
    // 3. up projections recomputed, activation backward in the epilogue: [da | db]
    moe::GemmParams u{};
    u.a = x; u.row_index = perm_token; u.offsets = offsets; u.nseg = E; u.rows = Tk; u.d = d;
    u.I = I; u.S = S; u.N = I; u.K = d; u.kblock = d; u.w_gate = wt_fwd.w_gate; u.w_up = wt_fwd.w_up;
    u.out = at(bc.dab_r); u.dact = at(bc.dh_r);
    if (ok()) e = moe::launch_up_backward(u, cfg->act, cus, stream);
    // 4. dx of the experts: [da | db] [W1 ; W3] per permuted row; W1 and W3 [I][d] are
    //    [K][N], stacked along K
    moe::GemmParams dxg{};
    dxg.a = at(bc.dab_r); dxg.offsets = offsets; dxg.nseg = E; dxg.rows = Tk; dxg.d = d; dxg.I = I;
    dxg.S = S; dxg.N = d; dxg.K = nab * I; dxg.kblock = nab * I; dxg.w_down = w->w_gate;
    dxg.w_up = w->w_up; dxg.trb_split = I; dxg.out = at(bc.dxp_r);
    if (ok()) e = moe::launch_down_trb(dxg, cus, stream);
    // 5. router: scores recomputed, routing-weight and logit gradients
    moe::RouteParams rp = route_params(cfg);
    rp.select_bias = w->select_bias;
    if (ok())
      e = moe::launch_route(rp, MOE_BF16, x, w->router, w->logit_bias, static_cast<float*>(at(bc.scores)),
                            static_cast<int32_t*>(at(bc.idx)), static_cast<float*>(at(bc.tw)), stream);
    if (ok()) e = moe::launch_routing_weight_grad(T, k, d, dout, y_r, slot_pos, topk_w, dw, stream);
    if (ok()) e = moe::launch_router_grad(rp, static_cast<const float*>(at(bc.scores)), idx, dw, dl, stream);
    if (ok() && (grads->d_router != nullptr || grads->d_logit_bias != nullptr))
      e = moe::launch_router_wgrad(T, d, E, x, dl, grads->d_router, grads->d_logit_bias, at(bc.rg), stream);
    // 6. dx = dl W_r + experts (+ dout)
    if (fork && ok()) e = hipStreamWaitEvent(stream, dxs_ev, 0);
    if (ok())
      e = moe::launch_dx_combine(T, d, E, k, dl, w->router, at(bc.dxp_r), slot_pos,
                                 shared ? at(bc.dx_s) : nullptr, cfg->residual ? dout : nullptr,
                                 grads->dx, stream);
    // 7. weight gradients of the routed experts: the x rows and the weighted dout rows are
    //    first copied into permuted order
    if (grads->d_w_down != nullptr) {
      if (ok()) e = moe::launch_gather_rows(dout, perm_token, perm_weight, offsets + E, Tk, d,
                                             at(bc.dy_perm), stream);
      wg(at(bc.dy_perm), d, 0, h_r, I, 0, offsets, E, Tk, d, I, I, grads->d_w_down, stream);
    }
    if (grads->d_w_gate != nullptr || (swiglu && grads->d_w_up != nullptr)) {
      if (ok()) e = moe::launch_gather_rows(x, perm_token, nullptr, offsets + E, Tk, d, at(bc.x_perm),
                                             stream);
      if (grads->d_w_gate != nullptr)
        wg(at(bc.dab_r), nab * I, 0, at(bc.x_perm), d, 0, offsets, E, Tk, I, d, d, grads->d_w_gate,
           stream);
      if (swiglu && grads->d_w_up != nullptr)
        wg(at(bc.dab_r), 2 * I, I, at(bc.x_perm), d, 0, offsets, E, Tk, I, d, d, grads->d_w_up,
           stream);
    }
    if (fork) {
      // also after an error: the side stream's work is ordered before what follows
      const hipError_t we = hipStreamWaitEvent(stream, join, 0);
      if (ok()) e = we;
    }
    return hip_status(e);
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

moe_status moe_gemm_kernel_path(const moe_config* cfg, moe_stage stage, moe_expert_set set,
                                int32_t rows, int32_t* path) {
  try {
    if (path == nullptr || rows < 0) return MOE_ERR_INVALID_ARG;
    moe_status st = check_config(cfg);
    if (st != MOE_OK) return st;
    if (stage != MOE_STAGE_UP && stage != MOE_STAGE_DOWN) return MOE_ERR_INVALID_ARG;
    if (set != MOE_EXPERTS_ROUTED && set != MOE_EXPERTS_SHARED) return MOE_ERR_INVALID_ARG;
    const bool routed = set == MOE_EXPERTS_ROUTED;
    if (!routed && cfg->num_shared == 0) return MOE_ERR_INVALID_ARG;
    // the shape fields of the launch parameters (pointers only as markers: never read)
    static const int32_t marker = 0;
    const int I_eff = routed ? cfg->inter_dim : cfg->num_shared * cfg->inter_dim;
    moe::GemmParams g{};
    g.offsets = routed ? &marker : nullptr;
    g.nseg = routed ? cfg->num_experts : 1;
    g.rows = rows;
    const bool up = stage == MOE_STAGE_UP;
    g.N = up ? I_eff : cfg->dim;
    g.K = up ? cfg->dim : I_eff;
    g.kblock = up ? cfg->dim : cfg->inter_dim;
    if (up && cfg->fp8_act) *path = MOE_GEMM_PATH_FP8_ACT;
    else if (cfg->act_dtype == MOE_F32) *path = MOE_GEMM_PATH_F32;
    else if (moe::tail_gemm_applies(g)) *path = MOE_GEMM_PATH_TAIL;
    else if (moe::decode_gemm_applies(g, cfg->act_dtype)) *path = MOE_GEMM_PATH_DECODE;
    else *path = MOE_GEMM_PATH_TILED;
    return MOE_OK;
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

moe_status moe_forward_ex(const moe_config* cfg, const moe_weights* w, const void* x, void* out,
                          void* ws, size_t ws_bytes, hipStream_t stream,
                          const moe_forward_opts* opts) {
  return forward_impl(cfg, w, x, out, ws, ws_bytes, stream, opts, true);
}

moe_status moe_forward(const moe_config* cfg, const moe_weights* w, const void* x, void* out,
                       void* ws, size_t ws_bytes, hipStream_t stream) {
  return moe_forward_ex(cfg, w, x, out, ws, ws_bytes, stream, nullptr);
}

moe_status moe_forward_noalloc(const moe_config* cfg, const moe_weights* w, const void* x,
                               void* out, hipStream_t stream) {
  try {
    moe_status st = check_config(cfg);
    if (st != MOE_OK) return st;
    if (carve(cfg).total > kScratchBytes) return MOE_ERR_WORKSPACE;
    if (cfg->num_tokens == 0) return MOE_OK;
    void* scratch_ptr = nullptr;
    st = device_scratch(&scratch_ptr);
    if (st != MOE_OK) return st;
    return forward_impl(cfg, w, x, out, scratch_ptr, kScratchBytes, stream, nullptr, false);
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

}  // extern "C"
