"""Plain fp64 CPU oracle of the fine-grained MoE FFN forward.

TEST INFRASTRUCTURE ONLY.  Imported by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``; nothing in the library (``include/``,
``sparse_mixture_experts_gemm_amd/``) imports, links or runs it, and it shares no code
with the HIP path.  It is slow on purpose: every step is the plain definition, in fp64,
on the exact values of the stored inputs (bf16 / fp32 / e4m3 x scale decoded exactly).

Sources (web pages, cited by title and section):

* [MoE-Eng] "大模型工程（一）：Transformer 到 MoE":
  - section "混合专家：更多参数，相同 FLOPs", the MoEBlock listing: a bias-free gate
    ``Linear(d_model, n_experts)``, top-k over the gate scores, softmax over the k
    selected values, and for every slot and expert a masked, weighted sum of SwiGLU
    expert outputs.
  - section "MoE 数学：路由、容量与平衡详解": the router is the linear map g(x) = W_g x,
    deterministic top-k with a fixed k per token, an always-on shared expert next to the
    routed ones, and capacity c = infinity at inference (no token is dropped).
  - section "变了什么，为什么变", item 3: SwiGLU (a gated FFN with gate, up and down
    projections), citing Shazeer's "GLU variants" paper.
* [FusionLLM] "FusionLLM：融合 MLA、GDN 与 MoE 的高效混合架构大模型训练框架":
  - section "混合专家（MoE）": fine-grained DeepSeekMoE, 64 routed / 6 active experts,
    group-limited routing and bias-free sigmoid gating.
  - section "融合内核": a fused Linear+ReLU^2 FFN kernel and grouped GEMM after routing.
  - section "模型配置与规模" (YAML): dim 2048, n_routed_experts 64,
    n_activated_experts 6, n_shared_experts 4, moe_inter_dim 1536.
* [MoE-Explainer] "开源混合架构大模型技术解析", section "四、工作原理：稀疏激活如何运行":
  gate scores -> top-k experts -> only those experts run -> outputs merged by the gate
  weights.

Readings where the pages are silent (each one is a convention, stated here and in the
design notes):

* Group-limited routing is only named.  Groups are contiguous blocks of E/G experts; a
  group's score is the sum of its n_g largest expert scores (n_g = 1: the group max);
  the Gk best groups are kept and the top-k is taken over experts of kept groups.
  PARITY UNPINNED as a reading: the pages fix no group-scoring rule; the brute-force
  tests pin only that this module computes the rule stated here.
* Ties: equal scores -> lower expert index first; equal group scores -> lower group
  index first.  Slot order: score descending.
* Weights: renormalised over the k selected scores, times route_scale (1.0).
* Selection is decided on fp32 scores (the kernel's precision): ``route`` rounds the
  fp64 scores to fp32 before selecting; group sums for n_g = 2 are fp32 adds.
  The weights use the fp64 scores.
* Shared experts: S independent FFNs of inter dim I, weight 1, applied to every token.
* ReLU^2 expert: W2 (max(W1 x, 0))^2, no gate/up pair.
* e4m3 expert weights: W[n, :] = scale[n] * e4m3(code[n, :]) (OCP e4m3, bias 7, max 448,
  0x7F/0xFF NaN); activations stay bf16.
* Selection-only expert bias b_e (the aux-loss-free balancing of [MoE-Eng] "负载均衡"):
  the selection compares the scores of l + b (sigmoid or softmax of the biased logits);
  the weights are the unbiased scores of the selected experts, renormalised.
* Load statistics: f_e counts routed (token, slot) assignments before any capacity drop,
  divided by T k; p_e averages each token's scores normalised to sum 1 over the E experts.
* Capacity: floor(c T k / E) rows per expert; each expert keeps its rows in token order
  and drops the rest (dropped slots contribute zero; weights are not renormalised).
* e4m3 activations (optional, with e4m3 weights): each token's x row is quantised with
  its own scale max|x|/448 in fp32 steps (RNE, saturating) before the up projections;
  the router and the down projections are unchanged.
* Pre-norm layer step (optional): the MoE input is RMSNorm(x) = x / sqrt(mean(x^2) + eps)
  * gamma (no mean subtraction, a learned per-channel gain gamma), stored in the
  activation dtype (one rounding of the exact value) before the router and the experts
  read it; with the residual option the unnormalised x is added to the output.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "decode_bf16", "decode_e4m3", "decode_weight", "router_logits", "gate_scores",
    "group_scores", "select_experts", "routing_weights", "route", "silu", "expert_ffn",
    "expert_up", "expert_down", "combine",
    "moe_forward", "permute", "expert_weights", "shared_weights", "decode_act",
    "selection_keys", "load_stats", "expert_capacity", "quantize_rows_e4m3",
    "dequantize_rows_e4m3", "rms_norm", "round_to_act", "normalized_input",
]


# ----------------------------------------------------------------------------- codecs
def decode_bf16(bits) -> np.ndarray:
    """bf16 bit patterns -> fp64.  A bf16 value is the upper half of an IEEE fp32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def decode_e4m3(codes) -> np.ndarray:
    """OCP e4m3 (FN) codes -> fp64: sign s, 4-bit exponent E (bias 7), 3-bit mantissa M.

    normal (E > 0): (-1)^s 2^(E-7) (1 + M/8); subnormal (E = 0): (-1)^s 2^-6 (M/8);
    E = 15 and M = 7 is NaN (no infinities).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    val = np.where(s == 1, -mag, mag)
    return np.where((e == 15) & (m == 7), np.nan, val)


def decode_act(a, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return decode_bf16(a)
    raise ValueError(dtype)


def decode_weight(w, dtype: str, scale=None) -> np.ndarray:
    """Stored expert weight -> fp64; e4m3 rows are multiplied by their fp32 scale."""
    if dtype in ("f32", "bf16"):
        return decode_act(w, dtype)
    if dtype == "e4m3":
        return decode_e4m3(w) * np.asarray(scale, dtype=np.float64)[..., None]
    raise ValueError(dtype)


# ----------------------------------------------------------------------------- routing
def router_logits(x, w_r, logit_bias=None) -> np.ndarray:
    """l[t, e] = sum_c x[t, c] W_r[e, c] (+ b[e]).  [MoE-Eng] g(x) = W_g x, no bias term
    in the gate itself; b is the optional per-expert logit offset of the skewed workload."""
    l = np.asarray(x, np.float64) @ np.asarray(w_r, np.float64).T
    if logit_bias is not None:
        l = l + np.asarray(logit_bias, np.float64)[None, :]
    return l


def gate_scores(logits, fn: str) -> np.ndarray:
    """sigmoid per expert ([FusionLLM] sigmoid gating) or softmax over all experts."""
    l = np.asarray(logits, np.float64)
    if fn == "sigmoid":
        return 1.0 / (1.0 + np.exp(-l))
    if fn == "softmax":
        z = np.exp(l - l.max(axis=-1, keepdims=True))
        return z / z.sum(axis=-1, keepdims=True)
    raise ValueError(fn)


def group_scores(scores, G: int, n_g: int) -> np.ndarray:
    """Score of each of G contiguous expert groups: sum of its n_g largest scores.

    Computed in the dtype of ``scores`` (fp32 input -> fp32 adds)."""
    s = np.asarray(scores)
    T, E = s.shape
    sg = np.sort(s.reshape(T, G, E // G), axis=-1)[..., ::-1]
    acc = sg[..., 0].copy()
    for i in range(1, n_g):
        acc = acc + sg[..., i]
    return acc


def select_experts(scores, k: int, G: int = 1, Gk: int = 1, n_g: int = 1) -> np.ndarray:
    """Group-limited top-k.  Returns idx [T, k] int32, slot order score-descending.

    1. rank groups by (group score desc, group index asc) and keep the first Gk;
    2. rank experts of kept groups by (score desc, expert index asc) and take k.
    The comparisons are made on the values of ``scores`` exactly as given."""
    s = np.asarray(scores)
    T, E = s.shape
    if G > 1 and Gk < G:
        gs = group_scores(s, G, n_g)
        gidx = np.broadcast_to(np.arange(G), (T, G))
        gorder = np.lexsort((gidx, -gs), axis=-1)          # primary: -gs, then index
        kept = np.zeros((T, G), dtype=bool)
        np.put_along_axis(kept, gorder[:, :Gk], True, axis=-1)
        eligible = np.repeat(kept, E // G, axis=1)
    else:
        eligible = np.ones((T, E), dtype=bool)
    eidx = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((eidx, -s, ~eligible), axis=-1)     # eligible first, -s, index
    return order[:, :k].astype(np.int32)


def routing_weights(scores64, idx, renormalize: bool = True, route_scale: float = 1.0):
    """w_j = route_scale * s_{e_j} / sum_i s_{e_i} (fp64).  [MoE-Eng] MoEBlock: softmax
    over the selected values, i.e. the selected probabilities renormalised to sum 1."""
    sel = np.take_along_axis(np.asarray(scores64, np.float64), np.asarray(idx, np.int64), axis=-1)
    if renormalize:
        sel = sel / sel.sum(axis=-1, keepdims=True)
    return sel * route_scale


def selection_keys(logits, fn: str, select_bias=None) -> np.ndarray:
    """The values the expert selection compares.  Without a selection bias these are the
    gate scores; with one, the scores of the biased logits l + b_e.  [MoE-Eng] section
    "MoE 数学：路由、容量与平衡详解" (and "负载均衡"): the per-expert bias b_e enters the
    gate logits for the assignment only; the weights keep coming from the unbiased
    scores."""
    l = np.asarray(logits, np.float64)
    if select_bias is not None:
        l = l + np.asarray(select_bias, np.float64)[None, :]
    return gate_scores(l, fn)


def route(layer, tokens=None, x=None):
    """Router of a stored layer: returns dict(logits, scores, keys, idx, w) in fp64 (idx
    int32).  The selection is decided on the fp32-rounded selection keys (group sums in
    fp32); the weights use the unbiased fp64 scores.  ``x`` (fp64 rows, already restricted
    to ``tokens``) replaces the layer's stored input, e.g. by its normalised rows."""
    s = layer.shape
    if x is None:
        x = decode_act(layer.x if tokens is None else layer.x[tokens], s.act_dtype)
    w_r = decode_act(layer.router, s.act_dtype)
    l = router_logits(x, w_r, layer.logit_bias)
    sc = gate_scores(l, s.score)
    sb = getattr(layer, "select_bias", None)
    keys = sc if sb is None else selection_keys(l, s.score, sb)
    idx = select_experts(keys.astype(np.float32), s.k, s.G, s.Gk, s.n_g)
    w = routing_weights(sc, idx, s.renormalize, s.route_scale)
    return {"x": x, "logits": l, "scores": sc, "keys": keys, "idx": idx, "w": w}


# ----------------------------------------------------------------------------- pre-norm
def rms_norm(x, gamma, eps: float):
    """RMSNorm of every row (fp64): y = x / sqrt(mean_c x_c^2 + eps) * gamma.

    [MoE-Eng] section "变了什么，为什么变": item 2 (RMSNorm drops LayerNorm's mean and keeps
    only the root-mean-square scaling) and the decoder-layer sketch, where the MoE reads
    rms_norm(h) and its output is added back to h; section "常见陷阱", item 3 (eps 1e-6
    for bf16 training).  The per-channel gain gamma is the reading taken for the learned
    scale the pages do not print."""
    x = np.asarray(x, np.float64)
    ms = np.mean(x * x, axis=1, keepdims=True)
    return x / np.sqrt(ms + float(eps)) * np.asarray(gamma, np.float64)[None, :]


def round_to_act(v, dtype: str) -> np.ndarray:
    """fp64 values to the nearest value of the activation dtype, ties to even, in one
    rounding step (bf16: 8 significant bits; fp32: IEEE single).  Returns fp64."""
    v = np.asarray(v, np.float64)
    if dtype == "f32":
        return v.astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        m, e = np.frexp(v)                           # v = m 2^e, 0.5 <= |m| < 1
        return np.ldexp(np.rint(m * 256.0), e - 8)   # rint: ties to even
    raise ValueError(dtype)


def normalized_input(layer, tokens=None):
    """The stored MoE input of a pre-norm layer: RMSNorm of the x rows with the layer's
    gain and eps (as fp32, the stored precision), rounded to the activation dtype."""
    s = layer.shape
    x = decode_act(layer.x if tokens is None else layer.x[tokens], s.act_dtype)
    eps = float(np.float32(s.norm_eps))
    return round_to_act(rms_norm(x, layer.norm_gamma, eps), s.act_dtype)


# ----------------------------------------------------------------------------- e4m3 activations
def _e4m3_rne_magnitude(v32):
    """|v| (fp32, <= 448) to the nearest e4m3 magnitude code, ties to even.  Normal codes
    (|v| >= 2^-6) keep 3 mantissa bits of the fp32 value; subnormals are multiples of
    2^-9.  Returns codes 0..126."""
    a = np.abs(np.asarray(v32, np.float64))
    codes = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    m_sub = np.rint(a[sub] * 512.0).astype(np.int64)        # exact scaling; rint = RNE
    codes[sub] = m_sub                                      # m = 8 is the smallest normal
    nrm = ~sub
    e = np.floor(np.log2(a[nrm])).astype(np.int64)          # exact for fp32 inputs
    frac = a[nrm] / np.ldexp(1.0, e) - 1.0                  # in [0, 1), exact
    m = np.rint(frac * 8.0).astype(np.int64)                # RNE on the 3-bit mantissa
    carry = m == 8
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 0, m)
    codes[nrm] = (e + 7) * 8 + m
    return codes


def quantize_rows_e4m3(a):
    """Per-row e4m3 quantisation of activations, in the kernel's fp32 steps: scale =
    fp32(max|a_row|) / 448 (fp32 division), v = a / scale (fp32 division), clamp |v| to
    448, round to the nearest e4m3 value with ties to even, keep the sign.  A row of zeros
    has scale 0 and codes 0.  Returns (codes uint8 [rows, cols], scales float32 [rows]).
    [MoE-Eng] section "生产现实：前沿实验室真正交付的内容", FP8 item (E4M3 products with FP32
    accumulation); the per-token
    scale is the reading taken for activations."""
    a32 = np.asarray(a, np.float32)
    amax = np.max(np.abs(a32), axis=1)
    scale = (amax / np.float32(448.0)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    v = (a32 / safe[:, None]).astype(np.float32)
    mag = np.minimum(np.abs(v), np.float32(448.0))
    codes = _e4m3_rne_magnitude(mag)
    codes = np.where(scale[:, None] > 0, codes, 0)
    sign = (v < 0) & (codes > 0)
    out = (codes | np.where(sign, 0x80, 0)).astype(np.uint8)
    return out, scale


def dequantize_rows_e4m3(codes, scale):
    return decode_e4m3(codes) * np.asarray(scale, np.float64)[:, None]


# ----------------------------------------------------------------------------- load statistics
def load_stats(scores, idx, E: int, alpha: float = 1.0):
    """Per-batch load statistics of the router and the Switch auxiliary-loss value.

    [MoE-Eng] section "负载均衡": loss = alpha * E * sum_e f_e p_e, with f_e the fraction of
    the routed (token, slot) assignments that went to expert e and p_e its mean routing
    probability.  The probability of expert e for token t is its gate score divided by the
    token's sum over all E experts (the softmax itself for softmax gating; the normalised
    sigmoid scores otherwise).  Returns (f [E], p [E], loss)."""
    sc = np.asarray(scores, np.float64)
    idx = np.asarray(idx, np.int64)
    T, k = idx.shape
    f = np.bincount(idx.reshape(-1), minlength=E).astype(np.float64) / float(T * k)
    prob = sc / sc.sum(axis=1, keepdims=True)
    p = prob.mean(axis=0)
    return f, p, float(alpha * E * np.sum(f * p))


# ----------------------------------------------------------------------------- experts
def silu(z):
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_up(x, w1, w3, act: str):
    """First half of an expert on rows x [n, d]: silu(W1 x) * (W3 x) for SwiGLU, or
    max(W1 x, 0)^2 for ReLU^2.  Weights in nn.Linear layout [out, in]."""
    a = x @ w1.T
    if act == "swiglu":
        return silu(a) * (x @ w3.T)
    if act == "relu2":
        return np.maximum(a, 0.0) ** 2
    raise ValueError(act)


def expert_down(h, w2):
    """Down projection W2 h of the inter activations h [n, I]; W2 is [d, I]."""
    return h @ w2.T


def expert_ffn(x, w1, w3, w2, act: str):
    """One expert on rows x [n, d]: SwiGLU W2 (silu(W1 x) * (W3 x)), or ReLU^2
    W2 (max(W1 x, 0))^2.  Weights in nn.Linear layout [out, in]."""
    return expert_down(expert_up(x, w1, w3, act), w2)


def combine(y_perm, slot_pos, y_shared, k: int):
    """out[t] = sum_j y_perm[slot_pos[t*k + j]] (+ y_shared[t]): the merge of the k weighted
    expert outputs of every token back into token order (slots dropped by a capacity limit,
    slot_pos -1, contribute nothing)."""
    y = np.asarray(y_perm, np.float64)
    sp = np.asarray(slot_pos, np.int64).reshape(-1, k)
    out = np.where((sp >= 0)[..., None], y[np.maximum(sp, 0)], 0.0).sum(axis=1)
    if y_shared is not None:
        out = out + np.asarray(y_shared, np.float64)
    return out


def expert_weights(layer, e: int):
    s = layer.shape
    dt = s.weight_dtype
    sc = lambda a: None if a is None else a[e]
    w1 = decode_weight(layer.w_gate[e], dt, sc(layer.s_gate))
    w3 = None if layer.w_up is None else decode_weight(layer.w_up[e], dt, sc(layer.s_up))
    w2 = decode_weight(layer.w_down[e], dt, sc(layer.s_down))
    return w1, w3, w2


def shared_weights(layer, i: int):
    s = layer.shape
    dt = s.weight_dtype
    sc = lambda a: None if a is None else a[i]
    w1 = decode_weight(layer.sh_gate[i], dt, sc(layer.sh_s_gate))
    w3 = None if layer.sh_up is None else decode_weight(layer.sh_up[i], dt, sc(layer.sh_s_up))
    w2 = decode_weight(layer.sh_down[i], dt, sc(layer.sh_s_down))
    return w1, w3, w2


def moe_forward(layer, tokens=None, idx=None):
    """out[t] = sum_j w_j FFN_{e_j}(x_t) + sum_s FFN^shared_s(x_t)  (fp64).

    The masked per-(slot, expert) loop of the MoEBlock listing, with the slot loop folded
    into the mask: for each expert, the tokens that picked it in any slot.  ``tokens``
    restricts the computation to a subset of rows (every step is per token).  With a
    capacity factor, slots dropped by the capacity limit contribute nothing; which slots
    are dropped depends on the whole batch, so the routing of all tokens decides it
    (computed from the fp32 capacity factor, as stored).  ``idx`` [T, k] replaces the
    selection with a given one for the whole batch (the weights stay the renormalised
    fp64 scores of those experts), for comparing outputs under a routing that was checked
    separately.  A pre-norm layer routes and runs its experts on the normalised rows
    (``normalized_input``) and, with the residual option, adds the stored x."""
    s = layer.shape
    pre = getattr(s, "pre_norm", False)
    x_in = normalized_input(layer, tokens) if pre else None
    r = route(layer, tokens, x=x_in)
    if idx is not None:
        idx_all = np.asarray(idx, np.int32)
        r["idx"] = idx_all if tokens is None else idx_all[np.asarray(tokens)]
        r["w"] = routing_weights(r["scores"], r["idx"], s.renormalize, s.route_scale)
    x, idx_t, w = r["x"], r["idx"], r["w"]
    kept = np.ones(idx_t.shape, dtype=bool)
    cf = getattr(s, "capacity_factor", None)
    if cf is not None:
        if idx is not None:
            full_idx = np.asarray(idx, np.int32)
        else:
            full_idx = (r if tokens is None else
                        route(layer, x=normalized_input(layer) if pre else None))["idx"]
        cap = expert_capacity(s.T, s.k, s.E, float(np.float32(cf)))
        _, _, _, slot_pos = permute(full_idx, s.E, cap)
        kept_all = slot_pos.reshape(s.T, s.k) >= 0
        kept = kept_all if tokens is None else kept_all[np.asarray(tokens)]
    r["kept"] = kept
    # with e4m3 activations the up projections see each token's quantised row (the router
    # keeps the unquantised x)
    xa = x
    if getattr(s, "fp8_act", False):
        xa = dequantize_rows_e4m3(*quantize_rows_e4m3(x))
    out = np.zeros_like(x)
    for e in range(s.E):
        rows, slots = np.nonzero((idx_t == e) & kept)
        if rows.size == 0:
            continue
        w1, w3, w2 = expert_weights(layer, e)
        out[rows] += w[rows, slots][:, None] * expert_ffn(xa[rows], w1, w3, w2, s.act)
    for i in range(s.S):
        w1, w3, w2 = shared_weights(layer, i)
        out += expert_ffn(xa, w1, w3, w2, s.act)
    if getattr(s, "residual", False):
        out = out + decode_act(layer.x if tokens is None else layer.x[tokens], s.act_dtype)
    r["out"] = out
    return r


# ----------------------------------------------------------------------------- permutation
def expert_capacity(T: int, k: int, E: int, factor: float) -> int:
    """Rows an expert may take in one batch: floor(c * T * k / E).  [MoE-Eng] section
    "MoE 数学：路由、容量与平衡详解" gives the capacity c |T| k / E; a row count is an
    integer, and the reading taken is to round down."""
    return int(math.floor(factor * T * k / E))


def permute(idx, E: int, capacity=None):
    """Rows grouped by expert: order of (expert asc, token asc) over all (t, j) slots.

    Returns counts [E], offsets [E+1] (exclusive scan of counts), perm_token [rows]
    (token of permuted row p) and slot_pos [T*k] (permuted row of slot t*k + j).  With a
    capacity, each expert keeps its first ``capacity`` slots in that order (the tokens
    beyond it are dropped: they bypass the expert and contribute nothing, [MoE-Eng]
    section "MoE 数学：路由、容量与平衡详解"); counts are the kept rows and dropped slots
    have slot_pos -1."""
    idx = np.asarray(idx, dtype=np.int64)
    T, k = idx.shape
    e_flat = idx.reshape(-1)
    t_flat = np.repeat(np.arange(T), k)
    order = np.lexsort((t_flat, e_flat))            # stable: expert, then token
    routed = np.bincount(e_flat, minlength=E)
    start = np.concatenate([[0], np.cumsum(routed)])
    rank = np.arange(T * k) - start[e_flat[order]]    # position inside the expert's run
    keep = np.ones(T * k, dtype=bool) if capacity is None else rank < capacity
    counts = np.minimum(routed, capacity if capacity is not None else routed).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    perm_token = t_flat[order][keep].astype(np.int32)
    slot_pos = np.full(T * k, -1, dtype=np.int32)
    slot_pos[order[keep]] = np.arange(int(keep.sum()), dtype=np.int32)
    return counts, offsets, perm_token, slot_pos
