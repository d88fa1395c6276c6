"""Plain fp64 CPU oracle of the MoE FFN layer's backward pass (gradients).

TEST INFRASTRUCTURE ONLY, like ``moe_oracle``: imported by ``tests/`` and nothing in the
library; it shares no code with the HIP path.

The layer's forward is the one in ``moe_oracle``; the backward is its chain rule, written
out step by step in fp64 on the exact values of the stored inputs.  The routing decision
(which experts a token uses, and which slots a capacity drops) is piecewise constant, so
its derivative is zero almost everywhere; everything else is differentiable:

* expert FFNs: SwiGLU W2 (silu(W1 x) * (W3 x)) or ReLU^2 W2 (max(W1 x, 0))^2
  ([MoE-Eng] "大模型工程（一）：Transformer 到 MoE", section "变了什么，为什么变", item 3;
  [FusionLLM] section "融合内核");
* routing weights w_j = c s_j / sum_i s_i over the selected experts (or c s_j), from
  sigmoid or softmax scores of the logits l = W_r x + b ([MoE-Eng] MoEBlock listing and
  section "MoE 数学：路由、容量与平衡详解");
* the router gradient flows through the full logits: with softmax scores every logit
  receives gradient, not only the selected ones, as the pitfall list of [MoE-Eng]
  (section "常见陷阱", item 4) requires;
* shared experts with weight 1; the optional residual adds dout to dx.

Readings: the selection-only bias has no gradient (it only moves the assignment); a slot
dropped by the capacity contributes nothing to the output, but its score still sits in
the renormalisation sum of the kept slots and receives gradient through it.  The pre-norm
step and e4m3 weights or activations are outside this backward.
"""
from __future__ import annotations

import numpy as np

from .moe_oracle import (decode_act, decode_weight, expert_capacity, gate_scores, permute,
                         route, routing_weights, silu)

__all__ = ["layer_params", "forward_params", "moe_backward", "routed_slots_kept"]


def layer_params(layer) -> dict:
    """Every differentiable input of a stored layer as fp64 arrays."""
    s = layer.shape
    if s.weight_dtype == "e4m3" or getattr(s, "pre_norm", False) or getattr(s, "fp8_act", False):
        raise ValueError("the backward oracle covers bf16/fp32 layers without the pre-norm step")
    dt = s.weight_dtype
    P = {
        "x": decode_act(layer.x, s.act_dtype),
        "router": decode_act(layer.router, s.act_dtype),
        "bias": (np.zeros(s.E) if layer.logit_bias is None
                 else np.asarray(layer.logit_bias, np.float64)),
        "w1": decode_weight(layer.w_gate, dt),
        "w3": None if layer.w_up is None else decode_weight(layer.w_up, dt),
        "w2": decode_weight(layer.w_down, dt),
    }
    if s.S > 0:
        P["sh_w1"] = decode_weight(layer.sh_gate, dt)
        P["sh_w3"] = None if layer.sh_up is None else decode_weight(layer.sh_up, dt)
        P["sh_w2"] = decode_weight(layer.sh_down, dt)
    return P


def routed_slots_kept(shape, idx) -> np.ndarray:
    """[T, k] mask of the slots that reach their expert (all, unless a capacity drops some)."""
    idx = np.asarray(idx, np.int32)
    cf = getattr(shape, "capacity_factor", None)
    if cf is None:
        return np.ones(idx.shape, dtype=bool)
    cap = expert_capacity(shape.T, shape.k, shape.E, float(np.float32(cf)))
    _, _, _, slot_pos = permute(idx, shape.E, cap)
    return slot_pos.reshape(idx.shape) >= 0


def _scores(shape, P):
    l = P["x"] @ P["router"].T + P["bias"][None, :]
    return gate_scores(l, shape.score)


def _up(x, w1, w3, act):
    a = x @ w1.T
    if act == "swiglu":
        b = x @ w3.T
        return a, b, silu(a) * b
    return a, None, np.maximum(a, 0.0) ** 2


def forward_params(shape, P, idx, kept=None) -> np.ndarray:
    """The layer output [T, d] from fp64 parameters with the selection ``idx`` held fixed
    (the function the backward differentiates)."""
    idx = np.asarray(idx, np.int64)
    kept = np.ones(idx.shape, bool) if kept is None else kept
    x = P["x"]
    w = routing_weights(_scores(shape, P), idx, shape.renormalize, shape.route_scale)
    out = np.zeros_like(x)
    for e in range(shape.E):
        rows, slots = np.nonzero((idx == e) & kept)
        if rows.size == 0:
            continue
        _, _, h = _up(x[rows], P["w1"][e], None if P["w3"] is None else P["w3"][e], shape.act)
        out[rows] += w[rows, slots][:, None] * (h @ P["w2"][e].T)
    for i in range(shape.S):
        _, _, h = _up(x, P["sh_w1"][i], None if P["sh_w3"] is None else P["sh_w3"][i], shape.act)
        out += h @ P["sh_w2"][i].T
    if getattr(shape, "residual", False):
        out = out + x
    return out


def _act_backward(a, b, dh, act):
    """Gradients of the activation's inputs: SwiGLU h = silu(a) b, ReLU^2 h = max(a, 0)^2."""
    if act == "swiglu":
        sig = 1.0 / (1.0 + np.exp(-a))
        return dh * b * sig * (1.0 + a * (1.0 - sig)), dh * silu(a)   # d silu(a)/da
    return dh * 2.0 * np.maximum(a, 0.0), None


def _weights_to_scores(dw, sel, c, renormalize):
    """d/ds of w_j = c s_j / sum_i s_i over the selected scores sel [T, k] (or w = c s)."""
    if not renormalize:
        return c * dw
    tot = sel.sum(axis=1, keepdims=True)
    return (c / tot) * (dw - np.sum(dw * sel, axis=1, keepdims=True) / tot)


def _scores_to_logits(ds, sc, fn):
    """d/dl of the scores: sigmoid per expert, softmax over all E logits."""
    if fn == "sigmoid":
        return ds * sc * (1.0 - sc)
    return sc * (ds - np.sum(ds * sc, axis=1, keepdims=True))


def _ffn_backward(x, w1, w3, w2, act, g):
    """One expert on rows x [n, d] with upstream gradient g [n, d] of its (unweighted)
    output: returns (y_hat, dx, dW1, dW3, dW2)."""
    a, b, h = _up(x, w1, w3, act)
    y = h @ w2.T
    dW2 = g.T @ h                       # [d, I]
    dh = g @ w2                         # [n, I]
    da, db = _act_backward(a, b, dh, act)
    if act == "swiglu":
        dW3 = db.T @ x
        dx = da @ w1 + db @ w3
    else:
        dW3 = None
        dx = da @ w1
    dW1 = da.T @ x
    return y, dx, dW1, dW3, dW2


def moe_backward(layer, dout, idx=None) -> dict:
    """Gradients of sum(dout * out) for a stored layer, fp64.

    ``idx`` [T, k] fixes the selection (default: the oracle's own routing).  Returns dx,
    dW1, dW3, dW2 (routed, [E, ...]), sh_dW1, sh_dW3, sh_dW2 ([S, ...]), drouter [E, d],
    dbias [E], dw [T, k] (gradient of each slot's routing weight), dl [T, E] (of the
    logits), and the idx and kept mask used."""
    s = layer.shape
    P = layer_params(layer)
    g = np.asarray(dout, np.float64)
    if idx is None:
        idx = route(layer)["idx"]
    idx = np.asarray(idx, np.int64)
    kept = routed_slots_kept(s, idx)
    x = P["x"]
    T, k = idx.shape
    sc = _scores(s, P)
    w = routing_weights(sc, idx, s.renormalize, s.route_scale)

    dx = np.zeros_like(x)
    dW1 = np.zeros_like(P["w1"])
    dW3 = None if P["w3"] is None else np.zeros_like(P["w3"])
    dW2 = np.zeros_like(P["w2"])
    dw = np.zeros((T, k))
    for e in range(s.E):
        rows, slots = np.nonzero((idx == e) & kept)
        if rows.size == 0:
            continue
        we = w[rows, slots][:, None]
        # the slot's output is w * y_hat: y_hat's upstream gradient is w * dout
        y, dxe, d1, d3, d2 = _ffn_backward(x[rows], P["w1"][e],
                                           None if P["w3"] is None else P["w3"][e],
                                           P["w2"][e], s.act, we * g[rows])
        dw[rows, slots] = np.sum(g[rows] * y, axis=1)
        np.add.at(dx, rows, dxe)
        dW1[e] += d1
        dW2[e] += d2
        if d3 is not None:
            dW3[e] += d3
    res = {}
    if s.S > 0:
        sh1, sh3, sh2 = (np.zeros_like(P["sh_w1"]),
                         None if P["sh_w3"] is None else np.zeros_like(P["sh_w3"]),
                         np.zeros_like(P["sh_w2"]))
        for i in range(s.S):
            _, dxs, d1, d3, d2 = _ffn_backward(x, P["sh_w1"][i],
                                               None if P["sh_w3"] is None else P["sh_w3"][i],
                                               P["sh_w2"][i], s.act, g)
            dx += dxs
            sh1[i], sh2[i] = d1, d2
            if d3 is not None:
                sh3[i] = d3
        res.update(sh_dW1=sh1, sh_dW3=sh3, sh_dW2=sh2)

    # routing weights -> scores: w_j = c s_j / S (S = sum of the selected scores)
    sel = np.take_along_axis(sc, idx, axis=1)
    ds_sel = _weights_to_scores(dw, sel, s.route_scale, s.renormalize)
    ds = np.zeros_like(sc)
    np.add.at(ds, (np.repeat(np.arange(T), k), idx.reshape(-1)), ds_sel.reshape(-1))
    # scores -> logits, through every logit
    dl = _scores_to_logits(ds, sc, s.score)
    dx += dl @ P["router"]
    if getattr(s, "residual", False):
        dx += g
    res.update(dx=dx, dW1=dW1, dW3=dW3, dW2=dW2, drouter=dl.T @ x, dbias=dl.sum(axis=0),
               dw=dw, dl=dl, idx=idx.astype(np.int32), kept=kept)
    return res
