"""GPU parity of moe_backward against the fp64 backward oracle (through the C ABI).

The forward runs first (moe_forward into its workspace); its selection is checked against
the oracle's routing (identical except at fp32 near ties), and the oracle's backward then
takes that selection, since gradients are only defined for a fixed selection.  Every
gradient must satisfy max|delta| <= 2e-2 max|ref| (the bf16 bar of the forward: h, dh,
[da | db] and the permuted dx rows are bf16 between stages, accumulation is fp32).
"""
import numpy as np
import pytest
import torch

import oracle as O
import sparse_mixture_experts_gemm_amd as moe
import workloads as W
from _dev import act_empty, act_to_f64, config, to_dev, weights, workspace
from test_gpu_parity import MARGIN, margins, valid_within_margin

pytestmark = pytest.mark.gpu

TOL = 2e-2

SHAPES = {
    # ragged: T, d and I give partial tiles; groups, two shared experts
    "bwd_swiglu": W.small_shape(T=300, d=320, E=16, k=4, G=4, Gk=2, S=2, I=192, seed=61),
    "bwd_relu2": W.small_shape(T=200, d=256, E=8, k=2, G=2, Gk=1, n_g=2, S=1, I=320, act="relu2",
                               seed=62),
    # softmax gating without renormalisation: the router gradient reaches every logit
    "bwd_softmax_raw": W.small_shape(T=150, d=192, E=16, k=3, score="softmax", G=1, Gk=1, S=1,
                                     I=128, renormalize=False, route_scale=2.0, seed=63),
    # capacity drops, a selection-only bias and Zipf logit offsets are not needed together:
    # capacity + bias here, residual below
    "bwd_capacity_bias": W.small_shape(T=333, d=256, E=32, k=4, G=8, Gk=3, n_g=2, S=1, I=128,
                                       select_bias_std=0.7, capacity_factor=1.0, seed=64),
    "bwd_residual_noshared": W.small_shape(T=257, d=256, E=16, k=4, G=1, Gk=1, S=0, I=128,
                                           residual=True, seed=65),
    # more slots per token than the combine keeps in flight (k = 12)
    "bwd_k12": W.small_shape(T=96, d=128, E=16, k=12, G=1, Gk=1, S=1, I=64, seed=68),
    # several tiles per workgroup in every GEMM
    "bwd_multi_tile": W.small_shape(T=8192, d=512, E=8, k=4, G=1, Gk=1, S=1, I=256, seed=66),
}

NAMES = {"dx": "dx", "d_router": "drouter", "d_logit_bias": "dbias", "d_w_gate": "dW1",
         "d_w_up": "dW3", "d_w_down": "dW2", "d_sh_gate": "sh_dW1", "d_sh_up": "sh_dW3",
         "d_sh_down": "sh_dW2"}


def run_backward(s, lay):
    cfg = config(s)
    wts = weights(lay)
    ws = workspace(cfg)
    x = to_dev(lay.x)
    out = act_empty((s.T, s.d), "bf16")
    moe.forward(cfg, wts, x, out, ws)
    dout_np = W.random_act((s.T, s.d), 99, "bf16", 1.0)
    dout = to_dev(dout_np)
    f32 = lambda *shape: torch.empty(shape, dtype=torch.float32, device="cuda")
    grads = {"dx": act_empty((s.T, s.d), "bf16"), "d_router": f32(s.E, s.d), "d_logit_bias": f32(s.E),
             "d_w_gate": f32(s.E, s.I, s.d), "d_w_down": f32(s.E, s.d, s.I)}
    if s.act == "swiglu":
        grads["d_w_up"] = f32(s.E, s.I, s.d)
    if s.S > 0:
        grads["d_sh_gate"] = f32(s.S, s.I, s.d)
        grads["d_sh_down"] = f32(s.S, s.d, s.I)
        if s.act == "swiglu":
            grads["d_sh_up"] = f32(s.S, s.I, s.d)
    bws = torch.empty(moe.backward_workspace_size(cfg), dtype=torch.uint8, device="cuda")
    moe.backward(cfg, wts, x, dout, ws, grads, bws)
    torch.cuda.synchronize()
    gpu_idx = ws[: s.T * s.k * 4].view(torch.int32).cpu().numpy().reshape(s.T, s.k)
    return cfg, wts, ws, x, dout, dout_np, grads, bws, gpu_idx


def checked_selection(s, lay, gpu_idx):
    r = O.route(lay)
    same = np.array([set(a.tolist()) == set(b.tolist()) for a, b in zip(gpu_idx, r["idx"])])
    assert np.all(same | (margins(r["keys"], s) <= MARGIN)), "routing differs away from a near tie"
    for t in np.nonzero(~same)[0]:
        assert valid_within_margin(gpu_idx[t], r["keys"][t], s)
    return gpu_idx


@pytest.mark.parametrize("name", list(SHAPES))
def test_backward_matches_oracle(name):
    s = SHAPES[name]
    lay = W.make_layer(s, cache=False)
    cfg, wts, ws, x, dout, dout_np, grads, bws, gpu_idx = run_backward(s, lay)
    idx = checked_selection(s, lay, gpu_idx)
    ref = O.backward.moe_backward(lay, O.decode_bf16(dout_np), idx=idx)
    for field, t in grads.items():
        want = ref[NAMES[field]]
        got = act_to_f64(t, "bf16") if field == "dx" else t.cpu().numpy().astype(np.float64)
        scale = np.max(np.abs(want))
        diff = np.max(np.abs(got - want))
        print(f"{name} {field}: max|d|/max|ref| = {diff / scale:.3e}")
        assert diff <= TOL * scale, field


def random_backward_shape(seed):
    """A seeded layer inside the backward's contract (bf16, dim and inter dim on the
    64-grid, no pre-norm or e4m3 activations): any activation, scoring, grouping, k up to
    the eligible experts, 0-2 shared experts, capacity, selection bias, residual, route
    scale, and 1 to 2500 tokens."""
    g = np.random.default_rng(8000 + seed)
    E = int(g.choice([4, 8, 16, 32, 64]))
    G = int(g.choice([x for x in (1, 2, 4, 8) if E % x == 0]))
    Gk = int(g.integers(1, G + 1))
    n_g = int(g.choice([1, 2])) if E // G >= 2 else 1
    return W.small_shape(
        T=int(g.choice([1, 5, 33, 64, 100, 257, 600, 1100, 2500])), d=64 * int(g.integers(1, 9)),
        E=E, k=int(g.integers(1, min(Gk * (E // G), 8) + 1)), G=G, Gk=Gk, n_g=n_g,
        S=int(g.integers(0, 3)), I=64 * int(g.integers(1, 7)),
        score=str(g.choice(["sigmoid", "softmax"])), act=str(g.choice(["swiglu", "relu2"])),
        renormalize=bool(g.integers(0, 2)), route_scale=float(g.choice([1.0, 2.5])),
        capacity_factor=float(g.choice([0.5, 1.0, 1.5])) if g.random() < 0.3 else None,
        select_bias_std=0.5 if g.random() < 0.3 else None, residual=bool(g.integers(0, 2)),
        seed=950 + seed)


@pytest.mark.parametrize("seed", range(32))
def test_backward_random_configs(seed):
    """Every gradient on seeded random layers, against the fp64 backward oracle under the
    forward's checked selection, at the bar of the fixed cases."""
    s = random_backward_shape(seed)
    print(s)
    lay = W.make_layer(s, cache=False)
    cfg, wts, ws, x, dout, dout_np, grads, bws, gpu_idx = run_backward(s, lay)
    idx = checked_selection(s, lay, gpu_idx)
    ref = O.backward.moe_backward(lay, O.decode_bf16(dout_np), idx=idx)
    # k = 1 with renormalised weights: the weight c s / s is constant, so the router
    # gradient is exactly zero and both sides hold rounding residue only
    no_router_grad = s.renormalize and s.k == 1
    for field, t in grads.items():
        want = ref[NAMES[field]]
        got = act_to_f64(t, "bf16") if field == "dx" else t.cpu().numpy().astype(np.float64)
        scale = np.max(np.abs(want))
        diff = np.max(np.abs(got - want))
        print(f"seed {seed} {field}: max|d| = {diff:.3e}, max|ref| = {scale:.3e}")
        if scale == 0 or (no_router_grad and field in ("d_router", "d_logit_bias")):
            assert diff <= 1e-4, field     # an exactly zero gradient (also: every slot dropped)
        else:
            assert diff <= TOL * scale, field


def test_backward_with_a_selected_expert_of_zero_weight():
    """Expert 3's logit is offset by -200, so its fp32 sigmoid score (and weight) is exactly
    0, and a selection-only bias of +1000 makes every token pick it anyway.  The exact
    gradient is finite (that weight's gradient enters the logits only multiplied by the
    score); every gradient must match the fp64 oracle, whose score is ~1e-87, not 0."""
    s = W.small_shape(T=200, d=256, E=16, k=4, G=1, Gk=1, S=1, I=128, select_bias_std=0.5,
                      seed=69)
    lay = W.make_layer(s, cache=False)
    lay.logit_bias = np.zeros(s.E, np.float32)
    lay.logit_bias[3] = -200.0
    lay.select_bias = lay.select_bias.copy()
    lay.select_bias[3] = 1000.0
    cfg, wts, ws, x, dout, dout_np, grads, bws, gpu_idx = run_backward(s, lay)
    assert (gpu_idx == 3).any(axis=1).all()
    off = (s.T * s.k * 4 + 255) // 256 * 256        # topk_w follows topk_idx in the workspace
    tw = ws[off: off + s.T * s.k * 4].view(torch.float32).cpu().numpy().reshape(s.T, s.k)
    assert np.all(tw[gpu_idx == 3] == 0.0)
    idx = checked_selection(s, lay, gpu_idx)
    ref = O.backward.moe_backward(lay, O.decode_bf16(dout_np), idx=idx)
    for field, t in grads.items():
        want = ref[NAMES[field]]
        got = act_to_f64(t, "bf16") if field == "dx" else t.cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(got)), field
        scale = np.max(np.abs(want))
        diff = np.max(np.abs(got - want))
        print(f"zero-weight {field}: max|d|/max|ref| = {diff / scale:.3e}")
        assert diff <= TOL * scale, field


def test_backward_is_deterministic_and_untouched_experts_get_zero():
    s = W.small_shape(T=12, d=128, E=32, k=2, G=1, Gk=1, S=1, I=64, seed=67)
    lay = W.make_layer(s, cache=False)
    cfg, wts, ws, x, dout, _, grads, bws, gpu_idx = run_backward(s, lay)
    first = {k: v.clone() for k, v in grads.items()}
    moe.backward(cfg, wts, x, dout, ws, grads, bws)
    torch.cuda.synchronize()
    for k in grads:
        assert torch.equal(grads[k], first[k]), k
    untouched = sorted(set(range(s.E)) - set(gpu_idx.reshape(-1).tolist()))
    assert untouched
    for k in ("d_w_gate", "d_w_up", "d_w_down"):
        assert torch.count_nonzero(grads[k][untouched]) == 0


def test_backward_at_the_prefill_shape():
    """The FusionLLM prefill layer: dx on sampled tokens, the weight gradients of sampled
    experts, and the router gradient, against the oracle."""
    s = W.SHAPES["fusionllm_bf16"]
    lay = W.make_layer(s)
    cfg, wts, ws, x, dout, dout_np, grads, bws, gpu_idx = run_backward(s, lay)
    idx = checked_selection(s, lay, gpu_idx)
    ref = O.backward.moe_backward(lay, O.decode_bf16(dout_np), idx=idx)
    rows = np.unique(np.r_[np.arange(16), np.random.default_rng(3).choice(s.T, 112, replace=False)])
    experts = [0, 17, 42, 63]
    checks = {"dx": (act_to_f64(grads["dx"], "bf16")[rows], ref["dx"][rows])}
    for field in ("d_w_gate", "d_w_up", "d_w_down"):
        checks[field] = (grads[field][experts].cpu().numpy().astype(np.float64), ref[NAMES[field]][experts])
    for field in ("d_sh_gate", "d_sh_up", "d_sh_down", "d_router", "d_logit_bias"):
        checks[field] = (grads[field].cpu().numpy().astype(np.float64), ref[NAMES[field]])
    for field, (got, want) in checks.items():
        scale = np.max(np.abs(want))
        diff = np.max(np.abs(got - want))
        print(f"prefill {field}: max|d|/max|ref| = {diff / scale:.3e}")
        assert diff <= TOL * scale, field
