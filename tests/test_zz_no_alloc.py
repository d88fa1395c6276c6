"""moe_forward_noalloc (the forward on the library's own per-device workspace) against
moe_forward through the C ABI, on the GPU.

Two calls in a row on the shared array, the second with fewer tokens, each compared with
moe_forward on a caller workspace: bit for bit against moe_forward_ex with stage events
(which, like moe_forward_noalloc, keeps every launch on the caller's stream), and within
the layer's float bar (max|delta| <= 2e-2 max|ref| for bf16, 1e-4 for fp32) against plain
moe_forward, which runs the shared experts on a second stream.  A config whose workspace
exceeds the 64 MiB array is refused before anything is enqueued.
"""
import ctypes

import numpy as np
import pytest
import torch

import sparse_mixture_experts_gemm_amd as moe
import workloads as W
from _dev import act_empty, act_to_f64, config, to_dev, weights, workspace

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}
SCRATCH_BYTES = 64 << 20

CASES = {
    # FusionLLM layer shape: 1024 tokens (the largest that fits the array), then 64
    "fusionllm_bf16": ("fusionllm_bf16", 1024, 64),
    "small_swiglu": (W.small_shape(T=300, d=320, E=16, k=4, G=4, Gk=2, S=2, I=192, seed=31),
                     300, 77),
    "small_relu2_e4m3": (W.small_shape(T=200, d=256, E=8, k=2, G=2, Gk=1, n_g=2, S=2, I=320,
                                       act="relu2", weight_dtype="e4m3", seed=32), 200, 33),
    "small_f32": (W.small_shape(T=77, d=48, E=8, k=3, score="softmax", G=1, Gk=1, S=1, I=32,
                                act_dtype="f32", weight_dtype="f32", seed=34), 77, 5),
}


def _reference(shape, w, x, T, staged):
    cfg = config(shape, T=T)
    out = act_empty((T, shape.d), shape.act_dtype)
    ws = workspace(cfg)
    if staged:
        ev = [torch.cuda.Event() for _ in range(8)]
        moe.forward(cfg, w, x, out, ws, stage_events=ev)
    else:
        moe.forward(cfg, w, x, out, ws)
    return out


@pytest.mark.parametrize("name", list(CASES))
def test_noalloc_matches_forward_on_two_calls(name):
    spec, t1, t2 = CASES[name]
    shape = W.SHAPES[spec] if isinstance(spec, str) else spec
    lay = W.make_layer(shape, cache=isinstance(spec, str))
    w = weights(lay)
    x_all = to_dev(lay.x)
    for T in (t1, t2):
        cfg = config(shape, T=T)
        assert moe.workspace_size(cfg) <= SCRATCH_BYTES
        x = x_all[:T].contiguous()
        out = act_empty((T, shape.d), shape.act_dtype)
        out.fill_(0)
        print(f"case {name} T={T}: moe_forward_noalloc", flush=True)
        moe.forward_noalloc(cfg, w, x, out)
        staged = _reference(shape, w, x, T, staged=True)
        plain = _reference(shape, w, x, T, staged=False)
        torch.cuda.synchronize()
        assert torch.equal(out, staged), f"{name} T={T}: differs from moe_forward_ex"
        got = act_to_f64(out, shape.act_dtype)
        ref = act_to_f64(plain, shape.act_dtype)
        assert np.isfinite(got).all()
        err = float(np.abs(got - ref).max())
        bound = TOL[shape.act_dtype] * float(np.abs(ref).max())
        assert err <= bound, f"{name} T={T}: max|delta| {err} > {bound}"


@pytest.mark.parametrize("seed", range(16))
def test_noalloc_random_configs(seed):
    """The seeded random layers of the forward parity tests, two calls in a row on the shared
    array (all tokens, then a third of them): bit for bit equal to moe_forward_ex."""
    from test_gpu_parity import random_shape
    shape = random_shape(seed)
    lay = W.make_layer(shape, cache=False)
    w = weights(lay)
    x_all = to_dev(lay.x)
    for T in (shape.T, max(1, shape.T // 3)):
        cfg = config(shape, T=T)
        assert moe.workspace_size(cfg) <= SCRATCH_BYTES
        x = x_all[:T].contiguous()
        out = act_empty((T, shape.d), shape.act_dtype)
        out.fill_(0)
        print(f"seed {seed} T={T}: moe_forward_noalloc", flush=True)
        moe.forward_noalloc(cfg, w, x, out)
        staged = _reference(shape, w, x, T, staged=True)
        torch.cuda.synchronize()
        assert torch.equal(out, staged), f"seed {seed} T={T}: differs from moe_forward_ex"


def test_noalloc_on_a_caller_stream():
    shape = W.small_shape(T=300, d=320, E=16, k=4, G=4, Gk=2, S=2, I=192, seed=31)
    lay = W.make_layer(shape, cache=False)
    w = weights(lay)
    x = to_dev(lay.x)
    cfg = config(shape)
    ref = _reference(shape, w, x, shape.T, staged=True)
    out = act_empty((shape.T, shape.d), shape.act_dtype)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        moe.forward_noalloc(cfg, w, x, out, stream=s)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_noalloc_refuses_a_workspace_above_the_array():
    shape = W.SHAPES["fusionllm_bf16"]
    cfg = config(shape, T=4096)
    assert moe.workspace_size(cfg) > SCRATCH_BYTES
    lay = W.make_layer(shape)
    w = weights(lay)
    x = to_dev(lay.x)[:4096].contiguous()
    out = act_empty((4096, shape.d), shape.act_dtype)
    out.fill_(0)
    torch.cuda.synchronize()
    st = moe.lib().moe_forward_noalloc(ctypes.byref(cfg), ctypes.byref(w.c),
                                       ctypes.c_void_p(x.data_ptr()),
                                       ctypes.c_void_p(out.data_ptr()), None)
    assert st == moe.MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert int(out.abs().max().item()) == 0     # nothing was enqueued
