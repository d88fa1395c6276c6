"""Test helpers: move seeded layers to the GPU and build libmoe configs (marshalling only)."""
import numpy as np
import torch

import sparse_mixture_experts_gemm_amd as moe

DEV = "cuda"


def to_dev(a):
    if a is None:
        return None
    if a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(DEV)


def from_dev_bf16(t):
    """bf16 bits held in an int16 tensor -> numpy uint16."""
    return t.cpu().numpy().view(np.uint16)


def config(shape, T=None):
    s = shape
    return moe.make_config(s.T if T is None else T, s.d, s.E, s.k, G=s.G, Gk=s.Gk, n_g=s.n_g,
                           S=s.S, I=s.I, score=s.score, renormalize=s.renormalize,
                           route_scale=s.route_scale, act=s.act, act_dtype=s.act_dtype,
                           weight_dtype=s.weight_dtype, capacity_factor=s.capacity_factor,
                           fp8_act=s.fp8_act, pre_norm=s.pre_norm, norm_eps=s.norm_eps,
                           residual=s.residual)


def weights(lay):
    names = ["w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down", "sh_gate", "sh_up",
             "sh_down", "sh_s_gate", "sh_s_up", "sh_s_down"]
    t = {n: to_dev(getattr(lay, n)) for n in names}
    t["router"] = to_dev(lay.router)
    t["logit_bias"] = to_dev(lay.logit_bias)
    t["select_bias"] = to_dev(lay.select_bias)
    t["norm_gamma"] = to_dev(lay.norm_gamma)
    return moe.Weights(**t)


def act_empty(shape, act_dtype):
    dt = torch.int16 if act_dtype == "bf16" else torch.float32
    return torch.empty(shape, dtype=dt, device=DEV)


def act_to_f64(t, act_dtype):
    import oracle as O
    if act_dtype == "bf16":
        return O.decode_bf16(from_dev_bf16(t))
    return t.cpu().numpy().astype(np.float64)


def workspace(cfg):
    n = moe.workspace_size(cfg)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=DEV)
