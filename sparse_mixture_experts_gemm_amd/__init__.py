"""Python binding of libmoe (MoE FFN forward on MI355X / gfx950).

Argument marshalling only: every step of the layer runs in the HIP kernels of
``libmoe.so``; torch tensors provide device memory and the current stream.  The entry
points mirror the C ABI in ``include/moe.h`` (same names without the ``moe_`` prefix).
If the library has not been built, every call raises ``LibraryMissing``; there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = [
    "MoeError", "LibraryMissing", "Config", "Weights", "lib", "library_path", "make_config",
    "workspace_size", "route", "rmsnorm_route", "select", "load_stats", "permute",
    "quantize_rows",
    "grouped_gemm", "gemm_kernel_path", "combine", "forward", "forward_noalloc",
    "backward_workspace_size", "backward", "GRAD_FIELDS",
    "status_string", "MOE_F32", "MOE_BF16", "MOE_FP8_E4M3", "MOE_SCORE_SOFTMAX",
    "MOE_SCORE_SIGMOID", "MOE_ACT_SWIGLU", "MOE_ACT_RELU2", "MOE_STAGE_UP", "MOE_STAGE_DOWN",
    "MOE_EXPERTS_ROUTED", "MOE_EXPERTS_SHARED", "EXPORTED_SYMBOLS",
]

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP, MOE_ERR_INTERNAL = range(6)
MOE_F32, MOE_BF16, MOE_FP8_E4M3 = 0, 1, 2
MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID = 0, 1
MOE_ACT_SWIGLU, MOE_ACT_RELU2 = 0, 1
MOE_STAGE_UP, MOE_STAGE_DOWN = 0, 1
MOE_EXPERTS_ROUTED, MOE_EXPERTS_SHARED = 0, 1
MOE_GEMM_PATH_TILED, MOE_GEMM_PATH_DECODE, MOE_GEMM_PATH_TAIL, MOE_GEMM_PATH_F32, \
    MOE_GEMM_PATH_FP8_ACT = range(5)

EXPORTED_SYMBOLS = ["moe_workspace_size", "moe_route", "moe_rmsnorm_route", "moe_select",
                    "moe_load_stats",
                    "moe_permute", "moe_quantize_rows", "moe_grouped_gemm",
                    "moe_gemm_kernel_path", "moe_combine",
                    "moe_forward", "moe_forward_ex", "moe_forward_noalloc",
                    "moe_backward_workspace_size", "moe_backward",
                    "moe_status_string", "moe_last_hip_error"]

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.path.join(_HERE, "libmoe.so")


class LibraryMissing(RuntimeError):
    pass


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


class Config(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int32), ("dim", ctypes.c_int32),
        ("num_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
        ("num_groups", ctypes.c_int32), ("topk_groups", ctypes.c_int32),
        ("group_score_topn", ctypes.c_int32), ("num_shared", ctypes.c_int32),
        ("inter_dim", ctypes.c_int32), ("score_fn", ctypes.c_int32),
        ("renormalize", ctypes.c_int32), ("route_scale", ctypes.c_float),
        ("act", ctypes.c_int32), ("act_dtype", ctypes.c_int32), ("weight_dtype", ctypes.c_int32),
        ("capacity_factor", ctypes.c_float), ("fp8_act", ctypes.c_int32),
        ("pre_norm", ctypes.c_int32), ("norm_eps", ctypes.c_float), ("residual", ctypes.c_int32),
    ]


_W_FIELDS = ["router", "logit_bias", "w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down",
             "sh_gate", "sh_up", "sh_down", "sh_s_gate", "sh_s_up", "sh_s_down", "select_bias",
             "norm_gamma"]


class _WeightsC(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _W_FIELDS]


class Weights:
    """Device weight tensors of a layer (``None`` for absent ones); keeps them alive."""

    def __init__(self, **tensors):
        unknown = set(tensors) - set(_W_FIELDS)
        if unknown:
            raise TypeError(f"unknown weight fields {sorted(unknown)}")
        self.tensors = {n: tensors.get(n) for n in _W_FIELDS}
        self.c = _WeightsC(**{n: _ptr(t) for n, t in self.tensors.items()})


GRAD_FIELDS = ["dx", "d_router", "d_logit_bias", "d_w_gate", "d_w_up", "d_w_down", "d_sh_gate",
               "d_sh_up", "d_sh_down"]


class _GradsC(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in GRAD_FIELDS]


class _OptsC(ctypes.Structure):
    _fields_ = [("stage_events", ctypes.c_void_p * 8), ("load_stats", ctypes.c_void_p),
                ("aux_alpha", ctypes.c_float)]


_LIB = None


def lib():
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise LibraryMissing(f"{path} is not built; run "
                                 "`python -m sparse_mixture_experts_gemm_amd.build`")
        L = ctypes.CDLL(path)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        cfgp = ctypes.POINTER(Config)
        wp = ctypes.POINTER(_WeightsC)
        sig = {
            "moe_workspace_size": [cfgp, ctypes.POINTER(sz)],
            "moe_route": [cfgp, vp, vp, vp, vp, vp, vp, vp, vp],
            "moe_rmsnorm_route": [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp],
            "moe_select": [cfgp, vp, vp, vp, vp, vp],
            "moe_load_stats": [cfgp, vp, vp, ctypes.c_float, vp, vp, vp, vp, sz, vp],
            "moe_permute": [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
            "moe_grouped_gemm": [cfgp, i32, i32, vp, vp, vp, i32, wp, vp, vp, vp, sz, vp],
            "moe_combine": [cfgp, vp, vp, vp, vp, vp],
            "moe_gemm_kernel_path": [cfgp, i32, i32, i32, ctypes.POINTER(i32)],
            "moe_quantize_rows": [cfgp, vp, i32, i32, vp, vp, vp],
            "moe_forward": [cfgp, wp, vp, vp, vp, sz, vp],
            "moe_forward_ex": [cfgp, wp, vp, vp, vp, sz, vp, ctypes.POINTER(_OptsC)],
            "moe_forward_noalloc": [cfgp, wp, vp, vp, vp],
            "moe_backward_workspace_size": [cfgp, ctypes.POINTER(sz)],
            "moe_backward": [cfgp, wp, vp, vp, vp, sz, ctypes.POINTER(_GradsC), vp, sz, vp],
            "moe_last_hip_error": [],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int32
        L.moe_status_string.argtypes = [ctypes.c_int32]
        L.moe_status_string.restype = ctypes.c_char_p
        _LIB = L
    return _LIB


def status_string(status: int) -> str:
    try:
        return lib().moe_status_string(int(status)).decode()
    except LibraryMissing:
        return "unknown"


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(status: int, what: str):
    if status != MOE_OK:
        raise MoeError(status, what)


def make_config(T, d, E, k, *, G=1, Gk=1, n_g=1, S=0, I, score="sigmoid", renormalize=True,
                route_scale=1.0, act="swiglu", act_dtype="bf16", weight_dtype="bf16",
                capacity_factor=0.0, fp8_act=False, pre_norm=False, norm_eps=1e-6,
                residual=False) -> Config:
    dt = {"f32": MOE_F32, "bf16": MOE_BF16, "e4m3": MOE_FP8_E4M3}
    return Config(num_tokens=T, dim=d, num_experts=E, top_k=k, num_groups=G, topk_groups=Gk,
                  group_score_topn=n_g, num_shared=S, inter_dim=I,
                  score_fn={"softmax": MOE_SCORE_SOFTMAX, "sigmoid": MOE_SCORE_SIGMOID}[score],
                  renormalize=int(bool(renormalize)), route_scale=float(route_scale),
                  act={"swiglu": MOE_ACT_SWIGLU, "relu2": MOE_ACT_RELU2}[act],
                  act_dtype=dt[act_dtype], weight_dtype=dt[weight_dtype],
                  capacity_factor=float(capacity_factor or 0.0), fp8_act=int(bool(fp8_act)),
                  pre_norm=int(bool(pre_norm)), norm_eps=float(norm_eps),
                  residual=int(bool(residual)))


def workspace_size(cfg: Config) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_workspace_size(ctypes.byref(cfg), ctypes.byref(n)), "moe_workspace_size")
    return n.value


def route(cfg, x, router, logit_bias, select_bias, scores, topk_idx, topk_w, stream=None):
    _check(lib().moe_route(ctypes.byref(cfg), _ptr(x), _ptr(router), _ptr(logit_bias),
                           _ptr(select_bias), _ptr(scores), _ptr(topk_idx), _ptr(topk_w),
                           _stream(stream)), "moe_route")


def rmsnorm_route(cfg, x, gamma, router, logit_bias, select_bias, x_norm, scores, topk_idx,
                  topk_w, stream=None):
    _check(lib().moe_rmsnorm_route(ctypes.byref(cfg), _ptr(x), _ptr(gamma), _ptr(router),
                                   _ptr(logit_bias), _ptr(select_bias), _ptr(x_norm),
                                   _ptr(scores), _ptr(topk_idx), _ptr(topk_w), _stream(stream)),
           "moe_rmsnorm_route")


def select(cfg, scores, keys, topk_idx, topk_w, stream=None):
    _check(lib().moe_select(ctypes.byref(cfg), _ptr(scores), _ptr(keys), _ptr(topk_idx),
                            _ptr(topk_w), _stream(stream)), "moe_select")


def load_stats(cfg, scores, topk_idx, alpha, f, p, loss, ws, ws_bytes=None, stream=None):
    nb = ws_bytes if ws_bytes is not None else (0 if ws is None else ws.numel() * ws.element_size())
    _check(lib().moe_load_stats(ctypes.byref(cfg), _ptr(scores), _ptr(topk_idx), float(alpha),
                                _ptr(f), _ptr(p), _ptr(loss), _ptr(ws), nb, _stream(stream)),
           "moe_load_stats")


def permute(cfg, topk_idx, topk_w, counts, offsets, perm_token, slot_pos, perm_weight, ws,
            ws_bytes=None, stream=None):
    nb = ws_bytes if ws_bytes is not None else (0 if ws is None else ws.numel() * ws.element_size())
    _check(lib().moe_permute(ctypes.byref(cfg), _ptr(topk_idx), _ptr(topk_w), _ptr(counts),
                             _ptr(offsets), _ptr(perm_token), _ptr(slot_pos), _ptr(perm_weight),
                             _ptr(ws), nb, _stream(stream)), "moe_permute")


def gemm_kernel_path(cfg, stage, expert_set, rows) -> int:
    """Kernel family of one grouped-GEMM stage (moe_gemm_kernel_path; host only)."""
    path = ctypes.c_int32(-1)
    _check(lib().moe_gemm_kernel_path(ctypes.byref(cfg), int(stage), int(expert_set), int(rows),
                                      ctypes.byref(path)), "moe_gemm_kernel_path")
    return path.value


def grouped_gemm(cfg, stage, expert_set, a, row_index, offsets, rows, weights: Weights,
                 row_weight, out, ws=None, ws_bytes=None, stream=None):
    nb = ws_bytes if ws_bytes is not None else (0 if ws is None else ws.numel() * ws.element_size())
    _check(lib().moe_grouped_gemm(ctypes.byref(cfg), int(stage), int(expert_set), _ptr(a),
                                  _ptr(row_index), _ptr(offsets), int(rows),
                                  ctypes.byref(weights.c), _ptr(row_weight), _ptr(out), _ptr(ws),
                                  nb, _stream(stream)), "moe_grouped_gemm")


def quantize_rows(cfg, a, rows, cols, q, scale, stream=None):
    _check(lib().moe_quantize_rows(ctypes.byref(cfg), _ptr(a), int(rows), int(cols), _ptr(q),
                                   _ptr(scale), _stream(stream)), "moe_quantize_rows")


def combine(cfg, y_perm, slot_pos, y_shared, out, stream=None):
    _check(lib().moe_combine(ctypes.byref(cfg), _ptr(y_perm), _ptr(slot_pos), _ptr(y_shared),
                             _ptr(out), _stream(stream)), "moe_combine")


def forward(cfg, weights: Weights, x, out, ws, ws_bytes=None, stream=None, stage_events=None,
            load_stats=None, aux_alpha=1.0):
    """The whole layer.  stage_events: optional list of 8 torch.cuda.Event (or None) recorded
    at the stage boundaries; load_stats: optional device fp32 buffer [2E + 1] for the load
    statistics (see moe_forward_opts in include/moe.h)."""
    nb = ws_bytes if ws_bytes is not None else ws.numel() * ws.element_size()
    if stage_events is None and load_stats is None:
        _check(lib().moe_forward(ctypes.byref(cfg), ctypes.byref(weights.c), _ptr(x), _ptr(out),
                                 _ptr(ws), nb, _stream(stream)), "moe_forward")
        return
    opts = _OptsC()
    for i, ev in enumerate(stage_events or []):
        if ev is not None and not ev.cuda_event:
            ev.record()          # torch creates its events lazily; the library re-records it
        opts.stage_events[i] = None if ev is None else ev.cuda_event
    opts.load_stats = _ptr(load_stats)
    opts.aux_alpha = float(aux_alpha)
    _check(lib().moe_forward_ex(ctypes.byref(cfg), ctypes.byref(weights.c), _ptr(x), _ptr(out),
                                _ptr(ws), nb, _stream(stream), ctypes.byref(opts)),
           "moe_forward_ex")


def forward_noalloc(cfg, weights: Weights, x, out, stream=None):
    """The whole layer on the library's own per-device workspace (moe_forward_noalloc: no
    allocation; moe_workspace_size(cfg) at most 64 MiB)."""
    _check(lib().moe_forward_noalloc(ctypes.byref(cfg), ctypes.byref(weights.c), _ptr(x),
                                     _ptr(out), _stream(stream)), "moe_forward_noalloc")


def backward_workspace_size(cfg: Config) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_backward_workspace_size(ctypes.byref(cfg), ctypes.byref(n)),
           "moe_backward_workspace_size")
    return n.value


def backward(cfg, weights: Weights, x, dout, fwd_ws, grads: dict, ws, fwd_ws_bytes=None,
             ws_bytes=None, stream=None):
    """Gradients of sum(dout * out) for the forward computed into fwd_ws.  grads maps the
    names of GRAD_FIELDS to device tensors (dx required; absent names are not computed)."""
    unknown = set(grads) - set(GRAD_FIELDS)
    if unknown:
        raise TypeError(f"unknown gradient fields {sorted(unknown)}")
    g = _GradsC(**{n: _ptr(grads.get(n)) for n in GRAD_FIELDS})
    fb = fwd_ws_bytes if fwd_ws_bytes is not None else fwd_ws.numel() * fwd_ws.element_size()
    nb = ws_bytes if ws_bytes is not None else ws.numel() * ws.element_size()
    _check(lib().moe_backward(ctypes.byref(cfg), ctypes.byref(weights.c), _ptr(x), _ptr(dout),
                              _ptr(fwd_ws), fb, ctypes.byref(g), _ptr(ws), nb, _stream(stream)),
           "moe_backward")
