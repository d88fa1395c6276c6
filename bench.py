"""Benchmark of the MoE FFN forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = one pass of the whole layer (route -> permute -> grouped GEMMs for routed and
shared experts -> combine) over one batch of seeded synthetic tokens, with inputs and
weights resident in HBM.  Prints ONE JSON line.  The headline workload is the
FusionLLM-shape layer (T=4096, dim 2048, 64 routed + 4 shared experts, top-6, bf16);
the decode-shaped layer (T=64, same weights) is reported alongside with its HBM rate.
Per-stage times come from HIP events that moe_forward_ex records between its launches on
the stream they run on.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E


def stage_flops(s, T):
    """Algorithmic FLOPs of each stage (padding and masked work excluded)."""
    c_up = 4 if s.act == "swiglu" else 2
    return {
        "route": 2 * T * s.d * s.E,
        "permute": 0,
        "up_routed": T * s.k * c_up * s.d * s.I,
        "up_shared": T * s.S * c_up * s.d * s.I,
        "down_routed": T * s.k * 2 * s.d * s.I,
        "down_shared": T * s.S * 2 * s.d * s.I,
        "combine": 0,
    }


def weight_bytes_per_expert(s):
    wb = 1 if s.weight_dtype == "e4m3" else (4 if s.weight_dtype == "f32" else 2)
    n_mats = 3 if s.act == "swiglu" else 2
    scales = 4 * (s.I * (n_mats - 1) + s.d) if s.weight_dtype == "e4m3" else 0
    return n_mats * s.d * s.I * wb + scales


def to_dev(a):
    """numpy array in its stored encoding -> device tensor (bf16 bits travel as int16)."""
    import torch
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    t = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a)
    return t.to("cuda")


class Runner:
    """Device-resident layer; one step = one moe_forward call.  Stage times come from
    separate passes of moe_forward_ex with HIP events at the stage boundaries, recorded on
    the stream the kernels run on."""

    def __init__(self, shape, lay, weights=None):
        import torch
        import sparse_mixture_experts_gemm_amd as moe
        self.torch, self.moe, self.s = torch, moe, shape
        s = shape
        self.cfg = moe.make_config(s.T, s.d, s.E, s.k, G=s.G, Gk=s.Gk, n_g=s.n_g, S=s.S, I=s.I,
                                   score=s.score, renormalize=s.renormalize,
                                   route_scale=s.route_scale, act=s.act, act_dtype=s.act_dtype,
                                   weight_dtype=s.weight_dtype, capacity_factor=s.capacity_factor,
                                   fp8_act=s.fp8_act, pre_norm=s.pre_norm, norm_eps=s.norm_eps,
                                   residual=s.residual)
        names = ["router", "logit_bias", "w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down",
                 "sh_gate", "sh_up", "sh_down", "sh_s_gate", "sh_s_up", "sh_s_down"]
        if weights is None:
            t = {n: to_dev(getattr(lay, n)) for n in names}
            t["select_bias"] = to_dev(lay.select_bias)
            t["norm_gamma"] = to_dev(lay.norm_gamma)
            weights = moe.Weights(**t)
        elif lay.select_bias is not None or lay.norm_gamma is not None:
            # the same device weights with this layer's selection bias and RMSNorm gain
            t = dict(weights.tensors)
            t["select_bias"] = to_dev(lay.select_bias)
            t["norm_gamma"] = to_dev(lay.norm_gamma)
            weights = moe.Weights(**t)
        self.w = weights
        self.x = to_dev(lay.x)
        adt = torch.int16 if s.act_dtype == "bf16" else torch.float32
        self.out = torch.empty((s.T, s.d), dtype=adt, device="cuda")
        self.ws = torch.empty(moe.workspace_size(self.cfg), dtype=torch.uint8, device="cuda")

    def counts(self):
        """Per-expert row counts of the last forward (from its workspace)."""
        s = self.s
        # the workspace starts with topk_idx [T*k] int32; counts follow topk_w, 256-aligned
        al = lambda n: (n + 255) // 256 * 256
        off = al(s.T * s.k * 4) * 2
        return self.ws[off: off + 4 * s.E].view(self.torch.int32).cpu().numpy()

    def timed(self, steps, warmup, load_stats=None):
        """K plain forwards bracketed by one event pair (the headline step time)."""
        torch = self.torch
        for _ in range(warmup):
            self.moe.forward(self.cfg, self.w, self.x, self.out, self.ws, load_stats=load_stats)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        a.record()
        for _ in range(steps):
            self.moe.forward(self.cfg, self.w, self.x, self.out, self.ws, load_stats=load_stats)
        b.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return a.elapsed_time(b) / steps, wall

    def step_distribution(self, steps, warmup):
        """Each of K forwards bracketed by its own event pair: median, p10, p90 and mean of
        the per-step times (ms).  The event records add a few microseconds per step."""
        torch = self.torch
        for _ in range(warmup):
            self.moe.forward(self.cfg, self.w, self.x, self.out, self.ws)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        torch.cuda.synchronize()
        for a, b in ev:
            a.record()
            self.moe.forward(self.cfg, self.w, self.x, self.out, self.ws)
            b.record()
        torch.cuda.synchronize()
        t = np.array([a.elapsed_time(b) for a, b in ev])
        return {"median": float(np.median(t)), "p10": float(np.percentile(t, 10)),
                "p90": float(np.percentile(t, 90)), "mean": float(t.mean()), "steps": steps}

    def rotated_timed(self, weight_sets, steps, warmup):
        """K forwards that cycle through several device copies of the same weights, so that
        no step finds the previous step's weights in the 256 MB Infinity Cache; one event
        pair around all K."""
        torch = self.torch
        n = len(weight_sets)
        for i in range(warmup):
            self.moe.forward(self.cfg, weight_sets[i % n], self.x, self.out, self.ws)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(steps):
            self.moe.forward(self.cfg, weight_sets[i % n], self.x, self.out, self.ws)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    def backward_timed(self, steps, warmup):
        """One forward, then K moe_backward calls on its workspace (all weight, router and
        input gradients), bracketed by one event pair."""
        torch, s = self.torch, self.s
        f32 = lambda *shape: torch.empty(shape, dtype=torch.float32, device="cuda")
        grads = {"dx": torch.empty_like(self.out), "d_router": f32(s.E, s.d),
                 "d_logit_bias": f32(s.E), "d_w_gate": f32(s.E, s.I, s.d),
                 "d_w_up": f32(s.E, s.I, s.d), "d_w_down": f32(s.E, s.d, s.I)}
        if s.S > 0:
            grads.update(d_sh_gate=f32(s.S, s.I, s.d), d_sh_up=f32(s.S, s.I, s.d),
                         d_sh_down=f32(s.S, s.d, s.I))
        dout = torch.randn((s.T, s.d), device="cuda").to(torch.bfloat16).view(torch.int16)
        bws = torch.empty(self.moe.backward_workspace_size(self.cfg), dtype=torch.uint8, device="cuda")
        self.moe.forward(self.cfg, self.w, self.x, self.out, self.ws)
        for _ in range(warmup):
            self.moe.backward(self.cfg, self.w, self.x, dout, self.ws, grads, bws)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            self.moe.backward(self.cfg, self.w, self.x, dout, self.ws, grads, bws)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps, bws.numel()

    def graph_timed(self, steps, warmup):
        """The same forward captured once into a HIP graph, then K replays bracketed by one
        event pair (launch overhead of the individual kernels removed)."""
        torch = self.torch
        self.moe.forward(self.cfg, self.w, self.x, self.out, self.ws)   # side stream exists
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.moe.forward(self.cfg, self.w, self.x, self.out, self.ws)
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    def staged(self, steps, warmup, stages=None):
        """K forwards with events at the given stage boundaries (indices into the eight of
        moe_forward_opts); returns the mean time between consecutive recorded events.  Every
        recorded event also adds a few microseconds to the stream, so the step time is taken
        from ``timed`` and these figures only attribute time to stages."""
        torch = self.torch
        stages = list(range(8)) if stages is None else stages
        names = ["route", "permute", "up_routed", "up_shared", "down_routed", "down_shared", "combine"]
        for _ in range(warmup):
            self.moe.forward(self.cfg, self.w, self.x, self.out, self.ws)
        ev = []
        for _ in range(steps):
            e = [None] * 8
            for i in stages:
                e[i] = torch.cuda.Event(enable_timing=True)
            ev.append(e)
        torch.cuda.synchronize()
        for i in range(steps):
            self.moe.forward(self.cfg, self.w, self.x, self.out, self.ws, stage_events=ev[i])
        torch.cuda.synchronize()
        out = {}
        for a, b in zip(stages[:-1], stages[1:]):
            key = "+".join(names[a:b])
            out[key] = float(np.mean([ev[i][a].elapsed_time(ev[i][b]) for i in range(steps)]))
        return out


def decode_bytes(s, counts):
    touched = int((counts > 0).sum())
    ab = 2 if s.act_dtype == "bf16" else 4
    return (touched + s.S) * weight_bytes_per_expert(s) + s.E * s.d * ab + 2 * s.T * s.d * ab, touched


def cpu_baseline(lay, n_tokens, min_seconds=10.0):
    """The fp64 oracle on the host cores: whole forwards of the first n_tokens tokens of the
    same layer, repeated until at least min_seconds of wall time have passed."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
                    or [1])
    except Exception:
        cores = os.cpu_count() or 1
    reps = 0
    t0 = time.perf_counter()
    while True:
        O.moe_forward(lay, tokens=np.arange(n_tokens))
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    return {"value": reps * n_tokens / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{reps} fp64 oracle forward(s) of {n_tokens} tokens of the same layer "
                      f"(routing, all expert FFNs, combine), {dt:.1f} s wall"}


GEMM_SOURCES = ["gemm.hip", "gemm_core.h", "common.h", "internal.h", "api.cpp"]
DECODE_SOURCES = ["decode.hip", "common.h", "internal.h", "api.cpp"]


def kernel_source_digest(names=GEMM_SOURCES):
    """sha256 over the sources that define a kernel and its launch."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_mixture_experts_gemm_amd", "csrc")
    for name in names:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def profiled_value(name, key, sources=GEMM_SOURCES):
    """A figure recorded in profiles/<name> (from rocprofv3 counter runs), or None when the
    file is absent or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith((" ", "#", "|")):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256") != kernel_source_digest(sources):
        return None
    try:
        return float(fields[key])
    except (KeyError, ValueError):
        return None


def profiled_traffic(name, sources=GEMM_SOURCES):
    """HBM bytes per launch (FETCH_SIZE and WRITE_SIZE runs, calibrated by a plain copy)."""
    return profiled_value(name, "traffic_bytes_per_launch", sources)


def only_kernel(workload, which, steps, warmup):
    """One grouped-GEMM launch of the workload repeated alone (for counter runs, where every
    matrix-core dispatch of the process is then this launch): the routing and permutation
    are computed once through moe_route / moe_permute, then K launches of the chosen stage
    through moe_grouped_gemm, bracketed by one event pair."""
    import torch
    import sparse_mixture_experts_gemm_amd as moe
    import workloads as W
    s = W.SHAPES[workload]
    run = Runner(s, W.make_layer(s))
    cfg, w = run.cfg, run.w
    T, k, E = s.T, s.k, s.E
    dev = "cuda"
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    tw = torch.empty((T, k), dtype=torch.float32, device=dev)
    moe.route(cfg, run.x, w.tensors["router"], w.tensors["logit_bias"], None, None, idx, tw)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    pt = torch.empty(T * k, dtype=torch.int32, device=dev)
    sp = torch.empty(T * k, dtype=torch.int32, device=dev)
    pw = torch.empty(T * k, dtype=torch.float32, device=dev)
    moe.permute(cfg, idx, tw, counts, offsets, pt, sp, pw, run.ws)
    adt = torch.int16 if s.act_dtype == "bf16" else torch.float32
    SI = s.S * s.I
    h_r = torch.zeros((T * k, s.I), dtype=adt, device=dev)
    h_s = torch.zeros((T, max(SI, 1)), dtype=adt, device=dev)
    y_r = torch.empty((T * k, s.d), dtype=adt, device=dev)
    y_s = torch.empty((T, s.d), dtype=adt, device=dev)
    R, SH = moe.MOE_EXPERTS_ROUTED, moe.MOE_EXPERTS_SHARED
    calls = {
        "up_routed": lambda: moe.grouped_gemm(cfg, moe.MOE_STAGE_UP, R, run.x, pt, offsets, T * k, w, None, h_r),
        "down_routed": lambda: moe.grouped_gemm(cfg, moe.MOE_STAGE_DOWN, R, h_r, None, offsets, T * k, w, pw, y_r),
        "up_shared": lambda: moe.grouped_gemm(cfg, moe.MOE_STAGE_UP, SH, run.x, None, None, T, w, None, h_s),
        "down_shared": lambda: moe.grouped_gemm(cfg, moe.MOE_STAGE_DOWN, SH, h_s, None, None, T, w, None, y_s),
    }
    # real h rows for the down projections
    calls["up_routed"]()
    if s.S > 0:
        calls["up_shared"]()
    f = calls[which]
    for _ in range(warmup):
        f()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        f()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    fl = stage_flops(s, T)[which]
    print(json.dumps({"workload": workload, "kernel": which, "steps": steps, "warmup": warmup,
                      "ms_per_launch": ms, "tflops": fl / (ms * 1e-3) / 1e12,
                      "frac_of_bf16_peak": fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}))
    return 0


def copy_probe(mib):
    """A plain device copy of a known size (torch's copy kernel), for scaling the TCC byte
    counters: run it under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "copies": 3}))
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="fusionllm_bf16")
    ap.add_argument("--cpu-tokens", type=int, default=4096)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--only-kernel", default="",
                    choices=["", "up_routed", "down_routed", "up_shared", "down_shared"],
                    help="only time this grouped-GEMM launch of the workload (counter runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-balance", action="store_true")
    ap.add_argument("--no-fp8", action="store_true")
    ap.add_argument("--no-prenorm", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-skewed", action="store_true")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the library runs the "
              "layer on one GPU and does not shard it across GPUs.", file=sys.stderr)
        return 2

    if args.copy_probe_mib > 0:
        return copy_probe(args.copy_probe_mib)
    if args.only_kernel:
        return only_kernel(args.workload, args.only_kernel, args.steps, args.warmup)

    import torch
    import workloads as W

    shape = W.SHAPES[args.workload]
    lay = W.make_layer(shape)
    run = Runner(shape, lay)
    step_ms, wall = run.timed(args.steps, args.warmup)
    T = shape.T
    fl = stage_flops(shape, T)
    total_flops = sum(fl.values())
    step_dist = run.step_distribution(args.steps, args.warmup)
    stage_ms = run.staged(args.steps, args.warmup)
    # the dominant kernel (the routed up projection), bracketed by its own two events
    dom = "up_routed"
    dom_ms = run.staged(args.steps, args.warmup, stages=[2, 3])[dom]
    achieved = fl[dom] / (dom_ms * 1e-3) / 1e12
    res = {
        "metric": "MoE fwd tokens/s & % MFMA peak, d2048 E64 k6 T4096; decode T64 % HBM BW",
        "value": T / (step_ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": shape.act_dtype if shape.weight_dtype != "e4m3" else "bf16-act/e4m3-weight",
        "data": "synthetic (seeded Gaussian x and weights, N(0,1/fan_in))",
        "config": {"workload": shape.name, "tokens": T, "dim": shape.d, "experts": shape.E,
                   "shared_experts": shape.S, "top_k": shape.k, "groups": shape.G,
                   "topk_groups": shape.Gk, "inter_dim": shape.I, "act": shape.act,
                   "weights": shape.weight_dtype},
        "layer_tflops": total_flops / (step_ms * 1e-3) / 1e12,
        "layer_mfma_frac": total_flops / (step_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "step_ms_per_step_events": step_dist,
        "stage_ms_with_events": stage_ms,
        "roofline": {"kernel": "grouped GEMM, routed up projection (SwiGLU epilogue)",
                     "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": profiled_traffic(f"traffic_up_routed_{shape.name}.txt"),
                     "kernel_ms": dom_ms, "algorithmic_tflop": fl[dom] / 1e12,
                     "mfma_busy_frac": profiled_value(f"counters_up_routed_{shape.name}.txt",
                                                      "mfma_busy_frac")},
    }
    if shape.name == "fusionllm_bf16":
        # the routed down projection, the kernel furthest below its roofline
        dn_ms = run.staged(args.steps, args.warmup, stages=[4, 5])["down_routed"]
        res["down_routed"] = {"kernel_ms": dn_ms,
                              "tflops": fl["down_routed"] / (dn_ms * 1e-3) / 1e12,
                              "frac": fl["down_routed"] / (dn_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                              "traffic": profiled_traffic(f"traffic_down_routed_{shape.name}.txt"),
                              "algorithmic_bytes": (shape.T * shape.k * (shape.I + shape.d) * 2
                                                    + shape.E * shape.d * shape.I * 2),
                              "mfma_busy_frac": profiled_value(
                                  f"counters_down_routed_{shape.name}.txt", "mfma_busy_frac")}
        # the tiny fp32 layer: latency-bound, reported in microseconds
        tshape = W.SHAPES["tiny_fp32"]
        trun = Runner(tshape, W.make_layer(tshape))
        t_ms, _ = trun.timed(args.steps, args.warmup)
        res["tiny"] = {"workload": tshape.name, "us_per_step": t_ms * 1e3,
                       "us_per_step_events": {k: (v * 1e3 if k != "steps" else v) for k, v in
                                              trun.step_distribution(args.steps, args.warmup).items()},
                       "tokens_per_s": tshape.T / (t_ms * 1e-3)}
        del trun
    if not args.no_decode:
        dshape = W.SHAPES["decode_bf16"]
        dlay = W.make_layer(dshape)
        drun = Runner(dshape, dlay, weights=run.w)     # same weights as the prefill layer
        d_ms_same, _ = drun.timed(args.steps, args.warmup)
        # two more device copies of the weights: consecutive steps read different copies,
        # so the 1.28 GB a step streams cannot come from the 256 MB Infinity Cache
        copies = [drun.w] + [run.moe.Weights(**{n: (None if t is None else t.clone())
                                                 for n, t in drun.w.tensors.items()})
                             for _ in range(2)]
        d_ms = drun.rotated_timed(copies, args.steps, args.warmup)
        del copies
        d_dist = drun.step_distribution(args.steps, args.warmup)
        d_graph_ms = drun.graph_timed(args.steps, args.warmup)
        d_stage = drun.staged(args.steps, args.warmup)
        d_up_ms = drun.staged(args.steps, args.warmup, stages=[2, 3])["up_routed"]
        counts = drun.counts()
        nbytes, touched = decode_bytes(dshape, counts)
        # the dominant decode kernel streams the up-projection weights of the touched
        # routed experts and of the shared experts in one launch
        up_bytes = (touched + dshape.S) * 2 * dshape.d * dshape.I * 2 + dshape.T * dshape.d * 2
        res["decode"] = {"workload": dshape.name, "tokens": dshape.T, "ms_per_step": d_ms,
                         "weights": "3 device copies, rotated every step",
                         "tokens_per_s": dshape.T / (d_ms * 1e-3),
                         "algorithmic_bytes": nbytes, "experts_touched": touched,
                         "hbm_GBps": nbytes / (d_ms * 1e-3) / 1e9,
                         "hbm_frac": nbytes / (d_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                         "same_weights_ms_per_step": d_ms_same,
                         "same_weights_hbm_frac": nbytes / (d_ms_same * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                         "step_ms_per_step_events": d_dist,
                         "graph_replay_ms_per_step": d_graph_ms,
                         "graph_replay_hbm_frac": nbytes / (d_graph_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                         "stage_ms_with_events": d_stage,
                         "roofline": {"kernel": "decode up projection (routed + shared experts, one launch)",
                                      "bound": "hbm",
                                      "achieved": up_bytes / (d_up_ms * 1e-3) / 1e9,
                                      "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                      "frac": up_bytes / (d_up_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                                      "traffic": profiled_traffic(
                                          f"traffic_decode_up_{dshape.name}.txt", DECODE_SOURCES),
                                      "kernel_ms": d_up_ms,
                                      "algorithmic_bytes": up_bytes}}
    if not args.no_balance and shape.name == "fusionllm_bf16":
        # the same layer with a selection-only expert bias, capacity factor 1.25 and the
        # load statistics written by every step
        bshape = W.SHAPES["balance_bf16"]
        blay = W.make_layer(bshape)
        brun = Runner(bshape, blay, weights=run.w)
        st = torch.empty(2 * bshape.E + 1, dtype=torch.float32, device="cuda")
        b_ms, _ = brun.timed(args.steps, args.warmup, load_stats=st)
        counts = brun.counts()
        stv = st.cpu().numpy()
        res["balance"] = {"workload": bshape.name, "capacity_factor": bshape.capacity_factor,
                          "select_bias": f"N(0, {bshape.select_bias_std}^2) per expert",
                          "ms_per_step": b_ms, "tokens_per_s": bshape.T / (b_ms * 1e-3),
                          "rows_kept_frac": float(counts.sum()) / (bshape.T * bshape.k),
                          "aux_loss_alpha1": float(stv[2 * bshape.E]),
                          "max_f_over_mean": float(stv[:bshape.E].max() * bshape.E)}
    if not args.no_prenorm and shape.name == "fusionllm_bf16":
        # the same layer as a pre-norm decoder step, h + MoE(RMSNorm(h)): the RMSNorm runs in
        # the routing launch and the residual in the combine
        pshape = W.SHAPES["prenorm_bf16"]
        prun = Runner(pshape, W.make_layer(pshape), weights=run.w)
        p_ms, _ = prun.timed(args.steps, args.warmup)
        p_route = prun.staged(args.steps, args.warmup, stages=[0, 1])["route"]
        p_comb = prun.staged(args.steps, args.warmup, stages=[6, 7])["combine"]
        res["prenorm"] = {"workload": pshape.name, "ms_per_step": p_ms,
                          "tokens_per_s": pshape.T / (p_ms * 1e-3),
                          "rmsnorm_route_ms": p_route, "plain_route_ms": stage_ms["route"],
                          "combine_with_residual_ms": p_comb,
                          "plain_combine_ms": stage_ms["combine"]}
    if not args.no_skewed and shape.name == "fusionllm_bf16":
        # the skewed prefill: 32768 tokens, Zipf(1.2) logit offsets (own weights)
        kshape = W.SHAPES["skewed_bf16"]
        krun = Runner(kshape, W.make_layer(kshape))
        k_ms, _ = krun.timed(max(5, args.steps // 5), args.warmup)
        kfl = sum(stage_flops(kshape, kshape.T).values())
        kc = krun.counts()
        res["skewed"] = {"workload": kshape.name, "ms_per_step": k_ms,
                         "tokens_per_s": kshape.T / (k_ms * 1e-3),
                         "layer_tflops": kfl / (k_ms * 1e-3) / 1e12,
                         "layer_mfma_frac": kfl / (k_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                         "expert_rows_max": int(kc.max()), "expert_rows_min": int(kc.min())}
        del krun
    if not args.no_backward and shape.name == "fusionllm_bf16":
        # gradients of the same layer: every data and weight gradient and the router's
        b_ms, b_ws = run.backward_timed(max(5, args.steps // 5), 2)
        c_act = 6 if shape.act == "swiglu" else 4
        gemm_fwd = (shape.k + shape.S) * T * c_act * shape.d * shape.I
        alg = 2 * gemm_fwd + 3 * 2 * T * shape.d * shape.E      # dgrad + wgrad of every GEMM
        res["backward"] = {"workload": shape.name, "ms_per_step": b_ms,
                           "tokens_per_s": T / (b_ms * 1e-3),
                           "algorithmic_tflop": alg / 1e12,
                           "tflops": alg / (b_ms * 1e-3) / 1e12,
                           "mfma_frac": alg / (b_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                           "recomputed_up_tflop": gemm_fwd * (2 / 3 if shape.act == "swiglu" else 1 / 2) / 1e12,
                           "workspace_gb": b_ws / 1e9}
    if not args.no_fp8 and shape.name == "fusionllm_bf16":
        # the e4m3-weight layer (T = 16384, ReLU^2): bf16 activations, then e4m3 activations
        # in the up projections (same device weights)
        f8 = {}
        base = None
        for name in ("fp8_relu2", "fp8a_relu2"):
            fshape = W.SHAPES[name]
            frun = Runner(fshape, W.make_layer(fshape), weights=base)
            base = frun.w
            f_ms, _ = frun.timed(max(5, args.steps // 4), args.warmup)
            up_ms = frun.staged(max(5, args.steps // 4), args.warmup, stages=[2, 3])["up_routed"]
            ffl = stage_flops(fshape, fshape.T)
            lfl = sum(ffl.values())
            f8[name] = {"ms_per_step": f_ms, "tokens_per_s": fshape.T / (f_ms * 1e-3),
                        "layer_tflops": lfl / (f_ms * 1e-3) / 1e12,
                        "layer_frac_of_bf16_peak": lfl / (f_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                        "up_routed_ms": up_ms,
                        "up_routed_tflops": ffl["up_routed"] / (up_ms * 1e-3) / 1e12}
        up_a8 = f8["fp8a_relu2"]["up_routed_tflops"]
        f8["fp8a_relu2"]["up_routed_frac_of_fp8_peak"] = up_a8 / PEAK_FP8_TFLOPS
        f8["fp8_relu2"]["up_routed_frac_of_bf16_peak"] = f8["fp8_relu2"]["up_routed_tflops"] / PEAK_BF16_TFLOPS
        res["fp8"] = f8
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(lay, min(args.cpu_tokens, shape.T), args.cpu_seconds)
    print(json.dumps(res))
    return 0


if __name__ == "__main__":
    sys.exit(main())
