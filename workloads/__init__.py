"""Seeded synthetic inputs for the MoE FFN forward.

This module is shared by the HIP-path tests, the oracle tests and the benchmark.  It
holds no step of the layer's arithmetic: it only draws Gaussian tensors and stores them
in the encodings the layer consumes (fp32, bf16 bit patterns, or e4m3 codes with a
per-output-channel fp32 scale).  Reading the stored encodings back into numbers is the
consumer's job (the oracle decodes them itself; the GPU kernels read the bits).

Workload recipe (the pages publish no dataset or trained weights for this layer, so
seeded Gaussian stand-ins are used):

* x ~ N(0, 1); every weight ~ N(0, 1/fan_in), fan_in = dim for router, gate and up
  projections and inter_dim for down projections.
* Each tensor has its own child stream of ``SeedSequence(seed)``, assigned in a fixed
  order: router; shared experts s = 0..S-1 (gate, up, down); routed experts
  e = 0..E-1 (gate, up, down); x; the Zipf permutation.  ReLU^2 layers have no up
  projection and skip that stream.
* Values are drawn in fp32 and then stored: fp32 as is, bf16 by round-to-nearest-even
  of the fp32 bit pattern, e4m3 by a per-output-channel scale max|W[n,:]|/448 and
  round-to-nearest-even onto the e4m3 grid, saturating at 448.
* Pre-norm shapes: every stored x row is scaled by exp(0.5 z), z ~ N(0, 1) (a residual
  stream whose rows differ in magnitude), and the RMSNorm gain is 1 + 0.1 N(0, 1) per
  channel; both from the stream ``SeedSequence([seed, 0x2A0E])``.

Shapes follow the FusionLLM MoE configuration ("FusionLLM：融合 MLA、GDN 与 MoE 的高效混合架构大模型训练框架",
section 模型配置与规模: dim 2048, 64 routed experts, 6 active, 4 shared, expert inter dim 1536).
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

__all__ = ["MoeShape", "Layer", "SHAPES", "make_layer", "encode_bf16", "encode_e4m3_rows",
           "shape_by_name"]


@dataclass(frozen=True)
class MoeShape:
    name: str
    T: int                 # tokens
    d: int                 # model dim
    E: int                 # routed experts
    k: int                 # experts per token
    score: str             # "softmax" | "sigmoid"
    G: int                 # expert groups
    Gk: int                # groups kept per token
    S: int                 # shared experts
    I: int                 # expert inter dim
    act: str               # "swiglu" | "relu2"
    act_dtype: str         # "f32" | "bf16"  (x, router, intermediates, output)
    weight_dtype: str      # "f32" | "bf16" | "e4m3"  (expert weights)
    seed: int
    n_g: int = 1           # experts summed into a group score (1 = group max)
    zipf_s: Optional[float] = None   # per-expert logit offsets -s*ln(1+rank)
    renormalize: bool = True
    route_scale: float = 1.0
    x_from: Optional[str] = None     # take x rows (and weights) of another shape
    capacity_factor: Optional[float] = None   # expert capacity c*T*k/E (None: unlimited)
    select_bias_std: Optional[float] = None   # selection-only per-expert bias ~ N(0, std^2)
    fp8_act: bool = False  # up projections take e4m3 activations with per-token scales
    pre_norm: bool = False     # the MoE reads RMSNorm(x) (gain norm_gamma, eps norm_eps)
    norm_eps: float = 1e-6
    residual: bool = False     # the output adds the unnormalised x

    @property
    def flops_per_token(self) -> int:
        c_act = 6 if self.act == "swiglu" else 4
        return 2 * self.d * self.E + (self.k + self.S) * c_act * self.d * self.I


SHAPES = {
    # tiny fp32 case the oracle finishes instantly
    "tiny_fp32": MoeShape("tiny_fp32", T=64, d=128, E=8, k=2, score="softmax", G=1, Gk=1,
                          S=0, I=256, act="swiglu", act_dtype="f32", weight_dtype="f32",
                          seed=0),
    # FusionLLM-shape prefill layer
    "fusionllm_bf16": MoeShape("fusionllm_bf16", T=4096, d=2048, E=64, k=6, score="sigmoid",
                               G=8, Gk=4, S=4, I=1536, act="swiglu", act_dtype="bf16",
                               weight_dtype="bf16", seed=1),
    # decode: 64 sequences x 1 step, weights and first 64 x rows of the prefill layer
    "decode_bf16": MoeShape("decode_bf16", T=64, d=2048, E=64, k=6, score="sigmoid", G=8,
                            Gk=4, S=4, I=1536, act="swiglu", act_dtype="bf16",
                            weight_dtype="bf16", seed=1, x_from="fusionllm_bf16"),
    # large prefill with Zipf(1.2) router logit offsets (highly imbalanced loads)
    "skewed_bf16": MoeShape("skewed_bf16", T=32768, d=2048, E=64, k=6, score="sigmoid", G=8,
                            Gk=4, S=4, I=1536, act="swiglu", act_dtype="bf16",
                            weight_dtype="bf16", seed=3, zipf_s=1.2),
    # e4m3 expert weights, bf16 activations, Linear+ReLU^2 experts
    "fp8_relu2": MoeShape("fp8_relu2", T=16384, d=2048, E=64, k=6, score="sigmoid", G=8,
                          Gk=4, S=4, I=1536, act="relu2", act_dtype="bf16",
                          weight_dtype="e4m3", seed=4),
    # the e4m3 layer with the up projections on e4m3 x e4m3 products (per-token scales)
    "fp8a_relu2": MoeShape("fp8a_relu2", T=16384, d=2048, E=64, k=6, score="sigmoid", G=8,
                           Gk=4, S=4, I=1536, act="relu2", act_dtype="bf16",
                           weight_dtype="e4m3", seed=4, x_from="fp8_relu2", fp8_act=True),
    # the prefill layer with a selection-only expert bias and capacity factor 1.25
    "balance_bf16": MoeShape("balance_bf16", T=4096, d=2048, E=64, k=6, score="sigmoid", G=8,
                             Gk=4, S=4, I=1536, act="swiglu", act_dtype="bf16",
                             weight_dtype="bf16", seed=1, x_from="fusionllm_bf16",
                             capacity_factor=1.25, select_bias_std=0.5),
    # the prefill layer as a pre-norm decoder step: h + MoE(RMSNorm(h))
    "prenorm_bf16": MoeShape("prenorm_bf16", T=4096, d=2048, E=64, k=6, score="sigmoid", G=8,
                             Gk=4, S=4, I=1536, act="swiglu", act_dtype="bf16",
                             weight_dtype="bf16", seed=1, x_from="fusionllm_bf16",
                             pre_norm=True, residual=True),
    # its decode step: 64 tokens of the pre-norm layer
    "prenorm_decode_bf16": MoeShape("prenorm_decode_bf16", T=64, d=2048, E=64, k=6,
                                    score="sigmoid", G=8, Gk=4, S=4, I=1536, act="swiglu",
                                    act_dtype="bf16", weight_dtype="bf16", seed=1,
                                    x_from="fusionllm_bf16", pre_norm=True, residual=True),
}
ORDER = ["tiny_fp32", "fusionllm_bf16", "decode_bf16", "skewed_bf16", "fp8_relu2", "balance_bf16",
         "fp8a_relu2", "prenorm_bf16", "prenorm_decode_bf16"]


def shape_by_name(name: str) -> MoeShape:
    return SHAPES[name]


# ----------------------------------------------------------------------------- encoders
def encode_bf16(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even (finite input)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def _e4m3_positive_grid() -> np.ndarray:
    # codes 0..126 (0x7F is NaN); value of code c = (e, m) = (c >> 3, c & 7)
    vals = np.empty(127, dtype=np.float64)
    for c in range(127):
        e, m = c >> 3, c & 7
        vals[c] = math.ldexp(m / 8.0, -6) if e == 0 else math.ldexp(1.0 + m / 8.0, e - 7)
    return vals


_E4M3_GRID = _e4m3_positive_grid()


def encode_e4m3_rows(w: np.ndarray):
    """Per-output-channel e4m3 quantisation of a [..., N, K] fp32 weight.

    Returns (codes uint8 [..., N, K], scale float32 [..., N]) with
    scale = max|W[n,:]| / 448 and codes = RNE(W / scale) on the e4m3 grid, saturating.
    """
    w = np.asarray(w, dtype=np.float32)
    amax = np.max(np.abs(w), axis=-1)
    scale = (amax / np.float32(448.0)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0))
    y = (w / safe[..., None]).astype(np.float64)
    ay = np.minimum(np.abs(y), 448.0)
    hi = np.searchsorted(_E4M3_GRID, ay, side="left")          # first grid value >= ay
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    dlo = ay - _E4M3_GRID[lo]
    dhi = _E4M3_GRID[hi] - ay
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((hi & 1) == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(ay == 0.0, np.uint8(0), code)
    code = code | np.where(y < 0, np.uint8(0x80), np.uint8(0))
    return code.astype(np.uint8), scale


# ----------------------------------------------------------------------------- layer
@dataclass
class Layer:
    shape: MoeShape
    x: np.ndarray                      # [T, d]  act encoding
    router: np.ndarray                 # [E, d]  act encoding
    logit_bias: Optional[np.ndarray]   # [E] fp32 or None
    w_gate: np.ndarray                 # [E, I, d]
    w_up: Optional[np.ndarray]         # [E, I, d] (None for relu2)
    w_down: np.ndarray                 # [E, d, I]
    sh_gate: Optional[np.ndarray]      # [S, I, d]
    sh_up: Optional[np.ndarray]
    sh_down: Optional[np.ndarray]      # [S, d, I]
    s_gate: Optional[np.ndarray] = None    # e4m3 scales [E, I]
    s_up: Optional[np.ndarray] = None
    s_down: Optional[np.ndarray] = None    # [E, d]
    sh_s_gate: Optional[np.ndarray] = None
    sh_s_up: Optional[np.ndarray] = None
    sh_s_down: Optional[np.ndarray] = None
    select_bias: Optional[np.ndarray] = None   # [E] fp32, selection only
    norm_gamma: Optional[np.ndarray] = None    # [d] fp32 RMSNorm gain (pre-norm layers)
    extra: dict = field(default_factory=dict)


def _store(a32: np.ndarray, dtype: str):
    if dtype == "f32":
        return a32.astype(np.float32), None
    if dtype == "bf16":
        return encode_bf16(a32), None
    if dtype == "e4m3":
        return encode_e4m3_rows(a32)
    raise ValueError(dtype)


def _normal(seed_seq, shape, std):
    g = np.random.Generator(np.random.PCG64(seed_seq))
    a = g.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


_CACHE: dict = {}


def _select_bias(s: MoeShape):
    """Selection-only expert bias of a shape: its own seeded stream (independent of the
    weight streams, so shapes that share weights can differ in bias)."""
    if s.select_bias_std is None:
        return None
    st = np.random.SeedSequence([s.seed, 0x5E1EC7])
    return _normal(st, (s.E,), s.select_bias_std).astype(np.float32)


def _decode_stored(a, dtype: str) -> np.ndarray:
    """Stored activations back to fp32 (bf16 bits are the upper half of an fp32)."""
    if dtype == "bf16":
        return (np.asarray(a, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    return np.asarray(a, np.float32)


def _pre_norm_inputs(s: MoeShape, x):
    """Pre-norm layers: the stored x stands for a residual stream whose rows differ in
    magnitude, so every row is scaled by exp(0.5 z), z ~ N(0, 1); the RMSNorm gain is
    1 + 0.1 N(0, 1) per channel.  Both come from the shape's own stream."""
    if not s.pre_norm:
        return x, None
    st = np.random.SeedSequence([s.seed, 0x2A0E]).spawn(2)
    gamma = (np.float32(1.0) + _normal(st[0], (s.d,), 0.1)).astype(np.float32)
    row = np.exp(_normal(st[1], (s.T, 1), 0.5)).astype(np.float32)
    x32 = _decode_stored(x, s.act_dtype) * row
    enc, _ = _store(x32.astype(np.float32), s.act_dtype)
    return enc, gamma


def make_layer(shape: MoeShape | str, threads: int = 8, cache: bool = True) -> Layer:
    """Build the seeded layer (inputs + weights) of a shape."""
    if isinstance(shape, str):
        shape = SHAPES[shape]
    if shape.x_from is not None:
        base = make_layer(shape.x_from, threads=threads, cache=cache)
        lay = Layer(**{**base.__dict__})
        lay.shape = shape
        lay.x, lay.norm_gamma = _pre_norm_inputs(shape, base.x[: shape.T].copy())
        lay.select_bias = _select_bias(shape)
        return lay
    if cache and shape.name in _CACHE:
        return _CACHE[shape.name]

    s = shape
    swiglu = s.act == "swiglu"
    n_mats = 3 if swiglu else 2
    n_streams = 1 + n_mats * (s.S + s.E) + 2
    streams = np.random.SeedSequence(s.seed).spawn(n_streams)
    it = iter(range(n_streams))

    router_stream = streams[next(it)]
    jobs = []   # (kind, index, which, stream)
    for kind, count in (("shared", s.S), ("routed", s.E)):
        for i in range(count):
            jobs.append((kind, i, "gate", streams[next(it)]))
            if swiglu:
                jobs.append((kind, i, "up", streams[next(it)]))
            jobs.append((kind, i, "down", streams[next(it)]))
    x_stream = streams[next(it)]
    perm_stream = streams[next(it)]

    wdt = s.weight_dtype
    np_w = {"f32": np.float32, "bf16": np.uint16, "e4m3": np.uint8}[wdt]
    np_a = {"f32": np.float32, "bf16": np.uint16}[s.act_dtype]

    def alloc(count, rows, cols):
        if count == 0:
            return None
        return np.empty((count, rows, cols), dtype=np_w)

    def alloc_scale(count, rows):
        if count == 0 or wdt != "e4m3":
            return None
        return np.empty((count, rows), dtype=np.float32)

    mats = {
        ("routed", "gate"): alloc(s.E, s.I, s.d), ("routed", "up"): alloc(s.E, s.I, s.d) if swiglu else None,
        ("routed", "down"): alloc(s.E, s.d, s.I),
        ("shared", "gate"): alloc(s.S, s.I, s.d), ("shared", "up"): alloc(s.S, s.I, s.d) if swiglu else None,
        ("shared", "down"): alloc(s.S, s.d, s.I),
    }
    scales = {
        ("routed", "gate"): alloc_scale(s.E, s.I), ("routed", "up"): alloc_scale(s.E, s.I) if swiglu else None,
        ("routed", "down"): alloc_scale(s.E, s.d),
        ("shared", "gate"): alloc_scale(s.S, s.I), ("shared", "up"): alloc_scale(s.S, s.I) if swiglu else None,
        ("shared", "down"): alloc_scale(s.S, s.d),
    }

    def run(job):
        kind, i, which, st = job
        if which == "down":
            a = _normal(st, (s.d, s.I), 1.0 / math.sqrt(s.I))
        else:
            a = _normal(st, (s.I, s.d), 1.0 / math.sqrt(s.d))
        enc, sc = _store(a, wdt)
        mats[(kind, which)][i] = enc
        if sc is not None:
            scales[(kind, which)][i] = sc

    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(run, jobs))

    router, _ = _store(_normal(router_stream, (s.E, s.d), 1.0 / math.sqrt(s.d)), s.act_dtype)
    x, _ = _store(_normal(x_stream, (s.T, s.d), 1.0), s.act_dtype)
    x, gamma = _pre_norm_inputs(s, x)
    bias = None
    if s.zipf_s is not None:
        g = np.random.Generator(np.random.PCG64(perm_stream))
        rank = g.permutation(s.E)
        bias = (-s.zipf_s * np.log1p(rank.astype(np.float64))).astype(np.float32)

    lay = Layer(shape=s, x=x.astype(np_a), router=router.astype(np_a), logit_bias=bias,
                w_gate=mats[("routed", "gate")], w_up=mats[("routed", "up")],
                w_down=mats[("routed", "down")], sh_gate=mats[("shared", "gate")],
                sh_up=mats[("shared", "up")], sh_down=mats[("shared", "down")],
                s_gate=scales[("routed", "gate")], s_up=scales[("routed", "up")],
                s_down=scales[("routed", "down")], sh_s_gate=scales[("shared", "gate")],
                sh_s_up=scales[("shared", "up")], sh_s_down=scales[("shared", "down")],
                select_bias=_select_bias(s), norm_gamma=gamma)
    if cache:
        _CACHE[shape.name] = lay
    return lay


def small_shape(**kw) -> MoeShape:
    """A custom shape for tests (defaults: a small bf16 sigmoid layer with groups)."""
    base = dict(name="custom", T=96, d=256, E=16, k=4, score="sigmoid", G=4, Gk=2, S=1,
                I=128, act="swiglu", act_dtype="bf16", weight_dtype="bf16", seed=11)
    base.update(kw)
    return MoeShape(**base)


def clear_cache():
    _CACHE.clear()


def random_act(shape, seed: int, dtype: str = "bf16", std: float = 1.0) -> np.ndarray:
    """Seeded N(0, std^2) tensor stored in an activation encoding (bf16 bits or fp32)."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    a = g.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return encode_bf16(a) if dtype == "bf16" else a
