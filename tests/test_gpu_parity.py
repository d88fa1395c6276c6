"""GPU parity of every libmoe entry point against the fp64 CPU oracle.

All inputs come from the seeded generator (workloads) or from the oracle; the only GPU
values handed to the oracle are the fp32 router scores and the selected experts, and
only after the parity protocol has checked them.  Bars:
* selection (moe_select on shared fp32 scores) and permutation: bit-exact;
* routing by moe_route: GPU scores within 1e-5 of the oracle's fp64 scores, and the
  oracle's selection applied to the GPU's own fp32 scores equal to the GPU's indices for
  every token, bit for bit; against the free-running fp64 oracle the indices are
  identical wherever the fp64 decision margin exceeds 1e-5 (a smaller margin is below
  the fp32 score error, so either choice is correct: those tokens are checked for
  validity instead);
* float outputs: every row, max|delta| <= 2e-2 max|ref| (bf16) and <= 1e-4 max|ref|
  (fp32), against the oracle run under the GPU's checked routing.
"""
import numpy as np
import pytest
import torch

import oracle as O
import sparse_mixture_experts_gemm_amd as moe
import workloads as W
from _dev import act_empty, act_to_f64, config, to_dev, weights, workspace

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}
MARGIN = 1e-5

SMALL = {
    # ragged everything: T not a multiple of the tiles, I and d give partial n-tiles
    "small_swiglu": W.small_shape(T=300, d=320, E=16, k=4, G=4, Gk=2, S=2, I=192, seed=31),
    "small_relu2_e4m3": W.small_shape(T=200, d=256, E=8, k=2, G=2, Gk=1, n_g=2, S=2, I=320,
                                      act="relu2", weight_dtype="e4m3", seed=32),
    "small_swiglu_e4m3": W.small_shape(T=150, d=192, E=16, k=3, G=1, Gk=1, S=1, I=128,
                                       weight_dtype="e4m3", seed=33),
    "small_f32": W.small_shape(T=77, d=48, E=8, k=3, score="softmax", G=1, Gk=1, S=1, I=32,
                               act_dtype="f32", weight_dtype="f32", seed=34),
    "single_token": W.small_shape(T=1, d=128, E=64, k=6, G=8, Gk=4, S=1, I=64, seed=35),
    "topk1_nogroups": W.small_shape(T=130, d=128, E=32, k=1, G=1, Gk=1, S=0, I=64, seed=36,
                                    renormalize=False, route_scale=2.5),
    # the largest selection: every token to every expert (k = E, softmax, no groups)
    "all_experts": W.small_shape(T=100, d=128, E=16, k=16, score="softmax", G=1, Gk=1, S=0, I=64,
                                 seed=53),
    # more tiles than workgroups: each persistent workgroup streams several tiles
    "multi_tile_swiglu": W.small_shape(T=8192, d=512, E=8, k=4, G=1, Gk=1, S=1, I=256, seed=37),
    "multi_tile_relu2_e4m3": W.small_shape(T=8192, d=512, E=8, k=4, G=2, Gk=1, S=1, I=256,
                                           act="relu2", weight_dtype="e4m3", seed=38),
    # enough rows for 256 x 256 tiles in the routed GEMMs (bf16; e4m3 weights, whose down
    # projection takes them with a single weight-scale block)
    "multi_tile_wide": W.small_shape(T=16384, d=512, E=8, k=4, G=1, Gk=1, S=1, I=512, seed=40),
    "multi_tile_wide_e4m3": W.small_shape(T=16384, d=512, E=8, k=4, G=1, Gk=1, S=1, I=512,
                                          act="relu2", weight_dtype="e4m3", seed=52),
    "multi_tile_wide_swiglu_e4m3": W.small_shape(T=16384, d=512, E=8, k=4, G=1, Gk=1, S=1,
                                                 I=512, weight_dtype="e4m3", seed=85),
    "multi_tile_wide_relu2_bf16": W.small_shape(T=16384, d=512, E=8, k=4, G=1, Gk=1, S=1,
                                                I=1024, act="relu2", seed=86),
    # selection-only expert bias: softmax gating (fp32) and n_g = 2 groups (bf16)
    "biased_softmax_f32": W.small_shape(T=257, d=128, E=16, k=3, score="softmax", G=1, Gk=1,
                                        S=0, I=64, act_dtype="f32", weight_dtype="f32",
                                        select_bias_std=1.0, seed=41),
    "biased_groups_n2": W.small_shape(T=333, d=256, E=32, k=4, G=8, Gk=3, n_g=2, S=1, I=128,
                                      select_bias_std=0.7, capacity_factor=1.0, seed=42),
    # e4m3 activations in the up projections (with e4m3 weights)
    "small_a8_swiglu": W.small_shape(T=300, d=256, E=16, k=4, G=4, Gk=2, S=2, I=192,
                                     weight_dtype="e4m3", fp8_act=True, seed=43),
    "multi_tile_a8_relu2": W.small_shape(T=8192, d=512, E=8, k=4, G=1, Gk=1, S=1, I=256,
                                         act="relu2", weight_dtype="e4m3", fp8_act=True, seed=44),
    # SwiGLU on e4m3 activations with 256 x 256 tiles in the routed up projection
    "wide_a8_swiglu": W.small_shape(T=16384, d=512, E=8, k=4, G=1, Gk=1, S=1, I=512,
                                    weight_dtype="e4m3", fp8_act=True, seed=54),
    # K = 64: one K-slice per tile, several tiles per workgroup
    "short_k": W.small_shape(T=40000, d=64, E=4, k=2, G=1, Gk=1, S=1, I=64, seed=39),
    # pre-norm layers (RMSNorm before the router and experts, optional residual)
    "small_prenorm_bf16": W.small_shape(T=300, d=320, E=16, k=4, G=4, Gk=2, S=2, I=192,
                                        pre_norm=True, residual=True, seed=45),
    "small_prenorm_noresid": W.small_shape(T=257, d=256, E=16, k=4, G=1, Gk=1, S=1, I=128,
                                           pre_norm=True, norm_eps=1e-5, seed=46),
    "small_prenorm_f32": W.small_shape(T=77, d=48, E=8, k=3, score="softmax", G=1, Gk=1, S=1,
                                       I=32, act_dtype="f32", weight_dtype="f32",
                                       pre_norm=True, residual=True, seed=47),
    "small_prenorm_a8": W.small_shape(T=300, d=256, E=16, k=4, G=4, Gk=2, S=2, I=192,
                                      weight_dtype="e4m3", fp8_act=True, pre_norm=True,
                                      residual=True, seed=48),
    # the widest rows staged in LDS by the pre-norm routing, and wider ones recomputed
    "prenorm_d4096": W.small_shape(T=33, d=4096, E=8, k=2, G=1, Gk=1, S=1, I=64,
                                   pre_norm=True, residual=True, seed=50),
    "prenorm_d4160": W.small_shape(T=40, d=4160, E=8, k=2, G=2, Gk=1, S=0, I=64,
                                   pre_norm=True, residual=True, seed=51),
    "biased_prenorm": W.small_shape(T=333, d=256, E=32, k=4, G=8, Gk=3, n_g=2, S=1, I=128,
                                    select_bias_std=0.7, capacity_factor=1.0, pre_norm=True,
                                    residual=True, seed=49),
    # dim and inter_dim off the 64-element grid (multiples of 8 for bf16, of 16 for e4m3
    # weights): the router's K tail and the tail grouped GEMM
    "tail_bf16": W.small_shape(T=300, d=200, E=16, k=4, G=4, Gk=2, S=2, I=136, seed=60),
    "tail_e4m3": W.small_shape(T=250, d=208, E=8, k=2, G=2, Gk=1, S=2, I=144,
                               weight_dtype="e4m3", seed=61),
    "tail_relu2_e4m3": W.small_shape(T=190, d=208, E=8, k=3, G=1, Gk=1, S=1, I=176,
                                     act="relu2", weight_dtype="e4m3", seed=62),
    "tail_d_only": W.small_shape(T=200, d=200, E=8, k=2, G=2, Gk=1, S=1, I=128, seed=63),
    "tail_i_only": W.small_shape(T=200, d=256, E=8, k=2, G=2, Gk=1, S=3, I=72, seed=64),
    # several tail tiles per workgroup
    "tail_multi": W.small_shape(T=16384, d=200, E=8, k=4, G=1, Gk=1, S=1, I=136, seed=65),
    "tail_prenorm": W.small_shape(T=150, d=200, E=16, k=4, G=4, Gk=2, S=1, I=136,
                                  pre_norm=True, residual=True, seed=66),
    # ReLU^2 with bf16 weights on every GEMM family (tiled, weight-streaming, tail), and
    # SwiGLU with e4m3 weights on the weight-streaming one
    "small_relu2_bf16": W.small_shape(T=300, d=256, E=16, k=4, G=4, Gk=2, S=1, I=256,
                                      act="relu2", seed=81),
    "decode_relu2_bf16": W.small_shape(T=40, d=256, E=16, k=4, G=4, Gk=2, S=1, I=256,
                                       act="relu2", seed=82),
    "decode_swiglu_e4m3": W.small_shape(T=48, d=256, E=16, k=4, G=4, Gk=2, S=1, I=256,
                                        weight_dtype="e4m3", seed=83),
    "tail_relu2_bf16": W.small_shape(T=200, d=200, E=8, k=2, G=2, Gk=1, S=1, I=136,
                                     act="relu2", seed=84),
}


def shape_of(name):
    return SMALL[name] if name in SMALL else W.SHAPES[name]


def layer_of(name):
    s = shape_of(name)
    return W.make_layer(s, cache=name in W.SHAPES)


def fp32_scores(lay, tokens=None):
    r = O.route(lay, tokens)
    return r


def margins(scores64, s):
    """Smallest fp64 decision margin per token (group boundary and top-k order)."""
    T, E = scores64.shape
    m = np.full(T, np.inf)
    if s.G > 1 and s.Gk < s.G:
        gs = O.group_scores(scores64, s.G, s.n_g)
        gsrt = -np.sort(-gs, axis=1)
        m = np.minimum(m, gsrt[:, s.Gk - 1] - gsrt[:, s.Gk])
        gorder = np.lexsort((np.broadcast_to(np.arange(s.G), gs.shape), -gs), axis=-1)
        kept = np.zeros_like(gs, dtype=bool)
        np.put_along_axis(kept, gorder[:, :s.Gk], True, axis=-1)
        elig = np.repeat(kept, E // s.G, axis=1)
    else:
        elig = np.ones((T, E), bool)
    se = np.where(elig, scores64, -1.0)
    srt = -np.sort(-se, axis=1)
    upto = min(s.k + 1, E)
    gaps = srt[:, :upto - 1] - srt[:, 1:upto]
    m = np.minimum(m, gaps.min(axis=1))
    return m


def valid_within_margin(row, sc, s, eps=2 * MARGIN):
    """Is ``row`` a correct group-limited top-k of the fp64 scores ``sc`` once every score
    may move by eps?  (Checked directly from the definition, without the oracle.)"""
    row = np.asarray(row)
    if len(set(row.tolist())) != s.k or row.min() < 0 or row.max() >= s.E:
        return False
    gsz = s.E // s.G
    limited = s.G > 1 and s.Gk < s.G
    if limited:
        gs = np.array([np.sort(sc[g * gsz:(g + 1) * gsz])[::-1][:s.n_g].sum() for g in range(s.G)])
        cut = np.sort(gs)[::-1][s.Gk - 1]
        used = set((row // gsz).tolist())
        if len(used) > s.Gk or any(gs[g] < cut - s.n_g * eps for g in used):
            return False
        # groups certainly kept (clearly above the Gk-th) plus the used ones are eligible
        sure = {g for g in range(s.G) if gs[g] > np.sort(gs)[::-1][s.Gk] + s.n_g * eps}
        elig = np.array([(e // gsz) in (used | sure) for e in range(s.E)])
    else:
        elig = np.ones(s.E, bool)
    low = sc[row].min()
    others = np.array([e for e in range(s.E) if elig[e] and e not in set(row.tolist())], dtype=int)
    return others.size == 0 or sc[others].max() <= low + eps


def sample_tokens(T, n=128, seed=0):
    if T <= n:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(32, T - 32), size=n - 64, replace=False)
    return np.unique(np.concatenate([np.arange(32), mid, np.arange(T - 32, T)]))


# ----------------------------------------------------------------------------- select
SELECT_CASES = ["tiny_fp32", "fusionllm_bf16", "skewed_bf16", "fp8_relu2", "small_swiglu",
                "small_relu2_e4m3", "topk1_nogroups"]


@pytest.mark.parametrize("name", SELECT_CASES)
def test_select_bit_exact_on_oracle_scores(name):
    s = shape_of(name)
    lay = layer_of(name)
    T = min(s.T, 8192)
    r = O.route(lay, np.arange(T))
    sc32 = r["scores"].astype(np.float32)
    cfg = config(s, T=T)
    idx = torch.empty((T, s.k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, s.k), dtype=torch.float32, device="cuda")
    moe.select(cfg, to_dev(sc32), None, idx, w)
    torch.cuda.synchronize()
    ref_idx = O.select_experts(sc32, s.k, s.G, s.Gk, s.n_g)
    assert np.array_equal(idx.cpu().numpy(), ref_idx)
    ref_w = O.routing_weights(sc32.astype(np.float64), ref_idx, s.renormalize, s.route_scale)
    assert np.allclose(w.cpu().numpy(), ref_w, rtol=2e-6, atol=1e-7)


@pytest.mark.parametrize("name", ["balance_bf16", "biased_softmax_f32", "biased_groups_n2"])
def test_select_on_keys_bit_exact(name):
    """Selection on given fp32 keys (the scores of the biased logits), weights from the
    unbiased scores: indices bit-exact against the oracle's selection on the same keys."""
    s = shape_of(name)
    lay = layer_of(name)
    r = O.route(lay)
    sc32 = r["scores"].astype(np.float32)
    k32 = r["keys"].astype(np.float32)
    cfg = config(s)
    idx = torch.empty((s.T, s.k), dtype=torch.int32, device="cuda")
    w = torch.empty((s.T, s.k), dtype=torch.float32, device="cuda")
    moe.select(cfg, to_dev(sc32), to_dev(k32), idx, w)
    torch.cuda.synchronize()
    ref_idx = O.select_experts(k32, s.k, s.G, s.Gk, s.n_g)
    assert np.array_equal(idx.cpu().numpy(), ref_idx)
    ref_w = O.routing_weights(sc32.astype(np.float64), ref_idx, s.renormalize, s.route_scale)
    assert np.allclose(w.cpu().numpy(), ref_w, rtol=2e-6, atol=1e-7)


def adversarial_scores(T, E, seed):
    rng = np.random.default_rng(seed)
    a = (rng.integers(0, 8, size=(T, E)) / 8.0).astype(np.float32)      # heavy ties
    a[0] = 0.5                                                         # all equal
    a[1] = 0.0                                                         # all zero
    a[2] = np.arange(E, dtype=np.float32) / E                          # ascending
    a[3] = np.arange(E, dtype=np.float32)[::-1] / E                    # descending
    a[4, ::2] = 0.75                                                   # ties across groups
    a[5] = 0.25
    a[5, -1] = 1.0                                                     # winner in last group
    return a


@pytest.mark.parametrize("E,k,G,Gk,n_g", [(64, 6, 8, 4, 1), (64, 6, 8, 4, 2), (64, 8, 1, 1, 1),
                                          (16, 4, 4, 1, 2), (8, 8, 1, 1, 1), (64, 1, 64, 3, 1),
                                          (12, 5, 3, 2, 2), (64, 64, 1, 1, 1), (64, 32, 8, 4, 2)])
def test_select_bit_exact_on_tie_laden_scores(E, k, G, Gk, n_g):
    T = 1000
    sc = adversarial_scores(T, E, seed=E * 100 + k * 10 + G + n_g)
    cfg = moe.make_config(T, 64, E, k, G=G, Gk=Gk, n_g=n_g, I=64)
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    moe.select(cfg, to_dev(sc), None, idx, w)
    torch.cuda.synchronize()
    ref = O.select_experts(sc, k, G, Gk, n_g)
    assert np.array_equal(idx.cpu().numpy(), ref)
    sel = np.take_along_axis(sc.astype(np.float64), ref.astype(np.int64), axis=1)
    tot = sel.sum(axis=1, keepdims=True)
    with np.errstate(invalid="ignore", divide="ignore"):
        ref_w = sel / tot
    ok = tot[:, 0] > 0
    assert np.allclose(w.cpu().numpy()[ok], ref_w[ok], rtol=2e-6, atol=1e-7)


@pytest.mark.parametrize("seed", range(24))
def test_select_random_bit_exact(seed):
    """Seeded random selection problems: any E up to 64 with any group count dividing it,
    Gk, n_g in {1, 2}, k up to the eligible experts, continuous or tie-laden (eighths)
    scores, with or without separate selection keys, renormalised or scaled weights:
    indices bit-exact against the oracle's selection, weights within 2e-6."""
    g = np.random.default_rng(6000 + seed)
    E = int(g.integers(1, 65))
    G = int(g.choice([x for x in range(1, E + 1) if E % x == 0]))
    Gk = int(g.integers(1, G + 1))
    n_g = int(g.choice([1, 2])) if E // G >= 2 else 1
    k = int(g.integers(1, Gk * (E // G) + 1))
    T = int(g.choice([1, 7, 100, 1000, 5000]))
    ties = bool(g.integers(0, 2))
    draw = lambda: ((g.integers(0, 8, size=(T, E)) / 8.0) if ties else g.random((T, E))).astype(np.float32)
    sc = draw()
    # keys, like scores, are >= 0 (the selection's contract)
    keys = ((sc + draw()) * np.float32(0.5)).astype(np.float32) if g.random() < 0.5 else None
    renorm, scale = bool(g.integers(0, 2)), float(g.choice([1.0, 2.5]))
    print(f"T={T} E={E} G={G} Gk={Gk} n_g={n_g} k={k} ties={ties} keys={keys is not None}")
    cfg = moe.make_config(T, 64, E, k, G=G, Gk=Gk, n_g=n_g, I=64, renormalize=renorm,
                          route_scale=scale)
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    moe.select(cfg, to_dev(sc), None if keys is None else to_dev(keys), idx, w)
    torch.cuda.synchronize()
    ref = O.select_experts(sc if keys is None else keys, k, G, Gk, n_g)
    assert np.array_equal(idx.cpu().numpy(), ref)
    with np.errstate(invalid="ignore", divide="ignore"):
        ref_w = O.routing_weights(sc.astype(np.float64), ref, renorm, scale)
    ok = np.all(np.isfinite(ref_w), axis=1)        # a renormalised all-zero selection has no weights
    assert np.allclose(w.cpu().numpy()[ok], ref_w[ok], rtol=2e-6, atol=1e-7)


# ----------------------------------------------------------------------------- route
ROUTE_CASES = ["tiny_fp32", "fusionllm_bf16", "decode_bf16", "skewed_bf16", "fp8_relu2",
               "small_swiglu", "small_f32", "single_token", "topk1_nogroups", "balance_bf16",
               "biased_softmax_f32", "biased_groups_n2", "tail_bf16", "tail_e4m3"]


@pytest.mark.parametrize("name", ROUTE_CASES)
def test_route_matches_oracle(name):
    """The routing protocol on moe_route's own output:
    (1) its fp32 scores against the oracle's fp64 scores;
    (2) the oracle's selection applied to those fp32 scores equals the GPU's indices for
        every token, bit for bit (cases without a selection bias, whose keys the kernel
        does not export), and the weights are the renormalised GPU scores within one ulp
        of their fp32 value;
    (3) against the free-running fp64 oracle: identical indices wherever the fp64 decision
        margin exceeds the fp32 score error; closer tokens must still be a valid top-k
        within that margin (informational count printed)."""
    _check_route(shape_of(name), layer_of(name), name)


def _check_route(s, lay, name):
    cfg = config(s)
    T = s.T
    scores = torch.empty((T, s.E), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, s.k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, s.k), dtype=torch.float32, device="cuda")
    moe.route(cfg, to_dev(lay.x), to_dev(lay.router), to_dev(lay.logit_bias),
              to_dev(lay.select_bias), scores, idx, w)
    torch.cuda.synchronize()
    r = O.route(lay)
    sc32 = scores.cpu().numpy()
    g_sc = sc32.astype(np.float64)
    assert np.max(np.abs(g_sc - r["scores"])) <= 1e-5
    g_idx = idx.cpu().numpy()
    g_w = w.cpu().numpy()
    if lay.select_bias is None:
        own = O.select_experts(sc32, s.k, s.G, s.Gk, s.n_g)
        bad = np.nonzero((own != g_idx).any(axis=1))[0]
        assert bad.size == 0, f"{bad.size} tokens differ from the oracle's selection on the GPU scores, first {bad[:8]}"
        # renormalisation in fp32 steps: the k selected scores summed in slot order, one
        # division, one product with route_scale
        sel = np.take_along_axis(sc32, g_idx.astype(np.int64), axis=1)
        tot = np.zeros(T, np.float32)
        for j in range(s.k):
            tot = (tot + sel[:, j]).astype(np.float32)
        ref_w = (sel / tot[:, None]).astype(np.float32) if s.renormalize else sel
        ref_w = (ref_w * np.float32(s.route_scale)).astype(np.float32).astype(np.float64)
        ulp = np.spacing(np.abs(ref_w).astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(g_w.astype(np.float64) - ref_w) <= ulp), \
            np.max(np.abs(g_w.astype(np.float64) - ref_w) / ulp)
    mar = margins(r["keys"], s)
    clear = mar > MARGIN
    assert np.array_equal(g_idx[clear], r["idx"][clear])
    # near-tie tokens: the GPU's pick must still be a valid top-k within the margin
    for t in np.nonzero(~clear)[0]:
        assert valid_within_margin(g_idx[t], r["keys"][t], s), (t, g_idx[t], r["idx"][t])
    differ = int((g_idx != r["idx"]).any(axis=1).sum())
    print(f"{name}: {differ} of {T} tokens route differently from the free-running fp64 "
          f"oracle ({int((~clear).sum())} within the fp32 margin)")
    same = (g_idx == r["idx"]).all(axis=1)
    assert np.allclose(g_w[same], r["w"][same], rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("seed", range(24))
def test_route_random(seed):
    """The routing protocol of moe_route on seeded random layers: bf16 or fp32, dim on or
    off the 32-element K-step (up to 4160), any E up to 64 with any group count dividing
    it, n_g in {1, 2}, k up to the eligible experts, sigmoid or softmax, a logit bias, a
    selection-only bias, and 1 to 3000 tokens."""
    g = np.random.default_rng(4000 + seed)
    f32 = bool(g.random() < 0.3)
    E = int(g.integers(2, 65))
    G = int(g.choice([x for x in range(1, E + 1) if E % x == 0]))
    Gk = int(g.integers(1, G + 1))
    s = W.small_shape(
        T=int(g.choice([1, 15, 16, 17, 300, 3000])),
        d=(16 if f32 else 8) * int(g.integers(2, 4160 // (16 if f32 else 8) + 1)), E=E,
        k=int(g.integers(1, min(Gk * (E // G), 8) + 1)), G=G, Gk=Gk,
        n_g=int(g.choice([1, 2])) if E // G >= 2 else 1, S=0, I=64,
        score=str(g.choice(["sigmoid", "softmax"])), renormalize=bool(g.integers(0, 2)),
        route_scale=float(g.choice([1.0, 2.5])), act_dtype="f32" if f32 else "bf16",
        weight_dtype="f32" if f32 else "bf16",
        select_bias_std=0.5 if g.random() < 0.3 else None, seed=800 + seed)
    print(s)
    _check_route(s, W.make_layer(s, cache=False), f"seed {seed}")


# ----------------------------------------------------------------------------- pre-norm routing
PRENORM_CASES = ["prenorm_bf16", "prenorm_decode_bf16", "small_prenorm_bf16",
                 "small_prenorm_noresid", "small_prenorm_f32", "biased_prenorm", "prenorm_d4096",
                 "prenorm_d4160", "tail_prenorm"]
# A normalised value that differs from the oracle's by one ulp moves a logit by about
# |W_r| * ulp (~1e-4 here); decisions closer than this are near ties of the pre-norm step.
PRENORM_MARGIN = 1e-3


def _ulp(v, dtype):
    mant = 7 if dtype == "bf16" else 23
    a = np.abs(v)
    return np.where(a > 0, np.ldexp(1.0, (np.floor(np.log2(np.where(a > 0, a, 1.0))) - mant).astype(int)), 0.0)


@pytest.mark.parametrize("name", PRENORM_CASES)
def test_rmsnorm_route_matches_oracle(name):
    """moe_rmsnorm_route: (1) the stored normalised rows are a faithful rounding of the exact
    RMSNorm (within one ulp; almost all equal to its nearest-even rounding); (2) its routing
    equals moe_route on those stored rows bit for bit; (3) moe_route on the oracle's own
    normalised rows matches the oracle's routing of them; (4) the fused routing matches the
    oracle's except at near ties of the pre-norm step."""
    s = shape_of(name)
    lay = layer_of(name)
    cfg = config(s)
    T, dt = s.T, s.act_dtype
    x, gamma, router = to_dev(lay.x), to_dev(lay.norm_gamma), to_dev(lay.router)
    lb, sb = to_dev(lay.logit_bias), to_dev(lay.select_bias)
    x_norm = act_empty((T, s.d), dt)
    scores = torch.empty((T, s.E), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, s.k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, s.k), dtype=torch.float32, device="cuda")
    moe.rmsnorm_route(cfg, x, gamma, router, lb, sb, x_norm, scores, idx, w)
    torch.cuda.synchronize()
    exact = O.rms_norm(O.decode_act(lay.x, dt), lay.norm_gamma, float(np.float32(s.norm_eps)))
    got = act_to_f64(x_norm, dt)
    # fp32 steps before the final rounding: the sum of d squares (relative error <= d u,
    # u = 2^-24), halved by the root, plus division, root, reciprocal and two products:
    # <= (d / 2 + 8) u.  For bf16 that is far below half an ulp (2^-9 relative), so the
    # stored value is one of the two neighbours of the exact one; fp32 outputs are held to
    # 16 ulp (the bound for d <= 48 is below 32 u = 16 ulp).
    assert dt == "bf16" or s.d <= 48
    n_ulp = 1 if dt == "bf16" else 16
    assert np.all(np.abs(got - exact) <= n_ulp * _ulp(exact, dt))
    rne = O.round_to_act(exact, dt)
    frac = np.mean(got == rne)
    print(f"{name}: {frac:.6f} of normalised values equal the nearest-even rounding")
    if dt == "bf16":
        assert frac >= 0.999
    # (2) the router saw exactly the stored rows
    sc2, idx2, w2 = torch.empty_like(scores), torch.empty_like(idx), torch.empty_like(w)
    moe.route(cfg, x_norm, router, lb, sb, sc2, idx2, w2)
    torch.cuda.synchronize()
    assert torch.equal(scores, sc2) and torch.equal(idx, idx2) and torch.equal(w, w2)
    # (3) moe_route on the oracle's normalised rows
    xo = rne.astype(np.float32)
    xo_dev = to_dev(W.encode_bf16(xo) if dt == "bf16" else xo)
    moe.route(cfg, xo_dev, router, lb, sb, sc2, idx2, w2)
    torch.cuda.synchronize()
    r = O.route(lay, x=rne)
    assert np.max(np.abs(sc2.cpu().numpy().astype(np.float64) - r["scores"])) <= 1e-5
    mar = margins(r["keys"], s)
    g2 = idx2.cpu().numpy()
    clear = mar > MARGIN
    assert np.array_equal(g2[clear], r["idx"][clear])
    for t in np.nonzero(~clear)[0]:
        assert valid_within_margin(g2[t], r["keys"][t], s), (t, g2[t], r["idx"][t])
    # (4) the fused routing against the oracle's
    g = idx.cpu().numpy()
    same = np.array([set(a.tolist()) == set(b.tolist()) for a, b in zip(g, r["idx"])])
    assert np.all(same | (mar <= PRENORM_MARGIN))
    assert (~same).sum() <= max(4, T // 200)


# ----------------------------------------------------------------------------- load statistics
@pytest.mark.parametrize("name", ["fusionllm_bf16", "skewed_bf16", "decode_bf16", "tiny_fp32",
                                  "biased_softmax_f32", "small_relu2_e4m3"])
def test_load_stats_match_oracle(name):
    s = shape_of(name)
    r = O.route(layer_of(name))
    sc32 = r["scores"].astype(np.float32)
    cfg = config(s)
    ws = workspace(cfg)
    f = torch.empty(s.E, dtype=torch.float32, device="cuda")
    p = torch.empty(s.E, dtype=torch.float32, device="cuda")
    loss = torch.empty(1, dtype=torch.float32, device="cuda")
    moe.load_stats(cfg, to_dev(sc32), to_dev(r["idx"]), 0.01, f, p, loss, ws)
    torch.cuda.synchronize()
    rf, rp, rl = O.load_stats(sc32.astype(np.float64), r["idx"], s.E, 0.01)
    # f: an integer count over T*k, rounded once to fp32
    assert np.array_equal(f.cpu().numpy(), rf.astype(np.float32))
    # p, loss: fp32 sums of T normalised scores
    assert np.allclose(p.cpu().numpy(), rp, rtol=1e-5, atol=1e-7)
    assert abs(loss.cpu().item() - rl) <= 1e-5 * abs(rl)


# ----------------------------------------------------------------------------- permute
def _check_permute(T, E, k, idx_np, topk_w_np, capacity_factor=0.0):
    cfg = moe.make_config(T, 64, E, k, I=64, capacity_factor=capacity_factor)
    ws = workspace(cfg)
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    pt = torch.empty(max(T * k, 1), dtype=torch.int32, device="cuda")
    sp = torch.empty(max(T * k, 1), dtype=torch.int32, device="cuda")
    pw = torch.empty(max(T * k, 1), dtype=torch.float32, device="cuda")
    moe.permute(cfg, to_dev(idx_np), to_dev(topk_w_np), counts, offsets, pt, sp, pw, ws)
    torch.cuda.synchronize()
    cap = None
    if capacity_factor > 0:
        cap = O.expert_capacity(T, k, E, float(np.float32(capacity_factor)))
    rc, ro, rpt, rsp = O.permute(idx_np, E, cap)
    rows = int(ro[-1])
    assert np.array_equal(counts.cpu().numpy(), rc)
    assert np.array_equal(offsets.cpu().numpy(), ro)
    assert np.array_equal(pt.cpu().numpy()[:rows], rpt)
    assert np.array_equal(sp.cpu().numpy()[:T * k], rsp)
    kept = rsp >= 0
    ref_pw = np.empty(rows, np.float32)
    ref_pw[rsp[kept]] = topk_w_np.reshape(-1)[kept]
    assert np.array_equal(pw.cpu().numpy()[:rows], ref_pw)


@pytest.mark.parametrize("name", ["fusionllm_bf16", "decode_bf16", "skewed_bf16", "fp8_relu2",
                                  "tiny_fp32", "small_swiglu", "single_token"])
def test_permute_bit_exact_on_oracle_routing(name):
    s = shape_of(name)
    r = O.route(layer_of(name))
    _check_permute(s.T, s.E, s.k, r["idx"], r["w"].astype(np.float32))


def test_permute_large_batch_with_capacity():
    """2.4 M slots (300000 tokens, k = 8 of 64 experts) with a capacity: each of the at most
    64 chunks of the two-launch path spans thousands of tokens; maps bit-exact."""
    T, E, k = 300000, 64, 8
    rng = np.random.default_rng(300)
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    _check_permute(T, E, k, idx, w, capacity_factor=0.9)


@pytest.mark.parametrize("name,cf", [("fusionllm_bf16", 1.25), ("fusionllm_bf16", 0.5),
                                     ("decode_bf16", 1.0), ("skewed_bf16", 1.25),
                                     ("small_swiglu", 0.3), ("single_token", 0.01),
                                     ("tiny_fp32", 1.1)])
def test_permute_with_capacity_bit_exact(name, cf):
    s = shape_of(name)
    r = O.route(layer_of(name))
    _check_permute(s.T, s.E, s.k, r["idx"], r["w"].astype(np.float32), capacity_factor=cf)


@pytest.mark.parametrize("T,E,k,pattern", [(1, 64, 6, "random"), (63, 64, 6, "random"),
                                           (257, 8, 8, "random"), (1000, 64, 1, "one_expert"),
                                           (700, 64, 6, "first_six"), (5000, 16, 3, "random"),
                                           (10000, 64, 6, "random"), (8192, 64, 6, "first_six"),
                                           (300000, 64, 8, "random")])
def test_permute_edge_cases(T, E, k, pattern):
    rng = np.random.default_rng(T + E + k)
    if pattern == "random":
        idx = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    elif pattern == "one_expert":
        idx = np.full((T, k), 5, np.int32)
    else:
        idx = np.tile(np.arange(k, dtype=np.int32)[::-1], (T, 1))
    w = rng.random((T, k)).astype(np.float32)
    _check_permute(T, E, k, idx, w)


@pytest.mark.parametrize("seed", range(24))
def test_permute_random_bit_exact(seed):
    """Seeded random routings (1 to 20000 tokens, 1 to 64 experts, k up to E, uniform or
    Zipf-skewed expert popularity, with and without a capacity) on both the one-launch and
    the two-launch path: every map bit-exact against the oracle's permutation."""
    g = np.random.default_rng(5000 + seed)
    T = int(g.choice([1, 2, 31, 64, 500, 1024, 1025, 3000, 20000]))
    E = int(g.choice([1, 3, 8, 16, 33, 64]))
    k = int(g.integers(1, min(E, 8) + 1))
    logp = -float(g.choice([0.0, 1.2])) * np.log1p(np.arange(E))     # Zipf exponent 0 or 1.2
    keys = logp[None, :] - np.log(-np.log(g.random((T, E))))          # Gumbel top-k
    idx = np.argsort(-keys, axis=1)[:, :k].astype(np.int32)
    w = g.random((T, k)).astype(np.float32)
    cf = float(g.choice([0.0, 0.0, 0.25, 1.0, 1.5]))
    print(f"T={T} E={E} k={k} capacity_factor={cf}")
    _check_permute(T, E, k, idx, w, capacity_factor=cf)


@pytest.mark.parametrize("T", [300, 3000])
def test_permute_skips_out_of_range_ids_and_combine_ignores_them(T):
    """Padding ids (-1 and E) in topk_idx get no row and slot_pos -1, on the one-launch
    (T <= 1024) and the two-launch path; the expected maps come from Python's sorted() of
    the valid (expert, token, slot) triples.  moe_combine then sums only the valid slots."""
    E, k, d = 16, 4, 64
    rng = np.random.default_rng(T + 7)
    idx = np.array([rng.choice(E, size=k, replace=False) for _ in range(T)], dtype=np.int32)
    pad = rng.random((T, k)) < 0.2
    idx[pad] = np.where(rng.random(int(pad.sum())) < 0.5, -1, E).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    cfg = moe.make_config(T, d, E, k, I=64)
    ws = workspace(cfg)
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    pt = torch.full((T * k,), -7, dtype=torch.int32, device="cuda")
    sp = torch.full((T * k,), 12345, dtype=torch.int32, device="cuda")
    pw = torch.empty(T * k, dtype=torch.float32, device="cuda")
    moe.permute(cfg, to_dev(idx), to_dev(w), counts, offsets, pt, sp, pw, ws)
    torch.cuda.synchronize()
    triples = sorted((int(idx[t, j]), t, j) for t in range(T) for j in range(k) if 0 <= idx[t, j] < E)
    exp_sp = np.full(T * k, -1, np.int32)
    for p, (_, t, j) in enumerate(triples):
        exp_sp[t * k + j] = p
    exp_counts = np.array([sum(1 for q in triples if q[0] == e) for e in range(E)], np.int32)
    rows = len(triples)
    assert np.array_equal(counts.cpu().numpy(), exp_counts)
    assert np.array_equal(offsets.cpu().numpy(), np.concatenate([[0], np.cumsum(exp_counts)]))
    assert np.array_equal(pt.cpu().numpy()[:rows], np.array([t for (_, t, _) in triples], np.int32))
    assert np.array_equal(sp.cpu().numpy(), exp_sp)
    assert np.array_equal(pw.cpu().numpy()[:rows], np.array([w[t, j] for (_, t, j) in triples], np.float32))
    y = W.random_act((T * k, d), seed=81, dtype="bf16")
    out = act_empty((T, d), "bf16")
    moe.combine(cfg, to_dev(y), sp, None, out)
    torch.cuda.synchronize()
    ref = O.combine(O.decode_act(y, "bf16"), exp_sp, None, k)
    got = act_to_f64(out, "bf16")
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6 * np.max(np.abs(ref)))


def _ws_maps(ws, T, k, E):
    """topk_idx, topk_w, counts, offsets, perm_token, slot_pos, perm_weight from the head of
    a forward workspace (each array 256-byte aligned, in that order; moe_forward's layout)."""
    out, off = [], 0
    for n, dt in ((T * k, torch.int32), (T * k, torch.float32), (E, torch.int32),
                  (E + 1, torch.int32), (T * k, torch.int32), (T * k, torch.int32),
                  (T * k, torch.float32)):
        out.append(ws[off: off + 4 * n].view(dt).cpu().numpy().copy())
        off += (4 * n + 255) // 256 * 256
    return out


@pytest.mark.parametrize("name,T", [("decode_bf16", 1), ("decode_bf16", 17), ("decode_bf16", 64),
                                    ("fusionllm_bf16", 128), ("biased_groups_n2", 100),
                                    ("tail_bf16", 77), ("small_relu2_e4m3", 128),
                                    # last split-logit batch, first one-launch batch; the last
                                    # and first batches of the 4-wave permutation
                                    ("fusionllm_bf16", 256), ("fusionllm_bf16", 257),
                                    ("fusionllm_bf16", 341), ("fusionllm_bf16", 342)])
def test_small_batch_forward_routes_and_permutes_like_the_separate_calls(name, T):
    """The routing (indices, weights) and permutation maps that moe_forward leaves in its
    workspace for a small batch equal those of moe_route followed by moe_permute on the same
    input, bit for bit (selection bias, capacity and a dim off the 32-grid included).  Up to
    256 tokens the forward computes the router logits as partial sums spread over many
    workgroups, moe_route in one launch per 16 tokens: both sum the same partials in the
    same order."""
    s = shape_of(name)
    lay = layer_of(name)
    assert T <= lay.x.shape[0], "the case must take its rows from the layer's input"
    wts = weights(lay)
    x = to_dev(lay.x)[:T].contiguous()
    cfg = config(s, T=T)
    ws = workspace(cfg)
    out = act_empty((T, s.d), s.act_dtype)
    moe.forward(cfg, wts, x, out, ws)
    torch.cuda.synchronize()
    fused = _ws_maps(ws, T, s.k, s.E)
    k, E = s.k, s.E
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    tw = torch.empty((T, k), dtype=torch.float32, device="cuda")
    moe.route(cfg, x, wts.tensors["router"], wts.tensors["logit_bias"], wts.tensors["select_bias"],
              None, idx, tw)
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    pt = torch.empty(T * k, dtype=torch.int32, device="cuda")
    sp = torch.empty(T * k, dtype=torch.int32, device="cuda")
    pw = torch.empty(T * k, dtype=torch.float32, device="cuda")
    moe.permute(cfg, idx, tw, counts, offsets, pt, sp, pw, workspace(cfg))
    torch.cuda.synchronize()
    rows = int(offsets[-1].item())
    sep = [idx.cpu().numpy().reshape(-1), tw.cpu().numpy().reshape(-1), counts.cpu().numpy(),
           offsets.cpu().numpy(), pt.cpu().numpy(), sp.cpu().numpy(), pw.cpu().numpy()]
    names = ["topk_idx", "topk_w", "counts", "offsets", "perm_token", "slot_pos", "perm_weight"]
    for nm, a, b in zip(names, fused, sep):
        if nm in ("perm_token", "perm_weight"):
            a, b = a[:rows], b[:rows]
        assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                              b.view(np.uint32) if b.dtype == np.float32 else b), nm


# ----------------------------------------------------------------------------- grouped GEMMs
def _dense(lay, which, e, shared=False):
    s = lay.shape
    w1, w3, w2 = (O.shared_weights(lay, e) if shared else O.expert_weights(lay, e))
    return {"up": (w1, w3), "down": w2}[which]


GEMM_CASES = ["small_swiglu", "small_relu2_e4m3", "small_swiglu_e4m3", "small_f32", "tiny_fp32",
              "single_token", "fusionllm_bf16", "fp8_relu2", "tail_bf16", "tail_e4m3",
              "tail_relu2_e4m3", "tail_d_only", "tail_i_only", "small_relu2_bf16",
              "decode_relu2_bf16", "decode_swiglu_e4m3", "tail_relu2_bf16"]


@pytest.mark.parametrize("name", GEMM_CASES)
def test_grouped_gemm_up_routed(name):
    s = shape_of(name)
    lay = layer_of(name)
    r = O.route(lay)
    counts, offsets, perm_token, _ = O.permute(r["idx"], s.E)
    Tk = s.T * s.k
    cfg = config(s)
    wts = weights(lay)
    h = act_empty((Tk, s.I), s.act_dtype)
    moe.grouped_gemm(cfg, moe.MOE_STAGE_UP, moe.MOE_EXPERTS_ROUTED, to_dev(lay.x),
                     to_dev(perm_token), to_dev(offsets), Tk, wts, None, h)
    torch.cuda.synchronize()
    got = act_to_f64(h, s.act_dtype)
    x64 = r["x"]
    rows = sample_tokens(Tk, n=512, seed=1)
    ref = np.zeros((len(rows), s.I))
    for e in range(s.E):
        sel = np.nonzero((rows >= offsets[e]) & (rows < offsets[e + 1]))[0]
        if sel.size:
            w1, w3 = _dense(lay, "up", e)
            ref[sel] = O.expert_up(x64[perm_token[rows[sel]]], w1, w3, s.act)
    err = np.max(np.abs(got[rows] - ref))
    assert err <= TOL[s.act_dtype] * np.max(np.abs(ref)), err


@pytest.mark.parametrize("name", GEMM_CASES)
def test_grouped_gemm_down_routed(name):
    s = shape_of(name)
    lay = layer_of(name)
    r = O.route(lay)
    counts, offsets, perm_token, slot_pos = O.permute(r["idx"], s.E)
    Tk = s.T * s.k
    pw = np.empty(Tk, np.float32)
    pw[slot_pos] = r["w"].astype(np.float32).reshape(-1)
    h_in = W.random_act((Tk, s.I), seed=77, dtype=s.act_dtype, std=0.5)
    cfg = config(s)
    wts = weights(lay)
    y = act_empty((Tk, s.d), s.act_dtype)
    moe.grouped_gemm(cfg, moe.MOE_STAGE_DOWN, moe.MOE_EXPERTS_ROUTED, to_dev(h_in), None,
                     to_dev(offsets), Tk, wts, to_dev(pw), y)
    torch.cuda.synchronize()
    got = act_to_f64(y, s.act_dtype)
    h64 = O.decode_act(h_in, s.act_dtype)
    rows = sample_tokens(Tk, n=512, seed=2)
    ref = np.zeros((len(rows), s.d))
    for e in range(s.E):
        sel = np.nonzero((rows >= offsets[e]) & (rows < offsets[e + 1]))[0]
        if sel.size:
            ref[sel] = pw[rows[sel]].astype(np.float64)[:, None] * O.expert_down(h64[rows[sel]], _dense(lay, "down", e))
    err = np.max(np.abs(got[rows] - ref))
    assert err <= TOL[s.act_dtype] * np.max(np.abs(ref)), err


@pytest.mark.parametrize("name", ["multi_tile_swiglu", "multi_tile_relu2_e4m3", "short_k",
                                  "multi_tile_wide", "multi_tile_wide_e4m3",
                                  "multi_tile_wide_swiglu_e4m3", "multi_tile_wide_relu2_bf16"])
def test_grouped_gemm_routed_every_row(name):
    """Up and down routed GEMMs with several tiles per workgroup, every output row checked."""
    s = shape_of(name)
    lay = layer_of(name)
    r = O.route(lay)
    counts, offsets, perm_token, slot_pos = O.permute(r["idx"], s.E)
    Tk = s.T * s.k
    pw = np.empty(Tk, np.float32)
    pw[slot_pos] = r["w"].astype(np.float32).reshape(-1)
    cfg = config(s)
    wts = weights(lay)
    h = act_empty((Tk, s.I), s.act_dtype)
    moe.grouped_gemm(cfg, moe.MOE_STAGE_UP, moe.MOE_EXPERTS_ROUTED, to_dev(lay.x),
                     to_dev(perm_token), to_dev(offsets), Tk, wts, None, h)
    h_in = W.random_act((Tk, s.I), seed=79, dtype=s.act_dtype, std=0.5)
    y = act_empty((Tk, s.d), s.act_dtype)
    moe.grouped_gemm(cfg, moe.MOE_STAGE_DOWN, moe.MOE_EXPERTS_ROUTED, to_dev(h_in), None,
                     to_dev(offsets), Tk, wts, to_dev(pw), y)
    torch.cuda.synchronize()
    got_h = act_to_f64(h, s.act_dtype)
    got_y = act_to_f64(y, s.act_dtype)
    x64 = r["x"]
    h64 = O.decode_act(h_in, s.act_dtype)
    ref_h = np.zeros((Tk, s.I))
    ref_y = np.zeros((Tk, s.d))
    for e in range(s.E):
        a, b = offsets[e], offsets[e + 1]
        if b > a:
            ref_h[a:b] = O.expert_up(x64[perm_token[a:b]], *_dense(lay, "up", e), s.act)
            ref_y[a:b] = pw[a:b].astype(np.float64)[:, None] * O.expert_down(h64[a:b], _dense(lay, "down", e))
    eh = np.abs(got_h - ref_h).max(axis=1)
    ey = np.abs(got_y - ref_y).max(axis=1)
    bad_h = np.nonzero(eh > TOL[s.act_dtype] * np.max(np.abs(ref_h)))[0]
    bad_y = np.nonzero(ey > TOL[s.act_dtype] * np.max(np.abs(ref_y)))[0]
    assert bad_h.size == 0, f"up: {bad_h.size} rows off, first {bad_h[:8]}"
    assert bad_y.size == 0, f"down: {bad_y.size} rows off, first {bad_y[:8]}"


# Segment sizes whose last tile ends at, and one row either side of, every 32-row block
# boundary of a wave's rows (the tiled kernel runs one K-loop copy per count of live row
# blocks), from one row to past a full tile, plus an empty segment.
BLOCK_EDGE_ROWS = [0, 1, 31, 32, 33, 63, 64, 65, 95, 96, 97, 127, 128, 129, 159, 160, 161, 191,
                   192, 193, 223, 224, 225, 255, 256, 257, 289, 320, 353, 384, 417, 448, 481, 512]


@pytest.mark.parametrize("case", ["wide", "narrow"])
def test_grouped_gemm_row_block_edges(case):
    """Routed UP and DOWN GEMMs on segments sized to every 32-row block edge of a tile's last
    m-tile, with gathered rows and routing weights; every output row against the oracle's
    expert FFN.  "wide": d = 2048, I = 1024 and 512 more rows per segment, so both stages
    take 256 x 256 tiles (four 32-row blocks per wave); "narrow": d = I = 256 and the
    sizes as listed, 128 x 256 tiles (two blocks per wave)."""
    wide = case == "wide"
    sizes = [r + (512 if wide else 0) for r in BLOCK_EDGE_ROWS]
    E = len(sizes)
    d, I = (2048, 1024) if wide else (256, 256)
    s = W.small_shape(T=4096, d=d, E=E, k=1, G=1, Gk=1, S=0, I=I, seed=67 if wide else 68)
    lay = W.make_layer(s, cache=False)
    wts = weights(lay)
    cfg = config(s)
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    rows = int(offsets[-1])
    rng = np.random.default_rng(69)
    row_index = rng.integers(0, s.T, size=rows).astype(np.int32)
    rw = rng.uniform(0.05, 1.0, size=rows).astype(np.float32)
    h = act_empty((rows, I), s.act_dtype)
    print(f"case {case}: {E} segments, {rows} rows", flush=True)
    moe.grouped_gemm(cfg, moe.MOE_STAGE_UP, moe.MOE_EXPERTS_ROUTED, to_dev(lay.x),
                     to_dev(row_index), to_dev(offsets), rows, wts, None, h)
    h_in = W.random_act((rows, I), seed=70, dtype=s.act_dtype, std=0.5)
    y = act_empty((rows, d), s.act_dtype)
    moe.grouped_gemm(cfg, moe.MOE_STAGE_DOWN, moe.MOE_EXPERTS_ROUTED, to_dev(h_in), None,
                     to_dev(offsets), rows, wts, to_dev(rw), y)
    torch.cuda.synchronize()
    got_h = act_to_f64(h, s.act_dtype)
    got_y = act_to_f64(y, s.act_dtype)
    x64 = O.decode_act(lay.x, s.act_dtype)
    h64 = O.decode_act(h_in, s.act_dtype)
    ref_h = np.zeros((rows, I))
    ref_y = np.zeros((rows, d))
    for e in range(E):
        a, b = offsets[e], offsets[e + 1]
        if b > a:
            ref_h[a:b] = O.expert_up(x64[row_index[a:b]], *_dense(lay, "up", e), s.act)
            ref_y[a:b] = rw[a:b].astype(np.float64)[:, None] * O.expert_down(h64[a:b], _dense(lay, "down", e))
    eh = np.abs(got_h - ref_h).max(axis=1)
    ey = np.abs(got_y - ref_y).max(axis=1)
    bad_h = np.nonzero(eh > TOL[s.act_dtype] * np.max(np.abs(ref_h)))[0]
    bad_y = np.nonzero(ey > TOL[s.act_dtype] * np.max(np.abs(ref_y)))[0]
    assert bad_h.size == 0, f"up: {bad_h.size} rows off, first {bad_h[:8]}"
    assert bad_y.size == 0, f"down: {bad_y.size} rows off, first {bad_y[:8]}"


@pytest.mark.parametrize("seed", range(24))
def test_grouped_gemm_random_segments(seed):
    """Routed UP (gathered rows) and DOWN (routing weights) on seeded random segment lists:
    1 to 64 segments whose sizes mix empty, decode-sized and multi-tile ones; bf16, e4m3 or
    fp32 weights; SwiGLU or ReLU^2; dim and inter dim on or off the 64-grid.  Every output
    row against the oracle's expert FFN."""
    g = np.random.default_rng(3000 + seed)
    kind = ("bf16", "e4m3", "f32")[seed % 3]
    q = 64 if g.random() < 0.5 else (8 if kind == "bf16" else 16)
    d = q * int(g.integers(-(-64 // q), 384 // q + 1))
    I = q * int(g.integers(-(-64 // q), 384 // q + 1))
    E = int(g.integers(1, 65))
    sizes = np.where(g.random(E) < 0.2, 0,
                     np.where(g.random(E) < 0.4, g.integers(1, 40, E), g.integers(1, 1500, E)))
    sizes = (sizes * min(1.0, 12000 / max(1, sizes.sum()))).astype(np.int64)
    s = W.small_shape(T=2000, d=d, E=E, k=1, G=1, Gk=1, S=0, I=I,
                      act=str(g.choice(["swiglu", "relu2"])),
                      act_dtype="f32" if kind == "f32" else "bf16", weight_dtype=kind,
                      seed=700 + seed)
    lay = W.make_layer(s, cache=False)
    wts = weights(lay)
    cfg = config(s)
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    rows = int(offsets[-1])
    print(f"{kind} {s.act} d={d} I={I} E={E} rows={rows} "
          f"paths up/down {moe.gemm_kernel_path(cfg, 0, 0, rows)}/{moe.gemm_kernel_path(cfg, 1, 0, rows)}")
    row_index = g.integers(0, s.T, size=max(rows, 1)).astype(np.int32)
    rw = g.uniform(0.05, 1.0, size=max(rows, 1)).astype(np.float32)
    h = act_empty((max(rows, 1), I), s.act_dtype)
    y = act_empty((max(rows, 1), d), s.act_dtype)
    h_in = W.random_act((max(rows, 1), I), seed=710 + seed, dtype=s.act_dtype, std=0.5)
    moe.grouped_gemm(cfg, moe.MOE_STAGE_UP, moe.MOE_EXPERTS_ROUTED, to_dev(lay.x),
                     to_dev(row_index), to_dev(offsets), rows, wts, None, h)
    moe.grouped_gemm(cfg, moe.MOE_STAGE_DOWN, moe.MOE_EXPERTS_ROUTED, to_dev(h_in), None,
                     to_dev(offsets), rows, wts, to_dev(rw), y)
    torch.cuda.synchronize()
    if rows == 0:
        return
    got_h = act_to_f64(h, s.act_dtype)[:rows]
    got_y = act_to_f64(y, s.act_dtype)[:rows]
    x64 = O.decode_act(lay.x, s.act_dtype)
    h64 = O.decode_act(h_in, s.act_dtype)[:rows]
    ref_h = np.zeros((rows, I))
    ref_y = np.zeros((rows, d))
    for e in range(E):
        a, b = offsets[e], offsets[e + 1]
        if b > a:
            ref_h[a:b] = O.expert_up(x64[row_index[a:b]], *_dense(lay, "up", e), s.act)
            ref_y[a:b] = rw[a:b].astype(np.float64)[:, None] * O.expert_down(h64[a:b], _dense(lay, "down", e))
    eh = np.abs(got_h - ref_h).max(axis=1)
    ey = np.abs(got_y - ref_y).max(axis=1)
    bad_h = np.nonzero(eh > TOL[s.act_dtype] * np.max(np.abs(ref_h)))[0]
    bad_y = np.nonzero(ey > TOL[s.act_dtype] * np.max(np.abs(ref_y)))[0]
    assert bad_h.size == 0, f"up: {bad_h.size} rows off, first {bad_h[:8]}"
    assert bad_y.size == 0, f"down: {bad_y.size} rows off, first {bad_y[:8]}"


@pytest.mark.parametrize("name", ["small_swiglu", "small_relu2_e4m3", "small_f32", "fusionllm_bf16",
                                  "fp8_relu2", "multi_tile_swiglu", "short_k"])
def test_grouped_gemm_shared(name):
    s = shape_of(name)
    lay = layer_of(name)
    cfg = config(s)
    wts = weights(lay)
    T = s.T
    SI = s.S * s.I
    h = act_empty((T, SI), s.act_dtype)
    moe.grouped_gemm(cfg, moe.MOE_STAGE_UP, moe.MOE_EXPERTS_SHARED, to_dev(lay.x), None, None, T,
                     wts, None, h)
    h_in = W.random_act((T, SI), seed=78, dtype=s.act_dtype, std=0.5)
    y = act_empty((T, s.d), s.act_dtype)
    moe.grouped_gemm(cfg, moe.MOE_STAGE_DOWN, moe.MOE_EXPERTS_SHARED, to_dev(h_in), None, None, T,
                     wts, None, y)
    torch.cuda.synchronize()
    rows = sample_tokens(T, n=256, seed=3)
    x64 = O.decode_act(lay.x[rows], s.act_dtype)
    h64 = O.decode_act(h_in[rows], s.act_dtype)
    ref_h = np.concatenate([O.expert_up(x64, *_dense(lay, "up", i, True), s.act) for i in range(s.S)], axis=1)
    ref_y = sum(O.expert_down(h64[:, i * s.I:(i + 1) * s.I], _dense(lay, "down", i, True)) for i in range(s.S))
    got_h = act_to_f64(h, s.act_dtype)[rows]
    got_y = act_to_f64(y, s.act_dtype)[rows]
    assert np.max(np.abs(got_h - ref_h)) <= TOL[s.act_dtype] * np.max(np.abs(ref_h))
    assert np.max(np.abs(got_y - ref_y)) <= TOL[s.act_dtype] * np.max(np.abs(ref_y))


# ----------------------------------------------------------------------------- e4m3 activations
@pytest.mark.parametrize("name", ["fusionllm_bf16", "small_a8_swiglu", "random_wide"])
def test_quantize_rows_bit_exact(name):
    if name == "random_wide":
        rng = np.random.default_rng(45)
        a32 = (rng.standard_normal((513, 1024)) * rng.random((513, 1)) * 30).astype(np.float32)
        a32[0] = 0.0
        a32[1] *= np.float32(1e-30)
        a32[2, 5] = np.float32(-3e4)
        x = W.encode_bf16(a32)
    else:
        x = layer_of(name).x
    rows, cols = x.shape
    cfg = moe.make_config(rows, cols, 8, 2, I=64, weight_dtype="e4m3", fp8_act=True)
    q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    sc = torch.empty(rows, dtype=torch.float32, device="cuda")
    moe.quantize_rows(cfg, to_dev(x), rows, cols, q, sc)
    torch.cuda.synchronize()
    rq, rs = O.quantize_rows_e4m3(O.decode_bf16(x))
    assert np.array_equal(sc.cpu().numpy(), rs)
    assert np.array_equal(q.cpu().numpy(), rq)


@pytest.mark.parametrize("name", ["small_a8_swiglu", "multi_tile_a8_relu2", "fp8a_relu2",
                                  "wide_a8_swiglu"])
def test_grouped_gemm_up_e4m3_activations(name):
    """Routed and shared up projections on e4m3 activations: the oracle's codes and scales
    in, every row (or a sample at full size) against the dequantised fp64 product."""
    s = shape_of(name)
    lay = layer_of(name)
    r = O.route(lay)
    counts, offsets, perm_token, _ = O.permute(r["idx"], s.E)
    Tk = s.T * s.k
    xq, xs = O.quantize_rows_e4m3(r["x"])
    xdq = O.dequantize_rows_e4m3(xq, xs)
    cfg = config(s)
    wts = weights(lay)
    h = act_empty((Tk, s.I), s.act_dtype)
    moe.grouped_gemm(cfg, moe.MOE_STAGE_UP, moe.MOE_EXPERTS_ROUTED, to_dev(xq), to_dev(perm_token),
                     to_dev(offsets), Tk, wts, to_dev(xs), h)
    hs = act_empty((s.T, s.S * s.I), s.act_dtype)
    moe.grouped_gemm(cfg, moe.MOE_STAGE_UP, moe.MOE_EXPERTS_SHARED, to_dev(xq), None, None, s.T,
                     wts, to_dev(xs), hs)
    torch.cuda.synchronize()
    rows = np.arange(Tk) if Tk <= 40000 else sample_tokens(Tk, n=1024, seed=5)
    got = act_to_f64(h, s.act_dtype)[rows]
    ref = np.zeros((len(rows), s.I))
    for e in range(s.E):
        sel = np.nonzero((rows >= offsets[e]) & (rows < offsets[e + 1]))[0]
        if sel.size:
            w1, w3 = _dense(lay, "up", e)
            ref[sel] = O.expert_up(xdq[perm_token[rows[sel]]], w1, w3, s.act)
    assert np.max(np.abs(got - ref)) <= TOL[s.act_dtype] * np.max(np.abs(ref))
    trows = sample_tokens(s.T, n=512, seed=6)
    ref_s = np.concatenate([O.expert_up(xdq[trows], *_dense(lay, "up", i, True), s.act)
                            for i in range(s.S)], axis=1)
    got_s = act_to_f64(hs, s.act_dtype)[trows]
    assert np.max(np.abs(got_s - ref_s)) <= TOL[s.act_dtype] * np.max(np.abs(ref_s))


# ----------------------------------------------------------------------------- combine
@pytest.mark.parametrize("name,with_shared,cf", [("small_swiglu", True, None), ("small_f32", True, None),
                                                 ("fusionllm_bf16", True, None),
                                                 ("topk1_nogroups", False, None),
                                                 ("fusionllm_bf16", True, 0.8),
                                                 ("small_f32", False, 0.5)])
def test_combine(name, with_shared, cf):
    s = shape_of(name)
    r = O.route(layer_of(name))
    cap = None if cf is None else O.expert_capacity(s.T, s.k, s.E, cf)
    _, _, _, slot_pos = O.permute(r["idx"], s.E, cap)
    if cap is not None:
        assert (slot_pos < 0).any()
    y = W.random_act((s.T * s.k, s.d), seed=79, dtype=s.act_dtype)
    ysh = W.random_act((s.T, s.d), seed=80, dtype=s.act_dtype) if with_shared else None
    out = act_empty((s.T, s.d), s.act_dtype)
    moe.combine(config(s), to_dev(y), to_dev(slot_pos), to_dev(ysh), out)
    torch.cuda.synchronize()
    ref = O.combine(O.decode_act(y, s.act_dtype), slot_pos,
                    None if ysh is None else O.decode_act(ysh, s.act_dtype), s.k)
    got = act_to_f64(out, s.act_dtype)
    # fp32 sum of k+1 terms, then one rounding to the output dtype
    rel = 2.0 ** -8 if s.act_dtype == "bf16" else 1e-6
    assert np.all(np.abs(got - ref) <= rel * np.abs(ref) + 1e-6 * np.max(np.abs(ref)))


@pytest.mark.parametrize("seed", range(16))
def test_combine_random(seed):
    """Seeded random slot maps (any T, k and dim on the 8 / 16 grid, slots dropped at random,
    with and without a shared row, bf16 or fp32): the fixed-order sum against the oracle's
    combine, one output rounding."""
    g = np.random.default_rng(2000 + seed)
    dt = "f32" if seed % 3 == 2 else "bf16"
    T = int(g.choice([1, 3, 64, 777, 5000]))
    k = int(g.integers(1, 13))
    d = (16 if dt == "f32" else 8) * int(g.integers(1, 520 // (16 if dt == "f32" else 8) + 1))
    slot_pos = g.permutation(T * k).astype(np.int32)
    slot_pos[g.random(T * k) < float(g.choice([0.0, 0.2, 0.9]))] = -1
    y = W.random_act((T * k, d), seed=2100 + seed, dtype=dt)
    ysh = W.random_act((T, d), seed=2200 + seed, dtype=dt) if g.random() < 0.5 else None
    print(f"{dt} T={T} k={k} d={d} dropped={int((slot_pos < 0).sum())} shared={ysh is not None}")
    cfg = moe.make_config(T, d, max(k, 2), k, I=64, act_dtype=dt, weight_dtype=dt)
    out = act_empty((T, d), dt)
    moe.combine(cfg, to_dev(y), to_dev(slot_pos), to_dev(ysh), out)
    torch.cuda.synchronize()
    ref = O.combine(O.decode_act(y, dt), slot_pos, None if ysh is None else O.decode_act(ysh, dt), k)
    got = act_to_f64(out, dt)
    rel = 2.0 ** -8 if dt == "bf16" else 1e-6
    assert np.all(np.abs(got - ref) <= rel * np.abs(ref) + 1e-6 * max(np.max(np.abs(ref)), 1e-30))


@pytest.mark.parametrize("seed", range(16))
def test_quantize_rows_random(seed):
    """Seeded random bf16 rows for the e4m3 row quantiser: per-row magnitudes from 1e-30 to
    3e4, zero rows, single-spike rows and sign mixes, 1 to 3000 rows of 8 to 8192 columns:
    codes and scales bit-exact against the oracle's quantiser."""
    g = np.random.default_rng(1000 + seed)
    rows = int(g.choice([1, 2, 63, 300, 3000]))
    cols = 8 * int(g.integers(1, 1025))
    mag = np.exp(g.uniform(np.log(1e-30), np.log(3e4), size=(rows, 1)))
    a32 = (g.standard_normal((rows, cols)) * mag).astype(np.float32)
    a32[g.random(rows) < 0.1] = 0.0
    spikes = np.nonzero(g.random(rows) < 0.1)[0]
    a32[spikes, g.integers(0, cols, size=spikes.size)] = np.float32(-2e4)
    x = W.encode_bf16(a32)
    print(f"rows={rows} cols={cols}")
    cfg = moe.make_config(rows, 128, 8, 2, I=64, weight_dtype="e4m3", fp8_act=True)
    q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    sc = torch.empty(rows, dtype=torch.float32, device="cuda")
    moe.quantize_rows(cfg, to_dev(x), rows, cols, q, sc)
    torch.cuda.synchronize()
    rq, rs = O.quantize_rows_e4m3(O.decode_bf16(x))
    assert np.array_equal(sc.cpu().numpy(), rs)
    assert np.array_equal(q.cpu().numpy(), rq)


# ----------------------------------------------------------------------------- forward
FORWARD_CASES = ["tiny_fp32", "fusionllm_bf16", "decode_bf16", "skewed_bf16", "fp8_relu2",
                 "small_swiglu", "small_relu2_e4m3", "small_swiglu_e4m3", "small_f32",
                 "single_token", "topk1_nogroups", "balance_bf16", "biased_softmax_f32",
                 "biased_groups_n2", "fp8a_relu2", "small_a8_swiglu", "multi_tile_a8_relu2",
                 "all_experts", "tail_bf16", "tail_e4m3", "tail_relu2_e4m3", "tail_d_only",
                 "tail_i_only", "tail_multi", "small_relu2_bf16", "decode_relu2_bf16",
                 "decode_swiglu_e4m3", "tail_relu2_bf16"]


def run_forward(name):
    s = shape_of(name)
    lay = layer_of(name)
    cfg = config(s)
    wts = weights(lay)
    ws = workspace(cfg)
    x = to_dev(lay.x)
    out = act_empty((s.T, s.d), s.act_dtype)
    moe.forward(cfg, wts, x, out, ws)
    torch.cuda.synchronize()
    gpu_idx = ws[: s.T * s.k * 4].view(torch.int32).cpu().numpy().reshape(s.T, s.k)
    return s, lay, cfg, wts, ws, x, out, gpu_idx


def check_forward_routing(s, lay, gpu_idx, x=None, margin=MARGIN):
    """The forward's routing against the free-running oracle: every token identical as a
    set of experts, except near ties (fp64 margin below ``margin``), which must still be a
    valid top-k within it.  Returns the number of tokens routed differently."""
    full = O.route(lay, x=x)
    mar = margins(full["keys"], s)
    same = np.array([set(a.tolist()) == set(b.tolist()) for a, b in zip(gpu_idx, full["idx"])])
    assert np.all(same | (mar <= margin)), "routing differs away from a near tie"
    if margin == MARGIN:
        for t in np.nonzero(~same)[0]:
            assert valid_within_margin(gpu_idx[t], full["keys"][t], s)
    return int((~same).sum())


@pytest.mark.parametrize("name", FORWARD_CASES)
def test_forward_matches_oracle(name):
    """Every output row of the forward against the oracle forward run under the GPU's
    checked routing (parity protocol step 4; with a capacity this is the only comparison
    possible, since dropped slots depend on the whole batch's routing)."""
    s, lay, cfg, wts, ws, x, out, gpu_idx = run_forward(name)
    differ = check_forward_routing(s, lay, gpu_idx)
    ref = O.moe_forward(lay, idx=gpu_idx)
    if s.capacity_factor is not None:
        assert (~ref["kept"]).any() or s.capacity_factor >= 1.0
    got = act_to_f64(out, s.act_dtype)
    err = np.abs(got - ref["out"]).max(axis=1)
    scale = np.max(np.abs(ref["out"]))
    print(f"{name}: max|d|/max|ref| = {err.max() / scale:.3e} over all {s.T} rows "
          f"({differ} near-tie tokens routed differently from the free-running oracle)")
    bad = np.nonzero(err > TOL[s.act_dtype] * scale)[0]
    assert bad.size == 0, f"{bad.size} rows off, first {bad[:8]}"


PRENORM_FORWARD_CASES = PRENORM_CASES + ["small_prenorm_a8"]


@pytest.mark.parametrize("name", PRENORM_FORWARD_CASES)
def test_forward_prenorm_matches_oracle(name):
    """The pre-norm layer step: routing identical to moe_rmsnorm_route on the same input,
    the oracle's own routing except at near ties of the pre-norm step, and every output row
    (against the oracle run under the GPU's checked routing) within TOL * max|MoE part| +
    half an ulp of the output (the final rounding of a sum that includes the residual x)."""
    s, lay, cfg, wts, ws, x, out, gpu_idx = run_forward(name)
    idx = torch.empty((s.T, s.k), dtype=torch.int32, device="cuda")
    w = torch.empty((s.T, s.k), dtype=torch.float32, device="cuda")
    x_norm = act_empty((s.T, s.d), s.act_dtype)
    moe.rmsnorm_route(cfg, x, to_dev(lay.norm_gamma), to_dev(lay.router), to_dev(lay.logit_bias),
                      to_dev(lay.select_bias), x_norm, None, idx, w)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), gpu_idx)
    check_forward_routing(s, lay, gpu_idx, x=O.normalized_input(lay), margin=PRENORM_MARGIN)
    ref = O.moe_forward(lay, idx=gpu_idx)
    got = act_to_f64(out, s.act_dtype)
    xr = O.decode_act(lay.x, s.act_dtype)
    moe_part = ref["out"] - (xr if s.residual else 0.0)
    scale = np.max(np.abs(moe_part))
    bound = TOL[s.act_dtype] * scale + 0.5 * _ulp(np.maximum(np.abs(got), np.abs(ref["out"])), s.act_dtype)
    err = np.abs(got - ref["out"])
    print(f"{name}: max|d|/max|moe part| = {np.max(err) / scale:.3e} over all {s.T} rows")
    assert np.all(err <= bound)


def random_shape(seed):
    """A seeded layer drawn from what the boundary accepts: any dtype pairing, activation,
    scoring, grouping (n_g of 1 or 2), k up to the eligible experts, shared experts, a
    capacity, a selection bias, the pre-norm step, tokens from 1 to 2500, and dim / inter
    dim on their grids (multiples of 8 for bf16 weights, 16 for e4m3 or fp32, 128 / 64 with
    e4m3 activations; half of them on the 64-element grid)."""
    g = np.random.default_rng(7000 + seed)
    kind = ("bf16", "e4m3", "f32", "a8")[seed % 4]
    E = int(g.choice([4, 8, 16, 32, 64]))
    G = int(g.choice([x for x in (1, 2, 4, 8) if E % x == 0]))
    Gk = int(g.integers(1, G + 1))
    n_g = int(g.choice([1, 2])) if E // G >= 2 else 1
    k = int(g.integers(1, min(Gk * (E // G), 8) + 1))
    if kind == "a8":
        d, I = 128 * int(g.integers(1, 4)), 64 * int(g.integers(1, 7))
    else:
        # half of the layers on the 64-element grid of the tiled kernels
        q = 64 if g.random() < 0.5 else (8 if kind == "bf16" else 16)
        d, I = q * int(g.integers(-(-48 // q), 512 // q + 1)), q * int(g.integers(-(-32 // q), 384 // q + 1))
    pre = bool(g.random() < 0.3)
    return W.small_shape(
        T=int(g.choice([1, 5, 33, 64, 100, 257, 600, 1100, 2500])), d=d, E=E, k=k, G=G, Gk=Gk,
        n_g=n_g, S=int(g.integers(0, 3)), I=I, score=str(g.choice(["sigmoid", "softmax"])),
        act=str(g.choice(["swiglu", "relu2"])),
        act_dtype="f32" if kind == "f32" else "bf16",
        weight_dtype={"bf16": "bf16", "f32": "f32"}.get(kind, "e4m3"), fp8_act=kind == "a8",
        renormalize=bool(g.integers(0, 2)), route_scale=float(g.choice([1.0, 2.5])),
        capacity_factor=float(g.choice([0.5, 1.0, 1.5])) if g.random() < 0.3 else None,
        select_bias_std=0.5 if g.random() < 0.3 else None,
        pre_norm=pre, residual=pre and bool(g.integers(0, 2)), seed=900 + seed)


@pytest.mark.parametrize("seed", range(96))
def test_forward_random_configs(seed):
    """The whole forward on seeded random layers: routing against the free-running oracle
    (identical away from near ties), every output row against the oracle run under the
    GPU's routing, to the same bars as the fixed cases."""
    s = random_shape(seed)
    print(s)
    lay = W.make_layer(s, cache=False)
    cfg = config(s)
    wts = weights(lay)
    ws = workspace(cfg)
    x = to_dev(lay.x)
    out = act_empty((s.T, s.d), s.act_dtype)
    moe.forward(cfg, wts, x, out, ws)
    torch.cuda.synchronize()
    gpu_idx = ws[: s.T * s.k * 4].view(torch.int32).cpu().numpy().reshape(s.T, s.k)
    if s.pre_norm:
        check_forward_routing(s, lay, gpu_idx, x=O.normalized_input(lay), margin=PRENORM_MARGIN)
    else:
        check_forward_routing(s, lay, gpu_idx)
    ref = O.moe_forward(lay, idx=gpu_idx)
    got = act_to_f64(out, s.act_dtype)
    moe_part = ref["out"] - (O.decode_act(lay.x, s.act_dtype) if s.residual else 0.0)
    scale = np.max(np.abs(moe_part))
    bound = TOL[s.act_dtype] * scale
    if s.residual:
        bound = bound + 0.5 * _ulp(np.maximum(np.abs(got), np.abs(ref["out"])), s.act_dtype)
    err = np.abs(got - ref["out"])
    print(f"seed {seed}: max|d|/max|moe part| = {np.max(err) / max(scale, 1e-300):.3e}")
    assert np.all(err <= bound)


@pytest.mark.parametrize("name", ["balance_bf16", "small_f32"])
def test_forward_load_stats_match_oracle(name):
    """The statistics moe_forward_ex writes for its own routing: f from the GPU routing
    exactly, p and the loss against the oracle's fp64 scores."""
    s = shape_of(name)
    lay = layer_of(name)
    cfg = config(s)
    wts = weights(lay)
    ws = workspace(cfg)
    out = act_empty((s.T, s.d), s.act_dtype)
    st = torch.empty(2 * s.E + 1, dtype=torch.float32, device="cuda")
    moe.forward(cfg, wts, to_dev(lay.x), out, ws, load_stats=st, aux_alpha=0.5)
    torch.cuda.synchronize()
    gpu_idx = ws[: s.T * s.k * 4].view(torch.int32).cpu().numpy().reshape(s.T, s.k)
    r = O.route(lay)
    rf, rp, rl = O.load_stats(r["scores"], gpu_idx, s.E, 0.5)
    got = st.cpu().numpy()
    assert np.array_equal(got[: s.E], rf.astype(np.float32))
    assert np.allclose(got[s.E: 2 * s.E], rp, rtol=1e-4, atol=1e-6)
    assert abs(got[2 * s.E] - rl) <= 1e-4 * abs(rl)
    # the forward's output does not depend on whether statistics were asked for
    out2 = torch.empty_like(out)
    moe.forward(cfg, wts, to_dev(lay.x), out2, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


@pytest.mark.parametrize("name", ["decode_bf16", "small_swiglu", "prenorm_decode_bf16",
                                  "small_a8_swiglu"])
def test_forward_graph_replay_matches_eager(name):
    """moe_forward captured into a HIP graph (the shared experts' side stream joins the
    capture through its fork and join events) and replayed several times, with eager
    launches and host synchronisation between the replays: every replay equals the eager
    forward bit for bit, also after the input changed in place."""
    s, lay, cfg, wts, ws, x, out, _ = run_forward(name)    # eager run; creates the side stream
    ref = out.clone()
    g_out = torch.empty_like(out)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.forward(cfg, wts, x, g_out, ws)
    x2 = to_dev(W.random_act((s.T, s.d), 77, s.act_dtype, 1.0))
    ref2 = torch.empty_like(out)
    for i in range(4):
        g_out.zero_()
        if i == 2:
            x_saved = x.clone()
            x.copy_(x2)
            moe.forward(cfg, wts, x, ref2, ws)       # eager result on the new input
            torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(g_out, ref2 if i >= 2 else ref), f"replay {i}"
        torch.cuda.synchronize()
    x.copy_(x_saved)
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(g_out, ref)


@pytest.mark.parametrize("name", ["fusionllm_bf16", "small_swiglu_e4m3", "tiny_fp32",
                                  "small_prenorm_bf16"])
def test_forward_is_deterministic(name):
    s, lay, cfg, wts, ws, x, out, _ = run_forward(name)
    out2 = torch.empty_like(out)
    moe.forward(cfg, wts, x, out2, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


@pytest.mark.parametrize("name", ["small_swiglu", "decode_bf16", "fusionllm_bf16"])
def test_forwards_on_two_streams_match_serial(name):
    """Two forwards on different inputs, enqueued together on two caller streams (each with
    its own second stream for the shared experts), three times in a row, equal the same
    forwards run one after the other, bit for bit."""
    s = shape_of(name)
    lay = layer_of(name)
    wts = weights(lay)
    cfg = config(s)
    x1 = to_dev(lay.x)
    x2 = torch.flip(x1, dims=[0]).contiguous()   # the same rows in reverse token order
    refs = []
    for x in (x1, x2):
        out = act_empty((s.T, s.d), s.act_dtype)
        moe.forward(cfg, wts, x, out, workspace(cfg))
        refs.append(out)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    wss = [workspace(cfg), workspace(cfg)]
    outs = [act_empty((s.T, s.d), s.act_dtype) for _ in range(2)]
    torch.cuda.synchronize()
    for rep in range(3):
        for i, x in enumerate((x1, x2)):
            with torch.cuda.stream(streams[i]):
                moe.forward(cfg, wts, x, outs[i], wss[i], stream=streams[i])
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(outs[i], refs[i]), f"{name}: stream {i}, repetition {rep}"


def test_forward_error_paths_enqueue_nothing():
    s = shape_of("small_swiglu")
    lay = layer_of("small_swiglu")
    cfg = config(s)
    wts = weights(lay)
    ws = workspace(cfg)
    out = act_empty((s.T, s.d), s.act_dtype)
    out.fill_(7)
    with pytest.raises(moe.MoeError) as ei:
        moe.forward(cfg, wts, to_dev(lay.x), out, ws, ws_bytes=ws.numel() - 1)
    assert ei.value.status == 3
    torch.cuda.synchronize()
    assert bool((out == 7).all())


@pytest.mark.parametrize("name", ["decode_bf16", "small_swiglu"])
def test_forward_ex_records_stage_events_and_matches_forward(name):
    s, lay, cfg, wts, ws, x, out, _ = run_forward(name)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(8)]
    out2 = torch.empty_like(out)
    moe.forward(cfg, wts, x, out2, ws, stage_events=ev)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    times = [ev[i].elapsed_time(ev[i + 1]) for i in range(7)]
    assert all(t >= 0 for t in times) and sum(times) > 0
