"""Pins of the CPU oracle against what the pages and mathematics fix (no GPU).

Every check here compares the oracle with something other than itself: exhaustive
closed forms, library routines (torch dtype conversions, Python's sorted), brute force
in pure Python on tiny inputs, identities of the method, and values printed on the pages
(tests/golden).  The mutation tests at the end plant plausible mistakes in the oracle and
check that a pin catches each one.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32layer(**kw):
    """A tiny fp32 layer (values exact in fp64) built by the shared seeded generator."""
    base = dict(act_dtype="f32", weight_dtype="f32", T=5, d=6, E=4, k=2, S=0, I=3,
                G=1, Gk=1, score="softmax")
    base.update(kw)
    return W.make_layer(W.small_shape(**base), cache=False)


# ----------------------------------------------------------------------------- codecs
def test_decode_bf16_exhaustive_matches_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = O.decode_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_decode_bf16_closed_form_anchors():
    # 1.0 = 0x3F80, -2.0 = 0xC000, smallest subnormal 2^-133 = 0x0001, max finite
    assert O.decode_bf16([0x3F80])[0] == 1.0
    assert O.decode_bf16([0xC000])[0] == -2.0
    assert O.decode_bf16([0x0001])[0] == math.ldexp(1.0, -133)
    assert O.decode_bf16([0x7F7F])[0] == math.ldexp(1 + 127 / 128, 127)


def test_decode_e4m3_exhaustive_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.decode_e4m3(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_decode_e4m3_anchors():
    d = O.decode_e4m3
    assert d([0x7E])[0] == 448.0          # max normal
    assert d([0x08])[0] == 2.0 ** -6      # min normal
    assert d([0x01])[0] == 2.0 ** -9      # min subnormal
    assert d([0x38])[0] == 1.0
    assert np.isnan(d([0x7F])[0]) and np.isnan(d([0xFF])[0])
    pos = d(np.arange(127, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)       # strictly increasing over the finite codes
    assert np.array_equal(d(np.arange(128, 255, dtype=np.uint8)), -pos)


def test_generator_bf16_encoder_is_rne():
    rng = np.random.default_rng(5)
    a = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                        np.array([1.00390625, 1.01171875, -3.0e-39, 65504.0], np.float32)])
    ours = W.encode_bf16(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_generator_e4m3_quantiser_matches_torch_and_bounds_error():
    rng = np.random.default_rng(6)
    w = rng.standard_normal((16, 64)).astype(np.float32)
    codes, scale = W.encode_e4m3_rows(w)
    y = torch.from_numpy(w / scale[:, None])
    ref = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)
    deq = O.decode_weight(codes, "e4m3", scale)
    # RNE on a 3-bit mantissa: relative error <= 2^-4 for normals
    big = np.abs(w) > scale[:, None] * 2.0 ** -6
    assert np.all(np.abs(deq - w)[big] <= np.abs(w)[big] * 2.0 ** -4 + 1e-12)
    assert np.allclose(np.max(np.abs(deq), axis=1), np.max(np.abs(w), axis=1), rtol=1e-6)


# ----------------------------------------------------------------------------- router
def test_router_logits_brute_force():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((3, 5))
    w = rng.standard_normal((4, 5))
    b = rng.standard_normal(4)
    got = O.router_logits(x, w, b)
    for t in range(3):
        for e in range(4):
            ref = math.fsum([x[t, c] * w[e, c] for c in range(5)] + [b[e]])
            assert abs(got[t, e] - ref) <= 1e-12 * (1 + abs(ref))
    assert np.allclose(O.router_logits(x, w), got - b[None, :], atol=1e-13)


def test_sigmoid_closed_forms():
    s = O.gate_scores(np.array([[0.0, math.log(3.0), -math.log(3.0), 40.0, -40.0]]), "sigmoid")[0]
    assert s[0] == 0.5
    assert abs(s[1] - 0.75) < 1e-15 and abs(s[2] - 0.25) < 1e-15
    assert abs(s[3] - 1.0) < 1e-15 and 0.0 < s[4] < 1e-17


def test_softmax_closed_forms():
    l = np.array([[0.0, math.log(2.0), math.log(5.0)], [1000.0, 1000.0, -1000.0]])
    s = O.gate_scores(l, "softmax")
    assert np.allclose(s[0], [1 / 8, 2 / 8, 5 / 8], rtol=0, atol=1e-15)
    assert np.allclose(s[1], [0.5, 0.5, 0.0], rtol=0, atol=1e-15)
    rng = np.random.default_rng(8)
    r = O.gate_scores(rng.standard_normal((50, 9)), "softmax")
    assert np.allclose(r.sum(axis=1), 1.0, atol=1e-14)


# ----------------------------------------------------------------------------- selection
def _bf_select(s, k, G, Gk, n_g):
    """Brute force from the definition for DISTINCT values: the kept groups are the Gk-subset
    of groups with the largest total group score, and the selection is the k-subset of
    eligible experts with the largest total score, listed by score descending."""
    E = len(s)
    gsz = E // G
    def gscore(g):
        mem = [np.float32(s[g * gsz + i]) for i in range(gsz)]
        best = None
        for c in itertools.combinations(mem, n_g):
            acc = np.float32(0)
            for v in sorted(c, reverse=True):
                acc = np.float32(acc + v)           # fp32 adds, as the decision precision
            best = acc if best is None else max(best, acc)
        return float(best)
    best_groups = max(itertools.combinations(range(G), Gk), key=lambda c: sum(gscore(g) for g in c))
    elig = [e for e in range(E) if e // gsz in best_groups]
    best = max(itertools.combinations(elig, k), key=lambda c: sum(float(s[e]) for e in c))
    return sorted(best, key=lambda e: -float(s[e]))


@pytest.mark.parametrize("E,G,Gk,n_g,k", [(6, 1, 1, 1, 2), (8, 4, 2, 1, 3), (8, 4, 2, 2, 3),
                                          (12, 3, 1, 2, 4), (12, 6, 3, 1, 5), (9, 3, 2, 2, 1)])
def test_select_brute_force_distinct(E, G, Gk, n_g, k):
    rng = np.random.default_rng(100 + E * 7 + k)
    for trial in range(40):
        s = rng.random(E).astype(np.float32)                               # distinct values
        gs = O.group_scores(s[None, :], G, n_g)[0]
        if len(set(s.tolist())) < E or len(set(gs.tolist())) < G:
            continue
        got = O.select_experts(s[None, :], k, G, Gk, n_g)[0].tolist()
        assert got == _bf_select(s, k, G, Gk, n_g), (s, got)


def test_select_without_group_limit_is_stable_argsort():
    rng = np.random.default_rng(9)
    s = (rng.integers(0, 6, size=(200, 16)) / 8.0).astype(np.float32)      # many ties
    got = O.select_experts(s, 5)
    ref = np.argsort(-s, axis=1, kind="stable")[:, :5]
    assert np.array_equal(got, ref)
    # Gk = G gives the same result as no group limit
    assert np.array_equal(O.select_experts(s, 5, G=4, Gk=4, n_g=2), ref)


def test_select_k1_is_argmax():
    rng = np.random.default_rng(10)
    s = (rng.integers(0, 4, size=(300, 8)) / 4.0).astype(np.float32)
    assert np.array_equal(O.select_experts(s, 1)[:, 0], np.argmax(s, axis=1))


def test_select_hand_written_tie_cases():
    cases = json.load(open(os.path.join(GOLDEN, "tie_cases.json")))["cases"]
    for c in cases:
        s = np.array([c["scores"]], dtype=np.float32)
        got = O.select_experts(s, c["k"], c["G"], c["Gk"], c["n_g"])[0].tolist()
        assert got == c["expect"], c


def test_group_scores_top2_brute_force_fp32():
    rng = np.random.default_rng(11)
    s = rng.random((40, 12)).astype(np.float32)
    gs = O.group_scores(s, 4, 2)
    assert gs.dtype == np.float32
    for t in range(40):
        for g in range(4):
            mem = s[t, 3 * g:3 * g + 3]
            ref = max(np.float32(a) + np.float32(b) for a, b in itertools.combinations(mem, 2))
            assert gs[t, g] == ref


def test_every_token_lands_in_exactly_k_distinct_experts():
    rng = np.random.default_rng(12)
    s = rng.random((500, 64)).astype(np.float32)
    idx = O.select_experts(s, 6, 8, 4, 1)
    assert idx.shape == (500, 6)
    assert all(len(set(r)) == 6 for r in idx.tolist())
    assert np.all((idx >= 0) & (idx < 64))
    # at most Gk distinct groups are used per token
    assert all(len(set(e // 8 for e in r)) <= 4 for r in idx.tolist())


# ----------------------------------------------------------------------------- weights
def test_weights_sum_to_one_and_positive():
    rng = np.random.default_rng(13)
    sc = O.gate_scores(rng.standard_normal((100, 16)), "sigmoid")
    idx = O.select_experts(sc.astype(np.float32), 4, 4, 2, 1)
    w = O.routing_weights(sc, idx)
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-15)
    assert np.all(w > 0)
    w2 = O.routing_weights(sc, idx, renormalize=False, route_scale=2.5)
    assert np.allclose(w2, 2.5 * np.take_along_axis(sc, idx.astype(np.int64), axis=1))


def test_renormalised_topk_softmax_is_softmax_of_selected_logits():
    """MoEBlock listing: softmax over the top-k gate values.  Equal to renormalising the
    full softmax over the selected experts."""
    rng = np.random.default_rng(14)
    l = rng.standard_normal((64, 8)) * 2
    sc = O.gate_scores(l, "softmax")
    idx = O.select_experts(sc.astype(np.float32), 2)
    w = O.routing_weights(sc, idx)
    top_l = torch.from_numpy(np.take_along_axis(l, idx.astype(np.int64), axis=1))
    ref = torch.softmax(top_l, dim=-1).numpy()
    assert np.allclose(w, ref, rtol=0, atol=1e-14)
    # and the top-k over softmax scores equals the top-k over the logits
    assert np.array_equal(idx, np.argsort(-l, axis=1, kind="stable")[:, :2])


# ----------------------------------------------------------------------------- experts
def _bf_ffn(xr, w1, w3, w2, act):
    I, d = len(w1), len(xr)
    h = []
    for i in range(I):
        a = math.fsum(w1[i][c] * xr[c] for c in range(d))
        if act == "swiglu":
            b = math.fsum(w3[i][c] * xr[c] for c in range(d))
            h.append(a / (1.0 + math.exp(-a)) * b)
        else:
            h.append(max(a, 0.0) ** 2)
    return [math.fsum(w2[n][i] * h[i] for i in range(I)) for n in range(len(w2))]


def test_silu_closed_forms_and_torch():
    z = np.array([0.0, math.log(3.0), -math.log(3.0), 30.0, -30.0, 1.5])
    got = O.silu(z)
    assert got[0] == 0.0
    assert abs(got[1] - 0.75 * math.log(3.0)) < 1e-15
    assert abs(got[2] + 0.25 * math.log(3.0)) < 1e-15
    assert np.allclose(got, torch.nn.functional.silu(torch.from_numpy(z)).numpy(), rtol=1e-15, atol=1e-15)


@pytest.mark.parametrize("act", ["swiglu", "relu2"])
def test_expert_ffn_brute_force(act):
    rng = np.random.default_rng(15)
    x = rng.standard_normal((3, 5))
    w1, w3, w2 = rng.standard_normal((4, 5)), rng.standard_normal((4, 5)), rng.standard_normal((6, 4))
    got = O.expert_ffn(x, w1, w3 if act == "swiglu" else None, w2, act)
    for t in range(3):
        ref = _bf_ffn(x[t].tolist(), w1.tolist(), w3.tolist(), w2.tolist(), act)
        assert np.allclose(got[t], ref, rtol=1e-12, atol=1e-12)


def test_relu2_closed_form():
    # W1 = I, W2 = I: out = max(x, 0)^2 elementwise
    x = np.array([[-2.0, -0.5, 0.0, 0.5, 3.0]])
    eye = np.eye(5)
    assert np.array_equal(O.expert_ffn(x, eye, None, eye, "relu2")[0], [0, 0, 0, 0.25, 9.0])


# ----------------------------------------------------------------------------- whole layer
def test_single_expert_equals_dense_swiglu_ffn():
    lay = f32layer(E=1, k=1, G=1, Gk=1, score="sigmoid", T=4, d=5, I=3)
    out = O.moe_forward(lay)["out"]
    w1, w3, w2 = [a.astype(np.float64).tolist() for a in (lay.w_gate[0], lay.w_up[0], lay.w_down[0])]
    for t in range(4):
        ref = _bf_ffn(lay.x[t].astype(np.float64).tolist(), w1, w3, w2, "swiglu")
        assert np.allclose(out[t], ref, rtol=1e-12, atol=1e-12)


def test_k_equals_E_softmax_is_dense_gate_weighted_sum():
    lay = f32layer(E=4, k=4, G=1, Gk=1, score="softmax", T=5, d=6, I=3)
    out = O.moe_forward(lay)["out"]
    for t in range(5):
        xr = lay.x[t].astype(np.float64).tolist()
        logits = [math.fsum(xr[c] * float(lay.router[e, c]) for c in range(6)) for e in range(4)]
        m = max(logits)
        z = [math.exp(v - m) for v in logits]
        p = [v / math.fsum(z) for v in z]
        ref = [0.0] * 6
        for e in range(4):
            y = _bf_ffn(xr, lay.w_gate[e].astype(np.float64).tolist(), lay.w_up[e].astype(np.float64).tolist(),
                        lay.w_down[e].astype(np.float64).tolist(), "swiglu")
            ref = [a + p[e] * b for a, b in zip(ref, y)]
        assert np.allclose(out[t], ref, rtol=1e-11, atol=1e-12)


def test_sparse_mixture_brute_force_with_groups_and_shared():
    """Full layer on a tiny case: brute force per token from the definition."""
    lay = f32layer(E=6, k=2, G=3, Gk=2, n_g=2, score="sigmoid", T=4, d=5, I=3, S=2)
    r = O.moe_forward(lay)
    for t in range(4):
        xr = lay.x[t].astype(np.float64).tolist()
        logits = [math.fsum(xr[c] * float(lay.router[e, c]) for c in range(5)) for e in range(6)]
        s = [1.0 / (1.0 + math.exp(-v)) for v in logits]
        sel = _bf_select(np.array(s, np.float32), 2, 3, 2, 2)
        tot = math.fsum(s[e] for e in sel)
        ref = [0.0] * 5
        for e in sel:
            y = _bf_ffn(xr, lay.w_gate[e].astype(np.float64).tolist(), lay.w_up[e].astype(np.float64).tolist(),
                        lay.w_down[e].astype(np.float64).tolist(), "swiglu")
            ref = [a + s[e] / tot * b for a, b in zip(ref, y)]
        for i in range(2):
            y = _bf_ffn(xr, lay.sh_gate[i].astype(np.float64).tolist(), lay.sh_up[i].astype(np.float64).tolist(),
                        lay.sh_down[i].astype(np.float64).tolist(), "swiglu")
            ref = [a + b for a, b in zip(ref, y)]
        assert r["idx"][t].tolist() == sel
        assert np.allclose(r["out"][t], ref, rtol=1e-11, atol=1e-12)


def test_shared_experts_equal_one_concatenated_ffn():
    lay = f32layer(E=2, k=1, S=3, T=6, d=8, I=4, score="sigmoid")
    no_routed = O.moe_forward(lay)["out"] - _routed_part(lay)
    x = lay.x.astype(np.float64)
    w1 = np.concatenate(list(lay.sh_gate.astype(np.float64)), axis=0)     # [S*I, d]
    w3 = np.concatenate(list(lay.sh_up.astype(np.float64)), axis=0)
    w2 = np.concatenate(list(lay.sh_down.astype(np.float64)), axis=1)     # [d, S*I]
    ref = np.array([_bf_ffn(x[t].tolist(), w1.tolist(), w3.tolist(), w2.tolist(), "swiglu") for t in range(6)])
    assert np.allclose(no_routed, ref, rtol=1e-11, atol=1e-12)


def _routed_part(lay):
    r = O.route(lay)
    out = np.zeros((lay.shape.T, lay.shape.d))
    for t in range(lay.shape.T):
        for j in range(lay.shape.k):
            e = int(r["idx"][t, j])
            out[t] += r["w"][t, j] * np.array(_bf_ffn(r["x"][t].tolist(), lay.w_gate[e].astype(np.float64).tolist(),
                                                      lay.w_up[e].astype(np.float64).tolist(),
                                                      lay.w_down[e].astype(np.float64).tolist(), "swiglu"))
    return out


def test_e4m3_layer_equals_dequantised_fp64_layer():
    """e4m3 weights: the oracle's expert is the bf16/fp64 expert of the dequantised weights."""
    lay = W.make_layer(W.small_shape(T=4, d=32, E=4, k=2, G=1, Gk=1, S=1, I=16, act="relu2",
                                     weight_dtype="e4m3", seed=21), cache=False)
    r = O.moe_forward(lay)
    x = O.decode_bf16(lay.x)
    for t in range(4):
        ref = np.zeros(32)
        for j, e in enumerate(r["idx"][t]):
            w1 = O.decode_e4m3(lay.w_gate[e]) * lay.s_gate[e][:, None].astype(np.float64)
            w2 = O.decode_e4m3(lay.w_down[e]) * lay.s_down[e][:, None].astype(np.float64)
            ref += r["w"][t, j] * np.array(_bf_ffn(x[t].tolist(), w1.tolist(), None, w2.tolist(), "relu2"))
        w1 = O.decode_e4m3(lay.sh_gate[0]) * lay.sh_s_gate[0][:, None].astype(np.float64)
        w2 = O.decode_e4m3(lay.sh_down[0]) * lay.sh_s_down[0][:, None].astype(np.float64)
        ref += np.array(_bf_ffn(x[t].tolist(), w1.tolist(), None, w2.tolist(), "relu2"))
        assert np.allclose(r["out"][t], ref, rtol=1e-11, atol=1e-12)


# ----------------------------------------------------------------------------- permutation
def test_permute_matches_python_sorted():
    rng = np.random.default_rng(16)
    s = rng.random((37, 16)).astype(np.float32)
    idx = O.select_experts(s, 3, 4, 2, 1)
    counts, offsets, perm_token, slot_pos = O.permute(idx, 16)
    pairs = sorted((int(idx[t, j]), t, j) for t in range(37) for j in range(3))
    assert perm_token.tolist() == [t for (_, t, _) in pairs]
    assert [slot_pos[t * 3 + j] for (_, t, j) in pairs] == list(range(37 * 3))
    assert counts.tolist() == [sum(1 for p in pairs if p[0] == e) for e in range(16)]
    assert offsets[0] == 0 and offsets[-1] == 37 * 3
    assert np.array_equal(np.diff(offsets), counts)
    # inverse bijection: the slot at permuted row p belongs to token perm_token[p]
    assert np.array_equal(perm_token[slot_pos], np.repeat(np.arange(37), 3))
    assert sorted(slot_pos.tolist()) == list(range(37 * 3))


def test_permute_empty_experts_and_single_token():
    idx = np.array([[5, 2]], dtype=np.int32)
    counts, offsets, perm_token, slot_pos = O.permute(idx, 8)
    assert counts.tolist() == [0, 0, 1, 0, 0, 1, 0, 0]
    assert offsets.tolist() == [0, 0, 0, 1, 1, 1, 2, 2, 2]
    assert perm_token.tolist() == [0, 0] and slot_pos.tolist() == [1, 0]


# ----------------------------------------------------------------------------- combine
def _combine_case(with_shared, drop):
    """Per-slot values v[t, j] (distinct powers-of-two sums, exact in fp64) laid out in
    expert-major order by Python's sorted() of (expert, token, slot), optionally with a
    capacity of one row per expert (later slots of an expert dropped, slot_pos -1), and
    the expected per-token result written out with pure-Python loops."""
    T, k, E, d = 7, 3, 5, 4
    rng = np.random.default_rng(91)
    idx = np.array([rng.choice(E, size=k, replace=False) for _ in range(T)], dtype=np.int32)
    v = {(t, j): [float(2 ** (t + 8 * j)) + c / 8.0 for c in range(d)] for t in range(T) for j in range(k)}
    pairs = sorted((int(idx[t, j]), t, j) for t in range(T) for j in range(k))
    seen, rows, slot_pos = {}, [], [-1] * (T * k)
    for e, t, j in pairs:
        seen[e] = seen.get(e, 0) + 1
        if drop and seen[e] > 1:
            continue
        slot_pos[t * k + j] = len(rows)
        rows.append(v[(t, j)])
    # a row that no slot points at: picking it up (e.g. through index -1) shows
    rows.append([1e6] * d)
    y_perm = np.array(rows, dtype=np.float64)
    y_sh = np.array([[float(-(c + 1) * (t + 1)) for c in range(d)] for t in range(T)]) if with_shared else None
    expect = []
    for t in range(T):
        acc = [0.0] * d
        for j in range(k):
            if slot_pos[t * k + j] < 0:
                continue
            acc = [a + b for a, b in zip(acc, v[(t, j)])]
        if with_shared:
            acc = [a + b for a, b in zip(acc, y_sh[t].tolist())]
        expect.append(acc)
    return y_perm, np.array(slot_pos, np.int32), y_sh, k, np.array(expect), drop


@pytest.mark.parametrize("with_shared,drop", [(True, False), (False, False), (True, True), (False, True)])
def test_combine_brute_force(with_shared, drop):
    """out[t] = sum of the kept slots' expert outputs + the shared row: per-token loops
    over (token, slot) pairs laid out by sorted(), with dropped slots skipped."""
    y_perm, slot_pos, y_sh, k, expect, drop = _combine_case(with_shared, drop)
    assert (slot_pos < 0).any() == drop
    got = O.combine(y_perm, slot_pos, y_sh, k)
    assert np.array_equal(got, expect)


def test_combine_inverts_the_permutation_of_the_oracle():
    """Round trip: rows laid out by O.permute (itself pinned by sorted()) and summed back by
    O.combine give each token the sum of its own k values, with or without a capacity."""
    rng = np.random.default_rng(92)
    T, E, k, d = 50, 8, 3, 5
    idx = np.array([rng.choice(E, size=k, replace=False) for _ in range(T)], dtype=np.int32)
    vals = rng.standard_normal((T, k, d))
    for cap in (None, 10):
        _, offsets, perm_token, slot_pos = O.permute(idx, E, cap)
        kept = (slot_pos >= 0).reshape(T, k)
        y = np.zeros((int(offsets[-1]), d))
        flat = vals.reshape(T * k, d)
        y[slot_pos[slot_pos >= 0]] = flat[slot_pos >= 0]
        got = O.combine(y, slot_pos, None, k)
        want = np.array([sum((vals[t, j] for j in range(k) if kept[t, j]), np.zeros(d)) for t in range(T)])
        assert np.allclose(got, want, rtol=1e-14, atol=1e-14)
        assert cap is None or (~kept).any()


# ----------------------------------------------------------------------------- selection bias
def _with_bias(lay, b):
    lay.select_bias = None if b is None else np.asarray(b, np.float32)
    return lay


def test_zero_selection_bias_is_the_unbiased_router():
    lay = f32layer(E=8, k=3, G=4, Gk=2, T=40, d=6, score="sigmoid")
    ref = O.route(lay)
    got = O.route(_with_bias(lay, np.zeros(8)))
    assert np.array_equal(ref["idx"], got["idx"]) and np.array_equal(ref["w"], got["w"])


@pytest.mark.parametrize("score", ["sigmoid", "softmax"])
def test_large_selection_bias_forces_the_biased_experts(score):
    """A bias far above every logit makes those experts the selection of every token, while
    the weights stay the renormalised UNBIASED scores of the selected experts."""
    lay = f32layer(E=8, k=3, T=30, d=6, score=score)
    b = np.zeros(8)
    chosen = [1, 4, 6]
    b[chosen] = 60.0
    r = O.route(_with_bias(lay, b))
    for t in range(30):
        assert sorted(r["idx"][t].tolist()) == chosen
        xr = lay.x[t].astype(np.float64).tolist()
        logits = [math.fsum(xr[c] * float(lay.router[e, c]) for c in range(6)) for e in range(8)]
        if score == "sigmoid":
            sc = [1.0 / (1.0 + math.exp(-v)) for v in logits]
        else:
            m = max(logits)
            z = [math.exp(v - m) for v in logits]
            sc = [v / math.fsum(z) for v in z]
        tot = math.fsum(sc[e] for e in chosen)
        for j in range(3):
            assert abs(r["w"][t, j] - sc[int(r["idx"][t, j])] / tot) < 1e-12


def test_selection_bias_brute_force_with_groups():
    """Selection on sigma(l + b) from the definition (brute force over group and expert
    subsets), weights from sigma(l)."""
    lay = f32layer(E=8, k=3, G=4, Gk=2, n_g=2, T=12, d=5, score="sigmoid")
    rng = np.random.default_rng(41)
    b = rng.standard_normal(8)
    r = O.route(_with_bias(lay, b))
    b32 = np.asarray(b, np.float32).astype(np.float64)
    for t in range(12):
        xr = lay.x[t].astype(np.float64).tolist()
        logits = [math.fsum(xr[c] * float(lay.router[e, c]) for c in range(5)) for e in range(8)]
        keys = np.array([1.0 / (1.0 + math.exp(-(logits[e] + b32[e]))) for e in range(8)], np.float32)
        if len(set(keys.tolist())) < 8:
            continue
        sel = _bf_select(keys, 3, 4, 2, 2)
        assert r["idx"][t].tolist() == sel
        sc = [1.0 / (1.0 + math.exp(-v)) for v in logits]
        tot = math.fsum(sc[e] for e in sel)
        assert np.allclose(r["w"][t], [sc[e] / tot for e in sel], rtol=1e-12, atol=0)


@pytest.mark.parametrize("score", ["sigmoid", "softmax"])
def test_common_shift_of_the_selection_bias_changes_nothing(score):
    """Without groups the selection is a ranking of l + b: adding one constant to every b_e
    leaves it unchanged (sigmoid and softmax are monotone in each logit)."""
    lay = f32layer(E=8, k=2, T=50, d=6, score=score)
    rng = np.random.default_rng(42)
    b = rng.standard_normal(8) * 0.5
    a = O.route(_with_bias(lay, b))["idx"]
    c = O.route(_with_bias(lay, b + 0.75))["idx"]
    assert np.array_equal(a, c)


# ----------------------------------------------------------------------------- load statistics
def test_load_stats_uniform_routing_gives_alpha():
    """[MoE-Eng] "负载均衡": the loss is minimal, alpha * E * E * (1/E)^2 = alpha, when every
    f_e = p_e = 1/E."""
    E = 4
    idx = np.arange(E, dtype=np.int32)[:, None]
    scores = np.full((E, E), 0.3)
    f, p, loss = O.load_stats(scores, idx, E, alpha=0.01)
    assert np.allclose(f, 0.25) and np.allclose(p, 0.25)
    assert abs(loss - 0.01) < 1e-15


def test_load_stats_hand_examples():
    # softmax probabilities, both tokens to expert 0: f = [1, 0], p = [0.75, 0.25]
    f, p, loss = O.load_stats(np.array([[0.9, 0.1], [0.6, 0.4]]), np.array([[0], [0]]), 2, 1.0)
    assert f.tolist() == [1.0, 0.0] and np.allclose(p, [0.75, 0.25]) and abs(loss - 1.5) < 1e-15
    # sigmoid scores are normalised per token: [0.75, 0.25] and [0.5, 0.5]
    f, p, loss = O.load_stats(np.array([[0.9, 0.3], [0.2, 0.2]]), np.array([[0], [1]]), 2, 2.0)
    assert f.tolist() == [0.5, 0.5] and np.allclose(p, [0.625, 0.375]) and abs(loss - 2.0) < 1e-15
    # top-2 of 3 experts: f counts assignments over T * k
    f, _, _ = O.load_stats(np.ones((2, 3)), np.array([[0, 1], [0, 2]]), 3, 1.0)
    assert f.tolist() == [0.5, 0.25, 0.25]


def test_load_stats_fractions_sum_to_one():
    lay = f32layer(E=8, k=3, G=4, Gk=2, T=60, d=6, score="sigmoid")
    r = O.route(lay)
    f, p, loss = O.load_stats(r["scores"], r["idx"], 8, 0.5)
    assert abs(f.sum() - 1.0) < 1e-14 and abs(p.sum() - 1.0) < 1e-14 and loss > 0


# ----------------------------------------------------------------------------- capacity
def test_expert_capacity_values():
    assert O.expert_capacity(4096, 6, 64, 1.25) == 480
    assert O.expert_capacity(10, 1, 3, 1.0) == 3         # 3.33 rounds down
    assert O.expert_capacity(4, 1, 2, 1.0) == 2


def test_capacity_hand_example():
    idx = np.array([[0], [0], [0], [1]], dtype=np.int32)
    counts, offsets, perm_token, slot_pos = O.permute(idx, 2, capacity=2)
    assert counts.tolist() == [2, 1] and offsets.tolist() == [0, 2, 3]
    assert perm_token.tolist() == [0, 1, 3] and slot_pos.tolist() == [0, 1, -1, 2]


def test_capacity_keeps_each_experts_first_tokens_python_sorted():
    rng = np.random.default_rng(43)
    s = rng.random((53, 8)).astype(np.float32)
    idx = O.select_experts(s, 3, 1, 1, 1)
    for cap in (0, 1, 7, 19, 1000):
        counts, offsets, perm_token, slot_pos = O.permute(idx, 8, capacity=cap)
        pairs = sorted((int(idx[t, j]), t, j) for t in range(53) for j in range(3))
        kept, seen = [], {}
        for e, t, j in pairs:
            seen[e] = seen.get(e, 0) + 1
            if seen[e] <= cap:
                kept.append((e, t, j))
        assert perm_token.tolist() == [t for (_, t, _) in kept]
        assert [slot_pos[t * 3 + j] for (_, t, j) in kept] == list(range(len(kept)))
        dropped = set((t, j) for (_, t, j) in pairs) - set((t, j) for (_, t, j) in kept)
        assert all(slot_pos[t * 3 + j] == -1 for (t, j) in dropped)
        assert counts.tolist() == [min(cap, sum(1 for p in pairs if p[0] == e)) for e in range(8)]
    unlimited = O.permute(idx, 8)
    large = O.permute(idx, 8, capacity=10 ** 6)
    assert all(np.array_equal(a, b) for a, b in zip(unlimited, large))


def test_forward_with_capacity_brute_force():
    """Dropped slots contribute nothing: brute force per token over the kept slots."""
    shape = W.small_shape(act_dtype="f32", weight_dtype="f32", T=6, d=5, E=4, k=2, S=1, I=3,
                          G=1, Gk=1, score="softmax", capacity_factor=0.5)
    lay = W.make_layer(shape, cache=False)
    r = O.moe_forward(lay)
    cap = O.expert_capacity(6, 2, 4, 0.5)
    assert cap == 1
    pairs = sorted((int(r["idx"][t, j]), t, j) for t in range(6) for j in range(2))
    kept, seen = set(), {}
    for e, t, j in pairs:
        seen[e] = seen.get(e, 0) + 1
        if seen[e] <= cap:
            kept.add((t, j))
    assert r["kept"].sum() == len(kept)
    for t in range(6):
        xr = lay.x[t].astype(np.float64).tolist()
        ref = np.array(_bf_ffn(xr, lay.sh_gate[0].astype(np.float64).tolist(),
                               lay.sh_up[0].astype(np.float64).tolist(),
                               lay.sh_down[0].astype(np.float64).tolist(), "swiglu"))
        for j in range(2):
            if (t, j) not in kept:
                continue
            e = int(r["idx"][t, j])
            ref = ref + r["w"][t, j] * np.array(_bf_ffn(xr, lay.w_gate[e].astype(np.float64).tolist(),
                                                        lay.w_up[e].astype(np.float64).tolist(),
                                                        lay.w_down[e].astype(np.float64).tolist(), "swiglu"))
        assert np.allclose(r["out"][t], ref, rtol=1e-11, atol=1e-12)
    # a subset of tokens sees the same drops as the whole batch
    sub = O.moe_forward(lay, tokens=np.array([4, 1]))
    assert np.allclose(sub["out"], r["out"][[4, 1]], rtol=1e-13, atol=0)


def test_forward_with_its_own_routing_given_is_unchanged():
    shape = W.small_shape(act_dtype="f32", weight_dtype="f32", T=9, d=6, E=4, k=2, S=1, I=3,
                          G=2, Gk=1, score="sigmoid", capacity_factor=0.75, select_bias_std=0.5)
    lay = W.make_layer(shape, cache=False)
    a = O.moe_forward(lay)
    b = O.moe_forward(lay, idx=a["idx"])
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["kept"], b["kept"])
    c = O.moe_forward(lay, tokens=np.array([2, 7]), idx=a["idx"])
    assert np.allclose(c["out"], a["out"][[2, 7]], rtol=1e-13, atol=0)


# ----------------------------------------------------------------------------- e4m3 activations
def _quant_inputs():
    rng = np.random.default_rng(44)
    a = (rng.standard_normal((40, 256)) * rng.random((40, 1)) * 20).astype(np.float32)
    a[0] = 0.0                                                   # zero row
    a[1] = np.float32(1e-3) * rng.standard_normal(256).astype(np.float32)
    a[2, :] = 0.0
    a[2, 0] = 7.0                                                # a single non-zero
    a[3] = np.linspace(-448 * 2.0 ** -9, 448 * 2.0 ** -9, 256, dtype=np.float32)   # subnormals
    return a


def test_activation_quantiser_matches_torch_e4m3():
    """Codes: torch's float8_e4m3fn conversion (round to nearest even) of the same fp32
    quotients a / scale, each computed with one fp32 division."""
    a = _quant_inputs()
    codes, scale = O.quantize_rows_e4m3(a)
    amax = np.abs(a).max(axis=1)
    assert np.array_equal(scale, (amax / np.float32(448.0)).astype(np.float32))
    safe = np.where(scale > 0, scale, np.float32(1)).astype(np.float32)
    v = np.clip((a / safe[:, None]).astype(np.float32), -448, 448)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ref = np.where(scale[:, None] > 0, ref, 0)
    ref = np.where(ref == 0x80, 0, ref)                          # -0 is stored as +0
    assert np.array_equal(codes, ref)
    assert codes[0].max() == 0 and scale[0] == 0
    assert codes[2, 0] == 0x7E                                   # the row max maps to 448


def test_activation_quantiser_error_bound():
    """Half an e4m3 ulp: 2^-4 relative for normals, 2^-10 * scale absolute below 2^-6."""
    a = _quant_inputs()
    codes, scale = O.quantize_rows_e4m3(a)
    dq = O.dequantize_rows_e4m3(codes, scale)
    a64 = a.astype(np.float64)
    for r in range(a.shape[0]):
        if scale[r] == 0:
            assert np.all(dq[r] == 0)
            continue
        v = np.abs(a64[r]) / float(scale[r])
        err = np.abs(dq[r] - a64[r])
        normal = v >= 2.0 ** -6
        assert np.all(err[normal] <= 2.0 ** -4 * np.abs(a64[r][normal]) * (1 + 1e-6))
        assert np.all(err[~normal] <= 2.0 ** -10 * float(scale[r]) * (1 + 1e-6))


def test_forward_with_e4m3_activations_is_the_forward_of_the_dequantised_rows():
    shape = W.small_shape(act_dtype="bf16", weight_dtype="e4m3", T=7, d=64, E=4, k=2, S=1, I=64,
                          G=1, Gk=1, act="relu2", fp8_act=True)
    lay = W.make_layer(shape, cache=False)
    r = O.moe_forward(lay)
    x = O.decode_bf16(lay.x)
    xq = O.dequantize_rows_e4m3(*O.quantize_rows_e4m3(x))
    assert not np.array_equal(xq, x)
    for t in range(7):
        ref = np.zeros(64)
        for j in range(2):
            e = int(r["idx"][t, j])
            w1, _, w2 = O.expert_weights(lay, e)
            ref += r["w"][t, j] * np.array(_bf_ffn(xq[t].tolist(), w1.tolist(), None, w2.tolist(), "relu2"))
        w1, _, w2 = O.shared_weights(lay, 0)
        ref += np.array(_bf_ffn(xq[t].tolist(), w1.tolist(), None, w2.tolist(), "relu2"))
        assert np.allclose(r["out"][t], ref, rtol=1e-10, atol=1e-12)
    # routing uses the unquantised x: same selection as the layer without e4m3 activations
    plain = W.make_layer(W.small_shape(act_dtype="bf16", weight_dtype="e4m3", T=7, d=64, E=4, k=2,
                                       S=1, I=64, G=1, Gk=1, act="relu2"), cache=False)
    assert np.array_equal(O.route(plain)["idx"], r["idx"])


# ----------------------------------------------------------------------------- pre-norm
def test_round_to_act_bf16_matches_the_fp32_encoder_and_rounds_once():
    """On fp32 inputs the single rounding equals the bf16 encoder of the fp32 bits (an
    independent integer implementation); ties go to even; an fp64 value just above a tie
    rounds up, which a detour through fp32 (a tie there) would round down."""
    rng = np.random.default_rng(7)
    v = (rng.standard_normal(20000) * np.exp(rng.standard_normal(20000) * 4)).astype(np.float32)
    ours = O.round_to_act(v.astype(np.float64), "bf16")
    ref = O.decode_bf16(W.encode_bf16(v))
    assert np.array_equal(ours, ref)
    t = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 1 + 2.0 ** -8 + 2.0 ** -30])
    assert list(O.round_to_act(t, "bf16")) == [1.0, 1 + 2.0 ** -6, -1.0, 1 + 2.0 ** -7]
    assert O.round_to_act(np.array([0.0]), "bf16")[0] == 0.0


def test_rms_norm_hand_example():
    y = O.rms_norm(np.array([[3.0, 4.0]]), np.array([2.0, -1.0]), 0.0)
    r = math.sqrt((9 + 16) / 2)
    assert np.allclose(y, [[6 / r, -4 / r]], rtol=1e-15)


def test_rms_norm_unit_rms_and_scale_invariance():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((6, 37)) * rng.random((6, 1)) * 10
    y = O.rms_norm(x, np.ones(37), 0.0)
    assert np.allclose(np.mean(y * y, axis=1), 1.0, rtol=1e-13)
    assert np.allclose(O.rms_norm(3.5 * x, np.ones(37), 0.0), y, rtol=1e-13)
    # homogeneity with eps: scaling x by c and eps by c^2 changes nothing
    assert np.allclose(O.rms_norm(3.5 * x, np.ones(37), 0.3 * 3.5 ** 2),
                       O.rms_norm(x, np.ones(37), 0.3), rtol=1e-13)
    g = rng.standard_normal(37)
    assert np.allclose(O.rms_norm(x, g, 0.1), O.rms_norm(x, np.ones(37), 0.1) * g, rtol=1e-13)


def test_rms_norm_keeps_the_mean_and_puts_eps_under_the_root():
    # a constant row is not centred (LayerNorm would give zeros)
    assert np.allclose(O.rms_norm(np.full((1, 8), -2.5), np.ones(8), 0.0), -1.0, rtol=1e-15)
    # x = 1e-3, eps = 1e-6: 1e-3 / sqrt(1e-6 + 1e-6) = 1 / sqrt(2)
    assert np.allclose(O.rms_norm(np.full((1, 4), 1e-3), np.ones(4), 1e-6), 2 ** -0.5, rtol=1e-12)
    assert np.all(O.rms_norm(np.zeros((1, 4)), np.ones(4), 1e-6) == 0.0)


def _prenorm_layer(**kw):
    base = dict(act_dtype="f32", weight_dtype="f32", T=6, d=8, E=4, k=2, S=1, I=5, G=2, Gk=1,
                score="sigmoid", pre_norm=True, residual=True, norm_eps=0.0)
    base.update(kw)
    return W.make_layer(W.small_shape(**base), cache=False)


def test_prenorm_forward_is_residual_plus_the_layer_on_the_normalised_rows():
    lay = _prenorm_layer()
    pre = O.moe_forward(lay)
    x = O.decode_act(lay.x, "f32")
    xn = O.rms_norm(x, lay.norm_gamma, 0.0).astype(np.float32)
    plain = W.Layer(**{**lay.__dict__})
    plain.shape = W.replace(lay.shape, pre_norm=False, residual=False)
    plain.x = xn
    ref = O.moe_forward(plain)
    assert np.array_equal(pre["idx"], ref["idx"])
    assert np.allclose(pre["out"], x + ref["out"], rtol=1e-13, atol=1e-13)
    # brute force for one token: residual + weighted experts + shared expert on x_norm
    t = 3
    acc = x[t].copy()
    for j in range(2):
        w1, w3, w2 = O.expert_weights(lay, int(pre["idx"][t, j]))
        acc += pre["w"][t, j] * np.array(_bf_ffn(xn[t].astype(np.float64).tolist(), w1.tolist(),
                                                 w3.tolist(), w2.tolist(), "swiglu"))
    w1, w3, w2 = O.shared_weights(lay, 0)
    acc += np.array(_bf_ffn(xn[t].astype(np.float64).tolist(), w1.tolist(), w3.tolist(),
                            w2.tolist(), "swiglu"))
    assert np.allclose(pre["out"][t], acc, rtol=1e-10, atol=1e-12)


def test_prenorm_layer_update_is_invariant_to_power_of_two_row_scaling():
    """With eps = 0 RMSNorm removes any row scale; a power of two scales the stored x
    exactly, so out(4 x) - 4 x equals out(x) - x bit for bit."""
    for dt in ("f32", "bf16"):
        lay = _prenorm_layer(act_dtype=dt, weight_dtype=dt, d=16, I=8)
        a = O.moe_forward(lay)
        big = W.Layer(**{**lay.__dict__})
        x32 = O.decode_act(lay.x, dt).astype(np.float32) * np.float32(4.0)
        big.x = x32 if dt == "f32" else W.encode_bf16(x32)
        b = O.moe_forward(big)
        xa = O.decode_act(lay.x, dt)
        assert np.array_equal(a["idx"], b["idx"])
        assert np.allclose(b["out"] - 4 * xa, a["out"] - xa, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- workloads
def test_fusionllm_shapes_match_the_yaml():
    y = json.load(open(os.path.join(GOLDEN, "fusionllm_moe_yaml.json")))
    for name in ("fusionllm_bf16", "decode_bf16", "skewed_bf16", "fp8_relu2"):
        s = W.SHAPES[name]
        assert (s.d, s.E, s.k, s.S, s.I) == (y["dim"], y["n_routed_experts"], y["n_activated_experts"],
                                            y["n_shared_experts"], y["moe_inter_dim"])


def test_ffn_flop_and_param_accounting_matches_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "llama70b_ffn_counts.json")))
    s = W.small_shape(d=g["d_model"], I=g["d_ffn"], E=1, k=1, S=0, G=1, Gk=1)
    ffn_flops = s.flops_per_token - 2 * s.d * s.E       # one SwiGLU FFN, no router
    assert abs(ffn_flops - g["ffn_flops_per_token_printed"]) <= g["ffn_flops_rounding"]
    assert abs(3 * s.d * s.I - g["ffn_params_printed"]) <= g["ffn_params_rounding"]
    assert W.SHAPES["fusionllm_bf16"].flops_per_token == 189_005_824


def test_decode_routing_is_prefix_of_prefill_routing():
    """Routing is per token, and the decode workload takes the prefill layer's first 64
    x rows and weights, so its selection equals rows 0..63 of the prefill selection."""
    pre = W.make_layer("fusionllm_bf16")
    dec = W.make_layer("decode_bf16")
    r_pre = O.route(pre, tokens=np.arange(64))
    r_dec = O.route(dec)
    assert np.array_equal(r_pre["idx"], r_dec["idx"])
    assert np.array_equal(r_pre["w"], r_dec["w"])


# ----------------------------------------------------------------------------- mutations
def _swapped_ffn(x, w1, w3, w2, act):
    return O.expert_ffn(x, w3 if w3 is not None else w1, w1, w2, act)


@pytest.mark.parametrize("mutation", ["swap_gate_up", "no_renorm", "tie_high_index",
                                      "token_desc_perm", "drop_shared", "transpose_down",
                                      "biased_weights", "keep_last_at_capacity",
                                      "truncating_quantiser", "layernorm_centering",
                                      "eps_outside_root", "sum_not_mean", "no_residual",
                                      "double_rounding", "combine_no_shared",
                                      "combine_dropped_as_last_row", "combine_slot_major"])
def test_planted_oracle_mistakes_are_caught(monkeypatch, mutation):
    """Each mutation is a plausible slip in the oracle; the named pin must then fail."""
    if mutation == "swap_gate_up":
        monkeypatch.setattr(O.moe_oracle, "expert_ffn", _swapped_ffn)
        check = test_single_expert_equals_dense_swiglu_ffn
    elif mutation == "no_renorm":
        orig = O.moe_oracle.routing_weights
        monkeypatch.setattr(O.moe_oracle, "routing_weights",
                            lambda s, i, renormalize=True, route_scale=1.0: orig(s, i, False, route_scale))
        check = test_k_equals_E_softmax_is_dense_gate_weighted_sum
        # softmax scores over all E already sum to 1 at k = E; use the grouped case instead
        check = test_sparse_mixture_brute_force_with_groups_and_shared
    elif mutation == "tie_high_index":
        orig_sel = O.select_experts
        def bad(s, k, G=1, Gk=1, n_g=1):
            s = np.asarray(s)
            E = s.shape[1]
            return (E - 1 - orig_sel(s[:, ::-1], k, 1, 1, n_g)) if (G == 1 or Gk == G) else orig_sel(s, k, G, Gk, n_g)
        monkeypatch.setattr(O, "select_experts", bad)
        check = test_select_hand_written_tie_cases
    elif mutation == "token_desc_perm":
        orig_perm = O.permute
        def bad(idx, E):
            c, o, _, _ = orig_perm(idx, E)
            idx = np.asarray(idx)
            T, k = idx.shape
            order = np.lexsort((-np.repeat(np.arange(T), k), idx.reshape(-1)))
            pt = np.repeat(np.arange(T), k)[order].astype(np.int32)
            sp = np.empty(T * k, np.int32)
            sp[order] = np.arange(T * k)
            return c, o, pt, sp
        monkeypatch.setattr(O, "permute", bad)
        check = test_permute_matches_python_sorted
    elif mutation == "biased_weights":
        # weights taken from the biased selection keys instead of the unbiased scores
        orig_route = O.moe_oracle.route
        def bad_route(layer, tokens=None):
            r = orig_route(layer, tokens)
            s = layer.shape
            r["w"] = O.moe_oracle.routing_weights(r["keys"], r["idx"], s.renormalize, s.route_scale)
            return r
        monkeypatch.setattr(O, "route", bad_route)
        check = lambda: test_large_selection_bias_forces_the_biased_experts("sigmoid")
    elif mutation == "keep_last_at_capacity":
        orig_perm = O.permute
        def bad(idx, E, capacity=None):
            if capacity is None:
                return orig_perm(idx, E)
            idx = np.asarray(idx)
            T, k = idx.shape
            rev = orig_perm(idx[::-1], E, capacity)     # keeps the LAST tokens of each expert
            sp = rev[3].reshape(T, k)[::-1].reshape(-1)
            return rev[0], rev[1], (T - 1 - rev[2]).astype(np.int32), sp
        monkeypatch.setattr(O, "permute", bad)
        check = test_capacity_keeps_each_experts_first_tokens_python_sorted
    elif mutation == "truncating_quantiser":
        orig = O.moe_oracle._e4m3_rne_magnitude
        def trunc(v32):
            a = np.abs(np.asarray(v32, np.float64))
            c = orig(a)
            up = O.decode_e4m3(c.astype(np.uint8)) > a           # rounded up: step back
            return np.where(up, c - 1, c)
        monkeypatch.setattr(O.moe_oracle, "_e4m3_rne_magnitude", trunc)
        check = test_activation_quantiser_matches_torch_e4m3
    elif mutation == "layernorm_centering":
        orig = O.moe_oracle.rms_norm
        def centred(x, gamma, eps):
            x = np.asarray(x, np.float64)
            return orig(x - x.mean(axis=1, keepdims=True), gamma, eps)
        monkeypatch.setattr(O, "rms_norm", centred)
        check = test_rms_norm_keeps_the_mean_and_puts_eps_under_the_root
    elif mutation == "eps_outside_root":
        def outside(x, gamma, eps):
            x = np.asarray(x, np.float64)
            return x / (np.sqrt(np.mean(x * x, axis=1, keepdims=True)) + eps) * np.asarray(gamma)[None, :]
        monkeypatch.setattr(O, "rms_norm", outside)
        check = test_rms_norm_keeps_the_mean_and_puts_eps_under_the_root
    elif mutation == "sum_not_mean":
        def summed(x, gamma, eps):
            x = np.asarray(x, np.float64)
            return x / np.sqrt(np.sum(x * x, axis=1, keepdims=True) + eps) * np.asarray(gamma)[None, :]
        monkeypatch.setattr(O, "rms_norm", summed)
        check = test_rms_norm_unit_rms_and_scale_invariance
    elif mutation == "no_residual":
        orig_fwd = O.moe_oracle.moe_forward
        def no_res(layer, tokens=None, idx=None):
            lay = W.Layer(**{**layer.__dict__})
            lay.shape = W.replace(layer.shape, residual=False)
            return orig_fwd(lay, tokens, idx)
        monkeypatch.setattr(O, "moe_forward", no_res)
        check = test_prenorm_layer_update_is_invariant_to_power_of_two_row_scaling
    elif mutation == "double_rounding":
        orig = O.moe_oracle.round_to_act
        monkeypatch.setattr(O, "round_to_act",
                            lambda v, dt: orig(np.asarray(v, np.float64).astype(np.float32).astype(np.float64), dt))
        check = test_round_to_act_bf16_matches_the_fp32_encoder_and_rounds_once
    elif mutation == "drop_shared":
        monkeypatch.setattr(O.moe_oracle, "shared_weights",
                            lambda lay, i: tuple(np.zeros_like(a) if a is not None else None
                                                 for a in O.moe_oracle.expert_weights(lay, 0)))
        check = test_shared_experts_equal_one_concatenated_ffn
    elif mutation == "transpose_down":
        def bad_ffn(x, w1, w3, w2, act):
            a = x @ w1.T
            h = O.silu(a) * (x @ w3.T) if act == "swiglu" else np.maximum(a, 0) ** 2
            return h @ w2[:, ::-1].T                      # wrong column order of W2
        monkeypatch.setattr(O.moe_oracle, "expert_ffn", bad_ffn)
        check = test_single_expert_equals_dense_swiglu_ffn
    elif mutation == "combine_no_shared":
        orig = O.moe_oracle.combine
        monkeypatch.setattr(O, "combine", lambda y, sp, ysh, k: orig(y, sp, None, k))
        check = lambda: test_combine_brute_force(True, False)
    elif mutation == "combine_dropped_as_last_row":
        # a dropped slot (-1) gathers the last row instead of being skipped
        def bad(y, sp, ysh, k):
            y = np.asarray(y, np.float64)
            out = y[np.asarray(sp, np.int64).reshape(-1, k)].sum(axis=1)
            return out if ysh is None else out + np.asarray(ysh, np.float64)
        monkeypatch.setattr(O, "combine", bad)
        check = lambda: test_combine_brute_force(False, True)
    elif mutation == "combine_slot_major":
        # slot_pos read as [k, T] instead of [T, k]
        orig = O.moe_oracle.combine
        def bad(y, sp, ysh, k):
            sp = np.asarray(sp).reshape(k, -1).T.reshape(-1)
            return orig(y, sp, ysh, k)
        monkeypatch.setattr(O, "combine", bad)
        check = test_combine_inverts_the_permutation_of_the_oracle
    # a planted mistake may divide by zero (a centred constant row): that is part of the
    # failure the pin must report, not a warning of the suite
    with pytest.raises(AssertionError), np.errstate(divide="ignore", invalid="ignore"):
        check()
