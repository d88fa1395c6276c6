"""Pins of the fp64 backward oracle (no GPU): every gradient against central finite
differences of the layer's forward with the selection held fixed, on tiny fp32 layers of
every routing variant; the fixed-selection forward against the forward oracle; and planted
mistakes that a pin must catch."""
import numpy as np
import pytest

import oracle as O
import workloads as W

B = O.backward

GRAD_OF = {"x": "dx", "router": "drouter", "bias": "dbias", "w1": "dW1", "w3": "dW3", "w2": "dW2",
           "sh_w1": "sh_dW1", "sh_w3": "sh_dW3", "sh_w2": "sh_dW2"}

CASES = {
    # sigmoid, groups, renormalised, shared SwiGLU expert
    "sigmoid_groups": dict(T=7, d=6, E=8, k=3, G=4, Gk=2, S=1, I=5, score="sigmoid"),
    # renormalised softmax: the weights equal the softmax of the selected logits alone
    "softmax": dict(T=6, d=5, E=6, k=2, G=1, Gk=1, S=0, I=4, score="softmax"),
    # raw softmax weights: the normalisation over all E logits reaches every logit
    "softmax_raw": dict(T=6, d=5, E=6, k=2, G=1, Gk=1, S=1, I=4, score="softmax",
                        renormalize=False),
    "relu2": dict(T=6, d=6, E=4, k=2, G=1, Gk=1, S=1, I=5, score="sigmoid", act="relu2"),
    "no_renorm": dict(T=5, d=4, E=5, k=2, G=1, Gk=1, S=0, I=3, score="sigmoid", renormalize=False,
                      route_scale=2.5),
    # capacity drops (some tokens lose one of their two slots) and a selection-only bias
    "capacity_bias": dict(T=9, d=5, E=4, k=2, G=1, Gk=1, S=1, I=3, score="sigmoid",
                          capacity_factor=0.75, select_bias_std=0.5, seed=8),
    "residual_softmax": dict(T=5, d=6, E=4, k=2, G=1, Gk=1, S=1, I=4, score="softmax", residual=True),
}


def _layer(name, seed=5):
    kw = dict(act_dtype="f32", weight_dtype="f32", seed=seed)
    kw.update(CASES[name])
    return W.make_layer(W.small_shape(**kw), cache=False)


def _dout(lay, seed=9):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((lay.shape.T, lay.shape.d))


@pytest.mark.parametrize("name", list(CASES))
def test_fixed_selection_forward_is_the_forward_oracle(name):
    lay = _layer(name)
    r = O.moe_forward(lay)
    P = B.layer_params(lay)
    out = B.forward_params(lay.shape, P, r["idx"], B.routed_slots_kept(lay.shape, r["idx"]))
    assert np.allclose(out, r["out"], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("name", list(CASES))
def test_gradients_match_central_differences(name):
    lay = _layer(name)
    s = lay.shape
    g = _dout(lay)
    grads = B.moe_backward(lay, g)
    idx, kept = grads["idx"], grads["kept"]
    if name == "capacity_bias":
        # the case really drops slots, and some tokens keep one slot and lose the other
        assert (kept.any(axis=1) & ~kept.all(axis=1)).any()
    P = B.layer_params(lay)

    def loss(Q):
        return float(np.sum(g * B.forward_params(s, Q, idx, kept)))

    rng = np.random.default_rng(1)
    for key, gk in GRAD_OF.items():
        if P.get(key) is None:
            continue
        an = grads[gk]
        flat = P[key].reshape(-1)
        picks = rng.choice(flat.size, size=min(flat.size, 10), replace=False)
        for i in picks:
            eps = 1e-6 * max(1.0, abs(flat[i]))
            Q = {kk: (None if v is None else v.copy()) for kk, v in P.items()}
            Q[key].reshape(-1)[i] += eps
            up = loss(Q)
            Q[key].reshape(-1)[i] -= 2 * eps
            dn = loss(Q)
            fd = (up - dn) / (2 * eps)
            assert abs(fd - an.reshape(-1)[i]) <= 1e-6 * max(1.0, abs(fd)), (key, i, fd, an.reshape(-1)[i])


def test_softmax_router_gradient_reaches_unselected_logits():
    """With raw softmax weights every logit moves the selected weights, so every logit has
    gradient; renormalised over the selection, the weights are the softmax of the selected
    logits alone, so the unselected ones have none."""
    lay = _layer("softmax_raw")
    grads = B.moe_backward(lay, _dout(lay))
    unselected = np.ones(grads["dl"].shape, bool)
    np.put_along_axis(unselected, grads["idx"].astype(np.int64), False, axis=1)
    assert np.all(np.abs(grads["dl"][unselected]) > 1e-6)
    lay = _layer("softmax")
    grads = B.moe_backward(lay, _dout(lay))
    unselected = np.ones(grads["dl"].shape, bool)
    np.put_along_axis(unselected, grads["idx"].astype(np.int64), False, axis=1)
    assert np.all(np.abs(grads["dl"][unselected]) <= 1e-15)


def test_residual_adds_dout_to_dx():
    lay = _layer("residual_softmax")
    g = _dout(lay)
    with_res = B.moe_backward(lay, g)
    lay2 = W.Layer(**{**lay.__dict__})
    lay2.shape = W.replace(lay.shape, residual=False)
    without = B.moe_backward(lay2, g)
    assert np.allclose(with_res["dx"] - without["dx"], g, rtol=0, atol=1e-12)


@pytest.mark.parametrize("mutation,case", [("topk_logits_only", "softmax_raw"),
                                           ("no_renorm_jacobian", "sigmoid_groups"),
                                           ("swap_da_db", "sigmoid_groups"),
                                           ("dsilu_as_sigmoid", "sigmoid_groups"),
                                           ("no_dropped_score_gradient", "capacity_bias")])
def test_planted_backward_mistakes_are_caught(monkeypatch, mutation, case):
    if mutation == "topk_logits_only":
        orig = B._scores_to_logits
        monkeypatch.setattr(B, "_scores_to_logits", lambda ds, sc, fn: np.where(ds != 0, orig(ds, sc, fn), 0.0))
    elif mutation == "no_renorm_jacobian":
        monkeypatch.setattr(B, "_weights_to_scores",
                            lambda dw, sel, c, rn: (c / sel.sum(axis=1, keepdims=True)) * dw if rn else c * dw)
    elif mutation == "swap_da_db":
        orig = B._act_backward
        def swapped(a, b, dh, act):
            da, db = orig(a, b, dh, act)
            return (db, da) if db is not None else (da, db)
        monkeypatch.setattr(B, "_act_backward", swapped)
    elif mutation == "dsilu_as_sigmoid":
        def bad(a, b, dh, act):
            sig = 1.0 / (1.0 + np.exp(-a))
            return dh * b * sig, dh * O.silu(a)
        monkeypatch.setattr(B, "_act_backward", bad)
    elif mutation == "no_dropped_score_gradient":
        # dropped slots taken out of the renormalisation Jacobian
        orig = B._weights_to_scores
        state = {}
        real = B.moe_backward
        def patched(layer, dout, idx=None):
            state["kept"] = B.routed_slots_kept(layer.shape, idx if idx is not None else O.route(layer)["idx"])
            return real(layer, dout, idx)
        monkeypatch.setattr(B, "_weights_to_scores",
                            lambda dw, sel, c, rn: np.where(state["kept"], orig(dw, sel, c, rn), 0.0))
        monkeypatch.setattr(B, "moe_backward", patched)
    with pytest.raises(AssertionError):
        test_gradients_match_central_differences(case)
