"""Pins of the oracle's backward against things other than its own formulas.

The backward of the layer (section "SonicMoE" of "Experts backends" names
training as that backend's focus; the gradients are the forward differentiated
with the top-k selection held fixed) is checked three ways, on the CPU:

* central finite differences of the oracle's *forward* (route + combine, fp64),
  one parameter group at a time along a random direction; the perturbed fp32
  inputs are rounded, so the exact step taken is used, not the nominal one;
* an independent dense float64 formulation differentiated by torch.autograd;
* invariants: softmax keys are shift invariant (each row of dkey sums to 0),
  a sigmoid router only passes gradient to the selected experts, and a single
  renormalised expert gets a constant weight (dkey = 0).
"""
import numpy as np
import pytest
import torch

import oracle

GATES = [oracle.GATE_SILU, oracle.GATE_GELU, oracle.GATE_RELU]
# (score, renormalize, routed scale, bias)
ROUTERS = [
    (oracle.SOFTMAX, True, 1.0, False),
    (oracle.SOFTMAX, False, 1.0, True),
    (oracle.SIGMOID, True, 2.5, True),
    (oracle.SIGMOID, False, 1.0, False),
]


def _problem(seed, T=6, H=16, I=24, E=6, k=2):
    rng = np.random.default_rng(seed)
    f = lambda *s, sc=1.0: (rng.standard_normal(s) * sc).astype(np.float32)
    return dict(x=f(T, H), w_r=f(E, H, sc=0.5), bias=f(E, sc=0.3),
                w_gate=f(E, I, H, sc=H ** -0.5), w_up=f(E, I, H, sc=H ** -0.5),
                w_down=f(E, H, I, sc=I ** -0.5), dout=f(T, H), k=k)


def _loss(p, score, renorm, scale, gate, use_bias):
    ex = oracle.Experts(p["w_gate"], p["w_up"], p["w_down"], gate=gate)
    ids, w = oracle.route(p["x"], p["w_r"], p["bias"] if use_bias else None, p["k"], score, renorm, scale)
    out = ex.combine(p["x"], ids, w)
    return float((out * p["dout"].astype(np.float64)).sum()), ids


def _grads(p, score, renorm, scale, gate, use_bias):
    ex = oracle.Experts(p["w_gate"], p["w_up"], p["w_down"], gate=gate)
    return oracle.backward(p["x"], p["w_r"], p["bias"] if use_bias else None, ex, p["k"], score, renorm,
                           scale, p["dout"])


GROUPS = [("x", "dx"), ("w_r", "dw_router"), ("bias", "dbias"), ("w_gate", "dw_gate"),
          ("w_up", "dw_up"), ("w_down", "dw_down")]


@pytest.mark.parametrize("gate", GATES)
@pytest.mark.parametrize("router", ROUTERS)
def test_backward_matches_finite_differences(router, gate):
    score, renorm, scale, use_bias = router
    p = _problem(seed=11 + gate)
    g = _grads(p, score, renorm, scale, gate, use_bias)
    rng = np.random.default_rng(5)
    eps = 1e-4
    for name, gname in GROUPS:
        if name == "bias" and not use_bias:
            continue
        v = rng.standard_normal(p[name].shape)
        plus, minus = dict(p), dict(p)
        plus[name] = (p[name] + eps * v).astype(np.float32)
        minus[name] = (p[name] - eps * v).astype(np.float32)
        step = plus[name].astype(np.float64) - minus[name].astype(np.float64)   # the exact step taken
        lp, ids_p = _loss(plus, score, renorm, scale, gate, use_bias)
        lm, ids_m = _loss(minus, score, renorm, scale, gate, use_bias)
        assert (ids_p == g["ids"]).all() and (ids_m == g["ids"]).all(), "selection moved; pick another seed"
        fd = lp - lm
        pred = float((g[gname] * step).sum())
        assert abs(fd - pred) <= 2e-6 * (abs(pred) + 1e-3), (name, fd, pred)


def _autograd(p, score, renorm, scale, gate, use_bias, ids):
    """Dense float64 layer with fixed ids, differentiated by torch.autograd."""
    t = {n: torch.tensor(p[n], dtype=torch.float64, requires_grad=True)
         for n in ("x", "w_r", "bias", "w_gate", "w_up", "w_down")}
    key = t["x"] @ t["w_r"].T + (t["bias"] if use_bias else 0.0)
    s = torch.softmax(key, dim=1) if score == oracle.SOFTMAX else torch.sigmoid(key)
    ids_t = torch.tensor(ids, dtype=torch.int64)
    w = torch.gather(s, 1, ids_t)
    if renorm:
        w = w / w.sum(dim=1, keepdim=True)
    w = w * scale
    act = {oracle.GATE_SILU: torch.nn.functional.silu,
           oracle.GATE_GELU: lambda z: torch.nn.functional.gelu(z, approximate="none"),
           oracle.GATE_RELU: torch.relu}[gate]
    out = torch.zeros_like(t["x"])
    for i in range(ids.shape[1]):
        e = ids_t[:, i]
        g = torch.einsum("th,tjh->tj", t["x"], t["w_gate"][e])
        u = torch.einsum("th,tjh->tj", t["x"], t["w_up"][e])
        y = torch.einsum("tj,toj->to", act(g) * u, t["w_down"][e])
        out = out + w[:, i:i + 1] * y
    (out * torch.tensor(p["dout"], dtype=torch.float64)).sum().backward()
    return {gname: (torch.zeros_like(t[name]) if t[name].grad is None else t[name].grad).numpy()
            for name, gname in GROUPS}


@pytest.mark.parametrize("gate", GATES)
@pytest.mark.parametrize("router", ROUTERS)
def test_backward_matches_dense_autograd(router, gate):
    score, renorm, scale, use_bias = router
    p = _problem(seed=3, T=9, H=12, I=20, E=5, k=3)
    g = _grads(p, score, renorm, scale, gate, use_bias)
    ref = _autograd(p, score, renorm, scale, gate, use_bias, g["ids"])
    for _, gname in GROUPS:
        if gname == "dbias" and not use_bias:
            continue
        np.testing.assert_allclose(g[gname], ref[gname], rtol=1e-9, atol=1e-12, err_msg=gname)


def test_backward_router_invariants():
    p = _problem(seed=21, T=8, H=16, I=8, E=7, k=3)
    ex = oracle.Experts(p["w_gate"], p["w_up"], p["w_down"])
    # softmax: adding a constant to every key of a token changes nothing
    g = oracle.backward(p["x"], p["w_r"], p["bias"], ex, 3, oracle.SOFTMAX, True, 1.0, p["dout"])
    assert np.abs(g["dkey"].sum(axis=1)).max() < 1e-12
    assert abs(g["dbias"].sum()) < 1e-12
    # sigmoid: only the selected experts of a token receive gradient
    g = oracle.backward(p["x"], p["w_r"], p["bias"], ex, 3, oracle.SIGMOID, False, 1.0, p["dout"])
    for t in range(8):
        sel = np.zeros(7, bool)
        sel[g["ids"][t]] = True
        assert (g["dkey"][t][~sel] == 0).all() and (g["dkey"][t][sel] != 0).all()
    # one renormalised expert per token: its weight is the routed scale, constant
    g = oracle.backward(p["x"], p["w_r"], p["bias"], ex, 1, oracle.SIGMOID, True, 2.5, p["dout"])
    assert np.abs(g["dkey"]).max() < 1e-12 and np.abs(g["dw_router"]).max() < 1e-11
    np.testing.assert_allclose(g["w"], 2.5)


def test_backward_expert_rows_subset_matches_full():
    """Requested rows of a weight gradient equal the same rows of the whole matrix."""
    p = _problem(seed=8, T=10, H=16, I=24, E=4, k=2)
    ex = oracle.Experts(p["w_gate"], p["w_up"], p["w_down"], gate=oracle.GATE_GELU)
    g = oracle.backward(p["x"], p["w_r"], None, ex, 2, oracle.SOFTMAX, True, 1.0, p["dout"])
    e = int(g["ids"][0, 0])
    rows = np.array([5, 0, 13])
    for which, name in ((oracle.BWD_GATE, "dw_gate"), (oracle.BWD_UP, "dw_up"), (oracle.BWD_DOWN, "dw_down")):
        sub = oracle.bwd_expert_rows(ex, which, e, rows, p["x"], g["ids"], g["w"], p["dout"])
        np.testing.assert_array_equal(sub, g[name][e][rows])
