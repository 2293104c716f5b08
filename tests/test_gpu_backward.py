"""GPU parity of moe_backward against the fp64 oracle's backward.

Every gradient of the layer (dx, dW_router, dbias, dW_gate, dW_up, dW_down)
is compared with the oracle on the same seeded inputs, row by row, with the
bf16 tolerance of the forward (per-row relative L2 <= 2e-2): the backward
rounds the gated-activation gradients and the scaled activations to bf16
between its fp32-accumulating GEMMs, the same kind of rounding the forward
does to h.  Weight-gradient rows of experts that no token selected
must be exactly zero.  At the full Qwen-like prefill shape the oracle checks
sampled token rows of dx and sampled rows of the weight gradients of a few
experts.
"""
import numpy as np
import pytest
import torch

import mixture_experts_routed_softmax_amd as moe
import oracle
import synthetic
from moe_cases import desc_for, host, oracle_experts, row_rel_err, score_code

pytestmark = pytest.mark.gpu
TOL = 2e-2

# small layers that span several 128-row tiles, ragged tails and idle experts
SMALL = {
    "dsv3_like": dict(base="dsv3_bf16", T=100, H=256, I=384, E=16, k=4),
    "qwen_like": dict(base="qwen_prefill", T=300, H=256, I=256, E=12, k=4),
    "idle_experts": dict(base="qwen_prefill", T=9, H=128, I=128, E=40, k=2),
    "one_token": dict(base="dsv3_bf16", T=1, H=128, I=256, E=8, k=3),
    "many_rows": dict(base="dsv3_bf16", T=700, H=384, I=128, E=6, k=2),
    "max_experts_topk": dict(base="dsv3_bf16", T=24, H=128, I=128, E=256, k=32),
}


def _spec(case, gate="silu"):
    c = dict(SMALL[case])
    return synthetic.spec(c.pop("base"), gate=gate, **c)


def _run_gpu(s, L, dout):
    d = desc_for(s)
    dev = L["x"].device
    dx = torch.empty_like(L["x"])
    dwr = torch.empty_like(L["w_router"])
    db = torch.empty(s.E, dtype=torch.float32, device=dev)
    dwg = torch.empty_like(L["w_gate"])
    dwu = torch.empty_like(L["w_up"])
    dwd = torch.empty_like(L["w_down"])
    ws = moe.workspace(d, moe.MOE_OP_BACKWARD, dev)
    moe.moe_backward(d, L["x"], L["w_router"], L["router_bias"], L["w_gate"], L["w_up"], L["w_down"], dout,
                     dx, dwr, db, dwg, dwu, dwd, ws)
    torch.cuda.synchronize()
    return dict(dx=dx, dw_router=dwr, dbias=db, dw_gate=dwg, dw_up=dwu, dw_down=dwd)


def _f64(t):
    return t.detach().cpu().double().numpy()


def _compare_full(s, got, ref, tol=TOL):
    assert row_rel_err(_f64(got["dx"]), ref["dx"]) <= tol, "dx"
    used = np.zeros(s.E, bool)
    used[np.unique(ref["ids"])] = True
    for name in ("dw_gate", "dw_up", "dw_down"):
        g = _f64(got[name])
        for e in range(s.E):
            if used[e]:
                err = row_rel_err(g[e], ref[name][e])
                assert err <= tol, (name, e, err)
            else:
                assert (g[e] == 0).all(), (name, e, "idle expert must get zeros")
    assert row_rel_err(_f64(got["dw_router"]), ref["dw_router"]) <= tol, "dw_router"
    db = _f64(got["dbias"])
    if s.bias != "none":
        assert np.linalg.norm(db - ref["dbias"]) <= tol * max(np.linalg.norm(ref["dbias"]), 1e-30), "dbias"


@pytest.mark.parametrize("case", list(SMALL))
def test_backward_small(case):
    s = _spec(case)
    print("case", case, s, flush=True)
    L = synthetic.make_layer(s, seed=1, device="cuda")
    dout = synthetic.make_grad_out(s, seed=1, device="cuda")
    got = _run_gpu(s, L, dout)
    hl = host(L)
    ref = oracle.backward(hl["x"], hl["w_router"], hl["router_bias"], oracle_experts(s, hl), s.k, score_code(s),
                          s.renormalize, s.routed_scale, dout.cpu().double().numpy())
    _compare_full(s, got, ref)


@pytest.mark.parametrize("gate", ["gelu", "relu"])
def test_backward_gated_variants(gate):
    s = _spec("qwen_like", gate=gate)
    L = synthetic.make_layer(s, seed=2, device="cuda")
    dout = synthetic.make_grad_out(s, seed=2, device="cuda")
    got = _run_gpu(s, L, dout)
    hl = host(L)
    ref = oracle.backward(hl["x"], hl["w_router"], hl["router_bias"], oracle_experts(s, hl), s.k, score_code(s),
                          s.renormalize, s.routed_scale, dout.cpu().double().numpy())
    _compare_full(s, got, ref)


def test_backward_is_deterministic():
    s = _spec("dsv3_like")
    L = synthetic.make_layer(s, seed=3, device="cuda")
    dout = synthetic.make_grad_out(s, seed=3, device="cuda")
    a = _run_gpu(s, L, dout)
    b = _run_gpu(s, L, dout)
    for k in a:
        assert torch.equal(a[k], b[k]), k


def _full_sampled(s, quantiles):
    """dx on sampled tokens and weight-gradient rows of experts picked by load
    quantile, at a full workload shape."""
    L = synthetic.make_layer(s, seed=0, device="cuda")
    dout = synthetic.make_grad_out(s, seed=0, device="cuda")
    got = _run_gpu(s, L, dout)
    hl = host(L)
    ex = oracle_experts(s, hl)
    dout64 = dout.cpu().double().numpy()
    ids, w, keys = oracle.route(hl["x"], hl["w_router"], hl["router_bias"], s.k, score_code(s), s.renormalize,
                                s.routed_scale, want_keys=True)
    rng = np.random.default_rng(0)
    tokens = np.concatenate([[0, s.T - 1], rng.choice(s.T, 6, replace=False)])
    dx, _, _ = oracle.bwd_tokens(ex, hl["x"], hl["w_router"], score_code(s), s.renormalize, s.routed_scale, keys,
                                 ids, w, dout64, tokens)
    assert row_rel_err(_f64(got["dx"])[tokens], dx) <= TOL
    counts = np.bincount(ids.ravel(), minlength=s.E)
    order = np.argsort(counts, kind="stable")
    live = order[np.nonzero(counts[order])[0]]
    for e in sorted({int(live[min(int(q * len(live)), len(live) - 1)]) for q in quantiles}):
        for which, name, nrows in ((oracle.BWD_GATE, "dw_gate", s.I), (oracle.BWD_UP, "dw_up", s.I),
                                   (oracle.BWD_DOWN, "dw_down", s.H)):
            rows = np.array([0, nrows - 1, int(rng.integers(nrows))])
            ref = oracle.bwd_expert_rows(ex, which, e, rows, hl["x"], ids, w, dout64)
            err = row_rel_err(_f64(got[name])[e][rows], ref)
            assert err <= TOL, (name, e, err)


def test_backward_qwen_prefill_full_sampled():
    """Full Qwen-like prefill shape (T=4096, 60 experts, k=4, softmax): the
    least-loaded, the median and the 75th-percentile expert."""
    _full_sampled(synthetic.spec("qwen_prefill"), (0.0, 0.5, 0.75))


def test_backward_dsv3_full_sampled():
    """Full DeepSeek-like shape (T=8192, H=7168, 256 experts, k=8, sigmoid,
    renormalised x2.5): the least-loaded and the median expert."""
    _full_sampled(synthetic.spec("dsv3_bf16"), (0.0, 0.5))


def test_backward_no_tokens_zero_fills():
    s = _spec("dsv3_like")
    L = synthetic.make_layer(s, seed=4, device="cuda")
    d = desc_for(s, T=0)
    outs = [torch.full_like(L[n], 7.0) for n in ("w_router", "w_gate", "w_up", "w_down")]
    db = torch.full((s.E,), 7.0, device="cuda")
    moe.moe_backward(d, L["x"][:0], L["w_router"], L["router_bias"], L["w_gate"], L["w_up"], L["w_down"],
                     L["x"][:0], L["x"][:0], outs[0], db, outs[1], outs[2], outs[3])
    torch.cuda.synchronize()
    for t in outs + [db]:
        assert (t == 0).all()
