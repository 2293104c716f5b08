"""Routing on inputs off the exactness grids (a diagnostic of the router).

The other parity tests snap x, W_r and the bias to grids on which every fp32
partial sum of a logit is exact, so that the HIP router's ids are well posed
and compared bit for bit.  Here they are drawn from the same distributions
without snapping.  A logit then depends on the order of its additions: every
bf16 x bf16 product is exact in fp32, and summing the H products and the bias
in any order in fp32 is off by at most

    delta[t, e] = gamma_H * (sum_h |x[t,h] w_r[e,h]| + |b[e]|),
    gamma_n = n u / (1 - n u),  u = 2^-24

(the classical bound for n roundings of a recursive sum).  If every gap
between neighbours among a token's k+1 largest exact keys exceeds twice the
token's largest delta, no such error can change its ordered top-k: the HIP ids
must then equal the oracle's exactly.  On the other ("ambiguous") tokens any
k distinct valid experts are accepted.  On the unambiguous tokens the routing
weights must agree within the same bound and the layer output within the bf16
tolerance.
"""
import numpy as np
import pytest
import torch

import mixture_experts_routed_softmax_amd as moe
import synthetic
from moe_cases import desc_for, host, oracle_experts, oracle_route, row_rel_err, run_forward, tol_of
import oracle

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _ambiguous(hl, keys, k):
    """(ambiguous token mask, per-token largest delta) from the fp64 keys."""
    x = hl["x"].double().numpy()
    w = hl["w_router"].double().numpy()
    b = np.zeros(w.shape[0]) if hl["router_bias"] is None else np.abs(hl["router_bias"].double().numpy())
    H = x.shape[1]
    gamma = H * U / (1 - H * U)
    delta = gamma * (np.abs(x) @ np.abs(w).T + b)          # [T, E]
    dmax = delta.max(axis=1)
    E = keys.shape[1]
    order = np.lexsort((np.broadcast_to(np.arange(E), keys.shape), -keys), axis=1)
    top = np.take_along_axis(keys, order[:, :min(k + 1, E)], axis=1)
    gaps = top[:, :-1] - top[:, 1:]
    return (gaps <= 2 * dmax[:, None]).any(axis=1), dmax


def _check_ids(s, hl, got_ids, got_w):
    ids_o, w_o, keys = oracle.route(hl["x"], hl["w_router"], hl["router_bias"], s.k,
                                    oracle.SOFTMAX if s.score == "softmax" else oracle.SIGMOID,
                                    s.renormalize, s.routed_scale, want_keys=True)
    amb, dmax = _ambiguous(hl, keys, s.k)
    agree = ~amb
    diff = (got_ids != ids_o).any(axis=1)
    print("%s T=%d: %d ambiguous tokens, %d differ from the oracle (all ambiguous: %s)"
          % (s.name, s.T, int(amb.sum()), int(diff.sum()), bool((diff <= amb).all())))
    assert not (diff & agree).any(), "ids differ on %d unambiguous tokens" % int((diff & agree).sum())
    # every token: k distinct experts in range
    assert ((got_ids >= 0) & (got_ids < s.E)).all()
    srt = np.sort(got_ids, axis=1)
    assert (srt[:, 1:] != srt[:, :-1]).all()
    # weights on the unambiguous tokens, within the bound's first-order effect
    rtol = 4 * dmax[agree][:, None] + 1e-5
    err = np.abs(got_w[agree] - w_o[agree]) / np.abs(w_o[agree])
    assert (err <= rtol).all(), "routing weights off by %.3e" % float(err.max())
    return ids_o, w_o, agree


@pytest.mark.parametrize("name,T", [("qwen_prefill", 4096), ("qwen_decode", 8), ("qwen_decode", 64)])
def test_unsnapped_forward(name, T):
    s = synthetic.spec(name, T=T)
    L = synthetic.make_layer(s, seed=40 + T, device="cuda", snap=False)
    out, ids, w, counts = run_forward(s, L, layout="packed")
    hl = host(L)
    del L
    got_ids = ids.cpu().numpy()
    ids_o, w_o, agree = _check_ids(s, hl, got_ids, w.cpu().numpy().astype(np.float64))
    assert np.array_equal(counts.cpu().numpy(), np.bincount(got_ids.ravel(), minlength=s.E))
    toks = np.flatnonzero(agree)
    rng = np.random.default_rng(T)
    if toks.size > 96:
        toks = np.sort(rng.choice(toks, 96, replace=False))
    ref = oracle_experts(s, hl).combine(hl["x"], ids_o, w_o, toks)
    err = row_rel_err(out[torch.from_numpy(toks).cuda()].cpu().float().numpy(), ref)
    print("output: %d unambiguous tokens checked, max row rel err %.3e" % (toks.size, err))
    assert err <= tol_of(s)


def test_unsnapped_route_dsv3():
    s = synthetic.spec("dsv3_bf16")
    L = synthetic.make_layer(s, seed=44, device="cuda", snap=False, experts=False)
    d = desc_for(s, layout="packed")
    ids = torch.empty(s.T, s.k, dtype=torch.int32, device="cuda")
    w = torch.empty(s.T, s.k, dtype=torch.float32, device="cuda")
    moe.moe_route_topk(d, L["x"], L["w_router"], L["router_bias"], ids, w, moe.workspace(d, moe.MOE_OP_ROUTE))
    torch.cuda.synchronize()
    _check_ids(s, host(L), ids.cpu().numpy(), w.cpu().numpy().astype(np.float64))
