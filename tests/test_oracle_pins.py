"""Pins of the fp64 oracle against things other than itself.

Each test checks one step of the oracle against a closed form, a library routine
on a special case, brute force on tiny inputs, an invariant the "Experts
backends" page fixes, or the hand-derived worked example under tests/golden.
They run on the CPU only (no GPU marker).
"""
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle
import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ codecs

def test_e4m3_decode_exhaustive_vs_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        got = oracle.e4m3_to_f64(c)
        if math.isnan(ref[c]):
            assert math.isnan(got), c
        else:
            assert got == ref[c], (c, got, ref[c])
    assert oracle.e4m3_to_f64(0x7E) == 448.0
    assert oracle.e4m3_to_f64(0x01) == 2.0 ** -9


# OCP Microscaling (MX) formats, FP4 E2M1 element table: magnitudes of the
# eight codes 0..7 (the definition of the format; code + 8 negates)
_E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_decode_exhaustive():
    for c in range(16):
        v = _E2M1_TABLE[c & 7] * (-1.0 if c & 8 else 1.0)
        got = oracle.e2m1_to_f64(c)
        assert got == v and math.copysign(1.0, got) == math.copysign(1.0, v), (c, got, v)
    # every E2M1 value is an E4M3 value (torch's conversion is exact for them)
    for v in _E2M1_TABLE:
        assert torch.tensor(v).to(torch.float8_e4m3fn).float().item() == v


def _fp4_dense(codes, scales):
    """float64 weights from E2M1 code pairs [E, R, C/2] and UE8M0 bytes [E, R, C/32]."""
    lo = codes & 15
    hi = codes >> 4
    c = np.stack([lo, hi], axis=-1).reshape(codes.shape[0], codes.shape[1], -1)
    tab = np.array(_E2M1_TABLE + [-v for v in _E2M1_TABLE])
    s = np.repeat(np.exp2(scales.astype(np.float64) - 127.0), 32, axis=2)
    return tab[c] * s


def test_fp4_experts_equal_dense_weights():
    # int8-packed E2M1 with one UE8M0 scale per (row, 32 K) equals the dense
    # fp64 weights built from the format table: pins the nibble order, the
    # code table and the scale indexing of both matrix shapes
    E, H, I = 3, 64, 96
    rng = np.random.default_rng(30)
    cg = rng.integers(0, 256, (E, I, H // 2), dtype=np.uint8)
    cu = rng.integers(0, 256, (E, I, H // 2), dtype=np.uint8)
    cd = rng.integers(0, 256, (E, H, I // 2), dtype=np.uint8)
    sg = rng.integers(118, 126, (E, I, H // 32), dtype=np.uint8)
    su = rng.integers(118, 126, (E, I, H // 32), dtype=np.uint8)
    sd = rng.integers(118, 126, (E, H, I // 32), dtype=np.uint8)
    fp4 = oracle.Experts(cg, cu, cd, sg, su, sd, oracle.SCALE_UE8M0, fp4=True)
    dg, du, dd = _fp4_dense(cg, sg), _fp4_dense(cu, su), _fp4_dense(cd, sd)
    assert np.array_equal(dg.astype(np.float32), dg) and np.array_equal(dd.astype(np.float32), dd)
    dense = oracle.Experts(dg.astype(np.float32), du.astype(np.float32), dd.astype(np.float32))
    x = rng.normal(0, 1, (5, H)).astype(np.float32)
    tok = np.array([0, 1, 2, 3, 4, 0])
    ex = np.array([0, 1, 2, 1, 0, 2])
    h1, y1 = fp4.pairs(x, tok, ex)
    h2, y2 = dense.pairs(x, tok, ex)
    assert np.array_equal(h1, h2) and np.array_equal(y1, y2)


def test_e8m0_decode_exhaustive_vs_torch():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    for c in range(256):
        got = oracle.e8m0_to_f64(c)
        if math.isnan(ref[c]):
            assert math.isnan(got)
        else:
            assert got == ref[c], (c, got, ref[c])


def test_bf16_decode_vs_torch():
    bits = torch.arange(0, 65536, 7, dtype=torch.int32)
    ref = bits.to(torch.int16).view(torch.bfloat16).to(torch.float64).numpy()
    for i, b in enumerate(bits.tolist()):
        got = oracle.bf16_to_f64(b)
        assert (math.isnan(got) and math.isnan(ref[i])) or got == ref[i], b


def test_e4m3_encode_rne_vs_torch():
    rng = np.random.default_rng(1)
    vals = [rng.normal(0, 100, 2000), rng.uniform(-2.0 ** -6, 2.0 ** -6, 500),
            rng.uniform(-448, 448, 1000)]
    # exact midpoints between neighbouring codes exercise ties-to-even
    finite = [oracle.e4m3_to_f64(c) for c in range(0x7F)]
    mids = [(finite[c] + finite[c + 1]) / 2 for c in range(0x7E)]
    vals.append(np.array(mids))
    vals.append(-np.array(mids))
    v = np.concatenate(vals).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for x, r in zip(v.tolist(), ref.tolist()):
        got = oracle.e4m3_encode(x)
        if r == 0x80:  # torch keeps the sign of a negative value that rounds to zero
            r = 0
        assert got == r, (x, got, r)


def test_e4m3_encode_saturates():
    assert oracle.e4m3_encode(448.0) == 0x7E
    assert oracle.e4m3_encode(463.9) == 0x7E
    assert oracle.e4m3_encode(500.0) == 0x7E
    assert oracle.e4m3_encode(1e30) == 0x7E
    assert oracle.e4m3_encode(-1e30) == 0xFE


# --------------------------------------------------------- activation quant

def test_quant_group_amax_maps_to_448():
    rng = np.random.default_rng(2)
    v = rng.normal(0, 3, 128)
    v[17] = -9.75
    deq, codes, s = oracle.quant_group(v)
    assert s == np.float32(9.75 / 448.0)
    assert codes[17] == 0xFE  # -448
    assert abs(deq[17] - (-448.0 * s)) == 0


def test_quant_group_zero_group():
    deq, codes, s = oracle.quant_group(np.zeros(128))
    assert s == 1.0 and not codes.any() and not deq.any()


def test_quant_group_error_bound():
    rng = np.random.default_rng(3)
    for _ in range(20):
        v = rng.normal(0, rng.uniform(0.01, 10), 128)
        deq, codes, s = oracle.quant_group(v)
        r = v / s
        normal = np.abs(r) >= 2.0 ** -6
        # half an e4m3 ulp: 2^-4 relative in the normal range, 2^-10 absolute below it
        assert np.all(np.abs(deq - v)[normal] <= np.abs(v)[normal] * 2.0 ** -4 * (1 + 1e-6) + 1e-300)
        assert np.all(np.abs(deq - v)[~normal] <= s * 2.0 ** -10 * (1 + 1e-6))


def test_quant_group_roundtrip_codes():
    # a group whose amax is 448 has scale 1, so every e4m3 value maps to its own code
    vals = np.array([oracle.e4m3_to_f64(c) for c in list(range(0x7F)) + list(range(0x80, 0xFF))])
    for start in range(0, vals.size, 127):
        g = np.concatenate([vals[start:start + 127], [448.0]])
        deq, codes, s = oracle.quant_group(g)
        assert s == 1.0
        assert np.array_equal(deq, g)


def test_quant_rows_matches_groups():
    rng = np.random.default_rng(4)
    x = rng.normal(0, 1, (3, 256)).astype(np.float32)
    codes, scales = oracle.quant_rows(x, 128)
    for r in range(3):
        for g in range(2):
            _, c, s = oracle.quant_group(x[r, g * 128:(g + 1) * 128].astype(np.float64))
            assert np.array_equal(c, codes[r, g * 128:(g + 1) * 128]) and s == scales[r, g]


# ------------------------------------------------------------------ routing

def _tiny_router(T=32, H=16, E=8, seed=0, snap=True):
    rng = np.random.default_rng(seed)
    x = rng.normal(0, 1, (T, H))
    w = rng.normal(0, 0.3, (E, H))
    if snap:
        x = np.round(x * 16) / 16
        w = np.round(w * 4096) / 4096
    return x.astype(np.float32), w.astype(np.float32)


@pytest.mark.parametrize("score", [oracle.SOFTMAX, oracle.SIGMOID])
def test_route_brute_force_topk(score):
    x, w = _tiny_router(T=40, H=16, E=8)
    bias = np.linspace(-0.5, 0.5, 8).astype(np.float32)
    ids, wt, keys = oracle.route(x, w, bias, 3, score, False, 1.0, want_keys=True)
    ref_keys = x.astype(np.float64) @ w.astype(np.float64).T + bias.astype(np.float64)
    assert np.array_equal(keys, ref_keys)  # exact on these grids
    for t in range(x.shape[0]):
        order = np.lexsort((np.arange(8), -ref_keys[t]))  # key desc, then index asc
        assert list(ids[t]) == list(order[:3])


def test_route_ties_lowest_index():
    x, w = _tiny_router(T=16, H=8, E=6)
    w[3] = w[1]
    w[5] = w[1]
    w[0] = w[1]
    ids, _, keys = oracle.route(x, w, None, 4, oracle.SOFTMAX, True, 1.0, want_keys=True)
    for t in range(16):
        sel = list(ids[t])
        # equal keys appear in ascending expert order
        for a in range(4):
            for b in range(a + 1, 4):
                if keys[t, sel[a]] == keys[t, sel[b]]:
                    assert sel[a] < sel[b]
    # all experts identical -> selection is 0..k-1
    w[:] = w[2]
    ids, _ = oracle.route(x, w, None, 4, oracle.SOFTMAX, True, 1.0)
    assert np.array_equal(ids, np.tile(np.arange(4), (16, 1)))


def test_route_nan_keys_rank_as_neg_inf():
    # reading: a NaN key (from a NaN among the inputs) ranks as -inf, ties to
    # the lowest index; checked against a brute-force lexsort of the keys with
    # NaN replaced by -inf
    x, w = _tiny_router(T=12, H=8, E=6, seed=9)
    w[2, 3] = np.nan          # expert 2's key is NaN for every token
    x[5, 1] = np.nan          # every key of token 5 is NaN
    for score in (oracle.SOFTMAX, oracle.SIGMOID):
        ids, wt, keys = oracle.route(x, w, None, 4, score, False, 1.0, want_keys=True)
        ref = x.astype(np.float64) @ w.astype(np.float64).T
        ref = np.where(np.isnan(ref), -np.inf, ref)
        assert np.array_equal(keys, ref)
        for t in range(12):
            order = np.lexsort((np.arange(6), -ref[t]))
            assert list(ids[t]) == list(order[:4]), (score, t)
        assert list(ids[5]) == [0, 1, 2, 3]
        assert 2 not in ids[np.arange(12) != 5]
        assert np.isfinite(wt[np.arange(12) != 5]).all()


def test_route_k_equals_E_softmax_sums_to_one():
    x, w = _tiny_router(T=20, H=8, E=5)
    ids, wt, keys = oracle.route(x, w, None, 5, oracle.SOFTMAX, False, 1.0, want_keys=True)
    for t in range(20):
        assert sorted(ids[t]) == list(range(5))
        assert np.all(np.diff(keys[t, ids[t]]) <= 0)
    assert np.allclose(wt.sum(1), 1.0, rtol=0, atol=1e-14)


def test_route_two_experts_closed_form():
    x, w = _tiny_router(T=30, H=8, E=2, seed=5)
    ids, wt, keys = oracle.route(x, w, None, 2, oracle.SOFTMAX, False, 1.0, want_keys=True)
    for t in range(30):
        a, b = ids[t]
        assert abs(wt[t, 0] - expit(keys[t, a] - keys[t, b])) < 1e-15
        assert abs(wt[t, 1] - expit(keys[t, b] - keys[t, a])) < 1e-15


def test_route_weight_invariants():
    x, w = _tiny_router(T=50, H=16, E=8, seed=6)
    bias = np.linspace(-1, 1, 8).astype(np.float32)
    # softmax + renorm: weights sum to 1 and keep the ratios of exp(key)
    ids, wt, keys = oracle.route(x, w, bias, 3, oracle.SOFTMAX, True, 1.0, want_keys=True)
    assert np.allclose(wt.sum(1), 1.0, atol=1e-14)
    for t in range(50):
        assert abs(wt[t, 0] / wt[t, 1] - math.exp(keys[t, ids[t, 0]] - keys[t, ids[t, 1]])) < 1e-12
    # softmax, no renorm: the top-k share of the full softmax (<= 1)
    ids, wt, keys = oracle.route(x, w, bias, 3, oracle.SOFTMAX, False, 1.0, want_keys=True)
    full = np.exp(keys - keys.max(1, keepdims=True))
    full /= full.sum(1, keepdims=True)
    assert np.allclose(wt, np.take_along_axis(full, ids.astype(np.int64), 1), rtol=1e-13, atol=0)
    assert np.all(wt.sum(1) <= 1 + 1e-15)
    # sigmoid + renorm x 2.5: sums to the routed scale
    ids, wt, keys = oracle.route(x, w, bias, 3, oracle.SIGMOID, True, 2.5, want_keys=True)
    assert np.allclose(wt.sum(1), 2.5, atol=1e-13)
    # sigmoid, no renorm: the logistic function of the key (library routine)
    ids, wt, keys = oracle.route(x, w, bias, 3, oracle.SIGMOID, False, 1.0, want_keys=True)
    assert np.allclose(wt, expit(np.take_along_axis(keys, ids.astype(np.int64), 1)), rtol=1e-14)


def test_route_bf16_inputs_decode_exactly():
    s = synthetic.spec("qwen_prefill", T=16, H=256, E=12)
    L = synthetic.make_layer(s, seed=3)
    ids, wt, keys = oracle.route(L["x"], L["w_router"], L["router_bias"], 4, oracle.SOFTMAX, False,
                                 1.0, want_keys=True)
    ref = (L["x"].double() @ L["w_router"].double().T + L["router_bias"].double()).numpy()
    assert np.array_equal(keys, ref)


# -------------------------------------------------------------- permutation

def test_permute_against_library_routines():
    rng = np.random.default_rng(7)
    for T, k, E in [(1, 1, 1), (64, 2, 8), (100, 4, 60), (33, 8, 256), (5, 3, 3)]:
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        counts, offsets, perm, inv = oracle.permute(ids, E)
        assert counts.sum() == T * k
        assert np.array_equal(counts, np.bincount(ids.ravel(), minlength=E))
        assert offsets[0] == 0 and offsets[-1] == T * k
        assert np.array_equal(offsets[1:], np.cumsum(counts))
        assert np.array_equal(perm, np.argsort(ids.ravel(), kind="stable"))
        assert np.array_equal(inv[perm], np.arange(T * k))
        assert np.array_equal(perm[inv], np.arange(T * k))
        flat = ids.ravel()
        for e in range(E):
            assert np.all(flat[perm[offsets[e]:offsets[e + 1]]] == e)


def test_permute_empty_experts_and_one_hot():
    ids = np.full((10, 1), 3, dtype=np.int32)
    counts, offsets, perm, inv = oracle.permute(ids, 5)
    assert list(counts) == [0, 0, 0, 10, 0]
    assert list(offsets) == [0, 0, 0, 0, 10, 10]
    assert np.array_equal(perm, np.arange(10))


# ------------------------------------------------------------------ experts

def _dense_mlp(x, wg, wu, wd):
    g = x @ wg.T
    u = x @ wu.T
    return (g * expit(g) * u) @ wd.T


def _rand_experts(E, H, I, seed):
    rng = np.random.default_rng(seed)
    wg = rng.normal(0, 1 / math.sqrt(H), (E, I, H)).astype(np.float32)
    wu = rng.normal(0, 1 / math.sqrt(H), (E, I, H)).astype(np.float32)
    wd = rng.normal(0, 1 / math.sqrt(I), (E, H, I)).astype(np.float32)
    return wg, wu, wd


@pytest.mark.parametrize("score,renorm,scale,wexp", [
    (oracle.SOFTMAX, True, 1.0, 1.0), (oracle.SOFTMAX, False, 1.0, 1.0),
    (oracle.SIGMOID, True, 2.5, 2.5)])
def test_single_expert_is_dense_gated_mlp(score, renorm, scale, wexp):
    H, I, T = 32, 48, 12
    wg, wu, wd = _rand_experts(1, H, I, 8)
    x, wr = _tiny_router(T=T, H=H, E=1, seed=9)
    ex = oracle.Experts(wg, wu, wd)
    ids, w, counts, offsets, perm, inv, out = oracle.forward(x, wr, None, ex, 1, score, renorm, scale)
    assert np.all(ids == 0) and np.allclose(w, wexp, atol=1e-15)
    ref = wexp * _dense_mlp(x.astype(np.float64), wg[0].astype(np.float64), wu[0].astype(np.float64),
                            wd[0].astype(np.float64))
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_sigmoid_no_renorm_single_expert_weight():
    H, I, T = 16, 16, 6
    wg, wu, wd = _rand_experts(1, H, I, 10)
    x, wr = _tiny_router(T=T, H=H, E=1, seed=11)
    ex = oracle.Experts(wg, wu, wd)
    ids, w, *_ , out = oracle.forward(x, wr, None, ex, 1, oracle.SIGMOID, False, 1.0)
    key = x.astype(np.float64) @ wr.astype(np.float64).T
    assert np.allclose(w, expit(key), rtol=1e-14)
    ref = expit(key) * _dense_mlp(x.astype(np.float64), wg[0].astype(np.float64),
                                  wu[0].astype(np.float64), wd[0].astype(np.float64))
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_identical_experts_independent_of_routing():
    H, I, E, T, k = 16, 24, 6, 20, 3
    wg, wu, wd = _rand_experts(1, H, I, 12)
    ex = oracle.Experts(np.repeat(wg, E, 0), np.repeat(wu, E, 0), np.repeat(wd, E, 0))
    x, wr = _tiny_router(T=T, H=H, E=E, seed=13)
    ids, w, *_, out = oracle.forward(x, wr, None, ex, k, oracle.SIGMOID, False, 1.0)
    ref = w.sum(1, keepdims=True) * _dense_mlp(x.astype(np.float64), wg[0].astype(np.float64),
                                                wu[0].astype(np.float64), wd[0].astype(np.float64))
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_zero_up_projection_gives_zero():
    H, I, E = 16, 16, 4
    wg, wu, wd = _rand_experts(E, H, I, 14)
    ex = oracle.Experts(wg, np.zeros_like(wu), wd)
    x, wr = _tiny_router(T=8, H=H, E=E, seed=15)
    *_, out = oracle.forward(x, wr, None, ex, 2, oracle.SOFTMAX, True, 1.0)
    assert not out.any()


def test_linear_in_down_projection_and_gate_is_silu_branch():
    H, I, E = 16, 16, 4
    wg, wu, wd = _rand_experts(E, H, I, 16)
    x, wr = _tiny_router(T=8, H=H, E=E, seed=17)
    *_, out1 = oracle.forward(x, wr, None, oracle.Experts(wg, wu, wd), 2, oracle.SOFTMAX, True, 1.0)
    *_, out2 = oracle.forward(x, wr, None, oracle.Experts(wg, wu, 2 * wd), 2, oracle.SOFTMAX, True, 1.0)
    assert np.array_equal(out2, 2 * out1)
    # silu sits on the gate branch: doubling W_up doubles the output, doubling W_gate does not
    *_, out3 = oracle.forward(x, wr, None, oracle.Experts(wg, 2 * wu, wd), 2, oracle.SOFTMAX, True, 1.0)
    assert np.array_equal(out3, 2 * out1)
    *_, out4 = oracle.forward(x, wr, None, oracle.Experts(2 * wg, wu, wd), 2, oracle.SOFTMAX, True, 1.0)
    assert not np.allclose(out4, 2 * out1)


# ------------------------------------------------- GeGLU / ReGLU gates
# Section "SonicMoE" of "Experts backends" lists gated activations silu, gelu
# and relu (SwiGLU / GeGLU / ReGLU); gelu is read as the exact x * Phi(x).

_GATES = {oracle.GATE_GELU: lambda g: torch.nn.functional.gelu(torch.from_numpy(g)).numpy(),
          oracle.GATE_RELU: lambda g: np.maximum(g, 0.0)}


@pytest.mark.parametrize("gate", [oracle.GATE_GELU, oracle.GATE_RELU])
def test_single_expert_is_dense_glu_variant(gate):
    # k = 1, E = 1: the layer is one dense gated MLP; torch's float64 gelu
    # (exact form) and numpy's maximum are independent implementations
    H, I, T = 32, 48, 12
    wg, wu, wd = _rand_experts(1, H, I, 18)
    x, wr = _tiny_router(T=T, H=H, E=1, seed=19)
    ex = oracle.Experts(wg, wu, wd, gate=gate)
    *_, out = oracle.forward(x, wr, None, ex, 1, oracle.SOFTMAX, True, 1.0)
    xd = x.astype(np.float64)
    g = xd @ wg[0].astype(np.float64).T
    u = xd @ wu[0].astype(np.float64).T
    ref = (_GATES[gate](g) * u) @ wd[0].astype(np.float64).T
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("gate", [oracle.GATE_SILU, oracle.GATE_GELU, oracle.GATE_RELU])
def test_gate_odd_part_is_identity(gate):
    # act(g) - act(-g) = g for silu, gelu (Phi(g) + Phi(-g) = 1) and relu, so
    # negating W_gate changes the layer by exactly W_down (g * u): a closed
    # form that catches a dropped factor or a wrong sign in any of the gates
    H, I, E, T = 16, 24, 3, 10
    wg, wu, wd = _rand_experts(E, H, I, 20)
    x, wr = _tiny_router(T=T, H=H, E=E, seed=21)
    ids, w, *_, out_p = oracle.forward(x, wr, None, oracle.Experts(wg, wu, wd, gate=gate), 2,
                                       oracle.SOFTMAX, True, 1.0)
    *_, out_n = oracle.forward(x, wr, None, oracle.Experts(-wg, wu, wd, gate=gate), 2,
                               oracle.SOFTMAX, True, 1.0)
    xd = x.astype(np.float64)
    ref = np.zeros_like(out_p)
    for t in range(T):
        for i in range(2):
            e = ids[t, i]
            g = wg[e].astype(np.float64) @ xd[t]
            u = wu[e].astype(np.float64) @ xd[t]
            ref[t] += w[t, i] * (wd[e].astype(np.float64) @ (g * u))
    assert np.allclose(out_p - out_n, ref, rtol=1e-10, atol=1e-12)


def test_gelu_gate_textbook_values():
    # Phi(1) = 0.8413447460685429, Phi(-1) = 0.15865525393145707 and
    # Phi(2) = 0.9772498680518208 (standard normal table): with H = I = 1 and
    # all three weights 1, g = u = x and the layer returns gelu(x) * x =
    # x^2 Phi(x)
    x = np.array([[1.0], [-1.0], [0.0], [2.0]], dtype=np.float32)
    one = np.ones((1, 1, 1), dtype=np.float32)
    ex = oracle.Experts(one, one, one, gate=oracle.GATE_GELU)
    h, y = ex.pairs(x, np.arange(4), [0, 0, 0, 0])
    assert abs(y[0, 0] - 0.8413447460685429) < 1e-15
    assert abs(y[1, 0] - 0.15865525393145707) < 1e-15
    assert y[2, 0] == 0.0
    assert abs(y[3, 0] - 4.0 * 0.9772498680518208) < 1e-14
    exr = oracle.Experts(one, one, one, gate=oracle.GATE_RELU)
    _, yr = exr.pairs(x, np.arange(4), [0, 0, 0, 0])
    assert list(yr[:, 0]) == [1.0, 0.0, 0.0, 4.0]


def _load_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, rhs = line.split("=", 1)
            vals[key.strip()] = np.array([float(v) for v in rhs.split()])
    return vals


def test_worked_example_golden():
    g = _load_golden("worked_example_two_experts.txt")
    x = g["x"].reshape(1, 2).astype(np.float32)
    wr = g["w_router"].reshape(2, 2).astype(np.float32)
    wg = g["w_gate"].reshape(2, 1, 2).astype(np.float32)
    wu = g["w_up"].reshape(2, 1, 2).astype(np.float32)
    wd = g["w_down"].reshape(2, 2, 1).astype(np.float32)
    ex = oracle.Experts(wg, wu, wd)
    ids, w, counts, offsets, perm, inv, out = oracle.forward(x, wr, None, ex, 2, oracle.SOFTMAX,
                                                             False, 1.0)
    assert list(ids[0]) == list(g["ids"].astype(int))
    assert np.allclose(w[0], g["weights"], rtol=1e-15, atol=0)
    h, y = ex.pairs(x, [0, 0], [0, 1])
    assert np.allclose(y[0], g["y_expert0"], rtol=1e-15) and np.allclose(y[1], g["y_expert1"], rtol=1e-15)
    assert np.allclose(h[:, 0], [g["h_expert0"][0], g["h_expert1"][0]], rtol=1e-15)
    assert np.allclose(out[0], g["out"], rtol=1e-14, atol=0)
    assert list(counts) == [1, 1] and list(perm) == [1, 0]


def test_token_permutation_equivariance():
    s = synthetic.spec("tiny", T=24)
    L = synthetic.make_layer(s, seed=1)
    ex = oracle.Experts(L["w_gate"], L["w_up"], L["w_down"])
    ids, w, *_, out = oracle.forward(L["x"], L["w_router"], None, ex, 2, oracle.SOFTMAX, True, 1.0)
    p = np.random.default_rng(0).permutation(24)
    ids2, w2, *_, out2 = oracle.forward(L["x"][p], L["w_router"], None, ex, 2, oracle.SOFTMAX, True, 1.0)
    assert np.array_equal(ids2, ids[p]) and np.array_equal(w2, w[p])
    assert np.array_equal(out2, out[p])


def test_combine_k1_is_unpermuted_expert_output():
    s = synthetic.spec("tiny", T=16)
    L = synthetic.make_layer(s, seed=2)
    ex = oracle.Experts(L["w_gate"], L["w_up"], L["w_down"])
    ids, w, counts, offsets, perm, inv, out = oracle.forward(L["x"], L["w_router"], None, ex, 1,
                                                             oracle.SOFTMAX, True, 1.0)
    assert np.all(w == 1.0)
    _, y = ex.pairs(L["x"], np.arange(16), ids[:, 0])
    assert np.array_equal(out, y)


# --------------------------------------------------------------- fp8 experts

def _e4m3_exact_weights(E, rows, cols, seed):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 0x7F, (E, rows, cols)).astype(np.uint8)
    codes |= (rng.integers(0, 2, codes.shape) << 7).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x30
    vals = np.vectorize(oracle.e4m3_to_f64)(codes).astype(np.float32)
    return codes, vals


@pytest.mark.parametrize("fmt", [oracle.SCALE_F32, oracle.SCALE_UE8M0])
def test_fp8_unit_scales_equal_dense(fmt):
    E, H, I = 2, 128, 128
    cg, vg = _e4m3_exact_weights(E, I, H, 20)
    cu, vu = _e4m3_exact_weights(E, I, H, 21)
    cd, vd = _e4m3_exact_weights(E, H, I, 22)
    one = np.ones((E, 1, 1), np.float32) if fmt == oracle.SCALE_F32 else np.full((E, 1, 1), 127, np.uint8)
    fp8 = oracle.Experts(cg, cu, cd, one, one, one, fmt, 128, act_fp8=False)
    dense = oracle.Experts(vg, vu, vd)
    x = (np.random.default_rng(23).normal(0, 0.05, (4, H))).astype(np.float32)
    h1, y1 = fp8.pairs(x, np.arange(4), [0, 1, 0, 1])
    h2, y2 = dense.pairs(x, np.arange(4), [0, 1, 0, 1])
    assert np.array_equal(y1, y2) and np.array_equal(h1, h2)


def test_fp8_activation_quant_sits_on_x_and_on_a():
    E, H, I = 1, 128, 128
    cg, vg = _e4m3_exact_weights(E, I, H, 24)
    cu, vu = _e4m3_exact_weights(E, I, H, 25)
    # W_down = identity (code 0x38 = 1.0), so y equals the quantized SwiGLU output
    cd = np.zeros((E, H, I), np.uint8)
    cd[0][np.arange(H), np.arange(I)] = 0x38
    one = np.ones((E, 1, 1), np.float32) * 0.01
    onedown = np.ones((E, 1, 1), np.float32)
    fp8 = oracle.Experts(cg, cu, cd, one, one, onedown, oracle.SCALE_F32, 128, act_fp8=True)
    x = np.random.default_rng(26).normal(0, 1, (1, H)).astype(np.float32)
    h, y = fp8.pairs(x, [0], [0])
    # composition of pinned pieces: quantize x, dense gated MLP in fp64, quantize a
    xq, _, _ = oracle.quant_group(x[0].astype(np.float64))
    g = xq @ (vg[0].astype(np.float64) * 0.01).T
    u = xq @ (vu[0].astype(np.float64) * 0.01).T
    aq, _, _ = oracle.quant_group(g * expit(g) * u)
    assert np.allclose(h[0], aq, rtol=1e-13, atol=1e-300)
    assert np.allclose(y[0], aq, rtol=1e-13, atol=1e-300)


@pytest.mark.parametrize("fmt", [oracle.SCALE_F32, oracle.SCALE_UE8M0])
def test_fp8_block_scales_index_the_right_block(fmt):
    E, H, I = 2, 256, 384
    cg, _ = _e4m3_exact_weights(E, I, H, 27)
    cu, _ = _e4m3_exact_weights(E, I, H, 28)
    cd, _ = _e4m3_exact_weights(E, H, I, 29)
    rng = np.random.default_rng(30)
    if fmt == oracle.SCALE_F32:
        sg = (rng.uniform(0.5, 2, (E, I // 128, H // 128)) * 1e-3).astype(np.float32)
        su = (rng.uniform(0.5, 2, (E, I // 128, H // 128)) * 1e-3).astype(np.float32)
        sd = (rng.uniform(0.5, 2, (E, H // 128, I // 128)) * 1e-3).astype(np.float32)
    else:
        sg = rng.integers(115, 119, (E, I // 128, H // 128)).astype(np.uint8)
        su = rng.integers(115, 119, (E, I // 128, H // 128)).astype(np.uint8)
        sd = rng.integers(115, 119, (E, H // 128, I // 128)).astype(np.uint8)
    x = rng.normal(0, 1, (2, H)).astype(np.float32)
    base = oracle.Experts(cg, cu, cd, sg, su, sd, fmt, 128, act_fp8=False)
    _, y = base.pairs(x, [0, 1], [1, 1])
    # double one W_down block (output block 1, input block 2) of expert 1
    sd2 = sd.copy()
    if fmt == oracle.SCALE_F32:
        sd2[1, 1, 2] *= 2
    else:
        sd2[1, 1, 2] += 1
    _, y2 = oracle.Experts(cg, cu, cd, sg, su, sd2, fmt, 128, act_fp8=False).pairs(x, [0, 1], [1, 1])
    diff = y2 - y
    # only output rows 128..255 move, by that block's contribution
    assert not diff[:, :128].any()
    h, _ = base.pairs(x, [0, 1], [1, 1])
    if fmt == oracle.SCALE_F32:
        sblk = float(sd[1, 1, 2])
    else:
        sblk = 2.0 ** (int(sd[1, 1, 2]) - 127)
    wblk = np.vectorize(oracle.e4m3_to_f64)(cd[1, 128:256, 256:384]) * sblk
    contrib = h[:, 256:384] @ wblk.T
    assert np.allclose(diff[:, 128:], contrib, rtol=1e-12, atol=1e-14)
