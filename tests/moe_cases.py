"""Shared helpers of the GPU parity tests: descriptions from workload specs,
host copies for the oracle, row sampling and the error metric.

The error metric is the one the layer is judged by: for each token row,
||out_t - ref_t||_2 / ||ref_t||_2, and the maximum over the compared rows.
"""
from __future__ import annotations

import numpy as np
import torch

import mixture_experts_routed_softmax_amd as moe
import oracle
import synthetic

# fp4 experts quantize activations and h exactly as fp8 experts do (their
# weights are exact on both sides), so they share the fp8 tolerance
TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2, "fp4": 6e-2}


def tol_of(s: synthetic.LayerSpec) -> float:
    return TOL[s.experts]


def desc_for(s: synthetic.LayerSpec, T: int | None = None, path: str = "auto", y_dtype=None,
             layout: str = "rowmajor"):
    return moe.make_desc(s.T if T is None else T, s.H, s.I, s.E, s.k, score=s.score,
                         renormalize=s.renormalize, routed_scale=s.routed_scale,
                         act_dtype=s.act, w_dtype=s.experts,
                         w_scale_fmt=s.scale_fmt if s.experts in ("fp8", "fp4") else "none",
                         y_dtype=y_dtype, path=path, layout=layout, gate=s.gate)


def expert_weights(d, L: dict):
    """(w_gate, w_up, w_down) as the GEMMs take them for d's layout."""
    if d.w_layout == moe.MOE_LAYOUT_PACKED:
        gu, dn = moe.pack_experts(d, L["w_gate"], L["w_up"], L["w_down"], L["x"].device)
        return gu, None, dn
    return L["w_gate"], L["w_up"], L["w_down"]


def score_code(s):
    return oracle.SOFTMAX if s.score == "softmax" else oracle.SIGMOID


def host(layer: dict) -> dict:
    return {k: (None if v is None else v.detach().cpu()) for k, v in layer.items()}


def oracle_experts(s, hl: dict) -> oracle.Experts:
    gate = {"silu": oracle.GATE_SILU, "gelu": oracle.GATE_GELU, "relu": oracle.GATE_RELU}[s.gate]
    if s.experts in ("fp8", "fp4"):
        fmt = oracle.SCALE_UE8M0 if s.scale_fmt == "ue8m0" else oracle.SCALE_F32
        return oracle.Experts(hl["w_gate"], hl["w_up"], hl["w_down"], hl["s_gate"], hl["s_up"],
                              hl["s_down"], fmt, s.block, act_fp8=True, gate=gate, fp4=s.experts == "fp4")
    return oracle.Experts(hl["w_gate"], hl["w_up"], hl["w_down"], gate=gate)


def oracle_route(s, hl):
    return oracle.route(hl["x"], hl["w_router"], hl["router_bias"], s.k, score_code(s),
                        s.renormalize, s.routed_scale)


def act_dtype(s):
    return torch.float32 if s.act == "f32" else torch.bfloat16


def row_rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.linalg.norm(got - ref, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max()) if num.size else 0.0


def coverage_rows(offsets, n_random: int, seed: int = 0, limit: int | None = None):
    """Sorted rows to check: first and last row of every non-empty expert
    segment (the ragged tail tiles) plus n_random seeded random rows."""
    offsets = np.asarray(offsets)
    P = int(offsets[-1])
    rows = set()
    for e in range(offsets.size - 1):
        if offsets[e + 1] > offsets[e]:
            rows.add(int(offsets[e]))
            rows.add(int(offsets[e + 1]) - 1)
    rng = np.random.default_rng(seed)
    if P:
        rows.update(int(r) for r in rng.integers(0, P, n_random))
    rows = np.array(sorted(rows), dtype=np.int64)
    if limit is not None and rows.size > limit:
        rows = np.sort(rng.choice(rows, limit, replace=False))
    return rows


def coverage_tokens(perm, offsets, k, n_random: int, seed: int = 0, limit: int | None = None):
    rows = coverage_rows(offsets, 0, seed)
    toks = set(int(perm[r]) // k for r in rows)
    T = perm.size // k
    rng = np.random.default_rng(seed + 1)
    if T:
        toks.update(int(t) for t in rng.integers(0, T, n_random))
    toks = np.array(sorted(toks), dtype=np.int64)
    if limit is not None and toks.size > limit:
        toks = np.sort(rng.choice(toks, limit, replace=False))
    return toks


def dequant_rows(codes: torch.Tensor, scales: torch.Tensor, group: int = 128) -> np.ndarray:
    """fp8 e4m3 code rows [n, N] with per-group fp32 scales [n, N/group] -> fp64 values."""
    v = codes.cpu().view(torch.float8_e4m3fn).to(torch.float64).numpy()
    s = scales.cpu().to(torch.float64).numpy()
    return v * np.repeat(s, group, axis=1)


def run_forward(s, L: dict, T=None, path="auto", y_dtype=None, layout="rowmajor"):
    """moe_forward on device tensors L; returns (out, ids, w, counts)."""
    T = s.T if T is None else T
    d = desc_for(s, T, path, y_dtype, layout)
    wg, wu, wd = expert_weights(d, L)
    dev = L["x"].device
    out = torch.empty(T, s.H, dtype=act_dtype(s), device=dev)
    ids = torch.empty(T, s.k, dtype=torch.int32, device=dev)
    w = torch.empty(T, s.k, dtype=torch.float32, device=dev)
    counts = torch.empty(s.E, dtype=torch.int32, device=dev)
    ws = moe.workspace(d, moe.MOE_OP_FORWARD, dev)
    moe.moe_forward(d, L["x"], L["w_router"], L["router_bias"], wg, wu, wd, L.get("s_gate"),
                    L.get("s_up"), L.get("s_down"), out, ids, w, counts, ws)
    torch.cuda.synchronize()
    return out, ids, w, counts


def run_staged(s, L: dict, ids_in: torch.Tensor, w_in: torch.Tensor, y_dtype=None, layout="rowmajor",
               path="grouped"):
    """The five staged entry points on given routing; returns a dict of results."""
    T = ids_in.shape[0]
    d = desc_for(s, T, path, y_dtype, layout)
    wg, wu, wd = expert_weights(d, L)
    dev = L["x"].device
    P = T * s.k
    fp8 = s.experts in ("fp8", "fp4")
    r = {}
    r["counts"] = torch.empty(s.E, dtype=torch.int32, device=dev)
    r["offsets"] = torch.empty(s.E + 1, dtype=torch.int32, device=dev)
    r["perm"] = torch.empty(P, dtype=torch.int32, device=dev)
    r["inv"] = torch.empty(P, dtype=torch.int32, device=dev)
    if fp8:
        r["x_sorted"] = torch.empty(P, s.H, dtype=torch.uint8, device=dev)
        r["x_scales"] = torch.empty(P, s.H // 128, dtype=torch.float32, device=dev)
    else:
        r["x_sorted"] = torch.empty(P, s.H, dtype=act_dtype(s), device=dev)
        r["x_scales"] = None
    ws = moe.workspace(d, moe.MOE_OP_PERMUTE, dev)
    moe.moe_permute(d, ids_in, L["x"], r["counts"], r["offsets"], r["perm"], r["inv"],
                    r["x_sorted"], r["x_scales"], ws)
    if fp8:
        r["h"] = torch.empty(P, s.I, dtype=torch.uint8, device=dev)
        r["h_scales"] = torch.empty(P, s.I // 128, dtype=torch.float32, device=dev)
    else:
        r["h"] = torch.empty(P, s.I, dtype=act_dtype(s), device=dev)
        r["h_scales"] = None
    ws = moe.workspace(d, moe.MOE_OP_GATE_UP, dev)
    moe.moe_expert_gate_up_swiglu(d, r["x_sorted"], r["x_scales"], r["offsets"], wg, wu,
                                  L.get("s_gate"), L.get("s_up"), r["h"], r["h_scales"], ws)
    ydt = torch.float32 if d.y_dtype == moe.MOE_DT_F32 else torch.bfloat16
    r["y"] = torch.empty(P, s.H, dtype=ydt, device=dev)
    ws = moe.workspace(d, moe.MOE_OP_DOWN, dev)
    moe.moe_expert_down(d, r["h"], r["h_scales"], r["offsets"], wd, L.get("s_down"), r["y"], ws)
    r["out"] = torch.empty(T, s.H, dtype=act_dtype(s), device=dev)
    moe.moe_unpermute_combine(d, r["y"], r["inv"], w_in, r["out"])
    torch.cuda.synchronize()
    return r
