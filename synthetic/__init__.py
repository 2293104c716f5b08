"""Seeded synthetic inputs for routed mixture-of-experts layers.

This module only draws random inputs; it holds none of the method's arithmetic
(no routing, no quantization of activations, no matmul).  Both the HIP path and
the fp64 oracle receive exactly the tensors made here.

Workloads (stand-ins for the layer shapes of the models the "Experts backends"
page names; no checkpoint or dataset is used):

=============  =========  =====  =====  ===  =  ======  =============================
name           T          H      I      E    k  experts routing
=============  =========  =====  =====  ===  =  ======  =============================
tiny           64         128    256    8    2  fp32    softmax over all, top-k renorm
qwen_prefill   4096       2048   1408   60   4  bf16    softmax, no renorm, Zipf bias
qwen_decode    1/8/32/64  2048   1408   60   4  bf16    softmax, no renorm, zero bias
dsv3_bf16      8192       7168   2048   256  8  bf16    sigmoid, renorm, x2.5, Zipf bias
dsv3_fp8       64/8192    7168   2048   256  8  e4m3    as dsv3_bf16; 128x128 block scales
dsv3_fp4       64/8192    7168   2048   256  8  e2m1    as dsv3_bf16; UE8M0 per row per 32
dsv3_ep8_shard 8192       7168   2048   32   8  bf16    sigmoid, renorm, x2.5, zero bias
=============  =========  =====  =====  ===  =  ======  =============================

Router inputs are snapped to grids so that every router logit is an exact fp32
number whatever the order of summation (so the top-k choice is well posed and
bit-exact on any hardware):

* x on multiples of 2^-4, |x| <= 127/16 (7 significant bits, bf16-exact);
* W_r on multiples of 2^-11, |w| <= 255 * 2^-11 (bf16 configs, 8 bits,
  bf16-exact), or of 2^-12 with |w| <= 2047 * 2^-12 (fp32 config);
* the Zipf bias on multiples of 2^-15.

Every product x*w is then an integer multiple of 2^-15 (2^-16 for fp32) below
2^15 (2^18) units, and ``make_layer`` asserts that every |logit| + |bias| stays
below 2^24 units, so every partial sum is exact in fp32.  The check uses the
Cauchy-Schwarz bound max_t ||x_t|| * max_e ||W_r[e]||, which needs no matmul.

Expert weights: N(0, 0.02) rounded to bf16 (bf16 configs), N(0, 1/fan_in) in
fp32 (tiny).  FP8 experts are drawn directly as e4m3 codes (roughly N(0, 112),
clamped to +-448) with one positive scale per 128 x 128 block: fp32 scales
0.02/112 * 2^U(-1/2, 1/2), or E8M0 bytes 115 + {-1, 0, 1} (about 2^-12.5), so
code * scale has a spread close to N(0, 0.02).  The Zipf bias is
b_e = -1.1 * ln(1 + pi(e)) for a seeded permutation pi of the experts, which
skews the load so that the expert of rank r gets about r^-1.1 of the top-1
picks among otherwise equal logits.
"""
from __future__ import annotations

import math
import zlib
from dataclasses import dataclass, replace

import torch


@dataclass(frozen=True)
class LayerSpec:
    name: str
    T: int
    H: int
    I: int
    E: int
    k: int
    act: str            # "f32" | "bf16": x, W_r and the layer output
    experts: str        # "f32" | "bf16" | "fp8" | "fp4"
    score: str          # "softmax" | "sigmoid"
    renormalize: bool
    routed_scale: float
    bias: str           # "none" | "zero" | "zipf"
    scale_fmt: str = "none"   # fp8 weight scales: "f32" | "ue8m0"
    block: int = 128
    gate: str = "silu"        # gated activation of the expert MLPs: "silu" | "gelu" | "relu"

    @property
    def P(self) -> int:
        return self.T * self.k


_BASE = {
    "tiny": LayerSpec("tiny", 64, 128, 256, 8, 2, "f32", "f32", "softmax", True, 1.0, "none"),
    "qwen_prefill": LayerSpec("qwen_prefill", 4096, 2048, 1408, 60, 4, "bf16", "bf16", "softmax",
                              False, 1.0, "zipf"),
    "qwen_decode": LayerSpec("qwen_decode", 64, 2048, 1408, 60, 4, "bf16", "bf16", "softmax",
                             False, 1.0, "zero"),
    "dsv3_bf16": LayerSpec("dsv3_bf16", 8192, 7168, 2048, 256, 8, "bf16", "bf16", "sigmoid",
                           True, 2.5, "zipf"),
    "dsv3_fp8": LayerSpec("dsv3_fp8", 8192, 7168, 2048, 256, 8, "bf16", "fp8", "sigmoid",
                          True, 2.5, "zipf", "f32"),
    # the DeepSeek-like layer with int8-packed FP4 experts (UE8M0 scales per
    # row per 32 K; activations fp8 per row per 128)
    "dsv3_fp4": LayerSpec("dsv3_fp4", 8192, 7168, 2048, 256, 8, "bf16", "fp4", "sigmoid",
                          True, 2.5, "zipf", "ue8m0"),
    # one GPU's share of an 8-way expert-parallel DeepSeek-like layer: 32 local
    # experts, 8 of them per token, so each expert receives about 2048 rows
    "dsv3_ep8_shard": LayerSpec("dsv3_ep8_shard", 8192, 7168, 2048, 32, 8, "bf16", "bf16", "sigmoid",
                                True, 2.5, "zero"),
}

# token counts each workload is exercised at
TOKEN_COUNTS = {
    "tiny": (64,),
    "qwen_prefill": (4096,),
    "qwen_decode": (1, 8, 32, 64),
    "dsv3_bf16": (8192,),
    "dsv3_fp8": (64, 8192),
    "dsv3_fp4": (64, 8192),
    "dsv3_ep8_shard": (8192,),
}


def spec(name: str, **overrides) -> LayerSpec:
    """The named workload, with any field overridden (e.g. T=8, scale_fmt="ue8m0")."""
    return replace(_BASE[name], **overrides)


def _seed(root: int, *parts) -> int:
    s = "%d/" % root + "/".join(str(p) for p in parts)
    return zlib.crc32(s.encode()) ^ (root * 0x9E3779B1 & 0xFFFFFFFF)


def _gen(device, root, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(root, *parts))
    return g


def _snap(v: torch.Tensor, frac_bits: int, max_units: int) -> torch.Tensor:
    return torch.round(v * (1 << frac_bits)).clamp_(-max_units, max_units) / (1 << frac_bits)


def _act_dtype(s: LayerSpec):
    return torch.float32 if s.act == "f32" else torch.bfloat16


def make_layer(s: LayerSpec, seed: int = 0, device="cpu", snap: bool = True, experts: bool = True) -> dict:
    """All inputs of one layer call, generated on `device` with seeded generators.

    Keys: x [T,H], w_router [E,H], router_bias [E] fp32 or None, w_gate, w_up
    [E,I,H], w_down [E,H,I], and for fp8 s_gate, s_up [E,I/128,H/128], s_down
    [E,H/128,I/128] (float32, or uint8 E8M0 bytes).

    snap=False draws x, W_r and the bias from the same distributions without
    snapping them to the grids that keep every partial sum of a logit exact in
    fp32 (router outputs then depend on the summation order); experts=False
    leaves out the expert weights."""
    device = torch.device(device)
    out = {}
    out["x"] = make_tokens(s, seed, device, snap)

    g = _gen(device, seed, s.name, "w_router")
    if s.act == "f32":
        wr = torch.randn(s.E, s.H, generator=g, device=device) * math.sqrt(1.0 / 128.0)
        wr = _snap(wr, 12, 2047) if snap else wr
    else:
        wr = torch.randn(s.E, s.H, generator=g, device=device) * 0.02
        wr = _snap(wr, 11, 255) if snap else wr
    out["w_router"] = wr.to(_act_dtype(s))

    if s.bias == "none":
        out["router_bias"] = None
    elif s.bias == "zero":
        out["router_bias"] = torch.zeros(s.E, dtype=torch.float32, device=device)
    else:
        g = _gen("cpu", seed, s.name, "zipf_rank")
        rank = torch.randperm(s.E, generator=g).to(torch.float64) + 1.0
        b = -1.1 * torch.log(rank)
        out["router_bias"] = (_snap(b, 15, 1 << 22) if snap else b).to(torch.float32).to(device)

    if snap:
        _check_router_exact(s, out["x"], out["w_router"], out["router_bias"])
    if not experts:
        return out

    if s.experts == "fp8":
        out.update(_fp8_experts(s, seed, device))
    elif s.experts == "fp4":
        out.update(_fp4_experts(s, seed, device))
    else:
        out.update(_dense_experts(s, seed, device))
    return out


def make_tokens(s: LayerSpec, seed: int, device, snap: bool = True) -> torch.Tensor:
    g = _gen(device, seed, s.name, "x", s.T)
    x = torch.randn(s.T, s.H, generator=g, device=device)
    return (_snap(x, 4, 127) if snap else x).to(_act_dtype(s))


def _check_router_exact(s, x, wr, bias):
    # Units of the logit grid: 2^-15 (bf16 grids) or 2^-16 (fp32 grid).  Every
    # partial sum of x*w stays exact in fp32 while |sum| < 2^24 units.
    unit = 2.0 ** (-16 if s.act == "f32" else -15)
    if s.T == 0:
        return
    xn = x.double().norm(dim=1).max().item()
    wn = wr.double().norm(dim=1).max().item()
    bmax = 0.0 if bias is None else bias.double().abs().max().item()
    bound = xn * wn + bmax
    assert bound < (2 ** 24) * unit * 0.999, (
        "router grid bound violated: %.3f >= %.3f" % (bound, 2 ** 24 * unit))


def _dense_experts(s: LayerSpec, seed: int, device) -> dict:
    dt = torch.float32 if s.experts == "f32" else torch.bfloat16
    res = {}
    for name, (rows, cols) in (("w_gate", (s.I, s.H)), ("w_up", (s.I, s.H)),
                               ("w_down", (s.H, s.I))):
        w = torch.empty(s.E, rows, cols, dtype=dt, device=device)
        std = math.sqrt(1.0 / cols) if s.experts == "f32" else 0.02
        for e in range(s.E):
            g = _gen(device, seed, s.name, name, e)
            w[e] = (torch.randn(rows, cols, generator=g, device=device) * std).to(dt)
        res[name] = w
    return res


def _fp8_experts(s: LayerSpec, seed: int, device) -> dict:
    b = s.block
    res = {}
    for name, (rows, cols) in (("w_gate", (s.I, s.H)), ("w_up", (s.I, s.H)),
                               ("w_down", (s.H, s.I))):
        codes = torch.empty(s.E, rows, cols, dtype=torch.float8_e4m3fn, device=device)
        for e in range(s.E):
            g = _gen(device, seed, s.name, name, e)
            v = (torch.randn(rows, cols, generator=g, device=device) * 112.0).clamp_(-448.0, 448.0)
            codes[e] = v.to(torch.float8_e4m3fn)
        res[name] = codes
        sname = "s_" + name[2:]
        g = _gen(device, seed, s.name, sname)
        shape = (s.E, rows // b, cols // b)
        if s.scale_fmt == "ue8m0":
            res[sname] = torch.randint(114, 117, shape, generator=g, device=device, dtype=torch.int64).to(torch.uint8)
        else:
            u = torch.rand(shape, generator=g, device=device, dtype=torch.float32) - 0.5
            res[sname] = (0.02 / 112.0) * torch.exp2(u)
    return res


_E2M1_VALUES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def _fp4_experts(s: LayerSpec, seed: int, device) -> dict:
    """E2M1 code pairs [E, rows, cols/2] (even column in the low nibble) and
    UE8M0 scale bytes [E, rows, cols/32]; codes follow N(0, 2) snapped to the
    nearest E2M1 value, scales 2^-8 .. 2^-6 (weights of std about 0.02)."""
    mags = torch.tensor(_E2M1_VALUES, device=device)
    res = {}
    for name, (rows, cols) in (("w_gate", (s.I, s.H)), ("w_up", (s.I, s.H)),
                               ("w_down", (s.H, s.I))):
        codes = torch.empty(s.E, rows, cols // 2, dtype=torch.uint8, device=device)
        for e in range(s.E):
            g = _gen(device, seed, s.name, name, e)
            v = torch.randn(rows, cols, generator=g, device=device) * 2.0
            c = (v.abs().unsqueeze(-1) - mags).abs().argmin(-1)          # nearest magnitude
            c = c | ((v < 0) & (c > 0)).to(torch.int64) << 3            # sign (no -0)
            c = c.to(torch.uint8).view(rows, cols // 2, 2)
            codes[e] = c[..., 0] | (c[..., 1] << 4)
        res[name] = codes
        sname = "s_" + name[2:]
        g = _gen(device, seed, s.name, sname)
        res[sname] = torch.randint(119, 122, (s.E, rows, cols // 32), generator=g, device=device,
                                   dtype=torch.int64).to(torch.uint8)
    return res


def make_grad_out(s: LayerSpec, seed: int = 0, device="cpu") -> torch.Tensor:
    """Gradient of the layer output for the backward: N(0, 1) in the activation
    dtype, [T, H]."""
    g = _gen(device, seed, s.name, "dout", s.T)
    return torch.randn(s.T, s.H, generator=g, device=device).to(_act_dtype(s))


def to_device(layer: dict, device) -> dict:
    return {k: (None if v is None else v.to(device)) for k, v in layer.items()}
