"""fp64 CPU oracle of the routed mixture-of-experts forward ("Experts backends" page).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``mixture_experts_routed_softmax_amd``) never imports it, and this package
imports nothing from the product: the two share no code.

The arithmetic lives in ``moe_oracle.c`` (plain C, fp64, one token and one
selected expert at a time); this module only marshals numpy / CPU torch arrays
through ctypes.  See the header of ``moe_oracle.c`` for what each step computes
and which passage of the page it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")

F32, BF16, E4M3, E2M1 = 0, 1, 2, 3
SOFTMAX, SIGMOID = 0, 1
SCALE_NONE, SCALE_F32, SCALE_UE8M0 = 0, 1, 2
GATE_SILU, GATE_GELU, GATE_RELU = 0, 1, 2    # SwiGLU / GeGLU / ReGLU


def build(force: bool = False) -> str:
    """Compile moe_oracle.c with gcc (strict fp64: no fast-math, no contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-shared", "-fPIC", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


class _Experts(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("I", ctypes.c_int32), ("E", ctypes.c_int32),
                ("wdt", ctypes.c_int32), ("scale_fmt", ctypes.c_int32),
                ("block", ctypes.c_int32), ("act_fp8", ctypes.c_int32), ("gate", ctypes.c_int32),
                ("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
                ("s_gate", ctypes.c_void_p), ("s_up", ctypes.c_void_p), ("s_down", ctypes.c_void_p)]


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        L.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_f64.restype = dbl
        L.orc_e4m3_to_f64.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_to_f64.restype = dbl
        L.orc_e2m1_to_f64.argtypes = [ctypes.c_uint8]
        L.orc_e2m1_to_f64.restype = dbl
        L.orc_e8m0_to_f64.argtypes = [ctypes.c_uint8]
        L.orc_e8m0_to_f64.restype = dbl
        L.orc_e4m3_encode.argtypes = [dbl]
        L.orc_e4m3_encode.restype = ctypes.c_uint8
        L.orc_quant_group.argtypes = [vp, i32, vp, vp, vp]
        L.orc_quant_group.restype = None
        L.orc_route.argtypes = [i64, i32, i32, i32, vp, i32, vp, i32, vp, i32, i32, dbl, vp, vp, vp]
        L.orc_route.restype = None
        L.orc_permute.argtypes = [i64, i32, i32, vp, vp, vp, vp, vp]
        L.orc_permute.restype = None
        L.orc_expert_row.argtypes = [ctypes.POINTER(_Experts), i32, vp, vp, vp]
        L.orc_expert_row.restype = None
        L.orc_combine_tokens.argtypes = [ctypes.POINTER(_Experts), i32, vp, i32, vp, vp, vp, i64, vp]
        L.orc_combine_tokens.restype = None
        L.orc_expert_pairs.argtypes = [ctypes.POINTER(_Experts), vp, i32, vp, vp, i64, vp, vp]
        L.orc_expert_pairs.restype = None
        L.orc_quant_rows.argtypes = [vp, i32, i64, i32, i32, vp, vp]
        L.orc_quant_rows.restype = None
        L.orc_bwd_tokens.argtypes = [ctypes.POINTER(_Experts), i64, i32, vp, i32, vp, i32, i32, i32, dbl,
                                     vp, vp, vp, vp, vp, i64, vp, vp, vp]
        L.orc_bwd_tokens.restype = None
        L.orc_bwd_expert_rows.argtypes = [ctypes.POINTER(_Experts), i32, i32, vp, i32, i64, i32, vp, i32,
                                          vp, vp, vp, vp]
        L.orc_bwd_expert_rows.restype = None
        L.orc_bwd_router.argtypes = [i64, i32, i32, vp, i32, vp, vp, vp]
        L.orc_bwd_router.restype = None
        L.orc_num_threads.argtypes = []
        L.orc_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def num_threads() -> int:
    return int(lib().orc_num_threads())


# ------------------------------------------------------------------ marshalling

def _as_host(a):
    """(contiguous numpy array, oracle format code) for a numpy array or CPU torch tensor.

    bfloat16 arrives as raw uint16 bits and float8_e4m3fn as raw uint8 codes."""
    fmt = None
    if not isinstance(a, np.ndarray):  # a torch tensor
        import torch
        t = a.detach()
        if t.device.type != "cpu":
            raise ValueError("oracle inputs must be host tensors")
        t = t.contiguous()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16), BF16
        if t.dtype == torch.float8_e4m3fn:
            return t.view(torch.uint8).numpy(), E4M3
        if t.dtype == torch.float32:
            return t.numpy(), F32
        a = t.numpy()
        fmt = None
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        fmt = F32
    elif a.dtype == np.uint16:
        fmt = BF16
    elif a.dtype == np.uint8:
        fmt = E4M3
    return a, fmt


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------------- scalars

def bf16_to_f64(bits: int) -> float:
    return lib().orc_bf16_to_f64(bits)


def e4m3_to_f64(code: int) -> float:
    return lib().orc_e4m3_to_f64(code)


def e2m1_to_f64(code: int) -> float:
    return lib().orc_e2m1_to_f64(code)


def e8m0_to_f64(b: int) -> float:
    return lib().orc_e8m0_to_f64(b)


def e4m3_encode(v: float) -> int:
    return int(lib().orc_e4m3_encode(float(v)))


def quant_group(v):
    """Dynamic fp8 quantization of one group: (dequantized fp64, codes uint8, scale fp32)."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    deq = np.empty_like(v)
    codes = np.empty(v.shape, dtype=np.uint8)
    s = np.zeros(1, dtype=np.float32)
    lib().orc_quant_group(_p(v), v.size, _p(deq), _p(codes), _p(s))
    return deq, codes, float(s[0])


def quant_rows(x, group: int = 128):
    """Per-row, per-`group`-channel fp8 codes [R,N] uint8 and scales [R,N/group] fp32."""
    xa, xf = _as_host(x)
    R, N = xa.shape
    codes = np.empty((R, N), dtype=np.uint8)
    scales = np.empty((R, N // group), dtype=np.float32)
    lib().orc_quant_rows(_p(xa), xf, R, N, group, _p(codes), _p(scales))
    return codes, scales


# ---------------------------------------------------------------------- routing

def route(x, w_r, bias, k: int, score: int, renormalize: bool, routed_scale: float,
          want_keys: bool = False):
    """(ids [T,k] int32, weights [T,k] fp64[, keys [T,E] fp64]) of the router."""
    xa, xf = _as_host(x)
    wa, wf = _as_host(w_r)
    T, H = xa.shape
    E = wa.shape[0]
    b = None if bias is None else np.ascontiguousarray(
        bias.detach().cpu().numpy() if hasattr(bias, "detach") else bias, dtype=np.float32)
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    keys = np.empty((T, E), dtype=np.float64) if want_keys else None
    lib().orc_route(T, H, E, k, _p(xa), xf, _p(wa), wf, _p(b), int(score), int(bool(renormalize)),
                    float(routed_scale), _p(ids), _p(w), _p(keys))
    return (ids, w, keys) if want_keys else (ids, w)


def permute(ids, E: int):
    """(counts [E], offsets [E+1], perm [P], inv [P]) as int32."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    P = T * k
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    perm = np.empty(P, dtype=np.int32)
    inv = np.empty(P, dtype=np.int32)
    lib().orc_permute(T, k, E, _p(ids), _p(counts), _p(offsets), _p(perm), _p(inv))
    return counts, offsets, perm, inv


# ---------------------------------------------------------------------- experts

@dataclass
class Experts:
    """Host copies of the expert weights, in any of the formats the oracle decodes.

    w_gate, w_up [E,I,H] and w_down [E,H,I]: float32, bfloat16 or float8_e4m3fn
    (torch CPU tensors or numpy float32 / uint16 bits / uint8 codes).  For fp8,
    s_gate, s_up [E,I/b,H/b] and s_down [E,H/b,I/b] are float32 (SCALE_F32) or
    uint8 E8M0 bytes (SCALE_UE8M0), and act_fp8 turns on the dynamic per-row
    activation quantization.  gate picks the gated activation (section
    "SonicMoE" of "Experts backends": silu, gelu or relu)."""
    w_gate: object
    w_up: object
    w_down: object
    s_gate: object = None
    s_up: object = None
    s_down: object = None
    scale_fmt: int = SCALE_NONE
    block: int = 128
    act_fp8: bool = False
    gate: int = 0            # GATE_SILU, GATE_GELU or GATE_RELU
    fp4: bool = False        # uint8 weights hold two E2M1 codes per byte along K

    def __post_init__(self):
        self._arrs = []
        g, gf = _as_host(self.w_gate)
        u, uf = _as_host(self.w_up)
        d, df = _as_host(self.w_down)
        if not (gf == uf == df):
            raise ValueError("gate/up/down must share one format")
        E, I, H = g.shape
        sg = su = sd = None
        if self.fp4:
            if gf != E4M3 or self.scale_fmt != SCALE_UE8M0:
                raise ValueError("fp4 experts are uint8 code pairs with UE8M0 scales")
            gf = E2M1
            H *= 2
        if gf in (E4M3, E2M1):
            sg = _as_host_scale(self.s_gate, self.scale_fmt)
            su = _as_host_scale(self.s_up, self.scale_fmt)
            sd = _as_host_scale(self.s_down, self.scale_fmt)
        self._arrs = [g, u, d, sg, su, sd]
        self.E, self.I, self.H = E, I, H
        self._st = _Experts(H, I, E, gf, self.scale_fmt if gf in (E4M3, E2M1) else SCALE_NONE,
                            self.block, int(bool(self.act_fp8)), int(self.gate),
                            g.ctypes.data, u.ctypes.data, d.ctypes.data,
                            None if sg is None else sg.ctypes.data,
                            None if su is None else su.ctypes.data,
                            None if sd is None else sd.ctypes.data)

    def row(self, e: int, x_row):
        """(h [I], y [H]) of expert e on one fp64 row."""
        xr = np.ascontiguousarray(x_row, dtype=np.float64)
        h = np.empty(self.I, dtype=np.float64)
        y = np.empty(self.H, dtype=np.float64)
        lib().orc_expert_row(ctypes.byref(self._st), int(e), _p(xr), _p(h), _p(y))
        return h, y

    def pairs(self, x, tokens, experts, want_h: bool = True, want_y: bool = True):
        """(h [n,I], y [n,H]) for the (token, expert) pairs; x is the [T,H] input."""
        xa, xf = _as_host(x)
        tok = np.ascontiguousarray(tokens, dtype=np.int64)
        ex = np.ascontiguousarray(experts, dtype=np.int32)
        n = tok.size
        h = np.empty((n, self.I), dtype=np.float64) if want_h else None
        y = np.empty((n, self.H), dtype=np.float64) if want_y else None
        lib().orc_expert_pairs(ctypes.byref(self._st), _p(xa), xf, _p(tok), _p(ex), n, _p(h), _p(y))
        return h, y

    def combine(self, x, ids, w, tokens=None):
        """out [n,H] fp64 = sum_i w[t,i] * expert(ids[t,i])(x[t]) for t in tokens."""
        xa, xf = _as_host(x)
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        w = np.ascontiguousarray(w, dtype=np.float64)
        T, k = ids.shape
        tok = np.arange(T, dtype=np.int64) if tokens is None else np.ascontiguousarray(tokens, dtype=np.int64)
        out = np.empty((tok.size, self.H), dtype=np.float64)
        lib().orc_combine_tokens(ctypes.byref(self._st), k, _p(xa), xf, _p(ids), _p(w), _p(tok),
                                 tok.size, _p(out))
        return out


def _as_host_scale(s, fmt):
    if s is None:
        raise ValueError("fp8 experts need block scales")
    if not isinstance(s, np.ndarray):
        import torch
        t = s.detach().cpu().contiguous()
        s = t.view(torch.uint8).numpy() if t.dtype in (torch.uint8, torch.float8_e8m0fnu) else t.numpy()
    s = np.ascontiguousarray(s)
    if fmt == SCALE_F32 and s.dtype != np.float32:
        raise ValueError("float32 scales expected")
    if fmt == SCALE_UE8M0 and s.dtype != np.uint8:
        raise ValueError("E8M0 bytes expected")
    return s


def forward(x, w_r, bias, experts: Experts, k: int, score: int, renormalize: bool,
            routed_scale: float, tokens=None):
    """Whole layer on the host: (ids, w, counts, offsets, perm, inv, out[tokens])."""
    ids, w = route(x, w_r, bias, k, score, renormalize, routed_scale)
    counts, offsets, perm, inv = permute(ids, experts.E)
    out = experts.combine(x, ids, w, tokens)
    return ids, w, counts, offsets, perm, inv, out


# --------------------------------------------------------------------- backward

def _f64(a):
    if a is not None and not isinstance(a, np.ndarray):
        a = a.detach().cpu().double().numpy()
    return np.ascontiguousarray(a, dtype=np.float64)


def bwd_tokens(experts: Experts, x, w_r, score: int, renormalize: bool, routed_scale: float,
               keys, ids, w, dout, tokens=None):
    """(dx [n,H], dw [n,k], dkey [n,E]) fp64 for the listed tokens (all by default).

    keys [T,E], ids and w [T,k] come from ``route(..., want_keys=True)``;
    dout [T,H] is the gradient of the layer output."""
    xa, xf = _as_host(x)
    wa, wf = _as_host(w_r)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    keys, w, dout = _f64(keys), _f64(w), _f64(dout)
    tok = np.arange(T, dtype=np.int64) if tokens is None else np.ascontiguousarray(tokens, dtype=np.int64)
    n = tok.size
    dx = np.empty((n, experts.H), dtype=np.float64)
    dw = np.empty((n, k), dtype=np.float64)
    dkey = np.empty((n, experts.E), dtype=np.float64)
    lib().orc_bwd_tokens(ctypes.byref(experts._st), T, k, _p(xa), xf, _p(wa), wf, int(score),
                         int(bool(renormalize)), float(routed_scale), _p(keys), _p(ids), _p(w), _p(dout),
                         _p(tok), n, _p(dx), _p(dw), _p(dkey))
    return dx, dw, dkey


BWD_GATE, BWD_UP, BWD_DOWN = 0, 1, 2


def bwd_expert_rows(experts: Experts, which: int, e: int, rows, x, ids, w, dout):
    """Rows of dW_gate[e] / dW_up[e] ([I,H]) or dW_down[e] ([H,I]) as fp64 [n, cols]."""
    xa, xf = _as_host(x)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    w, dout = _f64(w), _f64(dout)
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    cols = experts.I if which == BWD_DOWN else experts.H
    out = np.empty((rows.size, cols), dtype=np.float64)
    lib().orc_bwd_expert_rows(ctypes.byref(experts._st), int(which), int(e), _p(rows), rows.size, T, k,
                              _p(xa), xf, _p(ids), _p(w), _p(dout), _p(out))
    return out


def bwd_router(x, dkey):
    """(dW_r [E,H], dbias [E]) fp64 from dkey [T,E]."""
    xa, xf = _as_host(x)
    dkey = _f64(dkey)
    T, E = dkey.shape
    H = xa.shape[1]
    dwr = np.empty((E, H), dtype=np.float64)
    db = np.empty(E, dtype=np.float64)
    lib().orc_bwd_router(T, H, E, _p(xa), xf, _p(dkey), _p(dwr), _p(db))
    return dwr, db


def backward(x, w_r, bias, experts: Experts, k: int, score: int, renormalize: bool, routed_scale: float,
             dout):
    """Every gradient of the layer for the output gradient dout [T,H], as a dict of
    fp64 arrays: dx, dw_router, dbias, dw_gate, dw_up, dw_down, plus ids, w, dw
    (gradient of the routing weights) and dkey."""
    ids, w, keys = route(x, w_r, bias, k, score, renormalize, routed_scale, want_keys=True)
    dx, dw, dkey = bwd_tokens(experts, x, w_r, score, renormalize, routed_scale, keys, ids, w, dout)
    dwr, db = bwd_router(x, dkey)
    E, I, H = experts.E, experts.I, experts.H
    dwg = np.zeros((E, I, H))
    dwu = np.zeros((E, I, H))
    dwd = np.zeros((E, H, I))
    for e in range(E):
        if not (ids == e).any():
            continue
        dwg[e] = bwd_expert_rows(experts, BWD_GATE, e, np.arange(I), x, ids, w, dout)
        dwu[e] = bwd_expert_rows(experts, BWD_UP, e, np.arange(I), x, ids, w, dout)
        dwd[e] = bwd_expert_rows(experts, BWD_DOWN, e, np.arange(H), x, ids, w, dout)
    return dict(ids=ids, w=w, keys=keys, dw=dw, dkey=dkey, dx=dx, dw_router=dwr, dbias=db,
                dw_gate=dwg, dw_up=dwu, dw_down=dwd)
