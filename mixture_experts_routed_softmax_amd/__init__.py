"""Routed mixture-of-experts forward on AMD MI355X (gfx950): Python binding.

This module only marshals arguments to libmoe.so (and checks, before each
call, that every tensor is a contiguous GPU tensor of an accepted dtype and
large enough for the shapes in the description), the HIP library whose C ABI
is declared in include/moe.h.  Every step of the layer runs in libmoe's
kernels; PyTorch provides device memory and the current HIP stream.  The
functions carry the names of the C entry points and take torch tensors (or
None for optional arguments); a failing status raises MoeError with the
library's message.

If libmoe.so has not been built this module raises ImportError: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "moe.h")

if not os.path.exists(LIB_PATH):
    raise ImportError("libmoe.so is not built; run __graft_entry__.build() (or python "
                      "mixture_experts_routed_softmax_amd/_build.py) first")

# torch ships its own HIP runtime; load it before libmoe so that libmoe binds to
# the same runtime instance (and so accepts torch's streams and device state)
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

# ---- enums (values of include/moe.h)
MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP = range(5)
MOE_DT_F32, MOE_DT_BF16, MOE_DT_FP8_E4M3, MOE_DT_FP4_E2M1 = range(4)
MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID = range(2)
MOE_SCALE_NONE, MOE_SCALE_F32, MOE_SCALE_UE8M0 = range(3)
MOE_ACT_NONE, MOE_ACT_DYNAMIC, MOE_ACT_STATIC = range(3)
MOE_PATH_AUTO, MOE_PATH_GROUPED, MOE_PATH_STREAM = range(3)
MOE_LAYOUT_ROWMAJOR, MOE_LAYOUT_PACKED = range(2)
MOE_GATE_SILU, MOE_GATE_GELU, MOE_GATE_RELU = range(3)
MOE_PACK_GATE_UP, MOE_PACK_DOWN = range(2)
(MOE_OP_ROUTE, MOE_OP_PERMUTE, MOE_OP_GATE_UP, MOE_OP_DOWN, MOE_OP_COMBINE,
 MOE_OP_FORWARD, MOE_OP_BACKWARD) = range(7)
STAGES = ("route", "hist", "scan", "scatter", "quant_x", "gate_up", "down", "combine",
          "bwd_recompute", "bwd_data", "bwd_weight", "bwd_router", "bwd_misc")
MOE_NUM_STAGES = len(STAGES)


class MoeDesc(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("E", ctypes.c_int32), ("k", ctypes.c_int32), ("score", ctypes.c_int32),
                ("renormalize", ctypes.c_int32), ("routed_scale", ctypes.c_float),
                ("act_dtype", ctypes.c_int32), ("w_dtype", ctypes.c_int32),
                ("w_scale_fmt", ctypes.c_int32), ("block", ctypes.c_int32),
                ("act_scheme", ctypes.c_int32), ("y_dtype", ctypes.c_int32),
                ("path", ctypes.c_int32), ("w_layout", ctypes.c_int32),
                ("gate_act", ctypes.c_int32), ("reserved", ctypes.c_int32 * 1)]


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s (%s)" % (message, _lib.moe_status_str(status).decode()))
        self.status = status


_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_DP = ctypes.POINTER(MoeDesc)
_sigs = {
    "moe_route_topk": [_DP, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp],
    "moe_permute": [_DP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp],
    "moe_expert_gate_up_swiglu": [_DP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                  ctypes.c_size_t, _vp],
    "moe_expert_down": [_DP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp],
    "moe_unpermute_combine": [_DP, _vp, _vp, _vp, _vp, _vp],
    "moe_forward": [_DP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                    ctypes.c_size_t, _vp],
    "moe_backward": [_DP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                     ctypes.c_size_t, _vp],
    "moe_forward_static": [_DP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp],
}
for _name, _args in _sigs.items():
    getattr(_lib, _name).argtypes = _args
    getattr(_lib, _name).restype = ctypes.c_int
_lib.moe_pack_weights.argtypes = [_DP, ctypes.c_int, _vp, _vp, _vp, _vp]
_lib.moe_pack_weights.restype = ctypes.c_int
_lib.moe_packed_weight_bytes.argtypes = [_DP, ctypes.c_int]
_lib.moe_packed_weight_bytes.restype = ctypes.c_size_t
_lib.moe_workspace_bytes.argtypes = [_DP, ctypes.c_int]
_lib.moe_workspace_bytes.restype = ctypes.c_size_t
_lib.moe_status_str.argtypes = [ctypes.c_int]
_lib.moe_status_str.restype = ctypes.c_char_p
_lib.moe_last_error.argtypes = []
_lib.moe_last_error.restype = ctypes.c_char_p
_lib.moe_timing_enable.argtypes = [ctypes.c_int]
_lib.moe_timing_enable.restype = ctypes.c_int
_lib.moe_timing_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
_lib.moe_timing_read.restype = ctypes.c_int


def exported_symbols_of_header(path: str = HEADER_PATH):
    """Names of the functions include/moe.h declares."""
    text = open(path).read()
    return sorted(set(re.findall(r"^\s*(?:moe_status|size_t|const char\*)\s+(moe_\w+)\s*\(", text, re.M)))


def library():
    return _lib


def make_desc(T, H, I, E, k, *, score="softmax", renormalize=False, routed_scale=1.0,
              act_dtype="bf16", w_dtype="bf16", w_scale_fmt="none", block=None,
              act_scheme=None, y_dtype=None, path="auto", layout="rowmajor", gate="silu") -> MoeDesc:
    dt = {"f32": MOE_DT_F32, "bf16": MOE_DT_BF16, "fp8": MOE_DT_FP8_E4M3, "fp4": MOE_DT_FP4_E2M1}
    d = MoeDesc()
    d.T, d.H, d.I, d.E, d.k = int(T), int(H), int(I), int(E), int(k)
    d.score = {"softmax": MOE_SCORE_SOFTMAX, "sigmoid": MOE_SCORE_SIGMOID}[score]
    d.renormalize = int(bool(renormalize))
    d.routed_scale = float(routed_scale)
    d.act_dtype = dt[act_dtype]
    d.w_dtype = dt[w_dtype]
    d.w_scale_fmt = {"none": MOE_SCALE_NONE, "f32": MOE_SCALE_F32, "ue8m0": MOE_SCALE_UE8M0}[w_scale_fmt]
    fp8 = w_dtype in ("fp8", "fp4")
    d.block = int(block if block is not None else (128 if fp8 else 0))
    if act_scheme is None:
        act_scheme = "dynamic" if fp8 else "none"
    d.act_scheme = {"none": MOE_ACT_NONE, "dynamic": MOE_ACT_DYNAMIC, "static": MOE_ACT_STATIC}[act_scheme]
    if y_dtype is None:
        y_dtype = "f32" if act_dtype == "f32" else "bf16"
    d.y_dtype = dt[y_dtype]
    d.path = {"auto": MOE_PATH_AUTO, "grouped": MOE_PATH_GROUPED, "stream": MOE_PATH_STREAM}[path]
    d.w_layout = {"rowmajor": MOE_LAYOUT_ROWMAJOR, "packed": MOE_LAYOUT_PACKED}[layout]
    d.gate_act = {"silu": MOE_GATE_SILU, "gelu": MOE_GATE_GELU, "relu": MOE_GATE_RELU}[gate]
    return d


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return ctypes.c_void_p(t.data_ptr())


# ---- argument checks (before the call: the library cannot see tensor metadata)

def _dtypes():
    import torch
    f8 = [getattr(torch, n) for n in ("float8_e4m3fn", "float8_e8m0fnu") if hasattr(torch, n)]
    return {
        "f32": (torch.float32,), "bf16": (torch.bfloat16,), "i32": (torch.int32,),
        "bytes": None,   # any dtype: a raw byte buffer
        "codes": (torch.uint8, torch.int8, *f8),
    }


_ELT = {MOE_DT_F32: 4, MOE_DT_BF16: 2, MOE_DT_FP8_E4M3: 1, MOE_DT_FP4_E2M1: 1}
_KIND = {MOE_DT_F32: "f32", MOE_DT_BF16: "bf16", MOE_DT_FP8_E4M3: "codes", MOE_DT_FP4_E2M1: "codes"}


def _arg(t, name: str, kind: str, nbytes: int):
    """Raise ValueError unless the device tensor t can hold nbytes of `kind`:
    a contiguous GPU tensor of an accepted dtype and at least nbytes long.
    None and raw integer addresses pass unchecked."""
    if t is None or isinstance(t, int):
        return
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    ok = _dtypes()[kind]
    if ok is not None and t.dtype not in ok:
        raise ValueError("%s has dtype %s, expected one of %s" % (name, t.dtype, [str(d) for d in ok]))
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError("%s holds %d bytes, %d needed" % (name, have, nbytes))
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)


def _known(desc) -> bool:
    """Whether desc's dtypes and sizes are ones the checks can size; anything
    else is left to the library's own validation (which rejects it)."""
    return (desc.act_dtype in _ELT and desc.w_dtype in _ELT and desc.y_dtype in _ELT and
            desc.w_scale_fmt in (MOE_SCALE_NONE, MOE_SCALE_F32, MOE_SCALE_UE8M0) and
            min(desc.T, desc.H, desc.I, desc.E, desc.k) >= 0)


def _fp8(desc) -> bool:
    return desc.w_dtype in (MOE_DT_FP8_E4M3, MOE_DT_FP4_E2M1)


def _w_bytes(desc, rows: int, cols: int) -> int:
    """Bytes of one row-major expert matrix stack [E, rows, cols] in desc's weight format."""
    per = cols // 2 if desc.w_dtype == MOE_DT_FP4_E2M1 else cols * _ELT[desc.w_dtype]
    return desc.E * rows * per


def _scale_bytes(desc, rows: int, cols: int) -> int:
    if desc.w_dtype == MOE_DT_FP4_E2M1:
        return desc.E * rows * (cols // 32)
    per = 1 if desc.w_scale_fmt == MOE_SCALE_UE8M0 else 4
    return desc.E * ((rows + 127) // 128) * ((cols + 127) // 128) * per


def _check_weights(desc, w_gate, w_up, w_down, sg, su, sd):
    H, I = desc.H, desc.I
    if desc.w_layout == MOE_LAYOUT_PACKED:
        _arg(w_gate, "w_gate (packed gate/up)", "bytes", moe_packed_weight_bytes(desc, MOE_PACK_GATE_UP))
        _arg(w_down, "w_down (packed)", "bytes", moe_packed_weight_bytes(desc, MOE_PACK_DOWN))
    else:
        kind = _KIND[desc.w_dtype]
        _arg(w_gate, "w_gate", kind, _w_bytes(desc, I, H))
        _arg(w_up, "w_up", kind, _w_bytes(desc, I, H))
        _arg(w_down, "w_down", kind, _w_bytes(desc, H, I))
    if _fp8(desc):
        skind = "f32" if desc.w_scale_fmt == MOE_SCALE_F32 and desc.w_dtype == MOE_DT_FP8_E4M3 else "codes"
        _arg(sg, "w_gate_scales", skind, _scale_bytes(desc, I, H))
        _arg(su, "w_up_scales", skind, _scale_bytes(desc, I, H))
        _arg(sd, "w_down_scales", skind, _scale_bytes(desc, H, I))


def _check_router(desc, x, w_router, router_bias):
    ea = _ELT[desc.act_dtype]
    _arg(x, "x", _KIND[desc.act_dtype], desc.T * desc.H * ea)
    _arg(w_router, "w_router", _KIND[desc.act_dtype], desc.E * desc.H * ea)
    _arg(router_bias, "router_bias", "f32", desc.E * 4)


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status: int):
    if status != MOE_OK:
        raise MoeError(status, _lib.moe_last_error().decode())


def moe_workspace_bytes(desc: MoeDesc, op: int) -> int:
    return int(_lib.moe_workspace_bytes(ctypes.byref(desc), int(op)))


def moe_status_str(status: int) -> str:
    return _lib.moe_status_str(int(status)).decode()


def moe_last_error() -> str:
    return _lib.moe_last_error().decode()


def workspace(desc: MoeDesc, op: int, device="cuda"):
    """A uint8 device tensor of moe_workspace_bytes(desc, op) bytes (or None)."""
    import torch
    n = moe_workspace_bytes(desc, op)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def moe_packed_weight_bytes(desc: MoeDesc, which: int) -> int:
    return int(_lib.moe_packed_weight_bytes(ctypes.byref(desc), int(which)))


def moe_pack_weights(desc, which, w0, w1, dst, stream=None):
    if _known(desc):
        kind = _KIND[desc.w_dtype]
        rows, cols = (desc.I, desc.H) if which == MOE_PACK_GATE_UP else (desc.H, desc.I)
        _arg(w0, "w0", kind, _w_bytes(desc, rows, cols))
        _arg(w1, "w1", kind, _w_bytes(desc, rows, cols))
        _arg(dst, "dst", "bytes", moe_packed_weight_bytes(desc, which))
    _check(_lib.moe_pack_weights(ctypes.byref(desc), int(which), _ptr(w0), _ptr(w1), _ptr(dst),
                                 _stream(stream)))


def pack_experts(desc, w_gate, w_up, w_down, device="cuda"):
    """(packed gate/up, packed down) uint8 device tensors for desc's shapes."""
    import torch
    gu = torch.empty(moe_packed_weight_bytes(desc, MOE_PACK_GATE_UP), dtype=torch.uint8, device=device)
    dn = torch.empty(moe_packed_weight_bytes(desc, MOE_PACK_DOWN), dtype=torch.uint8, device=device)
    moe_pack_weights(desc, MOE_PACK_GATE_UP, w_gate, w_up, gu)
    moe_pack_weights(desc, MOE_PACK_DOWN, w_down, None, dn)
    return gu, dn


def moe_route_topk(desc, x, w_router, router_bias, topk_ids, topk_w, ws=None, stream=None):
    if _known(desc):
        _check_router(desc, x, w_router, router_bias)
        _arg(topk_ids, "topk_ids", "i32", desc.T * desc.k * 4)
        _arg(topk_w, "topk_w", "f32", desc.T * desc.k * 4)
    _check(_lib.moe_route_topk(ctypes.byref(desc), _ptr(x), _ptr(w_router), _ptr(router_bias),
                               _ptr(topk_ids), _ptr(topk_w), _ptr(ws), _nbytes(ws), _stream(stream)))


def moe_permute(desc, topk_ids, x, counts, offsets, perm, inv, x_sorted=None, x_sorted_scales=None,
                ws=None, stream=None):
    if _known(desc):
        P = desc.T * desc.k
        _arg(topk_ids, "topk_ids", "i32", P * 4)
        for t, n, b in ((counts, "counts", desc.E), (offsets, "offsets", desc.E + 1), (perm, "perm", P),
                        (inv, "inv", P)):
            _arg(t, n, "i32", b * 4)
        _arg(x, "x", _KIND[desc.act_dtype], desc.T * desc.H * _ELT[desc.act_dtype])
        if _fp8(desc):
            _arg(x_sorted, "x_sorted", "codes", P * desc.H)
            _arg(x_sorted_scales, "x_sorted_scales", "f32", P * (desc.H // 128) * 4)
        else:
            _arg(x_sorted, "x_sorted", _KIND[desc.act_dtype], P * desc.H * _ELT[desc.act_dtype])
    _check(_lib.moe_permute(ctypes.byref(desc), _ptr(topk_ids), _ptr(x), _ptr(counts), _ptr(offsets),
                            _ptr(perm), _ptr(inv), _ptr(x_sorted), _ptr(x_sorted_scales), _ptr(ws),
                            _nbytes(ws), _stream(stream)))


def moe_expert_gate_up_swiglu(desc, x_sorted, x_scales, offsets, w_gate, w_up, w_gate_scales,
                              w_up_scales, h, h_scales, ws=None, stream=None):
    if _known(desc):
        P = desc.T * desc.k
        _check_weights(desc, w_gate, w_up, None, w_gate_scales, w_up_scales, None)
        _arg(offsets, "offsets", "i32", (desc.E + 1) * 4)
        if _fp8(desc):
            _arg(x_sorted, "x_sorted", "codes", P * desc.H)
            _arg(x_scales, "x_scales", "f32", P * (desc.H // 128) * 4)
            _arg(h, "h", "codes", P * desc.I)
            _arg(h_scales, "h_scales", "f32", P * (desc.I // 128) * 4)
        else:
            _arg(x_sorted, "x_sorted", _KIND[desc.act_dtype], P * desc.H * _ELT[desc.act_dtype])
            _arg(h, "h", _KIND[desc.act_dtype], P * desc.I * _ELT[desc.act_dtype])
    _check(_lib.moe_expert_gate_up_swiglu(ctypes.byref(desc), _ptr(x_sorted), _ptr(x_scales),
                                          _ptr(offsets), _ptr(w_gate), _ptr(w_up),
                                          _ptr(w_gate_scales), _ptr(w_up_scales), _ptr(h),
                                          _ptr(h_scales), _ptr(ws), _nbytes(ws), _stream(stream)))


def moe_expert_down(desc, h, h_scales, offsets, w_down, w_down_scales, y_sorted, ws=None, stream=None):
    if _known(desc):
        P = desc.T * desc.k
        _check_weights(desc, None, None, w_down, None, None, w_down_scales)
        _arg(offsets, "offsets", "i32", (desc.E + 1) * 4)
        if _fp8(desc):
            _arg(h, "h", "codes", P * desc.I)
            _arg(h_scales, "h_scales", "f32", P * (desc.I // 128) * 4)
        else:
            _arg(h, "h", _KIND[desc.act_dtype], P * desc.I * _ELT[desc.act_dtype])
        _arg(y_sorted, "y_sorted", _KIND[desc.y_dtype], P * desc.H * _ELT[desc.y_dtype])
    _check(_lib.moe_expert_down(ctypes.byref(desc), _ptr(h), _ptr(h_scales), _ptr(offsets),
                                _ptr(w_down), _ptr(w_down_scales), _ptr(y_sorted), _ptr(ws),
                                _nbytes(ws), _stream(stream)))


def moe_unpermute_combine(desc, y_sorted, inv, topk_w, out, stream=None):
    if _known(desc):
        P = desc.T * desc.k
        _arg(y_sorted, "y_sorted", _KIND[desc.y_dtype], P * desc.H * _ELT[desc.y_dtype])
        _arg(inv, "inv", "i32", P * 4)
        _arg(topk_w, "topk_w", "f32", P * 4)
        _arg(out, "out", _KIND[desc.act_dtype], desc.T * desc.H * _ELT[desc.act_dtype])
    _check(_lib.moe_unpermute_combine(ctypes.byref(desc), _ptr(y_sorted), _ptr(inv), _ptr(topk_w),
                                      _ptr(out), _stream(stream)))


def moe_forward(desc, x, w_router, router_bias, w_gate, w_up, w_down, w_gate_scales, w_up_scales,
                w_down_scales, out, topk_ids_out=None, topk_w_out=None, counts_out=None, ws=None,
                stream=None):
    if _known(desc):
        _check_router(desc, x, w_router, router_bias)
        _check_weights(desc, w_gate, w_up, w_down, w_gate_scales, w_up_scales, w_down_scales)
        _arg(out, "out", _KIND[desc.act_dtype], desc.T * desc.H * _ELT[desc.act_dtype])
        _arg(topk_ids_out, "topk_ids_out", "i32", desc.T * desc.k * 4)
        _arg(topk_w_out, "topk_w_out", "f32", desc.T * desc.k * 4)
        _arg(counts_out, "counts_out", "i32", desc.E * 4)
    _check(_lib.moe_forward(ctypes.byref(desc), _ptr(x), _ptr(w_router), _ptr(router_bias),
                            _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(w_gate_scales),
                            _ptr(w_up_scales), _ptr(w_down_scales), _ptr(out), _ptr(topk_ids_out),
                            _ptr(topk_w_out), _ptr(counts_out), _ptr(ws), _nbytes(ws),
                            _stream(stream)))


MOE_STATIC_SCRATCH_BYTES = 256 << 20


def moe_forward_static(desc, x, w_router, router_bias, w_gate, w_up, w_down, w_gate_scales, w_up_scales,
                       w_down_scales, out, topk_ids_out=None, topk_w_out=None, counts_out=None, stream=None):
    """moe_forward on the library's static scratch (no workspace argument)."""
    if _known(desc):
        _check_router(desc, x, w_router, router_bias)
        _check_weights(desc, w_gate, w_up, w_down, w_gate_scales, w_up_scales, w_down_scales)
        _arg(out, "out", _KIND[desc.act_dtype], desc.T * desc.H * _ELT[desc.act_dtype])
        _arg(topk_ids_out, "topk_ids_out", "i32", desc.T * desc.k * 4)
        _arg(topk_w_out, "topk_w_out", "f32", desc.T * desc.k * 4)
        _arg(counts_out, "counts_out", "i32", desc.E * 4)
    _check(_lib.moe_forward_static(ctypes.byref(desc), _ptr(x), _ptr(w_router), _ptr(router_bias),
                                   _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(w_gate_scales),
                                   _ptr(w_up_scales), _ptr(w_down_scales), _ptr(out), _ptr(topk_ids_out),
                                   _ptr(topk_w_out), _ptr(counts_out), _stream(stream)))


def moe_backward(desc, x, w_router, router_bias, w_gate, w_up, w_down, d_out, dx, dw_router, d_bias,
                 dw_gate, dw_up, dw_down, ws=None, stream=None):
    if _known(desc):
        _check_router(desc, x, w_router, router_bias)
        _check_weights(desc, w_gate, w_up, w_down, None, None, None)
        ea = _ELT[desc.act_dtype]
        _arg(d_out, "d_out", _KIND[desc.act_dtype], desc.T * desc.H * ea)
        _arg(dx, "dx", _KIND[desc.act_dtype], desc.T * desc.H * ea)
        _arg(dw_router, "dw_router", _KIND[desc.act_dtype], desc.E * desc.H * ea)
        _arg(d_bias, "d_bias", "f32", desc.E * 4)
        _check_weights(desc, dw_gate, dw_up, dw_down, None, None, None)
    _check(_lib.moe_backward(ctypes.byref(desc), _ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(w_gate),
                             _ptr(w_up), _ptr(w_down), _ptr(d_out), _ptr(dx), _ptr(dw_router), _ptr(d_bias),
                             _ptr(dw_gate), _ptr(dw_up), _ptr(dw_down), _ptr(ws), _nbytes(ws),
                             _stream(stream)))


def moe_timing_enable(on: bool):
    _check(_lib.moe_timing_enable(int(bool(on))))


def moe_timing_read():
    """{stage: (total ms, launches)} of the stage events recorded since the last read."""
    ms = (ctypes.c_double * MOE_NUM_STAGES)()
    n = (ctypes.c_int64 * MOE_NUM_STAGES)()
    _check(_lib.moe_timing_read(ms, n))
    return {STAGES[i]: (ms[i], n[i]) for i in range(MOE_NUM_STAGES)}
