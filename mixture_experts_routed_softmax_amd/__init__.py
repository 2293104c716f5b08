"""Routed mixture-of-experts forward on AMD MI355X (gfx950): Python binding.

This module only marshals arguments to libmoe.so, the HIP library whose C ABI
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
    _check(_lib.moe_route_topk(ctypes.byref(desc), _ptr(x), _ptr(w_router), _ptr(router_bias),
                               _ptr(topk_ids), _ptr(topk_w), _ptr(ws), _nbytes(ws), _stream(stream)))


def moe_permute(desc, topk_ids, x, counts, offsets, perm, inv, x_sorted=None, x_sorted_scales=None,
                ws=None, stream=None):
    _check(_lib.moe_permute(ctypes.byref(desc), _ptr(topk_ids), _ptr(x), _ptr(counts), _ptr(offsets),
                            _ptr(perm), _ptr(inv), _ptr(x_sorted), _ptr(x_sorted_scales), _ptr(ws),
                            _nbytes(ws), _stream(stream)))


def moe_expert_gate_up_swiglu(desc, x_sorted, x_scales, offsets, w_gate, w_up, w_gate_scales,
                              w_up_scales, h, h_scales, ws=None, stream=None):
    _check(_lib.moe_expert_gate_up_swiglu(ctypes.byref(desc), _ptr(x_sorted), _ptr(x_scales),
                                          _ptr(offsets), _ptr(w_gate), _ptr(w_up),
                                          _ptr(w_gate_scales), _ptr(w_up_scales), _ptr(h),
                                          _ptr(h_scales), _ptr(ws), _nbytes(ws), _stream(stream)))


def moe_expert_down(desc, h, h_scales, offsets, w_down, w_down_scales, y_sorted, ws=None, stream=None):
    _check(_lib.moe_expert_down(ctypes.byref(desc), _ptr(h), _ptr(h_scales), _ptr(offsets),
                                _ptr(w_down), _ptr(w_down_scales), _ptr(y_sorted), _ptr(ws),
                                _nbytes(ws), _stream(stream)))


def moe_unpermute_combine(desc, y_sorted, inv, topk_w, out, stream=None):
    _check(_lib.moe_unpermute_combine(ctypes.byref(desc), _ptr(y_sorted), _ptr(inv), _ptr(topk_w),
                                      _ptr(out), _stream(stream)))


def moe_forward(desc, x, w_router, router_bias, w_gate, w_up, w_down, w_gate_scales, w_up_scales,
                w_down_scales, out, topk_ids_out=None, topk_w_out=None, counts_out=None, ws=None,
                stream=None):
    _check(_lib.moe_forward(ctypes.byref(desc), _ptr(x), _ptr(w_router), _ptr(router_bias),
                            _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(w_gate_scales),
                            _ptr(w_up_scales), _ptr(w_down_scales), _ptr(out), _ptr(topk_ids_out),
                            _ptr(topk_w_out), _ptr(counts_out), _ptr(ws), _nbytes(ws),
                            _stream(stream)))


def moe_backward(desc, x, w_router, router_bias, w_gate, w_up, w_down, d_out, dx, dw_router, d_bias,
                 dw_gate, dw_up, dw_down, ws=None, stream=None):
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
