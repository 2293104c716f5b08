"""moe_forward_static (the forward on the library's static scratch, for
callers that cannot allocate) against moe_forward on a caller workspace.

Through the C ABI: two calls in a row on one device, the second with a
smaller batch, each compared with moe_forward on the same inputs (ids,
weights and counts bit for bit; outputs within the layer tolerance), on the
weight-streaming (decode) and the grouped-GEMM (prefill) paths; and the
rejection of a layer whose workspace exceeds the static scratch."""
import numpy as np
import pytest
import torch

import mixture_experts_routed_softmax_amd as moe
import synthetic
from moe_cases import act_dtype, desc_for, expert_weights, row_rel_err, tol_of

pytestmark = pytest.mark.gpu


def _both(s, L, layout="packed"):
    d = desc_for(s, layout=layout)
    assert moe.moe_workspace_bytes(d, moe.MOE_OP_FORWARD) <= moe.MOE_STATIC_SCRATCH_BYTES
    wg, wu, wd = expert_weights(d, L)
    res = []
    for static in (False, True):
        out = torch.full((s.T, s.H), float("nan"), dtype=act_dtype(s), device="cuda")
        ids = torch.full((s.T, s.k), -5, dtype=torch.int32, device="cuda")
        w = torch.full((s.T, s.k), -5.0, dtype=torch.float32, device="cuda")
        counts = torch.full((s.E,), -5, dtype=torch.int32, device="cuda")
        args = (d, L["x"], L["w_router"], L["router_bias"], wg, wu, wd, L.get("s_gate"), L.get("s_up"),
                L.get("s_down"), out, ids, w, counts)
        if static:
            moe.moe_forward_static(*args)
        else:
            moe.moe_forward(*args, ws=moe.workspace(d, moe.MOE_OP_FORWARD))
        torch.cuda.synchronize()
        res.append((out.cpu().float().numpy(), ids.cpu().numpy(), w.cpu().numpy(), counts.cpu().numpy()))
    (o0, i0, w0, c0), (o1, i1, w1, c1) = res
    assert np.array_equal(i1, i0)
    assert np.array_equal(w1, w0)
    assert np.array_equal(c1, c0)
    assert np.isfinite(o1).all()
    err = row_rel_err(o1, o0)
    print("%s T=%d: static-scratch forward vs moe_forward max row rel err %.3e (bitwise equal: %s)"
          % (s.name, s.T, err, bool(np.array_equal(o1, o0))))
    assert err <= tol_of(s)


@pytest.mark.parametrize("name,T0,T1", [("qwen_decode", 64, 8), ("dsv3_fp8", 64, 1),
                                        ("qwen_prefill", 4096, 1000)])
def test_static_forward_twice(name, T0, T1):
    for i, T in enumerate((T0, T1)):
        s = synthetic.spec(name, T=T)
        L = synthetic.make_layer(s, seed=60 + i, device="cuda")
        _both(s, L)


def test_static_forward_rejects_large_layer():
    s = synthetic.spec("dsv3_bf16")
    d = desc_for(s, layout="packed")
    assert moe.moe_workspace_bytes(d, moe.MOE_OP_FORWARD) > moe.MOE_STATIC_SCRATCH_BYTES
    with pytest.raises(moe.MoeError) as ex:
        moe.moe_forward_static(d, None, None, None, None, None, None, None, None, None, None)
    assert ex.value.status == moe.MOE_EWORKSPACE
    assert "static scratch" in moe.moe_last_error()
