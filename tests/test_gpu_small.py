"""GPU parity of the HIP path against the fp64 oracle on shapes the oracle
finishes in seconds: the fp32 tiny layer, small bf16 / fp8 layers spanning
several tiles with ragged tails, and the degenerate cases of routing.

Router ids, counts, offsets, perm and inv are compared bit for bit; outputs by
the per-row relative L2 error (1e-5 fp32, 2e-2 bf16, 6e-2 fp8)."""
import numpy as np
import pytest
import torch

import mixture_experts_routed_softmax_amd as moe
import oracle
import synthetic
from moe_cases import (coverage_rows, desc_for, dequant_rows, host, oracle_experts, oracle_route,
                       row_rel_err, run_forward, run_staged, tol_of)

pytestmark = pytest.mark.gpu

SMALL = {
    "tiny": synthetic.spec("tiny"),
    "bf16_softmax": synthetic.spec("qwen_prefill", T=300, H=256, I=384, E=12),
    "bf16_ragged": synthetic.spec("qwen_prefill", T=77, H=192, I=320, E=7, k=3),
    "bf16_sigmoid": synthetic.spec("dsv3_bf16", T=130, H=256, I=256, E=16),
    # >= 256 tokens take the LDS-staged router; 100 experts pad to 128 rows
    "bf16_e100": synthetic.spec("dsv3_bf16", T=320, H=384, I=256, E=100, k=6),
    # 160 experts pad to 256 rows: 128-token router workgroups (the last one
    # ragged) over 4 K slices
    "bf16_e160": synthetic.spec("dsv3_bf16", T=300, H=1024, I=256, E=160, k=6),
    "fp8_f32": synthetic.spec("dsv3_fp8", T=100, H=256, I=384, E=16, k=4),
    "fp8_ue8m0": synthetic.spec("dsv3_fp8", T=100, H=256, I=384, E=16, k=4, scale_fmt="ue8m0"),
    "fp4": synthetic.spec("dsv3_fp4", T=100, H=256, I=384, E=16, k=4),
    # a long reduction (64 K steps of the grouped kernel's pipeline)
    "bf16_long_k": synthetic.spec("dsv3_bf16", T=96, H=4096, I=512, E=8, k=2),
    # fp8 / fp4 grouped kernels past their three-block head (17 blocks of 128
    # K), experts with several 32-row token tiles, and a down tile cut at
    # H = 2176 (8.5 tiles of 256 channels)
    "fp8_long_k": synthetic.spec("dsv3_fp8", T=160, H=2176, I=640, E=4, k=2),
    "fp4_long_k": synthetic.spec("dsv3_fp4", T=160, H=2176, I=640, E=4, k=2),
}


def _layer(s, seed=0):
    L = synthetic.make_layer(s, seed=seed, device="cuda")
    return L, host(L)


LAYOUTS = {name: (["rowmajor"] if s.experts == "f32" else (["packed"] if s.experts == "fp4" else ["rowmajor", "packed"]))
           for name, s in SMALL.items()}
CASES = [(n, lay) for n in SMALL for lay in LAYOUTS[n]]


def _check_forward(s, L, hl, seed=0, y_dtype=None, layout="rowmajor"):
    ids_o, w_o = oracle_route(s, hl)
    counts_o, offsets_o, perm_o, inv_o = oracle.permute(ids_o, s.E)
    out, ids, w, counts = run_forward(s, L, y_dtype=y_dtype, layout=layout)
    assert np.array_equal(ids.cpu().numpy(), ids_o), "router ids differ from the oracle"
    assert np.array_equal(counts.cpu().numpy(), counts_o)
    np.testing.assert_allclose(w.cpu().numpy(), w_o, rtol=1e-5, atol=1e-7)
    ex = oracle_experts(s, hl)
    out_o = ex.combine(hl["x"], ids_o, w_o)
    err = row_rel_err(out.cpu().float().numpy(), out_o)
    print("%s: max row rel err %.3e (tol %.0e)" % (s.name, err, tol_of(s)))
    assert err <= tol_of(s)
    return out


@pytest.mark.parametrize("name,layout", CASES)
def test_forward_small(name, layout):
    s = SMALL[name]
    L, hl = _layer(s)
    _check_forward(s, L, hl, layout=layout)


@pytest.mark.parametrize("name,layout", CASES)
def test_staged_small(name, layout):
    s = SMALL[name]
    L, hl = _layer(s, seed=1)
    ids_o, w_o = oracle_route(s, hl)
    # the router entry point alone
    ids = torch.empty(s.T, s.k, dtype=torch.int32, device="cuda")
    w = torch.empty(s.T, s.k, dtype=torch.float32, device="cuda")
    d = desc_for(s, layout=layout)
    moe.moe_route_topk(d, L["x"], L["w_router"], L["router_bias"], ids, w, moe.workspace(d, moe.MOE_OP_ROUTE))
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), ids_o)
    np.testing.assert_allclose(w.cpu().numpy(), w_o, rtol=1e-5, atol=1e-7)
    # the rest of the chain on the oracle's routing
    ids_in = torch.from_numpy(ids_o).cuda()
    w_in = torch.from_numpy(w_o.astype(np.float32)).cuda()
    r = run_staged(s, L, ids_in, w_in, layout=layout)
    counts_o, offsets_o, perm_o, inv_o = oracle.permute(ids_o, s.E)
    assert np.array_equal(r["counts"].cpu().numpy(), counts_o)
    assert np.array_equal(r["offsets"].cpu().numpy(), offsets_o)
    assert np.array_equal(r["perm"].cpu().numpy(), perm_o)
    assert np.array_equal(r["inv"].cpu().numpy(), inv_o)
    tok = perm_o // s.k
    if s.experts in ("fp8", "fp4"):
        codes_o, scales_o = oracle.quant_rows(hl["x"], 128)
        # compare code values (the GPU encodes -0 as 0x80, the oracle as 0x00)
        xs = r["x_sorted"].cpu().view(torch.float8_e4m3fn).float().numpy()
        xo = torch.from_numpy(codes_o[tok]).view(torch.float8_e4m3fn).float().numpy()
        sc = r["x_scales"].cpu().numpy()
        assert np.array_equal(sc, scales_o[tok])
        mism = np.mean(xs != xo)
        assert mism < 1e-3, "activation code mismatch rate %.2e" % mism
    else:
        assert torch.equal(r["x_sorted"].cpu(), hl["x"][torch.from_numpy(tok)])
    ex = oracle_experts(s, hl)
    rows = coverage_rows(offsets_o, 64)
    h_o, y_o = ex.pairs(hl["x"], tok[rows], ids_o.reshape(-1)[perm_o[rows]])
    if s.experts in ("fp8", "fp4"):
        h = dequant_rows(r["h"][torch.from_numpy(rows).cuda()], r["h_scales"][torch.from_numpy(rows).cuda()])
    else:
        h = r["h"].cpu().float().numpy()[rows]
    tol = tol_of(s)
    assert row_rel_err(h, h_o) <= tol
    assert row_rel_err(r["y"].cpu().float().numpy()[rows], y_o) <= tol
    out_o = ex.combine(hl["x"], ids_o, w_o)
    assert row_rel_err(r["out"].cpu().float().numpy(), out_o) <= tol


def test_forward_deterministic():
    s = SMALL["bf16_softmax"]
    L, _ = _layer(s, seed=3)
    a = run_forward(s, L)[0]
    b = run_forward(s, L)[0]
    assert torch.equal(a, b)


@pytest.mark.parametrize("layout", ["rowmajor", "packed"])
def test_forward_f32_intermediate_rows(layout):
    s = SMALL["bf16_sigmoid"]
    L, hl = _layer(s, seed=4)
    _check_forward(s, L, hl, y_dtype="f32", layout=layout)


@pytest.mark.parametrize("name", ["fp8_f32", "fp4_long_k"])
def test_fp8_forward_f32_intermediate_rows(name):
    """fp8 / fp4 experts with float32 y rows: the down projection then runs on
    the packed kernel (the grouped e4m3 kernel writes bf16 y only)."""
    s = SMALL[name]
    L, hl = _layer(s, seed=4)
    _check_forward(s, L, hl, y_dtype="f32", layout="packed")


@pytest.mark.parametrize("name", ["bf16_ragged", "fp8_f32"])
def test_packed_layout_bytes(name):
    """moe_pack_weights writes the layout include/moe.h documents (checked
    against a numpy construction of that description)."""
    s = SMALL[name]
    L = synthetic.make_layer(s, seed=2, device="cuda")
    d = desc_for(s, layout="packed")
    gu, dn = moe.pack_experts(d, L["w_gate"], L["w_up"], L["w_down"])
    torch.cuda.synchronize()

    def raw(t):
        t = t.cpu().contiguous()
        return t.view(torch.uint8).numpy().reshape(t.shape[0], t.shape[1], -1)

    def expect(mats, rows_per_tile):
        E, N, RB = mats[0].shape
        NT = -(-N // (rows_per_tile // len(mats)))
        KT = RB // 64
        out = np.zeros((E, NT, KT, 256, 4, 16), np.uint8)
        rows = np.arange(256)
        for nt in range(NT):
            for m, W in enumerate(mats):
                per = 256 // len(mats)
                n = nt * per + np.arange(per)
                ok = n < N
                for kt in range(KT):
                    for p in range(4):
                        r = m * per + np.arange(per)
                        c = p ^ ((r >> 2) & 3)
                        for i in np.nonzero(ok)[0]:
                            out[:, nt, kt, r[i], p, :] = W[:, n[i], kt * 64 + c[i] * 16: kt * 64 + c[i] * 16 + 16]
        return out.reshape(-1)

    assert np.array_equal(gu.cpu().numpy(), expect([raw(L["w_gate"]), raw(L["w_up"])], 256))
    assert np.array_equal(dn.cpu().numpy(), expect([raw(L["w_down"])], 256))


# ------------------------------------------------------------------ edge cases

def test_single_token():
    s = synthetic.spec("qwen_prefill", T=1, H=256, I=256, E=12)
    L, hl = _layer(s, seed=5)
    _check_forward(s, L, hl)


def test_empty_batch():
    s = synthetic.spec("qwen_prefill", T=0, H=256, I=256, E=12)
    L = synthetic.make_layer(s, device="cuda")
    d = desc_for(s)
    counts = torch.full((s.E,), -1, dtype=torch.int32, device="cuda")
    out = torch.empty(0, s.H, dtype=torch.bfloat16, device="cuda")
    ws = moe.workspace(d, moe.MOE_OP_FORWARD)
    moe.moe_forward(d, L["x"], L["w_router"], L["router_bias"], L["w_gate"], L["w_up"], L["w_down"],
                    None, None, None, out, None, None, counts, ws)
    torch.cuda.synchronize()
    assert not counts.cpu().any()


def test_k_equals_E():
    s = synthetic.spec("qwen_prefill", T=40, H=128, I=128, E=4, k=4)
    L, hl = _layer(s, seed=6)
    out = _check_forward(s, L, hl)


def test_one_expert():
    s = synthetic.spec("qwen_prefill", T=50, H=128, I=192, E=1, k=1, bias="none")
    L, hl = _layer(s, seed=7)
    _check_forward(s, L, hl)


def test_all_tokens_on_one_expert():
    s = synthetic.spec("qwen_prefill", T=260, H=128, I=256, E=8, k=1)
    L, hl = _layer(s, seed=8)
    b = torch.zeros(s.E, dtype=torch.float32, device="cuda")
    b[5] = 64.0
    L["router_bias"] = b
    hl["router_bias"] = b.cpu()
    out = _check_forward(s, L, hl)
    _, ids, _, counts = run_forward(s, L)
    assert counts.cpu().tolist() == [0, 0, 0, 0, 0, 260, 0, 0]


@pytest.mark.parametrize("layout", ["rowmajor", "packed"])
def test_max_experts_and_topk(layout):
    # the largest E and k the library takes (256 experts, 32 per token)
    s = synthetic.spec("dsv3_bf16", T=40, H=128, I=128, E=256, k=32)
    L, hl = _layer(s, seed=12)
    _check_forward(s, L, hl, layout=layout)


@pytest.mark.parametrize("T", [1024, 1025])
def test_permutation_chunk_boundary(T):
    # 1024 (token, slot) pairs run the one-workgroup permutation, 1025 the
    # histogram / scan / scatter launches
    s = synthetic.spec("qwen_prefill", T=T, H=128, I=128, E=12, k=1)
    L, hl = _layer(s, seed=13)
    ids_o, _ = oracle_route(s, hl)
    _, offsets_o, perm_o, inv_o = oracle.permute(ids_o, s.E)
    _check_forward(s, L, hl, layout="packed")
    d = desc_for(s)
    counts = torch.empty(s.E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(s.E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(T, dtype=torch.int32, device="cuda")
    inv = torch.empty(T, dtype=torch.int32, device="cuda")
    ids = torch.from_numpy(ids_o).cuda()
    ws = moe.workspace(d, moe.MOE_OP_PERMUTE)
    moe.moe_permute(d, ids, None, counts, offsets, perm, inv, ws=ws)
    torch.cuda.synchronize()
    assert np.array_equal(offsets.cpu().numpy(), offsets_o)
    assert np.array_equal(perm.cpu().numpy(), perm_o)
    assert np.array_equal(inv.cpu().numpy(), inv_o)


@pytest.mark.parametrize("T,k", [(1, 8), (16, 4), (16, 32), (17, 4), (32, 32)])
def test_small_batch_selection_in_permute(T, k):
    """Batches of at most 16 tokens select their experts inside the
    one-workgroup permutation launch (17 or more take the separate selection
    launch); ids, weights, counts and outputs must match the oracle on both
    sides of the boundary, with up to 32 experts per token."""
    s = synthetic.spec("dsv3_bf16", T=T, H=256, I=128, E=64, k=k)
    L, hl = _layer(s, seed=21)
    _check_forward(s, L, hl, layout="packed")


@pytest.mark.parametrize("T", [16, 64])
def test_exact_ties_break_to_lowest_index(T):
    s = synthetic.spec("qwen_prefill", T=T, H=128, I=128, E=10, k=3, bias="none")
    L, hl = _layer(s, seed=9)
    for dup in (4, 7, 9):
        L["w_router"][dup] = L["w_router"][2]
    hl = host(L)
    ids_o, _ = oracle_route(s, hl)
    _, ids, _, _ = run_forward(s, L)
    assert np.array_equal(ids.cpu().numpy(), ids_o)
    # duplicated experts appear together, in ascending order
    got = ids.cpu().numpy()
    for row in got:
        dup_pos = [list(row).index(e) for e in (2, 4, 7, 9) if e in row]
        assert dup_pos == sorted(dup_pos)


# ------------------------------------------------------- weight-streaming path

STREAM = {
    "bf16_decode": synthetic.spec("qwen_decode", T=40, H=256, I=384, E=12),
    "bf16_decode_t1": synthetic.spec("qwen_decode", T=1, H=256, I=384, E=12),
    "bf16_decode_hot": synthetic.spec("qwen_decode", T=64, H=256, I=256, E=4, k=2),   # > 32 rows per expert
    "fp8_decode_f32": synthetic.spec("dsv3_fp8", T=24, H=256, I=384, E=16, k=4),
    "fp8_decode_ue8m0": synthetic.spec("dsv3_fp8", T=64, H=256, I=256, E=6, k=3, scale_fmt="ue8m0"),
    # K deep enough that few touched experts split K over several workgroups
    # (split-K partials summed by the reduction launch)
    "bf16_decode_split_hot": synthetic.spec("qwen_decode", T=64, H=512, I=256, E=4, k=2),
    "fp8_decode_split": synthetic.spec("dsv3_fp8", T=8, H=1024, I=512, E=16, k=4),
    "fp8_decode_split_hot_ue8m0": synthetic.spec("dsv3_fp8", T=64, H=1024, I=512, E=4, k=2, scale_fmt="ue8m0"),
    # int8-packed FP4 experts (UE8M0 per row per 32 K): one tile per item,
    # split K, and experts with more than 32 rows
    "fp4_decode": synthetic.spec("dsv3_fp4", T=24, H=256, I=384, E=16, k=4),
    "fp4_decode_split": synthetic.spec("dsv3_fp4", T=8, H=1024, I=512, E=16, k=4),
    "fp4_decode_split_hot": synthetic.spec("dsv3_fp4", T=64, H=1024, I=512, E=4, k=2),
}


@pytest.mark.parametrize("name", list(STREAM))
def test_stream_forward(name):
    s = STREAM[name]
    L, hl = _layer(s, seed=12)
    ids_o, w_o = oracle_route(s, hl)
    out, ids, w, counts = run_forward(s, L, path="stream", layout="packed")
    assert np.array_equal(ids.cpu().numpy(), ids_o)
    ex = oracle_experts(s, hl)
    out_o = ex.combine(hl["x"], ids_o, w_o)
    err = row_rel_err(out.cpu().float().numpy(), out_o)
    print("%s stream: max row rel err %.3e" % (name, err))
    assert err <= tol_of(s)
    if "hot" in name:
        assert int(counts.max()) > 32


@pytest.mark.parametrize("y_dtype", [None, "f32"])
def test_stream_combine_sums_down_partials(y_dtype):
    """A decode batch whose down launch would be unsplit with as many
    touched experts as it could have (512 items on 512 workgroups), so the
    forward leaves out the down reduction launch; routing concentrated on 8
    experts makes the launch split after all, and the combine sums the
    partial tiles itself."""
    s = synthetic.spec("dsv3_bf16", T=64, H=512, I=256, E=256, k=8)
    L, hl = _layer(s, seed=21)
    b = torch.zeros(s.E, dtype=torch.float32, device="cuda")
    b[:8] = 64.0
    L["router_bias"] = b
    hl["router_bias"] = b.cpu()
    ids_o, w_o = oracle_route(s, hl)
    out, ids, w, counts = run_forward(s, L, path="stream", y_dtype=y_dtype, layout="packed")
    assert np.array_equal(ids.cpu().numpy(), ids_o)
    assert int((counts > 0).sum()) == 8
    out_o = oracle_experts(s, hl).combine(hl["x"], ids_o, w_o)
    err = row_rel_err(out.cpu().float().numpy(), out_o)
    print("concentrated stream (y %s): max row rel err %.3e" % (y_dtype, err))
    assert err <= tol_of(s)


# batches of at most 16 tokens: the combine takes one workgroup per (token, 32
# channels) and sums a split down launch's partial tiles itself
FINE = {
    # 16 slots x 16 splits: two chunks of (slot, split) pairs in LDS
    "t1_k16_split": synthetic.spec("qwen_decode", T=1, H=512, I=2048, E=64, k=16),
    # enough touched experts that the down launch is not split: y is read
    "t16_unsplit": synthetic.spec("dsv3_bf16", T=16, H=2048, I=256, E=256, k=8),
}


@pytest.mark.parametrize("y_dtype", [None, "f32"])
@pytest.mark.parametrize("name", list(FINE))
def test_stream_fine_combine(name, y_dtype):
    s = FINE[name]
    L, hl = _layer(s, seed=23)
    ids_o, w_o = oracle_route(s, hl)
    out, ids, w, counts = run_forward(s, L, path="stream", y_dtype=y_dtype, layout="packed")
    assert np.array_equal(ids.cpu().numpy(), ids_o)
    out_o = oracle_experts(s, hl).combine(hl["x"], ids_o, w_o)
    err = row_rel_err(out.cpu().float().numpy(), out_o)
    print("%s fine combine (y %s): max row rel err %.3e" % (name, y_dtype, err))
    assert err <= tol_of(s)


@pytest.mark.parametrize("name", ["bf16_decode", "fp8_decode_f32"])
def test_stream_staged_matches_oracle(name):
    s = STREAM[name]
    L, hl = _layer(s, seed=13)
    ids_o, w_o = oracle_route(s, hl)
    r = run_staged(s, L, torch.from_numpy(ids_o).cuda(), torch.from_numpy(w_o.astype(np.float32)).cuda(),
                   layout="packed", path="stream")
    out_o = oracle_experts(s, hl).combine(hl["x"], ids_o, w_o)
    assert row_rel_err(r["out"].cpu().float().numpy(), out_o) <= tol_of(s)


def test_stream_and_grouped_paths_agree():
    s = STREAM["bf16_decode"]
    L, _ = _layer(s, seed=14)
    a = run_forward(s, L, path="stream", layout="packed")[0].float()
    b = run_forward(s, L, path="grouped", layout="packed")[0].float()
    rel = ((a - b).norm(dim=1) / b.norm(dim=1)).max().item()
    assert rel < 1e-2


def test_forward_replays_as_graph():
    """The forward only enqueues work: captured once into a HIP graph, every
    replay (with eager work and synchronisation in between) reproduces the
    eager result bit for bit."""
    s = STREAM["fp8_decode_split"]
    L, _ = _layer(s, seed=15)
    d = desc_for(s, s.T, path="stream", layout="packed")
    gu, dn = moe.pack_experts(d, L["w_gate"], L["w_up"], L["w_down"], "cuda")
    out = torch.empty(s.T, s.H, dtype=torch.bfloat16, device="cuda")
    ws = moe.workspace(d, moe.MOE_OP_FORWARD, "cuda")

    def step():
        moe.moe_forward(d, L["x"], L["w_router"], L["router_bias"], gu, None, dn, L["s_gate"], L["s_up"],
                        L["s_down"], out, None, None, None, ws)

    step()
    torch.cuda.synchronize()
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        step()   # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, ref)


# GeGLU / ReGLU experts ("Experts backends", section "SonicMoE": gated
# activation silu, gelu or relu) on every expert-GEMM kernel family: fp32,
# bf16 and fp8 grouped GEMMs (row-major and packed weights) and the
# weight-streaming GEMMs with split-K reduction.
GATE_CASES = [(g, name, layout, path) for g in ("gelu", "relu") for name, layout, path in [
    ("tiny", "rowmajor", "grouped"), ("bf16_softmax", "rowmajor", "grouped"),
    ("bf16_softmax", "packed", "grouped"), ("fp8_f32", "rowmajor", "grouped"),
    ("fp8_ue8m0", "packed", "grouped"), ("bf16_decode_split_hot", "packed", "stream"),
    ("fp8_decode_split", "packed", "stream"), ("fp4_decode_split", "packed", "stream"),
    ("fp4", "packed", "grouped")]]


@pytest.mark.parametrize("gate,name,layout,path", GATE_CASES)
def test_gated_activation_variants(gate, name, layout, path):
    import dataclasses
    s = dataclasses.replace(SMALL[name] if name in SMALL else STREAM[name], gate=gate)
    L, hl = _layer(s, seed=16)
    ids_o, w_o = oracle_route(s, hl)
    out, ids, w, counts = run_forward(s, L, path=path, layout=layout)
    assert np.array_equal(ids.cpu().numpy(), ids_o)
    out_o = oracle_experts(s, hl).combine(hl["x"], ids_o, w_o)
    err = row_rel_err(out.cpu().float().numpy(), out_o)
    print("%s %s %s %s: max row rel err %.3e" % (gate, name, layout, path, err))
    assert err <= tol_of(s)


def test_stage_timing_counts_every_launch():
    """Stage timing: every launch of a forward is counted once under its
    stage with a positive duration (launches of one call are timed back to
    back), and the stage times of a call add up to no more than its wall time."""
    s = SMALL["bf16_softmax"]            # 1200 pairs: the multi-chunk permutation (histogram inside the scan)
    L, _ = _layer(s)
    run_forward(s, L, layout="packed")
    torch.cuda.synchronize()
    moe.moe_timing_enable(True)
    moe.moe_timing_read()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(3):
        run_forward(s, L, layout="packed")
    stop.record()
    torch.cuda.synchronize()
    st = moe.moe_timing_read()
    moe.moe_timing_enable(False)
    for name in ("route", "scan", "scatter", "gate_up", "down", "combine"):
        ms, n = st[name]
        assert n == 3 and ms > 0, (name, ms, n)
    assert st["hist"][1] == 0   # at most 32 chunks: no histogram launch of its own
    assert sum(ms for ms, _ in st.values()) <= start.elapsed_time(stop) * 1.001
    assert moe.moe_timing_read()["gate_up"][1] == 0


# ------------------------------------------------------------------ non-finite and invalid input

NAN_CASES = [
    ("qwen_prefill", 12, "packed"),      # selection inside the permutation launch, weight streaming
    ("qwen_prefill", 40, "packed"),      # separate selection launch, weight streaming
    ("qwen_prefill", 300, "packed"),     # LDS-staged router, grouped GEMM
    ("qwen_prefill", 300, "rowmajor"),
    ("dsv3_fp8", 40, "packed"),
    ("dsv3_fp8", 300, "packed"),
]


@pytest.mark.parametrize("name,T,layout", NAN_CASES)
def test_nan_token(name, T, layout):
    """A NaN in one token's hidden state makes all of its keys NaN; they rank
    as -inf, so the token takes experts 0..k-1 (as in the oracle), its output
    row is not finite and every other row still matches the oracle."""
    over = dict(T=T, H=256, I=384, E=16, k=4)
    s = synthetic.spec(name, **over)
    L = synthetic.make_layer(s, seed=31, device="cuda")
    t0 = T // 3
    L["x"][t0, 5] = float("nan")
    hl = host(L)
    ids_o, w_o = oracle_route(s, hl)
    assert list(ids_o[t0]) == list(range(s.k))
    out, ids, w, counts = run_forward(s, L, layout=layout)
    got_ids = ids.cpu().numpy()
    assert ((got_ids >= 0) & (got_ids < s.E)).all()
    assert np.array_equal(got_ids, ids_o)
    assert int(counts.cpu().sum()) == T * s.k
    o = out.cpu().float().numpy()
    assert not np.isfinite(o[t0]).any()
    rest = np.array([t for t in range(T) if t != t0])
    ref = oracle_experts(s, hl).combine(hl["x"], ids_o, w_o, rest)
    assert np.isfinite(o[rest]).all()
    assert row_rel_err(o[rest], ref) <= tol_of(s)


@pytest.mark.parametrize("T", [2049, 4096, 4097, 8193])
def test_permute_histogram_paths(T):
    """Up to 32 chunks of 1024 pairs the chunk histograms are taken inside the
    scan launch (T = 2049 and 4096 with k = 8: 17 and 32 chunks); above that
    a histogram launch precedes it (T = 4097 and 8193: 33 and 65 chunks).
    Skewed ids, checked bit for bit against the oracle's permutation."""
    s = synthetic.spec("dsv3_bf16", T=T, H=128, I=128, E=256, k=8)
    rng = np.random.default_rng(T)
    pz = 1.0 / np.arange(1, s.E + 1) ** 1.1
    ids = rng.choice(s.E, size=(T, s.k), p=pz / pz.sum()).astype(np.int32)
    counts_o, offsets_o, perm_o, inv_o = oracle.permute(ids, s.E)
    d = desc_for(s)
    P = T * s.k
    counts = torch.empty(s.E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(s.E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(P, dtype=torch.int32, device="cuda")
    inv = torch.empty(P, dtype=torch.int32, device="cuda")
    moe.moe_permute(d, torch.from_numpy(ids).cuda(), None, counts, offsets, perm, inv,
                    ws=moe.workspace(d, moe.MOE_OP_PERMUTE))
    torch.cuda.synchronize()
    assert np.array_equal(counts.cpu().numpy(), counts_o)
    assert np.array_equal(offsets.cpu().numpy(), offsets_o)
    assert np.array_equal(perm.cpu().numpy(), perm_o)
    assert np.array_equal(inv.cpu().numpy(), inv_o)


@pytest.mark.parametrize("T", [100, 1500])
def test_permute_out_of_range_ids(T):
    """Ids outside [0, E) (a caller's bad input to the staged calls) get no
    row: counts, offsets and perm cover the valid pairs in the stable order,
    inv is -1 for the others, and the combine skips them."""
    s = synthetic.spec("qwen_prefill", T=T, H=128, I=128, E=12, k=2)
    rng = np.random.default_rng(5)
    ids = rng.integers(0, s.E, (T, s.k)).astype(np.int32)
    bad = rng.random((T, s.k)) < 0.1
    ids[bad] = rng.choice(np.array([-1, s.E, 1000, -77], dtype=np.int32), int(bad.sum()))
    flat = ids.ravel()
    valid = (flat >= 0) & (flat < s.E)
    counts_ref = np.bincount(flat[valid], minlength=s.E)
    offsets_ref = np.concatenate([[0], np.cumsum(counts_ref)])
    perm_ref = np.flatnonzero(valid)[np.argsort(flat[valid], kind="stable")]
    inv_ref = np.full(flat.size, -1)
    inv_ref[perm_ref] = np.arange(perm_ref.size)
    d = desc_for(s)
    P = T * s.k
    counts = torch.empty(s.E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(s.E + 1, dtype=torch.int32, device="cuda")
    perm = torch.full((P,), -9, dtype=torch.int32, device="cuda")
    inv = torch.full((P,), -9, dtype=torch.int32, device="cuda")
    moe.moe_permute(d, torch.from_numpy(ids).cuda(), None, counts, offsets, perm, inv,
                    ws=moe.workspace(d, moe.MOE_OP_PERMUTE))
    torch.cuda.synchronize()
    assert np.array_equal(counts.cpu().numpy(), counts_ref)
    assert np.array_equal(offsets.cpu().numpy(), offsets_ref)
    n = perm_ref.size
    assert np.array_equal(perm.cpu().numpy()[:n], perm_ref)
    assert np.array_equal(inv.cpu().numpy(), inv_ref)
    # combine over the valid rows only
    y = torch.randn(P, s.H, device="cuda").to(torch.bfloat16)
    wt = torch.rand(T, s.k, device="cuda")
    out = torch.empty(T, s.H, dtype=torch.bfloat16, device="cuda")
    moe.moe_unpermute_combine(d, y, inv, wt, out)
    torch.cuda.synchronize()
    y64 = y.cpu().double().numpy()
    w64 = wt.cpu().double().numpy().ravel()
    ref = np.zeros((T, s.H))
    for p in np.flatnonzero(valid):
        ref[p // s.k] += w64[p] * y64[inv_ref[p]]
    np.testing.assert_allclose(out.cpu().double().numpy(), ref, rtol=1e-2, atol=1e-2)
