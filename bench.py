"""Throughput of the routed mixture-of-experts layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--T N]
                    [--scale-fmt f32|ue8m0] [--no-cpu-baseline] [--no-decode-extra]
                    [--decode-steps N] [--backward]

A step is one moe_forward call (router, permutation, gate/up + SwiGLU, down,
combine) over one batch of T synthetic tokens whose inputs and weights are
already resident in HBM.  W untimed warmup steps are followed by exactly K
timed steps (default 20), bracketed by torch.cuda.synchronize();
value = T / (elapsed / K).

Expert weights are packed into the tile-contiguous layout once before the
timed steps (moe_pack_weights, a model-load transform; --layout rowmajor
times the unpacked kernels instead).

The default workload is the largest prefill layer, the DeepSeek-V3-like one
(T=8192, H=7168, I=2048, E=256, top-8 sigmoid renormalised x 2.5,
Zipf-skewed router bias, bf16, 22.5 GB of expert weights).  Other workloads
(--config) print the same line.  The JSON line also carries:

* roofline: the gate/up grouped GEMM (two thirds of the layer's FLOPs) for
  prefill workloads, priced at its algorithmic FLOPs 2*P*H*2I against the dense
  MFMA peak of its dtype, plus the whole layer's fraction (layer_frac: expert
  FLOPs 6*P*H*I over the step time); for decode workloads (T <= 64) the whole
  step's touched-expert weight bytes against 8 TB/s.  Kernel durations come
  from HIP events the library records around each of its launches on the
  caller's stream during the timed steps.
* decode (prefill lines): the Qwen-like decode layer at T=1 and T=64, each
  the median of --decode-steps (default 200) individually timed steps with the
  last-level cache evicted before each, as the fraction of 8 TB/s that the
  touched experts' weight bytes give.  A decode workload's own line
  (--config qwen_decode) is timed the same way.
* cpu_baseline: the fp64 oracle (never tuned) on the host cores, on a bounded
  sample: the router over all T tokens plus the expert MLPs and the combine on
  a sample of tokens sized to about 10 s; tokens/s = 1 / (router time per
  token + expert time per token).

--backward times moe_backward instead (every gradient of the layer, bf16
row-major experts): value = T * K / elapsed, the roofline of its dominant GEMM
stage, and the oracle's backward on a bounded sample as cpu_baseline.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "fp4": 5000.0, "f32": 157.3}   # fp4 experts: fp8 x fp4 MFMA
PEAK_HBM_GBS = 8000.0
METRIC = "MoE-layer tokens/s; % MFMA peak (prefill), % HBM BW (decode)"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None,
                   help="timed steps (default 20; decode workloads: --decode-steps)")
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--decode-steps", type=int, default=200,
                   help="individually timed steps of a decode measurement (median reported)")
    p.add_argument("--no-decode-extra", dest="decode_extra", action="store_false",
                   help="prefill workloads: skip the Qwen-like decode measurements at T=1 and T=64")
    p.add_argument("--config", default="dsv3_bf16",
                   choices=["tiny", "qwen_prefill", "qwen_decode", "dsv3_bf16", "dsv3_fp8", "dsv3_fp4",
                            "dsv3_ep8_shard"])
    p.add_argument("--T", type=int, default=None)
    p.add_argument("--scale-fmt", default="f32", choices=["f32", "ue8m0"])
    p.add_argument("--gate", default="silu", choices=["silu", "gelu", "relu"],
                   help="gated activation of the experts (SwiGLU, GeGLU, ReGLU)")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device copy (to scale rocprofv3 byte counters) and exit")
    p.add_argument("--layout", default="packed", choices=["packed", "rowmajor"],
                   help="expert-weight layout; packed weights are written once before timing")
    p.add_argument("--graph", default="off", choices=["auto", "off"],
                   help="decode: replay each timed step as a captured HIP graph (auto) or launch eagerly "
                        "(off, the default: measured faster on this stack)")
    p.add_argument("--backward", action="store_true",
                   help="time moe_backward (every gradient of the layer) instead of the forward")
    p.add_argument("--flush", default="read", choices=["read", "write"],
                   help="decode: evict the last-level cache between timed steps by reading (default) "
                        "or by rewriting a 2 GiB buffer")
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def recorded_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from its committed rocprofv3 counter
    record (profiles/*.<workload>.traffic.json, FETCH_SIZE and WRITE_SIZE scaled
    by a plain-copy calibration), or None if there is none or the kernel's
    source changed since the counters were taken."""
    import glob
    import hashlib
    for path in glob.glob(os.path.join(ROOT, "profiles", "*.%s.traffic.json" % workload)):
        rec = json.load(open(path))
        if rec.get("kernel") != kernel:
            continue
        src = os.path.join(ROOT, rec["source"])
        if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest() != rec["source_sha256"]:
            return None
        return rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
    return None


def cpu_baseline(s, hl, budget_s: float):
    """Time the fp64 oracle on a bounded sample of this workload (hl: the
    layer's tensors in host memory)."""
    import numpy as np
    import oracle

    score = oracle.SOFTMAX if s.score == "softmax" else oracle.SIGMOID
    gate = {"silu": oracle.GATE_SILU, "gelu": oracle.GATE_GELU, "relu": oracle.GATE_RELU}[s.gate]
    t0 = time.perf_counter()
    ids, w = oracle.route(hl["x"], hl["w_router"], hl["router_bias"], s.k, score, s.renormalize,
                          s.routed_scale)
    t_route = time.perf_counter() - t0
    if s.experts in ("fp8", "fp4"):
        fmt = oracle.SCALE_UE8M0 if s.scale_fmt == "ue8m0" else oracle.SCALE_F32
        ex = oracle.Experts(hl["w_gate"], hl["w_up"], hl["w_down"], hl["s_gate"], hl["s_up"],
                            hl["s_down"], fmt, s.block, act_fp8=True, gate=gate, fp4=s.experts == "fp4")
    else:
        ex = oracle.Experts(hl["w_gate"], hl["w_up"], hl["w_down"], gate=gate)
    rng = np.random.default_rng(0)
    order = rng.permutation(s.T)
    n, t_exp, done = 8, 0.0, 0
    while done < s.T:
        batch = order[done:done + n]
        t0 = time.perf_counter()
        ex.combine(hl["x"], ids, w, batch)
        t_exp += time.perf_counter() - t0
        done += batch.size
        if t_exp + t_route >= budget_s:
            break
        per = t_exp / done
        n = int(min(max(8, (budget_s - t_exp - t_route) / per), s.T - done))
        if n <= 0:
            break
    per_token = t_route / s.T + t_exp / done
    return {"value": 1.0 / per_token, "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "fp64 oracle: router on all %d tokens (%.2f s) + expert MLPs and combine on "
                      "%d sampled tokens (%.2f s); tokens/s = 1/(router s/token + expert s/token)"
                      % (s.T, t_route, done, t_exp)}


def cpu_baseline_backward(s, L, dout, budget_s: float):
    """Time the fp64 oracle's backward on a bounded sample of this workload."""
    import numpy as np
    import oracle

    hl = {k: (None if v is None else v.detach().cpu()) for k, v in L.items()}
    d64 = dout.detach().cpu().double().numpy()
    score = oracle.SOFTMAX if s.score == "softmax" else oracle.SIGMOID
    gate = {"silu": oracle.GATE_SILU, "gelu": oracle.GATE_GELU, "relu": oracle.GATE_RELU}[s.gate]
    ex = oracle.Experts(hl["w_gate"], hl["w_up"], hl["w_down"], gate=gate)
    t0 = time.perf_counter()
    ids, w, keys = oracle.route(hl["x"], hl["w_router"], hl["router_bias"], s.k, score, s.renormalize,
                                s.routed_scale, want_keys=True)
    t_route = time.perf_counter() - t0
    rng = np.random.default_rng(0)
    order = rng.permutation(s.T)
    n, t_tok, done = 8, 0.0, 0
    while done < s.T and t_tok < budget_s / 2:
        batch = order[done:done + n]
        t0 = time.perf_counter()
        oracle.bwd_tokens(ex, hl["x"], hl["w_router"], score, s.renormalize, s.routed_scale, keys, ids, w, d64,
                          batch)
        t_tok += time.perf_counter() - t0
        done += batch.size
        n = int(min(max(8, (budget_s / 2 - t_tok) / (t_tok / done)), s.T - done))
    # weight gradients: every row of the three matrices of the expert with the
    # fewest (but at least 4) pairs, priced per pair
    counts = np.bincount(ids.ravel(), minlength=s.E)
    cand = np.nonzero(counts >= 4)[0]
    e = int(cand[np.argmin(counts[cand])])
    t0 = time.perf_counter()
    for which, rows in ((oracle.BWD_GATE, s.I), (oracle.BWD_UP, s.I), (oracle.BWD_DOWN, s.H)):
        oracle.bwd_expert_rows(ex, which, e, np.arange(rows), hl["x"], ids, w, d64)
    t_w = time.perf_counter() - t0
    per_token = t_route / s.T + t_tok / done + s.k * t_w / counts[e]
    return {"value": 1.0 / per_token, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "fp64 oracle backward: router on all %d tokens (%.2f s) + token gradients on %d sampled "
                      "tokens (%.2f s) + all weight-gradient rows of expert %d over its %d pairs (%.2f s); "
                      "tokens/s = 1/(router + token + k * weight-gradient-per-pair seconds)"
                      % (s.T, t_route, done, t_tok, e, counts[e], t_w)}


def bench_backward(args, s, L, dev):
    """One step = one moe_backward over the batch; prints the JSON line."""
    import torch
    import mixture_experts_routed_softmax_amd as moe
    import synthetic

    if s.experts != "bf16":
        print("the backward takes bf16 experts (workload %s has %s)" % (s.name, s.experts), file=sys.stderr)
        sys.exit(2)
    d = moe.make_desc(s.T, s.H, s.I, s.E, s.k, score=s.score, renormalize=s.renormalize,
                      routed_scale=s.routed_scale, gate=s.gate)
    dout = synthetic.make_grad_out(s, seed=args.seed, device=dev)
    dx = torch.empty_like(L["x"])
    dwr = torch.empty_like(L["w_router"])
    db = torch.empty(s.E, dtype=torch.float32, device=dev)
    dwg, dwu, dwd = torch.empty_like(L["w_gate"]), torch.empty_like(L["w_up"]), torch.empty_like(L["w_down"])
    ws = moe.workspace(d, moe.MOE_OP_BACKWARD, dev)

    def step():
        moe.moe_backward(d, L["x"], L["w_router"], L["router_bias"], L["w_gate"], L["w_up"], L["w_down"], dout,
                         dx, dwr, db, dwg, dwu, dwd, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    moe.moe_timing_enable(True)
    moe.moe_timing_read()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed_ms = (time.perf_counter() - t0) * 1e3
    stages = moe.moe_timing_read()
    moe.moe_timing_enable(False)
    ms_per_step = elapsed_ms / args.steps
    value = s.T / (ms_per_step / 1e3)
    for name, (ms, n) in stages.items():
        if n:
            log("  stage %-13s %8.1f us/step  (%d launches)" % (name, 1e3 * ms / args.steps, n))
    P = s.T * s.k
    # algorithmic FLOPs of the stages' GEMMs per step: data gradients e = W_down^T dout
    # (2 P H I) and dx = [dg|du] [W_gate; W_up] (2 P 2I H); weight gradients
    # dW_down (2 P H I) and dW_gate, dW_up (2 P 2I H); the recompute of g, u (2 P H 2I)
    gemm = {"bwd_data": 6.0 * P * s.H * s.I, "bwd_weight": 6.0 * P * s.H * s.I,
            "bwd_recompute": 4.0 * P * s.H * s.I}
    dom = max(gemm, key=lambda k: stages[k][0])
    ms_dom, n_dom = stages[dom]
    per_launch_ms = ms_dom / n_dom
    flops_per_launch = gemm[dom] * args.steps / n_dom
    achieved = flops_per_launch / (per_launch_ms / 1e3) / 1e12
    total_flops = 16.0 * P * s.H * s.I
    log("backward: %.3f ms/step, %.0f tokens/s, %.1f TFLOP/s over the expert GEMMs (recompute included)"
        % (ms_per_step, value, total_flops / (ms_per_step / 1e3) / 1e12))
    kname = {"bwd_data": "gemm_bwd_kernel<0, false>", "bwd_weight": "gemm_bwd_kernel<1, false>",
             "bwd_recompute": "gemm_bf16_kernel<0, false>"}[dom]
    traffic = recorded_traffic(s.name + "_backward", kname)
    roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_TFLOPS["bf16"], "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_TFLOPS["bf16"], 4),
            "traffic": None if traffic is None else round(traffic),
            "kernel": kname + {"bwd_data": " (data-gradient GEMMs)", "bwd_weight": " (weight-gradient GEMMs)",
                               "bwd_recompute": " (recompute of g, u)"}[dom],
            "avg_launch_us": round(per_launch_ms * 1e3, 2), "alg_flops_per_launch": flops_per_launch}
    cpu = None
    if not args.no_cpu_baseline:
        del ws, dwg, dwu, dwd
        cpu = cpu_baseline_backward(s, L, dout, args.cpu_seconds)
        log("cpu baseline: %.2f tokens/s on %d threads" % (cpu["value"], cpu["cores"]))
    line = {
        "metric": "MoE-layer backward tokens/s (every gradient of the layer); % MFMA peak of the dominant "
                  "backward GEMM",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": s.name + "_backward", "T": s.T, "H": s.H, "I": s.I, "E": s.E, "k": s.k,
                   "experts": s.experts, "score": s.score, "renormalize": s.renormalize,
                   "routed_scale": s.routed_scale, "router_bias": s.bias, "weights": "rowmajor",
                   **({"gate": s.gate} if s.gate != "silu" else {}),
                   "gemm_tflops": round(total_flops / (ms_per_step / 1e3) / 1e12, 1)},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def run_layer(args, s, L, dev, steps: int, warmup: int, decode: bool):
    """Times moe_forward on the resident layer L; returns the measurement.

    Prefill (decode=False): `steps` back-to-back steps between two
    synchronisations, with the library's per-launch stage events on (they
    give the gate/up kernel's duration).  Decode: `steps` individually timed
    steps (one event pair each, on the launch stream), each preceded by an
    untimed read of a 2 GiB buffer that evicts the last-level cache; the
    median step counts.  Packed weights are written once before timing."""
    import torch
    import mixture_experts_routed_softmax_amd as moe

    layout = args.layout if s.experts != "f32" else "rowmajor"
    d = moe.make_desc(s.T, s.H, s.I, s.E, s.k, score=s.score, renormalize=s.renormalize,
                      routed_scale=s.routed_scale, act_dtype=s.act, w_dtype=s.experts,
                      w_scale_fmt=s.scale_fmt if s.experts in ("fp8", "fp4") else "none", layout=layout,
                      gate=s.gate)
    if layout == "packed":
        # one-time model-load transform, outside the timed region
        wg, dn = moe.pack_experts(d, L["w_gate"], L["w_up"], L["w_down"], dev)
        wu = None
        del L["w_gate"], L["w_up"], L["w_down"]
        torch.cuda.synchronize()
    else:
        wg, wu, dn = L["w_gate"], L["w_up"], L["w_down"]
    out = torch.empty(s.T, s.H, dtype=torch.float32 if s.act == "f32" else torch.bfloat16, device=dev)
    counts = torch.empty(s.E, dtype=torch.int32, device=dev)
    ws = moe.workspace(d, moe.MOE_OP_FORWARD, dev)
    stream = torch.cuda.current_stream()

    def step():   # on the current stream (the capture stream while a graph is recorded)
        moe.moe_forward(d, L["x"], L["w_router"], L["router_bias"], wg, wu, dn, L.get("s_gate"),
                        L.get("s_up"), L.get("s_down"), out, None, None, counts, ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    run = step
    graph = None
    if decode and args.graph != "off":
        # A decode step is a chain of short kernels: replay it as one HIP graph
        # (the library only enqueues work, so the whole forward is capturable).
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
        torch.cuda.synchronize()
        run = graph.replay
    flush = None
    if decode:
        # touched weights of a decode step fit the 256 MB last-level cache: evict it
        # between timed steps by streaming a 2 GiB buffer through it (outside the
        # timed events).  Reading leaves clean lines behind; rewriting the buffer
        # would leave dirty lines whose write-back the next step would pay for.
        flush_buf = torch.ones(2 << 28, dtype=torch.int32, device=dev)
        flush_sink = torch.empty((), dtype=torch.int32, device=dev)

        def flush_cache():
            if args.flush == "read":
                torch.amax(flush_buf, dim=0, out=flush_sink)
            else:
                flush_buf.zero_()
        flush = flush_cache
    # Decode steps are timed with one event pair per step; per-launch events
    # would add their own cost to a ~0.1 ms step, so the per-stage breakdown
    # comes from extra steps after the timed region.
    moe.moe_timing_enable(not decode)
    moe.moe_timing_read()
    if decode:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            flush()
            ev[i][0].record(stream)
            run()
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        times = sorted(a.elapsed_time(b) for a, b in ev)
        ms_per_step = times[len(times) // 2]
    else:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        ms_per_step = (time.perf_counter() - t0) * 1e3 / steps
    stages = moe.moe_timing_read()
    moe.moe_timing_enable(False)
    if decode:
        moe.moe_timing_enable(True)
        moe.moe_timing_read()
        for _ in range(min(steps, 20)):
            flush()
            step()
        torch.cuda.synchronize()
        stages = moe.moe_timing_read()
        moe.moe_timing_enable(False)
    cnt = counts.cpu()
    del ws, wg, wu, dn, out
    return {"ms_per_step": ms_per_step, "stages": stages, "counts": cnt, "layout": layout,
            "graph": graph is not None, "n_stages": sum(n for _, n in stages.values()) / min(steps, 20)
            if decode else None}


def weight_bytes_per_expert(s) -> float:
    b = 3 * s.H * s.I * {"fp4": 0.5, "fp8": 1, "bf16": 2, "f32": 4}[s.experts]
    if s.experts == "fp4":
        b += 3 * s.H * s.I // 32    # one UE8M0 scale byte per 32 weights
    return b


def decode_record(s, m, steps: int) -> dict:
    """HBM roofline of a whole decode step: the touched experts' weight bytes
    (each read once) over the median step time."""
    touched = int((m["counts"] > 0).sum())
    alg = touched * weight_bytes_per_expert(s)
    gbs = alg / (m["ms_per_step"] / 1e3) / 1e9
    return {"workload": s.name, "T": s.T, "ms_per_step": round(m["ms_per_step"], 4),
            "tokens_per_s": round(s.T / (m["ms_per_step"] / 1e3), 1), "achieved_GBs": round(gbs, 1),
            "peak_GBs": PEAK_HBM_GBS, "frac": round(gbs / PEAK_HBM_GBS, 4), "touched_experts": touched,
            "alg_bytes": alg, "steps": steps, "timing": "median of %d individually timed steps, last-level "
            "cache evicted before each" % steps, "stages_per_step": m["n_stages"]}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import synthetic

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        # a plain copy kernel of known size: it reads and writes exactly 1 GiB
        src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 3 copies of %d bytes" % src.numel())
        return
    over = {}
    if args.T is not None:
        over["T"] = args.T
    if args.config == "dsv3_fp8":
        over["scale_fmt"] = args.scale_fmt
    if args.gate != "silu":
        over["gate"] = args.gate
    s = synthetic.spec(args.config, **over)
    decode = s.T <= 64
    steps = args.steps if args.steps is not None else (args.decode_steps if decode else 20)
    log("workload %s T=%d H=%d I=%d E=%d k=%d experts=%s" % (s.name, s.T, s.H, s.I, s.E, s.k, s.experts))
    t0 = time.perf_counter()
    L = synthetic.make_layer(s, seed=args.seed, device=dev)
    torch.cuda.synchronize()
    log("inputs generated in %.1f s" % (time.perf_counter() - t0))
    if args.backward:
        args.steps = steps
        bench_backward(args, s, L, dev)
        return

    m = run_layer(args, s, L, dev, steps, args.warmup, decode)
    del L
    torch.cuda.empty_cache()
    ms_per_step, stages, cnt, layout = m["ms_per_step"], m["stages"], m["counts"], m["layout"]
    value = s.T / (ms_per_step / 1e3)
    for name, (ms, n) in stages.items():
        if n:
            log("  stage %-8s %8.1f us/launch  (%d launches)" % (name, 1e3 * ms / n, n))

    P = s.T * s.k
    touched = int((cnt > 0).sum())
    layer_flops = 2.0 * P * 3 * s.H * s.I
    layer_tflops = layer_flops / (ms_per_step / 1e3) / 1e12
    if decode:
        rec = decode_record(s, m, steps)
        roof = {"bound": "hbm", "achieved": rec["achieved_GBs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": rec["frac"], "traffic": None,
                "kernel": "moe_forward (whole step%s, median of %d individually timed steps)"
                          % (", replayed as a HIP graph" if m["graph"] else "", steps),
                "alg_bytes_per_launch": rec["alg_bytes"], "touched_experts": touched}
    else:
        ms_gu, n_gu = stages["gate_up"]
        avg_ms = ms_gu / max(n_gu, 1)
        flops = 2.0 * P * s.H * 2 * s.I
        achieved = flops / (avg_ms / 1e3) / 1e12
        peak = PEAK_TFLOPS[s.experts]
        # the gate/up kernel the library launches for this layer (packed
        # weights: the one-wave-per-SIMD grouped GEMMs; fp8 and fp4 weights
        # share the e4m3-activation one)
        kname = {"bf16": "gemm_grouped_bf16_kernel<0, false>", "fp8": "gemm_grouped_fp8_kernel<0, false>",
                 "fp4": "gemm_grouped_fp8_kernel<0, true>"}.get(s.experts, "")
        traffic = recorded_traffic(s.name, kname) if layout == "packed" else None
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4),
                "traffic": None if traffic is None else round(traffic),
                "kernel": "gate_up grouped GEMM (%s)" % s.experts,
                "avg_launch_us": round(avg_ms * 1e3, 2), "alg_flops_per_launch": flops,
                "layer_tflops": round(layer_tflops, 1), "layer_frac": round(layer_tflops / peak, 4)}
        # the layer against the HBM roofline as well: the touched experts'
        # weights read once, x read and out written once (bf16), over the step
        act_b = 2 if s.act == "bf16" else 4
        layer_bytes = touched * weight_bytes_per_expert(s) + 2 * s.T * s.H * act_b
        layer_gbs = layer_bytes / (ms_per_step / 1e3) / 1e9
        roof["layer_hbm"] = {"alg_bytes": layer_bytes, "achieved_GBs": round(layer_gbs, 1),
                             "peak_GBs": PEAK_HBM_GBS, "frac": round(layer_gbs / PEAK_HBM_GBS, 4)}
    log("layer: %.3f ms/step, %.0f tokens/s, %.1f TFLOP/s expert GEMMs, touched %d/%d experts, "
        "max/mean tokens per expert %d/%.1f"
        % (ms_per_step, value, layer_tflops, touched, s.E, int(cnt.max()), P / s.E))

    # the decode regime next to a prefill line: the Qwen-like decode layer at
    # 1 and 64 tokens, HBM fraction of the whole step
    dec = None
    if not decode and args.decode_extra:
        dec = []
        for T in (1, 64):
            sd = synthetic.spec("qwen_decode", T=T)
            Ld = synthetic.make_layer(sd, seed=args.seed + T, device=dev)
            md = run_layer(args, sd, Ld, dev, args.decode_steps, max(args.warmup, 3), True)
            del Ld
            torch.cuda.empty_cache()
            r = decode_record(sd, md, args.decode_steps)
            log("decode %s T=%d: %.1f us/step, %.0f GB/s = %.1f%% of HBM (%d touched experts, %.1f timed stages)"
                % (sd.name, T, 1e3 * r["ms_per_step"], r["achieved_GBs"], 100 * r["frac"], r["touched_experts"],
                   r["stages_per_step"]))
            dec.append(r)

    cpu = None
    if not args.no_cpu_baseline:
        t0 = time.perf_counter()
        L = synthetic.make_layer(s, seed=args.seed, device=dev)   # the same seeded inputs, row-major
        hl = {k: (None if v is None else v.detach().cpu()) for k, v in L.items()}
        del L
        torch.cuda.empty_cache()
        log("host copy of the layer for the oracle: %.1f s" % (time.perf_counter() - t0))
        cpu = cpu_baseline(s, hl, args.cpu_seconds)
        log("cpu baseline: %.1f tokens/s on %d threads" % (cpu["value"], cpu["cores"]))

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "fp8": "fp8_e4m3", "fp4": "fp4_e2m1"}[s.experts],
        "data": "synthetic",
        "config": {"workload": s.name, "T": s.T, "H": s.H, "I": s.I, "E": s.E, "k": s.k,
                   "experts": s.experts, "score": s.score, "renormalize": s.renormalize,
                   "routed_scale": s.routed_scale, "router_bias": s.bias, "weights": layout,
                   **({"scale_fmt": s.scale_fmt} if s.experts in ("fp8", "fp4") else {}),
                   **({"gate": s.gate} if s.gate != "silu" else {}),
                   "layer_tflops": round(layer_tflops, 1)},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    if dec is not None:
        line["decode"] = dec
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
