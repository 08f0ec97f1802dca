"""Benchmark of the routed MoE layer forward pass on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
    python bench.py --backward [--no-saved] [--workload NAME]   (the local backward)
    python bench.py --copy-probe BYTES     (HBM counter calibration only)

A step is one whole layer forward (route -> permute -> expert FFN -> combine,
the four C-ABI calls that moe_forward makes) over one batch of seeded
synthetic tokens already resident in HBM.  The default workload is the
V4-Pro-shaped bf16 layer (T=8192, h=7168, 384 experts, top-6, f=3072, one
shared expert, Zipf(0.8) expert load).  HIP events recorded on the launch
stream between the four calls give per-stage times inside the timed region;
the grouped GEMM stage (moe_expert_ffn: Linear1+SwiGLU and Linear2) is the
dominant one and carries the roofline figures.

The same JSON line carries, measured in the same process: `routing`, the
router's ids on every token against the oracle's fp64 routing (the tokens
that differ, all of which must be near ties, and the near-tie count);
`cpu_baseline`, the oracle timed on a bounded sample; and `workloads`, the
other configurations (decode-shaped with hash and with score routing, the
Llama-shaped layer, one GPU's expert-parallel share, V4-Pro A8W8 e4m3), each
with its step time, stage times and the grouped GEMM's roofline figures
(--no-workloads leaves them out).

Prints one JSON line.  Runs on one GPU only: --gpus N with N > 1 exits.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE layer tokens/s and grouped-GEMM TFLOP/s (% of MFMA peak) at 1 GPU"
PEAK_HBM_GBS = 8000.0
PEAK_MFMA_TFLOPS = {"bf16": 2516.6, "fp8": 5033.2, "int8": 5033.2, "mxfp8": 5033.2,
                    "mxfp4": 10066.3, "fp32": 157.3}   # int8: tera-ops/s


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def stage_bytes(wl):
    """Algorithmic HBM bytes of the stages around the grouped GEMM (each
    tensor read or written once): route reads X and Wg and writes the ids and
    gate weights; permute reads the ids and X and writes the row maps and the
    k copies (e4m3: plus the quantised X and scales); combine reads the k
    expert rows, the gate weights and row map (and the shared row) and writes
    Y."""
    T, h, E, k = wl.T, wl.hidden, wl.experts, wl.topk
    ab = 4 if wl.precision == "fp32" else 2             # activation / output bytes
    q8 = wl.precision in ("fp8", "int8", "mxfp8", "mxfp4")
    xb = (0.5 if wl.precision == "mxfp4" else 1) if q8 else ab   # dispatched row bytes
    route = T * h * ab + h * E * ab + T * k * 8 + (T * 4 if wl.hash else 0)
    permute = 2 * T * k * 4 + T * h * ab + T * k * h * xb + 2 * T * k * 4
    if wl.precision in ("fp8", "int8"):      # Xq and the per-row scales
        permute += T * h + T * 4 + T * k * 4
    if wl.precision in ("mxfp8", "mxfp4"):    # Xq and the per-group E8M0 scales
        permute += T * h * xb + (T + T * k) * (h // 32)
    combine = T * k * h * ab + T * k * 8 + (T * h * ab if wl.shared else 0) + T * h * ab
    return {"route": route, "permute": permute, "combine": combine}


def algorithmic_work(wl, counts):
    """FLOPs and HBM bytes the grouped GEMM stage must do for these counts:
    every routed and shared row through Linear1 (h -> 2f) and Linear2 (f -> h);
    the weights of every expert that received a row, read once; the input rows
    read once and the output rows written once."""
    h, f, k, T = wl.hidden, wl.inter, wl.topk, wl.T
    rows = T * k + (T if wl.shared else 0)
    flops = 2.0 * rows * (h * 2 * f + f * h)
    q8 = wl.precision in ("fp8", "int8", "mxfp8", "mxfp4")
    wbytes = (0.5 if wl.precision == "mxfp4" else 1) if q8 else (4 if wl.precision == "fp32" else 2)
    xbytes = wbytes
    obytes = 4 if wl.precision == "fp32" else 2
    active = int((counts > 0).sum()) + (1 if wl.shared else 0)
    # MX: one E8M0 byte per 32 weights and per 32 input values
    sbytes = 1.0 / 32 if wl.precision in ("mxfp8", "mxfp4") else 0.0
    weight_bytes = active * 3.0 * h * f * (wbytes + sbytes)
    act_bytes = rows * h * (xbytes + sbytes + obytes)
    return flops, weight_bytes + act_bytes, active


def cpu_baseline(inp, gpu_ids, counts, target_s=12.0, max_s=30.0, log_fn=log):
    """Time the CPU oracle (as it stands) on a bounded sample of the workload.

    The sample: up to 1024 tokens whose selected experts all lie among the 96
    most loaded experts (every token costs the same k + shared expert FFNs, so
    this keeps the host copy of weights small without changing the per-token
    work); if fewer than 64 such tokens exist, the first 16 tokens.  The sample
    (fp64 routing of its tokens + the per-token expert loop) is repeated until
    about target_s seconds of CPU work have run."""
    import numpy as np
    import torch

    import oracle
    from tests.helpers import bits, f64

    wl = inp["workload"]
    hot = set(np.argsort(-counts, kind="stable")[:96].tolist())
    ok = np.array([all(int(e) in hot for e in row) for row in gpu_ids])
    toks = np.nonzero(ok)[0][:1024]
    how = "tokens whose experts are all among the 96 most loaded"
    if len(toks) < 64:
        toks = np.arange(min(16, wl.T))
        how = "the first tokens"
    ids_s = gpu_ids[toks]
    experts = sorted(set(int(e) for e in ids_s.ravel() if e >= 0))
    remap = np.full(wl.experts, -1, np.int32)
    remap[experts] = np.arange(len(experts), dtype=np.int32)
    idx = torch.tensor(experts, dtype=torch.long, device=inp["W1"].device)
    sel = lambda t: None if t is None else bits(t.index_select(0, idx))  # noqa: E731
    tsel = torch.from_numpy(toks).long().to(inp["X"].device)
    X = bits(inp["X"][tsel])
    Wg = bits(inp["Wg"])
    tok_ids = bits(inp["token_ids"][tsel]) if inp["token_ids"] is not None else None
    L = oracle.Layer(wl.precision, X, sel(inp["W1"]), sel(inp["W2"]), w1_scale=sel(inp["w1_scale"]),
                     w2_scale=sel(inp["w2_scale"]), Ws1=bits(inp["Ws1"]), Ws2=bits(inp["Ws2"]),
                     ws1_scale=bits(inp["ws1_scale"]), ws2_scale=bits(inp["ws2_scale"]),
                     k=wl.topk)
    ids_local = remap[ids_s]
    reps = 0
    t0 = time.perf_counter()
    while True:
        r = oracle.route(X, Wg, wl.topk, gate_bias=f64(inp["gate_bias"]), beta=f64(inp["beta"]),
                         score=wl.score, renorm=wl.renorm, alpha=wl.alpha, token_ids=tok_ids,
                         tid2eid=bits(inp["tid2eid"]))
        L.tokens(ids_local, r["G"])
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s or el * (reps + 1) / reps > max_s:
            break
    n = reps * len(toks)
    cores = oracle.set_threads(0)
    log_fn(f"[bench] cpu oracle: {n} tokens ({reps} x {len(toks)}) in {el:.2f} s on {cores} threads")
    # the same per-token work on one thread, over the first tokens of the sample
    one = min(len(toks), 32)
    oracle.set_threads(1)
    n1, t1 = 0, time.perf_counter()
    try:
        while True:
            r1 = oracle.route(X[:one], Wg, wl.topk, gate_bias=f64(inp["gate_bias"]),
                              beta=f64(inp["beta"]), score=wl.score, renorm=wl.renorm,
                              alpha=wl.alpha,
                              token_ids=None if tok_ids is None else tok_ids[:one],
                              tid2eid=bits(inp["tid2eid"]))
            G1 = r["G"].copy()
            G1[:one] = r1["G"]
            L.tokens(ids_local, G1, tokens=np.arange(one))
            n1 += one
            el1 = time.perf_counter() - t1
            if el1 >= 3.0:
                break
    finally:
        oracle.set_threads(0)
    log_fn(f"[bench] cpu oracle, one thread: {n1} tokens in {el1:.2f} s")
    return {"value": round(n / el, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{len(toks)} of the {wl.T} tokens ({how}), repeated {reps} times: fp64 "
                      f"routing of those tokens + the per-token loop over their {wl.topk} routed "
                      "experts" + (" and the shared expert" if wl.shared else ""),
            "seconds": round(el, 2),
            "value_1core": round(n1 / el1, 2),
            "sample_1core": f"the first {one} tokens of that sample, on one thread, "
                            f"repeated for {el1:.1f} s",
            "cpu": cpu_model()}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


TRAFFIC_SOURCES = ("mixture_experts_layer_09_amd/csrc/grouped_gemm.hip",
                   "mixture_experts_layer_09_amd/csrc/moe_internal.h",
                   "mixture_experts_layer_09_amd/csrc/lds_dma.h")


def grouped_gemm_source_hash() -> str:
    """sha256 over the sources the grouped GEMM kernels are built from."""
    import hashlib
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes of one moe_expert_ffn call on this workload, from the
    committed rocprofv3 counter summary (FETCH_SIZE + WRITE_SIZE of the two
    GEMM dispatches, scaled by the copy-probe calibration), or None when there
    is none or it was taken on other grouped GEMM sources than these."""
    import re
    path = os.path.join(ROOT, "profiles", f"expert_ffn_{workload}_hbm_bytes.md")
    try:
        with open(path) as fh:
            text = fh.read()
        sha = grouped_gemm_source_hash()
    except OSError:
        return None
    m = re.search(r"^bench-traffic: bytes_per_call=(\d+) sources_sha256=([0-9a-f]{64})\s*$",
                  text, re.M)
    if not m or m.group(2) != sha:
        return None
    return int(m.group(1))


def device_copy_gbs(nbytes: int = 1 << 30, reps: int = 5) -> float:
    """Context figure: read + write GB/s of a plain device-to-device copy."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    b.copy_(a)
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record()
    for _ in range(reps):
        b.copy_(a)
    s1.record()
    s1.synchronize()
    ms = s0.elapsed_time(s1) / reps
    del a, b
    return round(2 * nbytes / (ms / 1000.0) / 1e9, 1)


def copy_probe(nbytes: int, reps: int = 5):
    """A plain device-to-device copy of nbytes, for calibrating the HBM byte
    counters (FETCH_SIZE / WRITE_SIZE) against a known amount of traffic."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "reps": reps}))
    return 0


def backward_work(wl, counts):
    """FLOPs and HBM bytes the local backward must do: the recomputed Linear1
    over every row (dG comes out of Linear2's dgrad, so Linear2's forward is
    not recomputed), the dgrad and wgrad of both linears (each the forward's
    FLOPs again) and the router's two GEMMs; bytes: the active experts'
    weights read once and their gradients written once, X and dY read, dX
    written, the router's gradient."""
    h, f, k, T, E = wl.hidden, wl.inter, wl.topk, wl.T, wl.experts
    rows = T * k + (T if wl.shared else 0)
    fwd = 2.0 * rows * (h * 2 * f + f * h)
    flops = 2.0 * rows * h * 2 * f + 2.0 * fwd + 2 * (2.0 * T * h * E)
    active = int((counts > 0).sum()) + (1 if wl.shared else 0)
    nbytes = 2 * active * 3.0 * h * f * 2 + 3 * T * h * 2 + 2 * h * E * 2
    return flops, nbytes


def bench_backward(args, wl, inp, shape):
    """Times moe_backward (recompute + backward, router on) with HIP events on
    its launch stream; one JSON line."""
    import numpy as np
    import torch

    import mixture_experts_layer_09_amd as moe
    if wl.precision != "bf16":
        print(json.dumps({"error": "the backward is built for bf16 layers"}))
        return 2
    T, h, E, k, f = wl.T, wl.hidden, wl.experts, wl.topk, wl.inter
    ws = moe.alloc_workspace(shape)
    opts = moe.make_route_opts(wl.score, wl.renorm, wl.alpha, inp["beta"], inp["gate_bias"],
                               inp["token_ids"], inp["tid2eid"])
    weights = moe.make_weights(inp["W1"], inp["W2"], None, None, inp["Ws1"], inp["Ws2"])
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    G = torch.empty((T, k), dtype=torch.float32, device="cuda")
    moe.moe_route(shape, opts, inp["X"], inp["Wg"], ids, G, None, ws)
    gen = torch.Generator().manual_seed(4321)
    dY = torch.randn((T, h), generator=gen).to(torch.bfloat16).cuda()
    bf = dict(dtype=torch.bfloat16, device="cuda")
    g = dict(dX=torch.empty((T, h), **bf), dW1=torch.empty((E, h, 2 * f), **bf),
             dW2=torch.empty((E, f, h), **bf),
             dWs1=torch.empty((h, 2 * f), **bf) if wl.shared else None,
             dWs2=torch.empty((f, h), **bf) if wl.shared else None,
             dWg=torch.empty((h, E), **bf),
             dgate_bias=torch.empty(E, dtype=torch.float32, device="cuda"),
             dG=torch.empty((T, k), dtype=torch.float32, device="cuda"))
    grads = moe.make_grads(**g)
    wsb = moe.alloc_workspace(shape, backward=True)
    stream = torch.cuda.current_stream()

    def call():
        moe.moe_backward(shape, opts, inp["X"], inp["Wg"], weights, ids, G, dY, grads, wsb)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    assert moe.moe_check_device_error(wsb) == 0
    log(f"[bench] backward warmup done; timing {args.steps} calls")
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1000.0 / args.steps
    ms = e0.elapsed_time(e1) / args.steps
    # saved activations: the training forward keeps what moe_backward
    # recomputes, and moe_backward_saved starts from there
    Yt = torch.empty((T, h), dtype=torch.bfloat16, device="cuda")

    def fwd_train():
        moe.moe_forward_train(shape, opts, inp["X"], inp["Wg"], weights, ids, G, Yt, wsb)

    def bwd_saved():
        moe.moe_backward_saved(shape, opts, inp["X"], inp["Wg"], weights, ids, G, dY, grads, wsb)

    def timed(fn, pre=None):
        tot = 0.0
        for _ in range(args.steps):
            if pre:
                pre()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            tot += a.elapsed_time(b)
        return tot / args.steps

    if not args.no_saved:
        fwd_train()
        bwd_saved()
        torch.cuda.synchronize()
        ft_ms = timed(fwd_train)
        bs_ms = timed(bwd_saved, pre=fwd_train)
        assert moe.moe_check_device_error(wsb) == 0
    counts = np.bincount(ids.cpu().numpy().ravel(), minlength=E)
    flops, nbytes = backward_work(wl, counts)
    tflops = flops / (ms / 1000.0) / 1e12
    gbs = nbytes / (ms / 1000.0) / 1e9
    t_mfma = flops / (PEAK_MFMA_TFLOPS["bf16"] * 1e12)
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    bound = "hbm" if t_hbm >= t_mfma else "mfma"
    out = {
        "metric": "MoE layer local backward (recompute + dgrad + wgrad + router) tokens/s",
        "value": round(T / (ms / 1000.0), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "wall_ms_per_step": round(wall_ms, 4), "higher_is_better": True, "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded, random-init weights)",
        "config": {"workload": wl.name, "tokens": T, "hidden": h, "experts": E, "topk": k,
                   "inter": f, "shared_experts": wl.shared, "score": wl.score},
        "backward": {"tflops": round(tflops, 1), "frac_mfma_peak": round(tflops / PEAK_MFMA_TFLOPS["bf16"], 4),
                     "hbm_gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                     "algorithmic_flops": flops, "algorithmic_bytes": nbytes, "bound": bound,
                     "frac_of_roofline": round(max(t_mfma, t_hbm) / (ms / 1000.0), 4)},
        # moe_backward_saved after moe_forward_train (activations kept instead of
        # recomputed): its own time per call, and the training forward's
        "saved_activations": None if args.no_saved else {
            "backward_ms": round(bs_ms, 4), "tokens_per_s": round(T / (bs_ms / 1000.0), 1),
            "forward_train_ms": round(ft_ms, 4)},
    }
    print(json.dumps(out), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="v4pro_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-workloads", action="store_true",
                    help="measure the selected workload only (not the other configurations)")
    ap.add_argument("--no-routing-check", action="store_true",
                    help="skip the oracle's routing of every token (the 'routing' field)")
    ap.add_argument("--set", action="append", default=[], metavar="FIELD=VALUE",
                    help="override a workload field (exploration; e.g. --set zipf=False)")
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="only run a device copy of this many bytes (counter calibration)")
    ap.add_argument("--backward", action="store_true",
                    help="time the local backward (moe_backward, router on) instead")
    ap.add_argument("--no-saved", action="store_true",
                    help="with --backward: skip the saved-activation pair (moe_forward_train, "
                         "moe_backward_saved)")
    args = ap.parse_args(argv)
    if args.copy_probe:
        return copy_probe(args.copy_probe)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark measures one GPU's share of the layer; "
                                   "runs on more than one GPU are not supported",
                          "n_gpus": args.gpus}))
        return 2

    import numpy as np
    import torch

    import mixture_experts_layer_09_amd as moe
    import synth

    import ast
    wl = synth.WORKLOADS[args.workload]
    if args.set:
        wl = wl.replace(**{k: ast.literal_eval(v) for k, v in (x.split("=", 1) for x in args.set)})
    torch.cuda.set_device(0)
    log(f"[bench] generating {wl.name} on cuda:0")
    t = time.perf_counter()
    inp = synth.make_inputs(wl, device="cuda")
    torch.cuda.synchronize()
    log(f"[bench] inputs ready in {time.perf_counter() - t:.1f} s")

    shape = moe.make_shape(wl.T, wl.hidden, wl.experts, wl.topk, wl.inter, wl.shared, wl.precision)
    if args.backward:
        return bench_backward(args, wl, inp, shape)
    out, ids, cnt = measure_forward(wl, inp, args.steps, args.warmup,
                                    traffic=measured_traffic(wl.name) if not args.set else None)
    out = {"metric": METRIC, "value": out.pop("value"), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, **out}
    if not args.no_routing_check:
        out["routing"] = routing_check(wl, inp, ids)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, ids, cnt)
    out["hbm_copy_probe_gbs"] = device_copy_gbs()
    if not args.no_workloads and not args.set:
        del inp
        torch.cuda.empty_cache()
        out["workloads"] = other_workloads([w for w in EXTRA_WORKLOADS if w != wl.name], args)
    print(json.dumps(out), flush=True)
    return 0


# The other configurations, measured in the same run as the headline one:
# decode-shaped batches (hash and score routing), the Llama-shaped layer, one
# GPU's expert-parallel share and the V4-Pro A8W8 e4m3 layer.
EXTRA_WORKLOADS = ["decode_hash_bf16", "decode_score_bf16", "llama_bf16", "ep_share_bf16",
                   "v4pro_fp8"]


def other_workloads(names, args) -> dict:
    """measure_forward on each named workload (inputs generated, measured and
    freed one workload at a time); a short summary per workload."""
    import torch

    import synth
    res = {}
    for name in names:
        wl = synth.WORKLOADS[name]
        log(f"[bench] workload {name}: generating")
        inp = synth.make_inputs(wl, device="cuda")
        torch.cuda.synchronize()
        m, _, _ = measure_forward(wl, inp, args.steps, args.warmup,
                                  traffic=measured_traffic(name), with_forward=False)
        r = m["roofline"]
        res[name] = {"tokens_per_s": m["value"], "ms_per_step": m["ms_per_step"],
                     "stages_ms": m["stages_ms"], "expert_ffn_ms": m["stages_ms"]["expert_ffn"],
                     "bound": r["bound"], "roofline_frac": r["frac"],
                     "frac_of_roofline": r["frac_of_roofline"], "achieved": r["achieved"],
                     "unit": r["unit"], "traffic": r["traffic"],
                     "grouped_gemm": m["grouped_gemm"], "layer_hbm": m["layer_hbm"],
                     "config": m["config"]}
        del inp
        torch.cuda.empty_cache()
    return res


def routing_check(wl, inp, ids) -> dict:
    """The router's ids against the oracle's fp64 routing of every token: the
    tokens whose ids differ (all must be near ties: oracle margin between the
    k-th and (k+1)-th key below 1e-5) and the number of near ties."""
    import numpy as np

    import oracle
    from tests.helpers import bits, f64
    t0 = time.perf_counter()
    r = oracle.route(bits(inp["X"]), bits(inp["Wg"]), wl.topk, gate_bias=f64(inp["gate_bias"]),
                     beta=f64(inp["beta"]), score=wl.score, renorm=wl.renorm, alpha=wl.alpha,
                     token_ids=bits(inp["token_ids"]), tid2eid=bits(inp["tid2eid"]))
    near = r["margin"] < 1e-5
    differ = np.nonzero((ids != r["ids"]).any(axis=1))[0]
    log(f"[bench] routing check: {len(differ)} of {wl.T} tokens differ from the oracle, "
        f"{int(near.sum())} near ties ({time.perf_counter() - t0:.1f} s)")
    return {"tokens": wl.T, "checked_against": "oracle fp64 routing of every token",
            "near_tie_delta": 1e-5, "near_ties": int(near.sum()),
            "differ_from_oracle": [int(t) for t in differ],
            "differ_all_near_ties": bool(near[differ].all()) if len(differ) else True,
            "exact_at_clear_margin": bool((ids[~near] == r["ids"][~near]).all())}


def measure_forward(wl, inp, steps, warmup, traffic=None, with_forward=True):
    """Times the layer step (the four C-ABI calls moe_forward makes) with HIP
    events on the launch stream; returns (summary dict, ids [T,k], counts)."""
    import numpy as np
    import torch

    import mixture_experts_layer_09_amd as moe
    shape = moe.make_shape(wl.T, wl.hidden, wl.experts, wl.topk, wl.inter, wl.shared, wl.precision)
    ws = moe.alloc_workspace(shape)
    opts = moe.make_route_opts(wl.score, wl.renorm, wl.alpha, inp["beta"], inp["gate_bias"],
                               inp["token_ids"], inp["tid2eid"])
    weights = moe.make_weights(inp["W1"], inp["W2"], inp["w1_scale"], inp["w2_scale"], inp["Ws1"],
                               inp["Ws2"], inp["ws1_scale"], inp["ws2_scale"])
    dev = "cuda"
    mx = wl.precision in ("mxfp8", "mxfp4")
    fp4 = wl.precision == "mxfp4"
    fp8 = wl.precision in ("fp8", "int8", "mxfp8", "mxfp4")   # quantised activation codes
    odt = torch.float32 if wl.precision == "fp32" else torch.bfloat16
    xdt = (torch.int8 if wl.precision == "int8" else torch.float8_e4m3fn) if fp8 else odt
    T, k, h, E = wl.T, wl.topk, wl.hidden, wl.experts
    n = T * k
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    G = torch.empty((T, k), dtype=torch.float32, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    dst = torch.empty(n, dtype=torch.int32, device=dev)
    src = torch.empty(n, dtype=torch.int32, device=dev)
    Xp = (torch.empty((n, h // 2), dtype=torch.uint8, device=dev) if fp4
          else torch.empty((n, h), dtype=xdt, device=dev))
    sc_shape = (lambda r: (r, h // 32)) if mx else (lambda r: (r,))
    sc_dt = torch.uint8 if mx else torch.float32
    xps = torch.empty(sc_shape(n), dtype=sc_dt, device=dev) if fp8 else None
    Xq = ((torch.empty((T, h // 2), dtype=torch.uint8, device=dev) if fp4
           else torch.empty((T, h), dtype=xdt, device=dev)) if fp8 else None)
    xs = torch.empty(sc_shape(T), dtype=sc_dt, device=dev) if fp8 else None
    Yp = torch.empty((n, h), dtype=odt, device=dev)
    Ys = torch.empty((T, h), dtype=odt, device=dev) if wl.shared else None
    Y = torch.empty((T, h), dtype=odt, device=dev)
    X = inp["X"]
    Xs_in = (Xq if fp8 else X) if wl.shared else None
    xs_in = xs if (fp8 and wl.shared) else None
    stream = torch.cuda.current_stream()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        moe.moe_route(shape, opts, X, inp["Wg"], ids, G, None, ws)
        if ev:
            ev[1].record(stream)
        moe.moe_permute(shape, ids, X, counts, offsets, dst, src, Xp, xps, Xq, xs, ws)
        if ev:
            ev[2].record(stream)
        moe.moe_expert_ffn(shape, Xp, xps, offsets, Xs_in, xs_in, weights, Yp, Ys, ws)
        if ev:
            ev[3].record(stream)
        moe.moe_combine(shape, Yp, dst, G, Ys, Y)
        if ev:
            ev[4].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    assert moe.moe_check_device_error(ws) == 0
    log(f"[bench] {wl.name}: warmup done; timing {steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1000.0 / steps
    stage_ms = np.array([[e[s].elapsed_time(e[s + 1]) for s in range(4)] for e in evs]).mean(0)
    log(f"[bench] {wl.name}: {ms_per_step:.3f} ms/step; stages (route, permute, ffn, combine) "
        f"ms: {np.round(stage_ms, 4).tolist()}")

    fwd_ms = None
    if with_forward:
        # moe_forward (one call for all four stages) over the same inputs
        for _ in range(2):
            moe.moe_forward(shape, opts, X, inp["Wg"], weights, ids, G, Y, ws)
        torch.cuda.synchronize()
        tf0 = time.perf_counter()
        for _ in range(steps):
            moe.moe_forward(shape, opts, X, inp["Wg"], weights, ids, G, Y, ws)
        torch.cuda.synchronize()
        fwd_ms = (time.perf_counter() - tf0) * 1000.0 / steps

    cnt = counts.cpu().numpy()
    flops, nbytes, active = algorithmic_work(wl, cnt)
    ffn_s = stage_ms[2] / 1000.0
    tflops = flops / ffn_s / 1e12
    gbs = nbytes / ffn_s / 1e9
    prec = wl.precision
    t_mfma = flops / (PEAK_MFMA_TFLOPS[prec] * 1e12)
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    bound = "hbm" if t_hbm >= t_mfma else "mfma"
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_MFMA_TFLOPS[prec],
                "unit": "TFLOP/s", "frac": round(tflops / PEAK_MFMA_TFLOPS[prec], 4),
                "traffic": traffic}
    roof.update({"kernel": "moe_expert_ffn (grouped Linear1+SwiGLU, Linear2)",
                 "traffic_over_algorithmic": (round(traffic / nbytes, 3) if traffic else None),
                 "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
                 "ms": round(stage_ms[2], 4),
                 "frac_of_roofline": round(max(t_mfma, t_hbm) / ffn_s, 4)})
    sbytes = stage_bytes(wl)
    layer_bytes = nbytes + sum(sbytes.values())
    out = {
        "value": round(T / (ms_per_step / 1000.0), 1),
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp8": "fp8-e4m3 (bf16 activations/output)",
                  "int8": "i8 (int32 products; bf16 activations/output)",
                  "mxfp8": "mxfp8-e4m3 (group-32 E8M0 scales; bf16 input/output)",
                  "mxfp4": "mxfp4-e2m1 (group-32 E8M0 scales; bf16 input/output)",
                  "fp32": "f32"}[prec],
        "data": "synthetic (seeded, random-init weights)",
        "config": {"workload": wl.name, "tokens": T, "hidden": h, "experts": E, "topk": k,
                   "inter": wl.inter, "shared_experts": wl.shared, "score": wl.score,
                   "renorm": wl.renorm, "alpha": wl.alpha, "routing": "hash" if wl.hash else "score",
                   "expert_load": "zipf(0.8)" if wl.zipf else "random gate",
                   "active_experts": active},
        "grouped_gemm": {"tflops": round(tflops, 1),
                         "frac_mfma_peak": round(tflops / PEAK_MFMA_TFLOPS[prec], 4),
                         "hbm_gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)},
        "stages_ms": {"route": round(stage_ms[0], 4), "permute": round(stage_ms[1], 4),
                      "expert_ffn": round(stage_ms[2], 4), "combine": round(stage_ms[3], 4)},
        "moe_forward_ms": None if fwd_ms is None else round(fwd_ms, 4),
        "stages_hbm": {name: {"gbs": round(b / (stage_ms[i] / 1000.0) / 1e9, 1),
                              "frac_hbm_peak": round(b / (stage_ms[i] / 1000.0) / 1e9
                                                     / PEAK_HBM_GBS, 4),
                              "algorithmic_bytes": b}
                       for i, (name, b) in zip((0, 1, 3), sbytes.items())},
        "layer_hbm": {"gbs": round(layer_bytes / (ms_per_step / 1000.0) / 1e9, 1),
                      "frac_hbm_peak": round(layer_bytes / (ms_per_step / 1000.0) / 1e9
                                             / PEAK_HBM_GBS, 4),
                      "algorithmic_bytes": layer_bytes},
        "roofline": roof,
    }
    ids_h = ids.cpu().numpy()
    del ws, Xp, Yp, Ys, Y, xps, Xq, xs
    return out, ids_h, cnt


if __name__ == "__main__":
    sys.exit(main())
