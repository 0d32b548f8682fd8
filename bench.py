"""Benchmark: MoE decode FFN layer tokens/s and expert-weight HBM bandwidth on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode_bf16_t1]
                    [--also-tokens 8] [--mode auto|aux|seq|fused] [--eager]
                    [--no-cpu-baseline]

A step is one forward of the whole layer (router, top-k, bucketing, routed
gate/up, down, shared expert, join) over one batch of tokens.  The timed steps
cycle through L distinct device-resident copies of the layer and a pool of
token batches, so consecutive uses of a copy are hundreds of MB apart and the
256 MB Infinity Cache cannot serve them.  Steps are launched as HIP graphs of
a rotation window (the decode loop is graph-replayed) unless --eager.

Prints one JSON line.  `value` is tokens/s at the workload's batch; the decode
workload also times batch 8 on the same layer copies (key `batch_8`).  The
expert-weight bytes a step must read are the routed experts actually selected
(the used-expert count the kernels leave in their routing tables, read in an
untimed pass) plus the shared expert.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense
METRIC = "MoE-layer decode tokens/s at batch 1/8 + expert-weight HBM GB/s vs peak"
LAYER_COPIES = {"bf16": 16, "q4": 32, "f32": 16}
MIN_ROTATION_BYTES = 512 << 20
TOKEN_POOL = 8
WINDOW_REPEATS = 4
# the second batch size the metric names, timed beside the decode workload's batch 1
EXTRA_TOKENS = {"decode_bf16_t1": (8,), "decode_q4_t1_t4": (1,)}


def expert_bytes(shape) -> tuple[int, int]:
    """(gate+up bytes, down bytes) of one expert (or the shared expert) in its storage."""
    H, I = shape.hidden, shape.inter
    if shape.w_dtype == "q4":
        per = lambda rows, k: rows * (k // 2) + rows * (k // 32) * 2  # noqa: E731
    else:
        b = 2 if shape.w_dtype == "bf16" else 4
        per = lambda rows, k: rows * k * b  # noqa: E731
    return 2 * per(I, H), per(H, I)


def traffic_for(args, shape, T, shared_mode, dominant):
    """HBM bytes per launch of the dominant kernel from a rocprofv3 counter summary of a
    workload of this shape and batch, valid only while the kernel sources are the ones
    the counters were taken on."""
    from moe_decode_ffn_amd import synth
    from moe_decode_ffn_amd.traffic import kernel_source_hash, read_summary
    if args.input_block:
        return None
    names = [n for n, (s, _, c) in synth.WORKLOADS.items() if s == shape and c[-1] == T]
    if args.traffic:
        names = [None]
    for n in names:
        rec = read_summary(args.traffic or os.path.join(ROOT, "profiles", f"traffic_{n}.md"))
        if (rec and rec.get("kernel_source_hash") == kernel_source_hash()
                and (n is None or rec.get("workload") == n) and rec.get("shared_mode") == shared_mode
                and rec.get("kernel_id") == dominant):
            return rec.get("hbm_bytes_per_launch")
    return None


def measure(args, shape, layers, T, mode, regime, dev) -> dict:
    """Times K steps of batch T over the layer copies; per-kernel event times; roofline."""
    import numpy as np
    import torch

    from moe_decode_ffn_amd import ffn, synth

    L = len(layers)
    gu_b, d_b = expert_bytes(shape)
    xs = [synth.make_tokens_device(shape, T, 1000 + 97 * T + j, dev) for j in range(TOKEN_POOL)]
    mf = ffn.MoeFfn.for_layer(layers[0], max_tokens=T, flags=mode | regime)
    info = mf.info()
    ws = torch.empty(mf.workspace_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty(T, shape.hidden, dtype=torch.float32, device=dev)
    window = [(i % L, i % TOKEN_POOL) for i in range(L * WINDOW_REPEATS)]
    stream = torch.cuda.current_stream(dev)
    handle = stream.cuda_stream
    structs = {(li, xi): ffn.MoeFfn.tensors(layers[li], xs[xi], out) for li, xi in set(window)}

    def launch(step: int, h: int = handle) -> None:
        key = window[step % len(window)]
        ffn.moe_ffn_forward(mf.plan, structs[key], T, ws.data_ptr(), mf.workspace_bytes, h)

    # ---- untimed pass: used experts of every (copy, tokens) pair of the window, from the
    # kernels' own routing tables -------------------------------------------------------
    uniq = []
    for s in range(len(window)):
        launch(s)
        torch.cuda.synchronize()
        uniq.append(mf.routing_tables(ws, T)["n_used"])
    unique_mean = float(np.mean(uniq))
    bytes_per_step = unique_mean * (gu_b + d_b) + (gu_b + d_b)  # routed + shared expert weights

    # ---- graphs of whole rotation windows ----------------------------------------------
    graphs = {}

    def graph_for(n: int):
        if n not in graphs:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                h = torch.cuda.current_stream().cuda_stream  # the capture stream
                for s in range(n):
                    launch(s, h)
            graphs[n] = g
        return graphs[n]

    def run_steps(k: int) -> None:
        if args.eager:
            for s in range(k):
                launch(s)
            return
        full, rest = divmod(k, len(window))
        if full:
            g = graph_for(len(window))
            for _ in range(full):
                g.replay()
        if rest:
            graph_for(rest).replay()

    if not args.eager:
        graph_for(len(window))
        if args.steps % len(window):
            graph_for(args.steps % len(window))
        if args.warmup % len(window):
            graph_for(args.warmup % len(window))
        torch.cuda.synchronize()

    run_steps(args.warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps(args.steps)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_s = T * args.steps / elapsed
    gbps = bytes_per_step * args.steps / elapsed / 1e9

    # ---- per-kernel durations from HIP events in each kernel's own dispatch, on the
    # stream that kernel runs on --------------------------------------------------------
    prof_steps = max(len(window), min(args.steps, 4 * len(window)))
    mf.profile_enable(True)
    for s in range(prof_steps):
        launch(s)
    torch.cuda.synchronize()
    prof = mf.profile_read()
    mf.profile_enable(False)
    small = T <= info.matvec_max_tokens
    shared_mode = {1: "aux", 2: "seq", 3: "fused"}[info.shared_mode_matvec if small else info.shared_mode_gemm]
    # the routed (+ shared when fused) gate/up launch moves the most bytes; its name
    # says which regime ran (mat-vec or grouped GEMM)
    dominant = "gg_gate_up" if prof["gg_gate_up"][1] else "gate_up"
    ms_tot, n_launch = prof[dominant]
    avg_us = ms_tot * 1e3 / max(1, n_launch)
    gu_units = unique_mean + (1 if shared_mode == "fused" else 0)
    achieved = gu_units * gu_b / (avg_us * 1e-6) / 1e9
    # the contraction the dominant launch performs: gate and up (two H x I products) per
    # (token, slot) pair, plus the shared expert's per token when it is fused in
    gu_flops = 4.0 * shape.hidden * shape.inter * T * shape.top_k
    if shared_mode == "fused":
        gu_flops += 4.0 * shape.hidden * shape.shared_inter * T
    tflops = gu_flops / (avg_us * 1e-6) / 1e12
    # which roof binds the algorithm: the time its bytes take at peak bandwidth or the
    # time its flops take at the MFMA peak (only the grouped GEMM runs on MFMA)
    mfma_bound = dominant == "gg_gate_up" and (gu_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
                                               > gu_units * gu_b / (HBM_PEAK_GBPS * 1e9))
    kernels = {k: round(v[0] * 1e3 / v[1], 3) for k, v in prof.items() if v[1]}
    roofline = ({"bound": "mfma", "kernel": dominant, "achieved": round(tflops, 1),
                 "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)} if mfma_bound else
                {"bound": "hbm", "kernel": dominant, "achieved": round(achieved, 1),
                 "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4)})
    roofline |= {"traffic": traffic_for(args, shape, T, shared_mode, dominant), "avg_us": round(avg_us, 3),
                 "algorithmic_bytes_per_launch": int(gu_units * gu_b),
                 "algorithmic_flops_per_launch": int(gu_flops),
                 "hbm_frac": round(achieved / HBM_PEAK_GBPS, 4),
                 "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4) if dominant == "gg_gate_up" else None}
    mf.close()
    return {"tokens": T, "value": round(tokens_per_s, 1), "unit": "tokens/s",
            "ms_per_step": round(ms_per_step, 6), "expert_weight_GBps": round(gbps, 1),
            "expert_weight_hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
            "unique_experts_per_step": round(unique_mean, 3),
            "expert_weight_bytes_per_step": int(bytes_per_step), "kernel_avg_us": kernels,
            "roofline": roofline, "shared_mode": shared_mode,
            "regime": "gemm" if dominant == "gg_gate_up" else "matvec", "xs": xs}


def cpu_leg(layer_host, xs, n_cpu: int, threads: int, seconds: float) -> dict:
    """The oracle (test infrastructure, never tuned) on the host cores: forwards of n_cpu
    tokens of the same workload for a bounded time."""
    from oracle.oracle import Oracle
    from tests.helpers import oracle_tokens
    orc = Oracle()
    calls, c0 = 0, time.perf_counter()
    while True:
        orc.forward(layer_host, oracle_tokens(xs[calls % len(xs)][:n_cpu].cpu()), nthreads=threads)
        calls += 1
        if time.perf_counter() - c0 >= seconds:
            break
    c_el = time.perf_counter() - c0
    return {"value": round(n_cpu * calls / c_el, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{calls} forwards of {n_cpu} token(s) on layer copy 0 ({c_el:.1f} s, fp64, "
                      f"{threads} OpenMP thread(s) over rows)"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20000)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--workload", default="decode_bf16_t1")
    ap.add_argument("--also-tokens", type=str, default=None,
                    help="comma-separated extra batch sizes timed on the same layer copies "
                         "(default: 8 for decode_bf16_t1; '' for none)")
    ap.add_argument("--mode", default="auto", choices=["auto", "aux", "seq", "fused"])
    ap.add_argument("--regime", default="auto", choices=["auto", "matvec", "gemm"])
    ap.add_argument("--tokens", type=int, default=0, help="override the workload's batch (sweeps)")
    ap.add_argument("--eager", action="store_true")
    ap.add_argument("--input-block", action="store_true",
                    help="also run the FFN-input RMSNorm (eps 1e-6) and the residual add")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--cpu-seconds-1thread", type=float, default=8.0)
    ap.add_argument("--traffic", default=None,
                    help="traffic summary from rocprofv3 counters (default profiles/traffic_<workload>.md)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the layer runs on one GPU only; splitting it over several GPUs "
              "(experts or their rows sharded per GPU) is described, not implemented", file=sys.stderr)
        return 2

    import torch

    from moe_decode_ffn_amd import ffn, synth
    from moe_decode_ffn_amd.traffic import kernel_source_hash

    if args.workload not in synth.WORKLOADS:
        print(f"unknown workload {args.workload}; choose from {sorted(synth.WORKLOADS)}", file=sys.stderr)
        return 2
    shape, seed, counts = synth.WORKLOADS[args.workload]
    T = args.tokens or counts[-1]
    if args.also_tokens is None:
        extra = () if args.tokens else EXTRA_TOKENS.get(args.workload, ())
    else:
        extra = tuple(int(v) for v in args.also_tokens.split(",") if v.strip())
    dev = torch.device("cuda:0")
    mode = {"auto": ffn.SHARED_AUTO, "aux": ffn.SHARED_AUX, "seq": ffn.SHARED_SEQ,
            "fused": ffn.SHARED_FUSED}[args.mode]
    regime = {"auto": 0, "matvec": ffn.FORCE_MATVEC, "gemm": ffn.FORCE_GEMM}[args.regime]

    # ---- inputs resident in HBM ---------------------------------------------------------
    # enough copies that the calls between two uses of one copy read well over the 256 MB
    # cache even at one token (k routed experts + the shared one per call)
    gu_b, d_b = expert_bytes(shape)
    min_call_bytes = (shape.top_k + 1) * (gu_b + d_b)
    L = (max(LAYER_COPIES[shape.w_dtype], min(128, -(-MIN_ROTATION_BYTES // min_call_bytes) + 1))
         if shape.hidden >= 1024 else 2)
    layers = [synth.make_layer_device(shape, 100 + i, dev) for i in range(L)]
    if args.input_block:
        layers = [synth.with_input_block(ly, 500 + i, eps=1e-6) for i, ly in enumerate(layers)]

    main_leg = measure(args, shape, layers, T, mode, regime, dev)
    legs = [measure(args, shape, layers, t, mode, regime, dev) for t in extra if t != T]

    # ---- the oracle on the host cores (a bounded sample of the same workload) -------------
    cpu = None
    if not args.no_cpu_baseline:
        from tests.helpers import oracle_layer
        try:
            cores = len(os.sched_getaffinity(0))
        except AttributeError:
            cores = os.cpu_count() or 1
        host_layer = oracle_layer({k: (v.cpu() if isinstance(v, torch.Tensor) else v)
                                   for k, v in layers[0].items()})
        # each token's output depends on that token alone: large batches are sampled
        n_cpu = min(T, 64)
        cpu = cpu_leg(host_layer, main_leg["xs"], n_cpu, cores, args.cpu_seconds)
        if args.cpu_seconds_1thread > 0:
            cpu["one_thread"] = cpu_leg(host_layer, main_leg["xs"], n_cpu, 1, args.cpu_seconds_1thread)

    def public(leg: dict) -> dict:
        return {k: v for k, v in leg.items() if k not in ("xs", "shared_mode", "regime")}

    m = main_leg
    res = {
        "metric": METRIC,
        "value": m["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "q4": "q4_b32+bf16", "f32": "f32"}[shape.w_dtype],
        "data": "synthetic",
        "config": {"workload": args.workload, "hidden": shape.hidden, "experts": shape.n_experts,
                   "top_k": shape.top_k, "inter": shape.inter, "shared_inter": shape.shared_inter,
                   "tokens": T, "weights": shape.w_dtype, "accumulate": "fp32",
                   "layer_copies": L, "shared_mode": m["shared_mode"], "regime": m["regime"],
                   "launch": "eager" if args.eager else "hip_graph",
                   "input_block": "rmsnorm+residual" if args.input_block else "none"},
        "expert_weight_GBps": m["expert_weight_GBps"],
        "expert_weight_hbm_frac": m["expert_weight_hbm_frac"],
        "unique_experts_per_step": m["unique_experts_per_step"],
        "expert_weight_bytes_per_step": m["expert_weight_bytes_per_step"],
        "kernel_avg_us": m["kernel_avg_us"],
        "roofline": m["roofline"],
    }
    for leg in legs:
        res[f"batch_{leg['tokens']}"] = public(leg) | {"shared_mode": leg["shared_mode"], "regime": leg["regime"]}
    res["cpu_baseline"] = cpu
    res["kernel_source_hash"] = kernel_source_hash()
    print(json.dumps(res))
    return 0


if __name__ == "__main__":
    sys.exit(main())
