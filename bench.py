#!/usr/bin/env python
"""Benchmark of the fused MoE forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]

A step is one whole fused MoE forward (routing, align/sort, gate-up GEMM + SiLU*up, down GEMM,
shared expert if the workload has one, weighted combine) over one batch of seeded synthetic
inputs already resident in HBM.  The default workload is the DeepSeek-V3-style grouped prefill
(T=4096 tokens, H=7168, E=256 experts, F=2048, top-8 sigmoid routing with a correction bias,
8 groups / top-4, routed scaling 2.5), the largest single-GPU workload.

To keep the expert weights cold (the weights are what the pass streams), the inputs come in R
rotating sets -- separate weights, hidden states and gating per set -- with R chosen so the
sets together exceed 16x the 256 MB last-level cache; step i uses set i mod R.

Two timed loops of K steps each (W warm-up steps first), bracketed by synchronize():
  1. fused_moe_fwd calls -> ``value`` / ``ms_per_step``;
  2. the same pass as moe_route + fused_moe_experts_stage calls with HIP events between the
     stages on the stream they run on -> per-stage device times, and the dominant kernel's
     roofline (gate-up GEMM: its algorithmic bytes / its average duration vs 8 TB/s HBM).
The CPU oracle is then timed on the host's cores on a bounded sample of the same workload.
Prints ONE JSON line on stdout (diagnostics go to stderr).
"""
import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

LLC_BYTES = 256 * 2 ** 20
PROFILE_DIR = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default=None)
    ap.add_argument("--dtype", default="bf16", choices=["bf16", "f16"],
                    help="element type of the fused pass (activations, weights, output)")
    ap.add_argument("--weights", default="16bit", choices=["16bit", "mxfp4", "fp8"],
                    help="expert weight format: the pass's element type, MXFP4 (bf16 "
                         "activations), or FP8 e4m3 with 128x128 block scales (activations "
                         "quantised per 1x128 group)")
    ap.add_argument("--rotate", type=int, default=0, help="input sets (0 = automatic)")
    ap.add_argument("--path", default="auto", choices=["auto", "direct", "sorted"],
                    help="the library's path choice (auto: its own rule)")
    ap.add_argument("--skew", default=None, metavar="ALPHA|auto",
                    help="skewed routing (aiter MI308 decoding PR, 'Skewed routing'): add "
                         "-alpha*log(1+rank) to the router scores; 'auto' takes the alpha that "
                         "gives the workload's most popular expert twice the mean load.  The "
                         "line then also times the same pass on the unskewed scores")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="one device-to-device copy of BYTES before the timed loops (the "
                         "known-size reference for rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="DIR",
                    help="write profiles/<kernel>_<workload>_pmc.txt from rocprofv3 --pmc "
                         "output directories (FETCH_SIZE run, WRITE_SIZE run[, MFMA run])")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="write profiles/kernel_trace_<workload>.md from a rocprofv3 "
                         "--kernel-trace --stats output directory")
    ap.add_argument("--pmc-commands", nargs="*", default=[],
                    help="the rocprofv3 command lines that produced --summarize-pmc's inputs")
    return ap.parse_args()


def main():
    args = parse()
    if args.summarize_pmc:
        summarize_pmc(args)
        return
    if args.summarize_trace:
        summarize_trace(args)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (--gpus %d "
              "requested). Run with --gpus 1." % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mixture_experts_forward_amd as moe
    from moe_harness import perfmodel
    from moe_harness.workloads import (BENCH_CONFIG, CONFIGS, FP8_CONFIGS, MASKED_CONFIGS,
                                       make_fp8_weights, make_inputs, make_mxfp4_weights,
                                       skew_alpha, skew_gating)

    if args.config in MASKED_CONFIGS:
        bench_masked(args, MASKED_CONFIGS[args.config])
        return
    if args.config in FP8_CONFIGS:
        bench_fp8(args, FP8_CONFIGS[args.config])
        return
    cfg = CONFIGS[args.config or BENCH_CONFIG]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    moe.lib()

    mx = args.weights == "mxfp4"
    f8 = args.weights == "fp8"
    if (mx or f8) and (cfg.S > 0 or args.dtype != "bf16"):
        sys.exit("--weights %s takes bf16 activations and no shared expert" % args.weights)
    # bytes per routed expert's weights relative to 16-bit: MXFP4 half a byte per element plus
    # one scale byte per 32; FP8 one byte plus 4 bytes per 128 x 128 block
    wfac = 17.0 / 32.0 / 2.0 if mx else ((1.0 + 4.0 / 16384.0) / 2.0 if f8 else 1.0)
    wbytes = cfg.E * 6.0 * cfg.H * cfg.F * wfac + 6.0 * cfg.H * cfg.S
    R = args.rotate or max(1, min(8, math.ceil(16 * LLC_BYTES / wbytes)))
    log("workload %s, %d input sets of %.2f GB weights" % (cfg.name, R, wbytes / 1e9))
    tdt = torch.float16 if args.dtype == "f16" else torch.bfloat16
    if mx or f8:
        sets = []
        for i in range(R):
            d = make_inputs(cfg, dev, seed=42 + i, weights=False)
            d.update((make_mxfp4_weights if mx else make_fp8_weights)(cfg, dev, seed=42 + i))
            sets.append(d)
    else:
        sets = [make_inputs(cfg, dev, seed=42 + i, dtype=tdt) for i in range(R)]
    alpha = None
    if args.skew is not None:
        alpha = skew_alpha(cfg) if args.skew == "auto" else float(args.skew)
        for d in sets:
            d["gating_uniform"] = d["gating_output"]
            d["gating_output"] = skew_gating(d["gating_output"], alpha)
        log("skewed routing: alpha %.4f" % alpha)
    torch.cuda.synchronize()
    if args.copy_calibration:
        src = torch.ones(args.copy_calibration, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)      # one plain copy kernel of known size
        torch.cuda.synchronize()
        del src, dst

    S = cfg.S
    p = moe.make_params(cfg.T, cfg.H, cfg.E, cfg.F, cfg.k, cfg.scoring, cfg.renormalize,
                        cfg.num_expert_group, cfg.topk_group, cfg.rsf, path=args.path,
                        dtype=tdt)
    ws_need = (moe.mxfp4_workspace_bytes(p) if mx else
               moe.fp8_workspace_bytes(p) if f8 else moe.workspace_bytes(p, S))
    ws = torch.empty(max(256, ws_need), dtype=torch.uint8, device=dev)
    out = torch.empty((cfg.T, cfg.H), dtype=tdt, device=dev)
    ids = [torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=dev) for _ in range(R)]
    wts = [torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=dev) for _ in range(R)]

    def fused_step(i):
        d = sets[i % R]
        if f8:
            moe.fused_moe_fp8_fwd(d["hidden_states"], d["gating_output"], d["w_gate_up"],
                                  d["w_gate_up_scale"], d["w_down"], d["w_down_scale"], cfg.k,
                                  d["correction_bias"], cfg.scoring, cfg.renormalize,
                                  cfg.num_expert_group, cfg.topk_group, cfg.rsf, out=out,
                                  workspace=ws, path=args.path)
        elif mx:
            moe.fused_moe_mxfp4_fwd(d["hidden_states"], d["gating_output"], d["w_gate_up_q"],
                                    d["w_gate_up_scale"], d["w_down_q"], d["w_down_scale"],
                                    cfg.k, d["correction_bias"], cfg.scoring, cfg.renormalize,
                                    cfg.num_expert_group, cfg.topk_group, cfg.rsf,
                                    path=args.path, out=out, workspace=ws)
        elif S > 0:
            moe.fused_moe_shared_fwd(d["hidden_states"], d["gating_output"], d["w_gate_up"],
                                     d["w_down"], d["shared_w_gate_up"], d["shared_w_down"],
                                     cfg.k, d["correction_bias"], cfg.scoring, cfg.renormalize,
                                     cfg.num_expert_group, cfg.topk_group, cfg.rsf,
                                     path=args.path, out=out, workspace=ws)
        else:
            moe.fused_moe_fwd(d["hidden_states"], d["gating_output"], d["w_gate_up"],
                              d["w_down"], cfg.k, d["correction_bias"], cfg.scoring,
                              cfg.renormalize, cfg.num_expert_group, cfg.topk_group, cfg.rsf,
                              path=args.path, out=out, workspace=ws)

    stages = [moe.STAGE_ALIGN, moe.STAGE_GATE_UP, moe.STAGE_DOWN]
    if S > 0:
        stages.append(moe.STAGE_SHARED)
    stages.append(moe.STAGE_COMBINE)
    names = ["route"] + [moe.STAGE_NAMES[s] for s in stages]

    def staged_step(i, events=None):
        d = sets[i % R]
        j = i % R
        if events is not None:
            events[0].record()
        st = moe.lib().moe_route(moe._ptr(d["gating_output"]), moe._ptr(d["correction_bias"]),
                                 ctypes.byref(p), moe._ptr(ids[j]),
                                 moe._ptr(wts[j]), moe._stream(dev))
        if st != 0:
            raise moe.MoEError(st, "moe_route")
        if events is not None:
            events[1].record()
        for n, s in enumerate(stages):
            if f8:
                moe.fused_moe_fp8_stage(s, p, d["hidden_states"], d, ids[j], wts[j], out, ws)
            elif mx:
                moe.fused_moe_mxfp4_stage(s, p, d["hidden_states"], d, ids[j], wts[j], out, ws)
            else:
                moe.fused_moe_experts_stage(s, p, d["hidden_states"], d["w_gate_up"],
                                            d["w_down"], ids[j], wts[j], out, ws,
                                            d.get("shared_w_gate_up"), d.get("shared_w_down"))
            if events is not None:
                events[n + 2].record()

    # ---- loop 1: fused calls
    for i in range(args.warmup):
        fused_step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        fused_step(i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fused_ms = e0.elapsed_time(e1) / args.steps
    log("fused: %.4f ms/step (device), %.4f ms/step (wall)" % (fused_ms,
                                                                 wall * 1e3 / args.steps))
    skew_cmp = None
    if alpha is not None:
        # the same loop on the unskewed scores of the same input sets
        for d in sets:
            d["gating_output"], d["gating_uniform"] = d["gating_uniform"], d["gating_output"]
        for i in range(args.warmup):
            fused_step(i)
        torch.cuda.synchronize()
        e0.record()
        for i in range(args.steps):
            fused_step(i)
        e1.record()
        torch.cuda.synchronize()
        uniform_ms = e0.elapsed_time(e1) / args.steps
        for d in sets:
            d["gating_output"], d["gating_uniform"] = d["gating_uniform"], d["gating_output"]
        skew_cmp = {"alpha": alpha, "skewed_ms": round(fused_ms, 5),
                    "unskewed_ms": round(uniform_ms, 5),
                    "skewed_over_unskewed": round(fused_ms / uniform_ms, 4)}
        log("unskewed scores: %.4f ms/step; skewed / unskewed %.3f" % (uniform_ms,
                                                                       fused_ms / uniform_ms))

    # ---- loop 2: staged calls with events between the stages
    for i in range(args.warmup):
        staged_step(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
           for _ in range(args.steps)]
    for i in range(args.steps):
        staged_step(i, evs[i])
    torch.cuda.synchronize()
    per_stage = {n: 0.0 for n in names}
    for i in range(args.steps):
        for n, name in enumerate(names):
            per_stage[name] += evs[i][n].elapsed_time(evs[i][n + 1]) / args.steps
    staged_ms = evs[0][0].elapsed_time(evs[-1][-1]) / args.steps
    log("staged: %.4f ms/step; per stage (ms): %s" % (
        staged_ms, ", ".join("%s %.4f" % (k, v) for k, v in per_stage.items())))

    # ---- loop 3: the same fused calls replayed from HIP graphs (one graph per input set):
    # the pass without host launch overhead
    graphs = []
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for j in range(R):
            fused_step(j)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for j in range(R):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fused_step(j)
        graphs.append(g)
    for i in range(args.warmup):
        graphs[i % R].replay()
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        graphs[i % R].replay()
    e1.record()
    torch.cuda.synchronize()
    graph_ms = e0.elapsed_time(e1) / args.steps
    del graphs
    # ---- loop 3b: per-step events around single fused calls, for the median
    step_evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(args.steps)]
    for i in range(args.steps):
        step_evs[i][0].record()
        fused_step(i)
        step_evs[i][1].record()
    torch.cuda.synchronize()
    median_ms = float(np.median([a.elapsed_time(b) for a, b in step_evs]))
    # ---- loop 4: one input set over and over (weights partly cache-resident)
    for i in range(args.warmup):
        fused_step(0)
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        fused_step(0)
    e1.record()
    torch.cuda.synchronize()
    warm_ms = e0.elapsed_time(e1) / args.steps
    log("graph replay: %.4f ms/step; median single call %.4f ms; warm (one input set): "
        "%.4f ms/step" % (graph_ms, median_ms, warm_ms))
    ctx = context_numbers(torch, dev)
    log("context: streaming read %.0f GB/s, device copy %.0f GB/s, torch bf16 matmul %.0f "
        "TFLOP/s" % (ctx["stream_read_gbps"], ctx["device_copy_gbps"],
                     ctx["torch_matmul_bf16_tflops"]))

    # ---- roofline of the pass and of the dominant kernel, from the realized routing
    touched = []
    loads = []
    for j in range(R):
        idj = ids[j].cpu().numpy()
        touched.append(perfmodel.touched_experts(idj, cfg.E))
        loads.append(perfmodel.load_stats(idj, cfg.E))
    touched_mean = float(np.mean([touched[i % R] for i in range(args.steps)]))
    P = cfg.T * cfg.k
    pass_bytes = perfmodel.algorithmic_bytes(cfg.T, cfg.H, cfg.E, cfg.F, cfg.k, touched_mean,
                                             cfg.S, cfg.bias)
    # MXFP4: the touched experts' weights shrink to 17/64 of their bf16 bytes
    pass_bytes -= touched_mean * 6.0 * cfg.H * cfg.F * (1.0 - wfac)
    pass_flops = perfmodel.flops(cfg.T, cfg.k, cfg.H, cfg.F, cfg.S)
    gu_bytes = touched_mean * 4.0 * cfg.H * cfg.F * wfac + 2.0 * cfg.T * cfg.H + 2.0 * P * cfg.F
    gu_flops = 2.0 * P * 2 * cfg.F * cfg.H
    gu_ms = per_stage["gate_up"]
    gu_gbs = gu_bytes / (gu_ms * 1e-3) / 1e9
    gu_tflops = gu_flops / (gu_ms * 1e-3) / 1e12
    peak_gbs = perfmodel.HBM_PEAK_BYTES_PER_S / 1e9
    peak_tflops = perfmodel.BF16_MFMA_PEAK_FLOP_PER_S / 1e12
    # the gate-up kernel's own bound: its bytes at 8 TB/s or its FLOPs at the bf16 MFMA peak
    gu_mfma_bound = gu_flops / perfmodel.BF16_MFMA_PEAK_FLOP_PER_S > \
        gu_bytes / perfmodel.HBM_PEAK_BYTES_PER_S
    # algorithmic bytes of each HBM-bound stage (what it must read and write once) and its rate
    # against the 8 TB/s peak: touched experts' weights, the activation / intermediate rows it
    # reads and the rows it writes (16-bit elements; MXFP4 / FP8 weights scaled by wfac)
    eb = 2.0  # bytes per 16-bit element
    stage_bytes = {
        "route": 4.0 * cfg.T * cfg.E + (4.0 * cfg.E if cfg.bias else 0.0) + 8.0 * P,
        "gate_up": gu_bytes,
        "down": touched_mean * 2.0 * cfg.H * cfg.F * wfac + eb * P * cfg.F + eb * P * cfg.H,
        "combine": eb * P * cfg.H + 8.0 * P + eb * cfg.T * cfg.H * (2.0 if S > 0 else 1.0),
    }
    if S > 0:
        stage_bytes["shared"] = (6.0 * cfg.H * S * eb / 2.0 + eb * cfg.T * cfg.H
                                 + 2.0 * eb * cfg.T * S + eb * cfg.T * cfg.H)
    stage_flops = {"gate_up": gu_flops, "down": 2.0 * P * cfg.H * cfg.F,
                   "shared": 2.0 * cfg.T * 3.0 * cfg.H * S}
    stage_roofline = {}
    for name, b in stage_bytes.items():
        t = per_stage.get(name)
        if t:
            gbs = b / (t * 1e-3) / 1e9
            stage_roofline[name] = {"algorithmic_bytes": b, "achieved_gbps": round(gbs, 1),
                                    "frac_of_hbm_peak": round(gbs / peak_gbs, 4)}
            if stage_flops.get(name):
                tf = stage_flops[name] / (t * 1e-3) / 1e12
                stage_roofline[name].update(achieved_tflops=round(tf, 1),
                                            frac_of_mfma_peak=round(tf / peak_tflops, 4))
    # the committed counter summaries are of the bf16 kernels with bf16 weights
    traffic = None
    if args.dtype == "bf16" and args.weights in ("16bit", "mxfp4"):
        traffic = read_traffic(cfg.name, "_mxfp4" if args.weights == "mxfp4" else "")

    # ---- CPU baseline: the oracle on this host
    if args.no_cpu_baseline:
        cpu = None
    elif f8:
        cpu = cpu_baseline_fp8(cfg, sets[0], args.cpu_seconds)
    else:
        cpu = cpu_baseline(cfg, sets[0], args.cpu_seconds, args.dtype)
    base = None if args.weights != "16bit" else BASELINE_MS.get(
        cfg.name if args.dtype == "bf16" else cfg.name + ":" + args.dtype)

    ms = fused_ms
    t_hbm = pass_bytes / perfmodel.HBM_PEAK_BYTES_PER_S
    t_mfma = pass_flops / perfmodel.BF16_MFMA_PEAK_FLOP_PER_S
    floor_ms = max(t_hbm, t_mfma) * 1e3
    line = {
        "metric": "fused-MoE fwd ms; achieved TB/s (decode) / TFLOP/s (prefill) vs roofline",
        "value": round(ms, 5),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": False,
        "scaling": "weak",
        # the pages' figures come from other GPUs: context (baseline_context), not a target
        "vs_baseline": None,
        "dtype": "fp8e4m3" if f8 else args.dtype,
        "data": "synthetic (seeded; %d rotating input sets)" % R,
        "config": {"workload": cfg.name, "T": cfg.T, "H": cfg.H, "E": cfg.E, "F": cfg.F,
                   "top_k": cfg.k, "scoring": cfg.scoring, "renormalize": cfg.renormalize,
                   "num_expert_group": cfg.num_expert_group, "topk_group": cfg.topk_group,
                   "routed_scaling_factor": cfg.rsf, "correction_bias": cfg.bias,
                   "shared_inter": cfg.S, "path": args.path, "weights": args.weights,
                   "skew_alpha": alpha, "parallelism": "single GPU"},
        "achieved_tbps": round(pass_bytes / (ms * 1e-3) / 1e12, 4),
        "achieved_tflops": round(pass_flops / (ms * 1e-3) / 1e12, 3),
        "hbm_roofline_frac": round(pass_bytes / (ms * 1e-3) / perfmodel.HBM_PEAK_BYTES_PER_S, 4),
        "mfma_roofline_frac": round(pass_flops / (ms * 1e-3) /
                                    perfmodel.BF16_MFMA_PEAK_FLOP_PER_S, 4),
        "algorithmic_bytes": pass_bytes,
        "flops": pass_flops,
        "touched_experts": touched_mean,
        "rows_per_expert": loads[0],
        "binding_roofline": {"bound": "hbm" if t_hbm >= t_mfma else "mfma",
                             "floor_ms": round(floor_ms, 5), "frac": round(floor_ms / ms, 4)},
        "graph_ms_per_step": round(graph_ms, 5),
        "median_ms_single_call": round(median_ms, 5),
        "warm_ms_per_step": round(warm_ms, 5),
        "staged_ms_per_step": round(staged_ms, 5),
        "stage_ms": {k: round(v, 5) for k, v in per_stage.items()},
        "stage_roofline": stage_roofline,
        # the fused call runs the shared expert on a second stream beside the routed GEMMs;
        # the in-order stages give it the same three eighths of the CUs, so its stage time
        # alone is longer than its share of the fused call
        "stage_notes": ({"shared": "3/8 of the CUs, overlapped in the fused call"}
                        if S > 0 else {}),
        "roofline": ({"kernel": "gate-up GEMM of the routed experts", "bound": "mfma",
                      "achieved": round(gu_tflops, 1), "peak": peak_tflops, "unit": "TFLOP/s",
                      "frac": round(gu_tflops / peak_tflops, 4), "traffic": traffic,
                      "algorithmic_flops_per_launch": gu_flops,
                      "algorithmic_bytes_per_launch": gu_bytes}
                     if gu_mfma_bound else
                     {"kernel": "gate-up GEMM of the routed experts", "bound": "hbm",
                      "achieved": round(gu_gbs, 1), "peak": peak_gbs, "unit": "GB/s",
                      "frac": round(gu_gbs / peak_gbs, 4), "traffic": traffic,
                      "algorithmic_bytes_per_launch": gu_bytes,
                      # the same rate against what a plain streaming read reaches here
                      "stream_read_gbps": ctx["stream_read_gbps"],
                      "frac_of_stream_read": round(gu_gbs / ctx["stream_read_gbps"], 4)}),
        "cpu_baseline": cpu,
        "baseline_context": base,
        "context": ctx,
    }
    if skew_cmp is not None:
        line["skew"] = skew_cmp
    print(json.dumps(line), flush=True)


def bench_masked(args, cfg):
    """The masked-layout expert MLPs of one expert-parallel shard (fused_moe_masked_fwd): the
    whole call, and its stages with events between them; the roofline object is the gate-up
    GEMM's (the page's MoEGroupedGemmFwd on the same shapes)."""
    import numpy as np
    import torch

    import mixture_experts_forward_amd as moe
    from moe_harness import perfmodel
    from moe_harness.workloads import make_masked_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    moe.lib()
    wbytes = cfg.E * 6.0 * cfg.H * cfg.F
    R = args.rotate or max(1, min(8, math.ceil(16 * LLC_BYTES / wbytes)))
    sets = [make_masked_inputs(cfg, dev, seed=42 + i) for i in range(R)]
    ws = torch.empty(max(256, moe.masked_workspace_bytes(cfg.E, cfg.max_m, cfg.H, cfg.F)),
                     dtype=torch.uint8, device=dev)
    out = torch.zeros((cfg.E, cfg.max_m, cfg.H), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    def step(i):
        d = sets[i % R]
        moe.fused_moe_masked_fwd(d["a"], d["masked_m"], d["w_gate_up"], d["w_down"], out=out,
                                 workspace=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    stages = [moe.STAGE_ALIGN, moe.STAGE_GATE_UP, moe.STAGE_DOWN]
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        d = sets[i % R]
        evs[i][0].record()
        for n, st in enumerate(stages):
            moe.fused_moe_masked_stage(st, d["a"], d["masked_m"], d["w_gate_up"], d["w_down"],
                                       out, ws)
            evs[i][n + 1].record()
    torch.cuda.synchronize()
    per = {moe.STAGE_NAMES[st]: sum(e[n].elapsed_time(e[n + 1]) for e in evs) / args.steps
           for n, st in enumerate(stages)}
    log("masked %s: %.4f ms/call; stages (ms): %s" % (
        cfg.name, ms, ", ".join("%s %.4f" % kv for kv in per.items())))
    rows = float(np.mean([int(sd["masked_m"].clamp(0, cfg.max_m).sum()) for sd in sets]))
    pass_bytes = wbytes + 4.0 * rows * cfg.H + 4.0 * cfg.E
    pass_flops = 2.0 * rows * 3 * cfg.H * cfg.F
    gu_bytes = cfg.E * 4.0 * cfg.H * cfg.F + 2.0 * rows * cfg.H + 2.0 * rows * cfg.F
    gu_gbs = gu_bytes / (per["gate_up"] * 1e-3) / 1e9
    peak_gbs = perfmodel.HBM_PEAK_BYTES_PER_S / 1e9
    t_hbm = pass_bytes / perfmodel.HBM_PEAK_BYTES_PER_S
    t_mfma = pass_flops / perfmodel.BF16_MFMA_PEAK_FLOP_PER_S
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_masked(cfg, sets[0], args.cpu_seconds)
    line = {
        "metric": "masked expert-MLP ms (one expert-parallel shard); achieved TB/s vs roofline",
        "value": round(ms, 5), "unit": "ms", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; %d rotating input sets)" % R,
        "config": {"workload": cfg.name, "E": cfg.E, "max_m": cfg.max_m, "H": cfg.H,
                   "F": cfg.F, "rows_in_use_mean": rows, "parallelism": "single GPU"},
        "achieved_tbps": round(pass_bytes / (ms * 1e-3) / 1e12, 4),
        "achieved_tflops": round(pass_flops / (ms * 1e-3) / 1e12, 3),
        "binding_roofline": {"bound": "hbm" if t_hbm >= t_mfma else "mfma",
                             "floor_ms": round(max(t_hbm, t_mfma) * 1e3, 5),
                             "frac": round(max(t_hbm, t_mfma) * 1e3 / ms, 4)},
        "stage_ms": {k: round(v, 5) for k, v in per.items()},
        "roofline": {"kernel": "gate-up GEMM of the masked rows", "bound": "hbm",
                     "achieved": round(gu_gbs, 1), "peak": peak_gbs, "unit": "GB/s",
                     "frac": round(gu_gbs / peak_gbs, 4), "traffic": read_traffic(cfg.name),
                     "algorithmic_bytes_per_launch": gu_bytes},
        "cpu_baseline": cpu,
        "baseline_context": {"gate_up_ms": 0.4851, "source": "TileOPs MoE page, "
                             "MoEGroupedGemmFwd ds-v3-ep8-masked bf16 (the gate-up GEMM alone)",
                             "hardware": "not named on the page"},
    }
    print(json.dumps(line), flush=True)


# The pages' figures for the FP8 grouped GEMM workloads (TileOPs "MoE" page,
# MoEGroupedGemmFP8Fwd; GPU not named): context only.
FP8_BASELINE_MS = {"ds-v3-dec-b64-up": 0.2266, "ds-v3-dec-b64-down": 0.1157,
                   "ds-v3-dec-b256-up": 0.2420, "ds-v3-e8-up-masked": 0.0743}


def bench_fp8(args, cfg):
    """The block-scaled FP8 grouped GEMM of the masked layout (moe_grouped_gemm_fp8): one
    launch per step, against the 8 TB/s roofline of its bytes (e4m3 operands, f32 scales, bf16
    output) and the 5.0 PFLOP/s dense FP8 MFMA peak."""
    import numpy as np
    import torch

    import mixture_experts_forward_amd as moe
    from moe_harness import perfmodel
    from moe_harness.workloads import make_fp8_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    moe.lib()
    KB, NB = cfg.K // 128, (cfg.N + 127) // 128
    wbytes = cfg.E * (cfg.N * cfg.K + NB * KB * 4.0)
    R = args.rotate or max(1, min(8, math.ceil(16 * LLC_BYTES / wbytes)))
    sets = [make_fp8_inputs(cfg, dev, seed=42 + i) for i in range(R)]
    out = torch.zeros((cfg.E, cfg.max_m, cfg.N), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    def step(i):
        d = sets[i % R]
        moe.moe_grouped_gemm_fp8(d["a"], d["a_scale"], d["b"], d["b_scale"], d["masked_m"],
                                 out=out)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    rows = float(np.mean([int(sd["masked_m"].clamp(0, cfg.max_m).sum()) for sd in sets]))
    nbytes = wbytes + rows * (cfg.K + KB * 4.0 + 2.0 * cfg.N) + 4.0 * cfg.E
    flops = 2.0 * rows * cfg.N * cfg.K
    gbs = nbytes / (ms * 1e-3) / 1e9
    peak_gbs = perfmodel.HBM_PEAK_BYTES_PER_S / 1e9
    t_hbm, t_mfma = nbytes / perfmodel.HBM_PEAK_BYTES_PER_S, flops / 5.0e15
    log("fp8 %s: %.4f ms/call, %.0f GB/s, %.1f TFLOP/s" % (cfg.name, ms, gbs,
                                                          flops / (ms * 1e-3) / 1e12))
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        h = {k: v.cpu().numpy() for k, v in sets[0].items()}
        cols = 128
        t0 = time.perf_counter()
        oracle.grouped_gemm_fp8(h["a"][:1], h["a_scale"][:1], h["b"][:1, :cols],
                                h["b_scale"][:1, :1], h["masked_m"][:1])
        dt = time.perf_counter() - t0
        scale = cfg.E * (cfg.N / cols) * rows / cfg.E / max(1, int(h["masked_m"][0]))
        cpu = {"value": round(dt * scale * 1e3, 3), "unit": "ms", "cores": oracle.max_threads(),
               "kind": "oracle", "sample": "expert 0, first %d output columns, scaled to all "
               "experts, columns and rows in use" % cols}
        log("cpu oracle: sample %.2f s -> %.1f ms per call" % (dt, cpu["value"]))
    base = FP8_BASELINE_MS.get(cfg.name)
    line = {
        "metric": "FP8 grouped GEMM ms (masked layout, block scales); achieved TB/s vs roofline",
        "value": round(ms, 5), "unit": "ms", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8e4m3",
        "data": "synthetic (seeded e4m3 codes and scales; %d rotating input sets)" % R,
        "config": {"workload": cfg.name, "E": cfg.E, "max_m": cfg.max_m, "N": cfg.N,
                   "K": cfg.K, "rows_in_use_mean": rows, "parallelism": "single GPU"},
        "achieved_tbps": round(gbs / 1e3, 4),
        "achieved_tflops": round(flops / (ms * 1e-3) / 1e12, 3),
        "binding_roofline": {"bound": "hbm" if t_hbm >= t_mfma else "mfma",
                             "floor_ms": round(max(t_hbm, t_mfma) * 1e3, 5),
                             "frac": round(max(t_hbm, t_mfma) * 1e3 / ms, 4)},
        "roofline": {"kernel": "k_fp8_gemm", "bound": "hbm", "achieved": round(gbs, 1),
                     "peak": peak_gbs, "unit": "GB/s", "frac": round(gbs / peak_gbs, 4),
                     "traffic": read_traffic(cfg.name), "algorithmic_bytes_per_launch": nbytes},
        "cpu_baseline": cpu,
        "baseline_context": ({"ms": base, "source": "TileOPs MoE page, MoEGroupedGemmFP8Fwd "
                              "%s fp8e4m3" % cfg.name, "hardware": "not named on the page"}
                             if base else None),
    }
    print(json.dumps(line), flush=True)


def cpu_baseline_masked(cfg, d, seconds):
    """The oracle's masked MLP on the host for a sample of the experts, scaled to all E."""
    import numpy as np
    import oracle
    from moe_harness.workloads import to_u16
    a, m = to_u16(d["a"]), d["masked_m"].cpu().numpy()
    wgu, wd = to_u16(d["w_gate_up"]), to_u16(d["w_down"])
    t0 = time.perf_counter()
    oracle.masked_mlp(a[:1], m[:1], wgu[:1], wd[:1])
    one = max(time.perf_counter() - t0, 1e-6)
    n = int(max(1, min(cfg.E, seconds / one)))
    t0 = time.perf_counter()
    oracle.masked_mlp(a[:n], m[:n], wgu[:n], wd[:n])
    dt = time.perf_counter() - t0
    per_call = dt / n * cfg.E
    log("cpu oracle: %d of %d experts in %.2f s on %d threads -> %.1f ms per call" % (
        n, cfg.E, dt, oracle.max_threads(), per_call * 1e3))
    return {"value": round(per_call * 1e3, 3), "unit": "ms", "cores": oracle.max_threads(),
            "kind": "oracle", "sample": "%d of %d experts, scaled to all" % (n, cfg.E)}


def stream_read_gbps(torch, dev, nbytes=4 << 30, reps=5):
    """The library's streaming-read kernel (moe_stream_read) over a buffer 16x the last-level
    cache: the HBM read rate this GPU's CUs reach on a plain sequential stream."""
    import mixture_experts_forward_amd as moe
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device=dev).fill_(1)
    sink = moe.moe_stream_read(buf)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        moe.moe_stream_read(buf, sink)
    e1.record()
    torch.cuda.synchronize()
    gbps = nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del buf, sink
    return gbps


def context_numbers(torch, dev):
    """What this GPU reaches, for context: the library's streaming-read kernel over 4 GiB (the
    practical HBM read ceiling), a 1 GiB device-to-device copy (read + write bytes per second)
    and a torch bf16 8192^3 matmul."""
    read_gbps = stream_read_gbps(torch, dev)
    n = 1 << 30
    a = torch.ones(n, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    copy_gbps = 2.0 * n * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    m = 8192
    x = torch.randn((m, m), dtype=torch.bfloat16, device=dev)
    y = torch.randn((m, m), dtype=torch.bfloat16, device=dev)
    z = torch.matmul(x, y)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        z = torch.matmul(x, y)
    e1.record()
    torch.cuda.synchronize()
    tflops = 2.0 * m ** 3 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del x, y, z
    return {"stream_read_gbps": round(read_gbps, 1), "device_copy_gbps": round(copy_gbps, 1),
            "torch_matmul_bf16_tflops": round(tflops, 1)}


# The pages' own figure for this exact workload (another, unnamed GPU): context only.
BASELINE_MS = {
    "qwen3-30b-decode": {"ms": 0.2656, "source": "TileOPs MoE page, FusedMoEFwd "
                         "qwen3-30b-decode-b32 bf16", "hardware": "not named on the page"},
    "qwen3-235b-batch": {"ms": 1.2042, "source": "TileOPs MoE page, FusedMoEFwd "
                         "qwen3-235b-decode bf16", "hardware": "not named on the page"},
    "qwen3-235b-batch:f16": {"ms": 1.2004, "source": "TileOPs MoE page, FusedMoEFwd "
                             "qwen3-235b-decode f16", "hardware": "not named on the page"},
    "qwen3-30b-decode-b1": {"ms": 0.0396, "source": "TileOPs MoE page, FusedMoEFwd "
                            "qwen3-30b-decode-b1 bf16", "hardware": "not named on the page"},
    "qwen3-235b-prefill": {"ms": 2.5018, "source": "TileOPs MoE page, FusedMoEFwd "
                           "qwen3-235b-prefill bf16", "hardware": "not named on the page"},
    "ds-v3-grouped-decode": {"ms": 3.7285, "source": "TileOPs MoE page, FusedMoEFwd "
                             "ds-v3-grouped-decode bf16", "hardware": "not named on the page"},
    "kimi-k2-decode": {"ms": 3.6029, "source": "TileOPs MoE page, FusedMoEFwd kimi-k2-decode "
                       "bf16", "hardware": "not named on the page"},
    "kimi-k2-prefill": {"ms": 6.9423, "source": "TileOPs MoE page, FusedMoEFwd kimi-k2-prefill "
                        "bf16", "hardware": "not named on the page"},
    "ds-v3-grouped-prefill": {"ms": 7.1078, "source": "TileOPs MoE page, FusedMoEFwd "
                              "ds-v3-grouped-prefill bf16", "hardware": "not named on the page"},
    "kimi-k2-shared": {"ms": 5.0723, "source": "TileOPs MoE page, FusedMoESharedExpertFwd "
                       "kimi-k2-t512 bf16", "hardware": "not named on the page"},
}


def read_traffic(workload, suffix=""):
    """HBM traffic of the dominant kernel from the committed rocprofv3 counter summary
    (profiles/gate_up_<workload><suffix>_pmc.txt, suffix "_mxfp4" for MXFP4 weights: a line
    'traffic_bytes_per_launch: N' and the hash of the kernel sources it was taken on), or None
    when absent or taken on other sources."""
    path = os.path.join(PROFILE_DIR, "gate_up_%s%s_pmc.txt" % (workload, suffix))
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != kernel_source_hash(vals.get("kernel", "")):
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# kernel family (as it appears in a kernel name) -> its source files
KERNEL_FAMILY_SOURCES = {
    "k_ws_gemm": ("moe_ws_kernel.h", "moe_gemm_ws.hip"),
    "k_tiled_gemm": ("moe_tiled_kernel.h", "moe_gemm_tiled.hip"),
    "k_wide_gemm": ("moe_wide_kernel.h", "moe_gemm_wide.hip"),
    "k_mx_gemm": ("moe_mx_kernel.h", "moe_mx_dequant.h", "moe_gemm_mx.hip"),
    "k_mx_tiled": ("moe_mx_kernel.h", "moe_mx_dequant.h", "moe_gemm_mx.hip"),
    "k_wide_mx": ("moe_wide_kernel.h", "moe_mx_dequant.h", "moe_gemm_wide.hip"),
}
# template argument that holds the row source (SRC 2: the shared expert's dense rows), by
# family; the MXFP4 row-tiled and 256 x 256 kernels run on sorted rows only
KERNEL_FAMILY_SRC_ARG = {"k_ws_gemm": 1, "k_tiled_gemm": 1, "k_wide_gemm": 1, "k_mx_gemm": 1,
                         "k_mx_tiled": None, "k_wide_mx": None}

# GEMM roles with a counter summary each: profiles/<role>_<workload>_pmc.txt
PMC_ROLES = ("gate_up", "down", "shared_gate_up", "shared_down")


def kernel_source_hash(kernel_names):
    """Hash of the sources of the kernel family named in kernel_names (the summary's 'kernel'
    line; its template arguments record the tile shape the plan chose) and the shared device
    helpers: a counter summary taken on other sources of that kernel is stale.  Changes to
    other kernels leave it valid."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mixture_experts_forward_amd", "csrc")
    names = []
    for fam, files in KERNEL_FAMILY_SOURCES.items():
        if fam in kernel_names:
            names += files
    for name in names + ["moe_device.h"]:
        h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()[:16]


def _read_counters(d):
    """rocprofv3 --pmc CSV rows of directory d -> {dispatch_id: (kernel name, {counter: value})}"""
    import csv
    import glob
    out = {}
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for row in csv.DictReader(open(path)):
            did = int(row["Dispatch_Id"])
            name, vals = out.setdefault(did, (row["Kernel_Name"], {}))
            vals[row["Counter_Name"]] = vals.get(row["Counter_Name"], 0.0) + \
                float(row["Counter_Value"])
    return out


def _role(name):
    """GEMM role of a kernel name: gate_up / down of the routed experts (any row source but
    dense), shared_gate_up / shared_down (dense rows, SRC 2), or None for other kernels."""
    for fam in KERNEL_FAMILY_SOURCES:
        key = fam + "<"
        if key in name:
            args = name.split(key, 1)[1].split(">", 1)[0].split(",")
            gate_up = args[0].strip() == "true"
            src = KERNEL_FAMILY_SRC_ARG[fam]
            dense = src is not None and args[src].strip() == "2"
            return ("shared_" if dense else "") + ("gate_up" if gate_up else "down")
    return None


def _is_dominant(name):
    """The gate-up GEMM of the routed experts."""
    return _role(name) == "gate_up"


def _calibration_copy(disp):
    """Dispatch id of the calibration copy: the last copy kernel before the first routing
    kernel of the pass."""
    ids = sorted(disp)
    first_route = next(i for i in ids if "k_route" in disp[i][0])
    copies = [i for i in ids if i < first_route and "copy" in disp[i][0].lower()]
    return copies[-1]


def summarize_trace(args):
    """profiles/kernel_trace_<workload>.md from a rocprofv3 --kernel-trace --stats run of
    bench.py: per-kernel call counts and durations of the pass's kernels."""
    import csv
    import glob
    from moe_harness.workloads import BENCH_CONFIG, CONFIGS
    cfg = CONFIGS[args.config or BENCH_CONFIG]
    path = glob.glob(os.path.join(args.summarize_trace, "**", "*kernel_stats.csv"),
                     recursive=True)[0]
    wname = {"fp8": "FP8", "mxfp4": "MXFP4"}.get(args.weights)
    lines = ["# Kernel trace: fused MoE forward%s, workload %s (T=%d, H=%d, E=%d, F=%d, top-%d%s)"
             % (" with %s expert weights" % wname if wname else "", cfg.name, cfg.T, cfg.H,
                cfg.E, cfg.F, cfg.k, ", shared S=%d" % cfg.S if cfg.S else ""), ""]
    for c in args.pmc_commands:
        lines += ["Command (from /tmp, repository at $R):", "", "    " + c, ""]
    # per-dispatch durations for the median (the average includes the first, colder calls)
    durs = {}
    for tpath in glob.glob(os.path.join(args.summarize_trace, "**", "*kernel_trace.csv"),
                           recursive=True):
        for r in csv.DictReader(open(tpath)):
            if r.get("Kernel_Name") and r.get("Start_Timestamp") and r.get("End_Timestamp"):
                durs.setdefault(r["Kernel_Name"], []).append(
                    int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    lines += ["Input-generation and copy kernels, and the bench's context measurements (the "
              "streaming-read kernel and the library GEMM of its matmul), are omitted.  The "
              "median is over the kernel's dispatches; the average also weighs the first, colder "
              "ones.", "",
              "| kernel | calls | average us | median us | min us | max us |",
              "|---|---|---|---|---|---|"]
    for r in csv.DictReader(open(path)):
        n = r["Name"]
        if "at::native" in n or "rocclr" in n or n.startswith("Cijk_") or "k_stream_read" in n:
            continue
        short = n.replace("(anonymous namespace)::", "").replace("void ", "")
        short = short.split("(")[0] if "(" in short else short
        d = sorted(durs.get(n, []))
        med = "%.2f" % (0.5 * (d[(len(d) - 1) // 2] + d[len(d) // 2]) / 1e3) if d else "-"
        lines.append("| `%s` | %s | %.2f | %s | %.2f | %.2f |" % (
            short, r["Calls"], float(r["AverageNs"]) / 1e3, med, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3))
    lines += ["", "Template arguments: k_ws_gemm<GATE_UP, SRC, NT, MT, KSPLIT, STAGES, DT, SEGK> "
              "(SRC 0 sorted, 1 direct, 2 dense, 3 scan; DT 0 bf16, 1 f16; SEGK k-steps per weight "
              "load segment, STAGES counting segments); k_tiled_gemm<GATE_UP, SRC, "
              "BM, NTW, STAGES, DT>; "
              "k_wide_gemm<GATE_UP, SRC, WS, DT> (WS weight stages); k_wide_reduce<GATE_UP, DT> (sum "
              "of the K-split dense tiles' parts); k_combine<DT>."]
    if args.weights == "fp8":
        lines += ["", "FP8: k_fp8_direct<GATE_UP, NT, KSPLIT, STAGES, SEG> (routes straight from "
                  "topk_ids, rows quantised in the kernel; NT 16-column tiles, K split over KSPLIT "
                  "waves, STAGES segments in flight, SEG 128-element k-steps per weight load); "
                  "k_fp8_ws<NT, KSPLIT, STAGES, SEG> (contiguous layout); k_quant_fp8<MODE> (0 "
                  "plain rows, 2 SiLU(gate)*up of gate-up rows)."]
    if args.weights == "mxfp4":
        lines += ["", "MXFP4: k_mx_gemm<GATE_UP, SRC, NT, KSPLIT, STAGES> (weight streaming); "
                  "k_mx_tiled<GATE_UP, NTW, STAGES> (64-row tiles); k_wide_mx<GATE_UP> (256 x 256 "
                  "tiles, codes dequantised into the MFMA operands)."]
    suffix = "" if args.weights == "16bit" else "_" + args.weights
    out = os.path.join(PROFILE_DIR, "kernel_trace_%s%s.md" % (cfg.name, suffix))
    os.makedirs(PROFILE_DIR, exist_ok=True)
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_pmc(args):
    """profiles/<role>_<workload>_pmc.txt for each expert GEMM role present (routed gate-up and
    down, the shared expert's gate-up and down) from rocprofv3 --pmc runs of bench.py
    --copy-calibration (FETCH_SIZE run, WRITE_SIZE run, optional MFMA-busy run)."""
    from moe_harness.workloads import BENCH_CONFIG, CONFIGS
    cfg = CONFIGS[args.config or BENCH_CONFIG]
    runs = [_read_counters(d) for d in args.summarize_pmc]
    titles = {"gate_up": "the gate-up GEMM of the routed experts",
              "down": "the down GEMM of the routed experts",
              "shared_gate_up": "the shared expert's gate-up GEMM",
              "shared_down": "the shared expert's down GEMM"}
    wsuffix = "_mxfp4" if args.weights == "mxfp4" else ""
    wnote = " (MXFP4 expert weights)" if wsuffix else ""
    for role in PMC_ROLES:
        if not any(_role(n) == role for n, _ in runs[0].values()):
            continue
        res = {}
        lines = ["# HBM traffic and MFMA activity of %s%s, workload %s"
                 % (titles[role], wnote, cfg.name),
                 "# FETCH_SIZE / WRITE_SIZE are per-dispatch KiB; each is scaled by the reading of "
                 "the same counter for one plain device-to-device copy of known size in the same "
                 "run.", "#"]
        for c in args.pmc_commands:
            lines.append("command: %s" % c)
        for counter, disp in zip(("FETCH_SIZE", "WRITE_SIZE"), runs[:2]):
            dom = [v[counter] for i, (n, v) in disp.items() if _role(n) == role and counter in v]
            names = sorted({n for n, v in disp.values() if _role(n) == role})
            cal = disp[_calibration_copy(disp)][1][counter]
            copy_bytes = args.copy_calibration
            scale = copy_bytes / (cal * 1024.0)
            res[counter] = sum(dom) / len(dom) * 1024.0 * scale
            lines += ["%s_kib_per_dispatch: %.1f" % (counter.lower(), sum(dom) / len(dom)),
                      "%s_dispatches: %d" % (counter.lower(), len(dom)),
                      "%s_copy_kib: %.1f" % (counter.lower(), cal),
                      "%s_scale: %.5f" % (counter.lower(), scale)]
            res["kernels"] = names
        if len(runs) > 2:
            disp = runs[2]
            # GRBM_GUI_ACTIVE is summed over the 8 XCDs; MFMA-busy cycles over the 1024 SIMDs
            busy = [v["SQ_VALU_MFMA_BUSY_CYCLES"] / (v["GRBM_GUI_ACTIVE"] / 8.0 * 1024.0)
                    for n, v in disp.values() if _role(n) == role and "GRBM_GUI_ACTIVE" in v]
            if busy:
                lines.append("mfma_busy_pct: %.2f" % (100.0 * sum(busy) / len(busy)))
        lines += ["copy_bytes: %d" % args.copy_calibration,
                  "kernel: %s" % "; ".join(res["kernels"]),
                  "kernel_source_sha256: %s" % kernel_source_hash("; ".join(res["kernels"])),
                  "fetch_bytes_per_launch: %.0f" % res["FETCH_SIZE"],
                  "write_bytes_per_launch: %.0f" % res["WRITE_SIZE"],
                  "traffic_bytes_per_launch: %.0f" % (res["FETCH_SIZE"] + res["WRITE_SIZE"])]
        path = os.path.join(PROFILE_DIR, "%s_%s%s_pmc.txt" % (role, cfg.name, wsuffix))
        os.makedirs(PROFILE_DIR, exist_ok=True)
        open(path, "w").write("\n".join(lines) + "\n")
        print("\n".join(lines))


def _cpu_baseline_mx(cfg, d, seconds, x, ids, w, route_s):
    """MXFP4 weights: per sampled token, the oracle dequantises that token's experts
    (oracle.mxfp4_to_bf16) and evaluates them; scaled to one whole forward."""
    import numpy as np
    import torch

    import oracle

    def one_token(t):
        sel = torch.as_tensor(ids[t], device=d["w_gate_up_q"].device, dtype=torch.long)
        host = {k: d[k].index_select(0, sel).cpu().numpy() for k in
                ("w_gate_up_q", "w_gate_up_scale", "w_down_q", "w_down_scale")}
        t0 = time.perf_counter()
        wgu = oracle.mxfp4_to_bf16(host["w_gate_up_q"], host["w_gate_up_scale"])
        wd = oracle.mxfp4_to_bf16(host["w_down_q"], host["w_down_scale"])
        oracle.experts(x[t:t + 1], wgu, wd, np.arange(cfg.k, dtype=np.int32)[None, :],
                       w[t:t + 1])
        return time.perf_counter() - t0

    one = max(one_token(0), 1e-6)
    n = int(max(1, min(cfg.T, seconds / one)))
    tokens = np.linspace(0, cfg.T - 1, n).round().astype(np.int64)
    dt = sum(one_token(int(t)) for t in tokens)
    per_forward_ms = (route_s + dt * cfg.T / n) * 1e3
    log("cpu oracle (mxfp4 weights): %d of %d tokens in %.2f s -> %.1f ms per forward"
        % (n, cfg.T, dt, per_forward_ms))
    return {"value": round(per_forward_ms, 2), "unit": "ms", "cores": oracle.max_threads(),
            "kind": "oracle", "sample": "routing of all %d tokens + per sampled token the "
            "dequantisation and evaluation of its experts, %d of %d tokens, scaled to all"
            % (cfg.T, n, cfg.T)}


def cpu_baseline_fp8(cfg, d, seconds):
    """The oracle's FP8 pass (oracle.fp8_forward) on this host for a sample of tokens, scaled
    to one whole forward of T tokens (its routing runs on every token either way)."""
    import numpy as np

    import oracle
    from moe_harness.workloads import to_u16

    h = {k: d[k].cpu().numpy() for k in ("w_gate_up", "w_gate_up_scale", "w_down",
                                         "w_down_scale", "gating_output")}
    b = None if d["correction_bias"] is None else d["correction_bias"].cpu().numpy()
    x = to_u16(d["hidden_states"])
    args = (x, h["gating_output"], h["w_gate_up"], h["w_gate_up_scale"], h["w_down"],
            h["w_down_scale"], b, cfg.k, cfg.scoring, cfg.renormalize, cfg.num_expert_group,
            cfg.topk_group, float(np.float32(cfg.rsf)))
    t0 = time.perf_counter()
    oracle.fp8_forward(*args, tokens=[0])
    one = max(time.perf_counter() - t0, 1e-6)
    n = int(max(1, min(cfg.T, seconds / one)))
    tokens = np.linspace(0, cfg.T - 1, n).round().astype(np.int64)
    t0 = time.perf_counter()
    oracle.fp8_forward(*args, tokens=tokens)
    dt = time.perf_counter() - t0
    per_forward_ms = dt * cfg.T / n * 1e3
    log("cpu oracle (fp8 pass): %d of %d tokens in %.2f s -> %.1f ms per forward"
        % (n, cfg.T, dt, per_forward_ms))
    return {"value": round(per_forward_ms, 2), "unit": "ms", "cores": oracle.max_threads(),
            "kind": "oracle", "sample": "fp8 pass of %d of %d tokens (evenly spaced; routing of "
            "all tokens each call), scaled to all" % (n, cfg.T)}


def cpu_baseline(cfg, d, seconds, dtype="bf16"):
    """The oracle, as it stands, on this host: route every token, evaluate the experts of a
    sample of tokens; the time is scaled to one whole forward of T tokens."""
    import numpy as np

    import oracle
    from moe_harness.workloads import to_u16

    g = d["gating_output"].cpu().numpy()
    b = None if d["correction_bias"] is None else d["correction_bias"].cpu().numpy()
    x = to_u16(d["hidden_states"])
    t0 = time.perf_counter()
    ids, w = oracle.route(g, b, cfg.k, cfg.scoring, cfg.renormalize, cfg.num_expert_group,
                          cfg.topk_group, float(np.float32(cfg.rsf)))
    route_s = time.perf_counter() - t0
    import torch
    used = np.unique(ids)
    if "w_gate_up_q" in d:  # MXFP4 weights: the oracle dequantises a token's experts, then runs
        return _cpu_baseline_mx(cfg, d, seconds, x, ids, w, route_s)
    else:
        sel = torch.as_tensor(used, device=d["w_gate_up"].device)
        wgu = to_u16(d["w_gate_up"].index_select(0, sel))
        wd = to_u16(d["w_down"].index_select(0, sel))
    remap = np.full(cfg.E, -1, np.int64)
    remap[used] = np.arange(used.size)
    lids = remap[ids].astype(np.int32)
    sgu = to_u16(d["shared_w_gate_up"]) if cfg.S else None
    sd = to_u16(d["shared_w_down"]) if cfg.S else None
    threads = oracle.max_threads()
    # calibrate on one token, then size the sample to about `seconds`
    t0 = time.perf_counter()
    oracle.experts(x, wgu, wd, lids, w, sgu, sd, tokens=[0], dtype=dtype)
    one = max(time.perf_counter() - t0, 1e-6)
    n = int(max(1, min(cfg.T, seconds * max(1, threads) / one)))
    tokens = np.linspace(0, cfg.T - 1, n).round().astype(np.int32)
    t0 = time.perf_counter()
    oracle.experts(x, wgu, wd, lids, w, sgu, sd, tokens=tokens, dtype=dtype)
    exp_s = time.perf_counter() - t0
    per_forward_ms = (route_s + exp_s * cfg.T / n) * 1e3
    log("cpu oracle: %d of %d tokens in %.2f s on %d threads -> %.1f ms per forward"
        % (n, cfg.T, exp_s, threads, per_forward_ms))
    return {"value": round(per_forward_ms, 2), "unit": "ms", "cores": threads, "kind": "oracle",
            "sample": "routing of all %d tokens + experts of %d of %d tokens (evenly spaced), "
                      "scaled to %d tokens" % (cfg.T, n, cfg.T, cfg.T)}


if __name__ == "__main__":
    main()
