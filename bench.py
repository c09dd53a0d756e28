#!/usr/bin/env python3
"""Throughput of one Beam MoE block on one MI355X.

A step is one call of the whole hot path (router -> group-limited top-k ->
permutation -> gate/up GEMM + SwiGLU -> down GEMM -> combine) over one batch
of synthetic tokens, with inputs and weights already resident in HBM.

Default workload: the Beam-shape decode batch (T=64, hidden 5120,
intermediate 2560, 256 experts, 8 groups / keep 4 / top-8, x2.5), where
reading the chosen experts' weights dominates.  --workload verify|prefill|skewed|
stack|tiny measures the other shapes.

Prints one JSON line.  `roofline` describes the dominant kernel (gate/up):
its average launch time comes from HIP events the library records around it
on the launch stream during the timed loop; `achieved` is its algorithmic
bytes (decode: bound "hbm") or FLOPs (prefill sizes: bound "mfma") per launch
divided by that time.  `traffic` is the measured HBM traffic per launch from
the committed rocprofv3 counter summary, when that summary was taken on the
current kernel source.  `cpu_baseline` times the CPU oracle on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "MoE-layer tokens/s at H=5120,E=256,k=8; % of peak MFMA / HBM GB/s"
CSRC = os.path.join(ROOT, "sparse_moe_transformer_group_amd", "csrc")
# source file of each gate/up schedule (the stream kernel serves decode-size
# batches, the tiled kernel prefill sizes)
GEMM_SRC = {"stream": os.path.join(CSRC, "gemm_stream.hip"),
            "tiled": os.path.join(CSRC, "gemm_tiled.hip")}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None)
    p.add_argument("--warmup", type=int, default=None,
                   help="untimed warm-up steps (default: at least 5 and at least 0.3 s of work, "
                        "so the timed steps run at settled clocks)")
    p.add_argument("--workload", default="decode",
                   choices=["decode", "verify", "prefill", "skewed", "stack", "tiny",
                            "attn_swa", "attn_global", "dense_decode", "dense_prefill"],
                   help="MoE block shapes, or the attention sublayer of a sliding-window "
                        "(attn_swa) or global (attn_global) layer over one 8192-token sequence, "
                        "or a dense SwiGLU layer (I = 20480) at T = 64 or 8192")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-tokens", type=int, default=None)
    p.add_argument("--weights", default="bf16", choices=["bf16", "fp8"],
                   help="expert weight format: bf16 (the headline), or FP8 E4M3 with per-row "
                        "scales (bf16 activations)")
    p.add_argument("--no-context", action="store_true",
                   help="skip the dense bf16 GEMM context measurement")
    p.add_argument("--no-graph", action="store_true",
                   help="skip the HIP-graph replay measurement reported beside the eager value")
    p.add_argument("--copy-probe", action="store_true",
                   help="also run one 1 GiB device copy (HBM counter calibration)")
    p.add_argument("--no-sub", action="store_true",
                   help="MoE block workloads: skip the prefill and skewed records that the default "
                        "run times on the same resident weights")
    p.add_argument("--sub-steps", type=int, default=20,
                   help="timed steps of each prefill / skewed record")
    return p.parse_args()


def kernel_hash(schedule):
    src = GEMM_SRC.get(schedule, schedule)
    with open(src, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(workload, schedule, kernel="gateup"):
    """HBM bytes per launch of the kernel from the committed counter summary,
    if it was taken on this kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("gemm_source_sha256_16") != kernel_hash(schedule):
        return None
    return d.get("bytes_per_launch")


def measured_clock(workload, schedule, kernel="gateup"):
    """Shader clock and MFMA-busy share of the kernel from the committed
    counter summary (GRBM_GUI_ACTIVE, MfmaUtil), if taken on this kernel source."""
    path = os.path.join(ROOT, "profiles", f"clock_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("gemm_source_sha256_16") != kernel_hash(schedule):
        return None
    return {"clock_GHz": d.get("clock_GHz"), "mfma_busy_pct": d.get("MfmaUtil_pct_mean"),
            "bf16_mfma_peak_at_clock_TFLOPs": d.get("bf16_mfma_peak_at_this_clock_TFLOPs")}


def copy_probe(dev):
    """A plain elementwise copy of known size (reads 1 GiB, writes 1 GiB): the
    calibration dispatch for the HBM traffic counters."""
    import torch
    a = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(2):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    del a, b


def warm_up(step, warmup):
    """Untimed steps before the timed region; with warmup None at least 5
    steps and 0.3 s of work, so the timed steps run at a settled clock."""
    import torch
    if warmup is None:
        torch.cuda.synchronize()
        t_w, n_w = time.perf_counter(), 0
        while n_w < 5 or time.perf_counter() - t_w < 0.3:
            step()
            n_w += 1
            if n_w % 5 == 0:
                torch.cuda.synchronize()
        warmup = n_w
    else:
        for _ in range(warmup):
            step()
    torch.cuda.synchronize()
    return warmup


def timed_steps(bm, step, steps, calls_per_step, stages=None):
    """K timed steps between device synchronisations; the library's stage
    timer records HIP events around the given stages (every stage when None)
    of every call, on the launch stream.  Returns (elapsed s, sorted per-step
    ms, stage ms per call)."""
    import torch
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    with bm.StageTimer(steps * calls_per_step, stages=stages) as timer:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        marks[0].record()
        for i in range(steps):
            step()
            marks[i + 1].record()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    step_ms = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(steps))
    stage_ms = {n: v / max(timer.calls, 1) for n, v in timer.result.items()}
    return elapsed, step_ms, stage_ms


def gateup_roofline(tag, T, H, I, k, a_mean, wbytes, gu_ms):
    """Roofline of the gate/up launch: algorithmic bytes (touched experts'
    gate and up weights, x in, h out) or FLOPs (T k 4 H I) per launch over
    its mean HIP-event time; bound "hbm" below the bf16 MFMA/HBM ridge."""
    gu_bytes = a_mean * 2 * I * H * wbytes + T * H * 2 + T * k * I * 2
    gu_flops = T * k * 4 * H * I
    if (gu_flops / gu_bytes) < (PEAK_BF16_TFLOPS / PEAK_HBM_GBS * 1e3):
        ach = gu_bytes / (gu_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4)}
    else:
        ach = gu_flops / (gu_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4)}
    # both fractions: at prefill sizes the launch sits near the ridge
    roof["frac_of_peak_mfma"] = round(gu_flops / (gu_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
    roof["frac_of_peak_hbm"] = round(gu_bytes / (gu_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
    schedule = "stream" if T * k < 20 * 256 else "tiled"
    roof["traffic"] = measured_traffic(tag, schedule)
    roof["clock"] = measured_clock(tag, schedule)
    roof["kernel"] = "grouped_stream_kernel<2,1,*> (gate/up)" if schedule == "stream" else \
        "grouped_tiled_kernel<2,...> (gate/up)"
    roof["algorithmic_per_launch"] = {"bytes": int(gu_bytes), "flops": int(gu_flops)}
    roof["avg_launch_ms"] = round(gu_ms, 5)
    return roof


def expert_load(counts):
    """Realised per-expert load of one batch: tokens per expert (max, mean,
    min over active experts, the five largest) and the Zipf exponent s of a
    least-squares fit log(load) = c - s log(rank) over the active experts."""
    import numpy as np
    c = np.sort(np.asarray(counts, dtype=np.float64))[::-1]
    act = c[c > 0]
    rank = np.arange(1, act.size + 1, dtype=np.float64)
    s_fit = float(-np.polyfit(np.log(rank), np.log(act), 1)[0]) if act.size > 1 else None
    return {"max": int(c[0]), "mean": round(float(c.mean()), 2), "min_active": int(act[-1]),
            "max_over_mean": round(float(c[0] / c.mean()), 2), "top5": [int(v) for v in c[:5]],
            "fitted_zipf_s": round(s_fit, 3) if s_fit is not None else None}


def moe_workload(args, bm, name, wr, pk, host_weights, steps, warmup, graph_replay):
    """Time one MoE workload on resident packed weights; returns its record
    (value, stage times, roofline of gate/up, and the CPU oracle baseline
    with the parity of the GPU result on the oracle's sample)."""
    import torch

    import moe_inputs as MI

    dev = torch.device("cuda:0")
    shape = MI.WORKLOADS[name]
    T, H, I, E, k = shape.T, shape.H, shape.I, shape.E, shape.k
    layers = shape.layers
    x = MI.make_x(T, H).to(dev)
    off = MI.load_zipf_offsets(E).to(dev) if shape.offset == "zipf" else None
    y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    if layers == 1:
        def step():
            bm.block(x, wr[0], *pk[0], shape.groups, shape.topk_groups, k, shape.scale,
                     logit_offset=off, out=y, return_routing=False)
    else:
        stream0 = bm.stream_init(x)
        work = stream0.clone()

        def step():
            work.copy_(stream0)
            for l in range(layers):
                bm.sublayer(work, l + 2, wr[l], *pk[l], shape.groups,
                            shape.topk_groups, k, shape.scale, keep_io=False)

    # routing (active experts; ids and weights for the parity check) from one
    # untimed call
    routing = None
    if layers == 1:
        y_r, ids, w, counts = bm.block(x, wr[0], *pk[0], shape.groups, shape.topk_groups, k,
                                       shape.scale, logit_offset=off)
        active = [int((counts > 0).sum().item())]
        routing = (y_r, ids, w)
        load = expert_load(counts.cpu().numpy())
    else:
        load = None
        tmp = stream0.clone()
        active = []
        for l in range(layers):
            _, _, _, _, c = bm.sublayer(tmp, l + 2, wr[l], *pk[l], shape.groups,
                                        shape.topk_groups, k, shape.scale)
            active.append(int((c > 0).sum().item()))
        del tmp

    warmup = warm_up(step, warmup)
    print(f"[bench] {name}: timing {steps} steps", file=sys.stderr, flush=True)
    # the timed region carries the events of gate/up only (the roofline's
    # kernel); the per-stage breakdown comes from further steps after it
    elapsed, step_ms, stage_timed = timed_steps(bm, step, steps, layers, stages=("gateup",))
    n_breakdown = min(steps, 10)
    _, _, stage_all = timed_steps(bm, step, n_breakdown, layers)
    stage_ms = {n: v for n, v in stage_all.items() if not n.startswith("attn_")}
    ms_step = elapsed * 1e3 / steps

    # ---- algorithmic work (per step)
    flops_step = layers * T * (2 * H * E + k * 6 * H * I)
    wbytes = 1 if args.weights == "fp8" else 2   # bytes per expert weight
    sbytes = (lambda a: a * 4 * (2 * I + H)) if args.weights == "fp8" else (lambda a: 0)  # row scales
    bytes_step = sum(wbytes * (a * 3 * H * I) + sbytes(a) + 2 * E * H + 2 * T * H + 2 * T * H + 8 * T * k
                     for a in active)
    tflops = flops_step / (ms_step * 1e-3) / 1e12
    gbs = bytes_step / (ms_step * 1e-3) / 1e9
    tag = name + ("_fp8" if args.weights == "fp8" else "")
    roof = gateup_roofline(tag, T, H, I, k, sum(active) / len(active), wbytes, stage_timed["gateup"])

    if args.copy_probe:
        copy_probe(dev)

    graph = None
    if graph_replay:
        # the same step replayed from a HIP graph (serving-loop style: no
        # launch overhead between the kernels); reported beside the eager value
        step()                    # outputs and workspace exist before the capture
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            step()
        for _ in range(3):
            gr.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(steps):
            gr.replay()
        g1.record()
        torch.cuda.synchronize()
        gms = g0.elapsed_time(g1) / steps
        graph = {"ms_per_step": round(gms, 4), "tokens_per_s": round(T / (gms * 1e-3), 1),
                 "how": f"{steps} replays of one captured step, HIP events around them"}
        del gr

    rec = {
        "metric": METRIC,
        "value": round(T * steps / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_median": round(step_ms[len(step_ms) // 2], 4),
        "ms_per_step_min": round(step_ms[0], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if args.weights == "bf16" else "fp8-e4m3 weights x bf16 activations",
        "data": "synthetic",
        "config": {"workload": f"beam_moe_{name}", "weights": args.weights,
                   "T": T, "H": H, "I": I, "E": E,
                   "groups": shape.groups, "topk_groups": shape.topk_groups, "k": k,
                   "scale": shape.scale, "layers": layers,
                   "logit_offset": shape.offset, "active_experts": active,
                   "expert_load": load},
        "tflops": round(tflops, 1),
        "frac_peak_mfma": round(tflops / PEAK_BF16_TFLOPS, 4),
        "algorithmic_gbs": round(gbs, 1),
        "frac_peak_hbm": round(gbs / PEAK_HBM_GBS, 4),
        "stage_ms": {n: round(v, 5) for n, v in stage_ms.items()},
        "stage_ms_how": (f"HIP events around every stage of {n_breakdown} further steps after the "
                         "timed region; inside it only gate/up carries events (roofline)"),
        "roofline": roof,
        "graph_replay": graph,
    }
    if not args.no_cpu_baseline:
        print(f"[bench] {name}: timed loop done ({ms_step:.3f} ms/step); CPU oracle baseline next",
              file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(args, shape, x, wr[0], *host_weights, off, routing)
    del x, y
    return rec


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the expert-parallel multi-GPU path is not built)", file=sys.stderr)
        sys.exit(2)

    if args.workload.startswith("attn_"):
        return run_attention(args)
    if args.workload.startswith("dense_"):
        return run_dense(args)

    import numpy as np
    import torch

    import moe_inputs as MI
    import sparse_moe_transformer_group_amd as bm

    dev = torch.device("cuda:0")
    shape = MI.WORKLOADS[args.workload]
    steps = args.steps if args.steps is not None else (
        {"decode": 100, "verify": 50, "tiny": 200}.get(args.workload, 20))
    E, H, I = shape.E, shape.H, shape.I

    # ---- expert weights resident in HBM, packed once (model-load time);
    # the unpacked layer-0 copy is kept for the CPU baseline's sample
    wr, pk = [], []
    wg0 = wu0 = wd0 = None
    for l in range(shape.layers):
        wr.append(MI.make_router(E, H, layer=l).to(dev))
        g, u, d = MI.make_expert_weights(E, H, I, dev, layer=l)
        pk.append(bm.pack_experts_fp8(g, u, d) if args.weights == "fp8" else bm.pack_experts(g, u, d))
        if l == 0:
            wg0, wu0, wd0 = g, u, d
        del g, u, d
    torch.cuda.empty_cache()
    torch.cuda.synchronize()

    out = moe_workload(args, bm, args.workload, wr, pk, (wg0, wu0, wd0), steps, args.warmup,
                       not args.no_graph)

    # the MFMA-bound shapes on the same resident layer-0 weights: prefill
    # (T = 8192, near-uniform load) and skewed (T = 16384, Zipf(1.1) load)
    subs = [] if args.no_sub else [n for n in ("prefill", "skewed")
                                   if n != args.workload and MI.WORKLOADS[n].layers == 1
                                   and (MI.WORKLOADS[n].H, MI.WORKLOADS[n].I) == (H, I)
                                   and shape.layers == 1]
    if subs:
        out["sub_workloads"] = {}
        for n in subs:
            out["sub_workloads"][n] = moe_workload(args, bm, n, wr, pk, (wg0, wu0, wd0),
                                                   args.sub_steps, args.warmup, False)
            bm.release_workspaces()
            torch.cuda.empty_cache()

    if not args.no_context:
        # what a dense library GEMM sustains on this machine (hipBLASLt through
        # torch.matmul, random N(0,1) bf16 operands, 8192^3), for context
        ga = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
        gb = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
        torch.cuda.synchronize()
        tw = time.perf_counter()
        while time.perf_counter() - tw < 0.3:
            gc = torch.matmul(ga, gb)
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            gc = torch.matmul(ga, gb)
        e1.record()
        torch.cuda.synchronize()
        gt = 2.0 * 8192 ** 3 / (e0.elapsed_time(e1) / 20 * 1e-3) / 1e12
        out["context"] = {"dense_bf16_gemm_8192_tflops": round(gt, 1),
                          "frac_peak_mfma": round(gt / PEAK_BF16_TFLOPS, 4),
                          "how": "torch.matmul (hipBLASLt) on random bf16 operands, 20 runs after "
                                 "0.3 s warm-up"}
        del ga, gb, gc
    out["inputs"] = {"seed": MI.SEED, "numpy": np.__version__, "torch": torch.__version__,
                     "recipe": "x ~ N(0,1), router and expert weights ~ N(0,0.02), bf16 (RNE); "
                               "expert weights drawn on the device per expert from a seeded "
                               "generator; skewed: stored per-expert logit offsets (Zipf 1.1)"}
    print(json.dumps(out), flush=True)


ATTN_T, ATTN_H, ATTN_WINDOW = 8192, 5120, 512
ATTN_Q, ATTN_KV, ATTN_D = 48, 8, 128


def attention_pairs(T, window):
    """Allowed (query, key) pairs: causal, and within the window if one is given."""
    if window is None:
        return T * (T + 1) // 2
    w = min(window, T)
    return w * (w + 1) // 2 + (T - w) * w


def run_attention(args):
    """Attention sublayer of one sequence (projections, per-head norms and
    position, flash attention with the sigmoid gate, output projection)."""
    import torch

    import moe_inputs as MI
    import sparse_moe_transformer_group_amd as bm

    dev = torch.device("cuda:0")
    glob = args.workload == "attn_global"
    T, H = ATTN_T, ATTN_H
    steps = args.steps if args.steps is not None else 20
    u = MI.make_attention_input(T, H).to(dev)
    ws_cpu = MI.make_attention_weights(H)
    w_qkvg, w_o = bm.pack_attention_weights(*[w.to(dev) for w in ws_cpu])
    y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    def step():
        bm.attention(u, w_qkvg, w_o, glob, window=ATTN_WINDOW, out=y)

    if args.warmup is None:
        torch.cuda.synchronize()
        t_w, n_w = time.perf_counter(), 0
        while n_w < 5 or time.perf_counter() - t_w < 0.3:
            step()
            n_w += 1
            if n_w % 5 == 0:
                torch.cuda.synchronize()
        args.warmup = n_w
    else:
        for _ in range(args.warmup):
            step()
    torch.cuda.synchronize()

    # per-stage breakdown (events around every stage) before the timed region,
    # which then carries the events of the dominant stage only
    n_breakdown = min(steps, 10)
    _, _, stage_all = timed_steps(bm, step, n_breakdown, 1)
    stage_ms = {n: v for n, v in stage_all.items() if n.startswith("attn_")}

    pairs = attention_pairs(T, None if glob else ATTN_WINDOW)
    proj_rows = (2 * ATTN_Q + 2 * ATTN_KV) * ATTN_D
    flops = {"attn_proj": 2 * T * H * proj_rows,
             "attn_flash": 4 * ATTN_D * pairs * ATTN_Q,
             "attn_out": 2 * T * ATTN_Q * ATTN_D * H}
    # algorithmic bytes: each operand read once, each result written once
    nbytes = {"attn_proj": 2 * T * H + 2 * proj_rows * H + 4 * T * proj_rows,
              "attn_flash": 2 * T * (ATTN_Q + 2 * ATTN_KV) * ATTN_D + 4 * T * ATTN_Q * ATTN_D
              + 2 * T * ATTN_Q * ATTN_D,
              "attn_out": 2 * T * ATTN_Q * ATTN_D + 2 * ATTN_Q * ATTN_D * H + 2 * T * H}
    total_flops = sum(flops.values())
    dom = max(flops, key=lambda n: stage_ms[n])
    elapsed, step_ms, stage_timed = timed_steps(bm, step, steps, 1, stages=(dom,))
    ms_step = elapsed * 1e3 / steps
    kern = {"attn_proj": ("grouped_tiled_kernel<0,...> (q, k, v, gate projection)", "tiled"),
            "attn_flash": ("attn_flash_kernel", os.path.join(CSRC, "attention.hip")),
            "attn_out": ("grouped_tiled_kernel<0,...> (output projection)", "tiled")}[dom]
    ach = flops[dom] / (stage_timed[dom] * 1e-3) / 1e12
    roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(ach / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic(args.workload, kern[1], dom),
            "clock": measured_clock(args.workload, kern[1], dom),
            "kernel": kern[0], "stage": dom,
            "algorithmic_per_launch": {"bytes": int(nbytes[dom]), "flops": int(flops[dom])},
            "avg_launch_ms": round(stage_timed[dom], 5)}
    if args.copy_probe:
        copy_probe(dev)
    per_stage = {n: {"ms": round(stage_ms[n], 5),
                     "tflops": round(flops[n] / (stage_ms[n] * 1e-3) / 1e12, 1) if n in flops else None}
                 for n in stage_ms}
    out = {
        "metric": "attention-sublayer tokens/s (one sequence, prefill) at H=5120, 48/8 heads x 128",
        "value": round(T * steps / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_median": round(step_ms[len(step_ms) // 2], 4),
        "ms_per_step_min": round(step_ms[0], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"beam_{args.workload}", "T": T, "H": H, "q_heads": ATTN_Q,
                   "kv_heads": ATTN_KV, "head_dim": ATTN_D,
                   "window": None if glob else ATTN_WINDOW, "attended_pairs": pairs},
        "tflops": round(total_flops / (ms_step * 1e-3) / 1e12, 1),
        "frac_peak_mfma": round(total_flops / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "stages": per_stage,
        "stages_how": (f"HIP events around every stage of {n_breakdown} steps before the timed "
                       f"region; inside it only {dom} carries events (roofline)"),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        print(f"[bench] timed loop done ({ms_step:.3f} ms/step); CPU oracle baseline next",
              file=sys.stderr, flush=True)
        out["cpu_baseline"] = attention_cpu_baseline(args, u, ws_cpu, glob)
    print(json.dumps(out), flush=True)


DENSE_H, DENSE_I = 5120, 20480
# chunks of the intermediate dimension (a pack-time choice): more chunks give
# a decode-size batch more parallel work; one chunk spares a prefill the FP32
# chunk partials (measured: 8 chunks 0.155 ms at T = 64, 1 chunk 4.24 ms vs
# 4.68 ms with 8 at T = 8192)
DENSE_CHUNKS = {"dense_decode": 8, "dense_prefill": 1}


def run_dense(args):
    """Dense SwiGLU layer (the first three layers), I = 20480, as 8 chunks of
    its intermediate dimension on the expert GEMMs."""
    import numpy as np
    import torch

    import moe_inputs as MI
    import sparse_moe_transformer_group_amd as bm

    dev = torch.device("cuda:0")
    T = 64 if args.workload == "dense_decode" else 8192
    H, I = DENSE_H, DENSE_I
    steps = args.steps if args.steps is not None else (100 if T == 64 else 20)
    x = MI.make_x(T, H).to(dev)
    wg, wu, wd = MI.make_dense_weights(H, I, dev)
    chunks = DENSE_CHUNKS[args.workload]
    fp8 = args.weights == "fp8"
    packed = bm.pack_dense(wg, wu, wd, chunks=chunks, fp8=fp8)
    y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    def step():
        bm.dense_mlp(x, *packed, out=y)

    if args.warmup is None:
        t_w, n_w = time.perf_counter(), 0
        while n_w < 5 or time.perf_counter() - t_w < 0.3:
            step()
            n_w += 1
            if n_w % 5 == 0:
                torch.cuda.synchronize()
        args.warmup = n_w
    else:
        for _ in range(args.warmup):
            step()
    torch.cuda.synchronize()
    # the timed region carries gate/up's events only; the breakdown comes
    # from further steps after it
    elapsed, step_ms, stage_timed = timed_steps(bm, step, steps, 1, stages=("gateup",))
    ms_step = elapsed * 1e3 / steps
    n_breakdown = min(steps, 10)
    _, _, stage_all = timed_steps(bm, step, n_breakdown, 1)
    stage_ms = {n: v for n, v in stage_all.items()
                if n in ("select", "permute", "gateup", "down", "combine")}
    if args.copy_probe:
        copy_probe(dev)
    flops = 6 * T * H * I
    wb = 1 if fp8 else 2                                   # bytes per weight
    sb = (lambda rows: 4 * rows) if fp8 else (lambda rows: 0)  # FP8 row scales
    wbytes = 3 * H * I * wb + sb(2 * I + chunks * H)
    gu_ms = stage_timed["gateup"]
    gu_flops, gu_bytes = 4 * T * H * I, 2 * H * I * wb + sb(2 * I) + T * H * 2 + T * I * 2
    schedule = "stream" if T < 20 else "tiled"
    if gu_flops / gu_bytes < PEAK_BF16_TFLOPS / PEAK_HBM_GBS * 1e3:
        ach = gu_bytes / (gu_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4)}
    else:
        ach = gu_flops / (gu_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4)}
    tag = args.workload + ("_fp8" if fp8 else "")
    roof.update({"traffic": measured_traffic(tag, schedule),
                 "clock": measured_clock(tag, schedule),
                 "kernel": f"grouped_{schedule}_kernel<2,...> (gate/up + SwiGLU)",
                 "algorithmic_per_launch": {"bytes": int(gu_bytes), "flops": int(gu_flops)},
                 "avg_launch_ms": round(gu_ms, 5)})
    out = {
        "metric": "dense SwiGLU layer tokens/s at H=5120, I=20480",
        "value": round(T * steps / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_median": round(step_ms[len(step_ms) // 2], 4),
        "ms_per_step_min": round(step_ms[0], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 weights x bf16 activations" if fp8 else "bf16",
        "data": "synthetic",
        "config": {"workload": f"beam_{args.workload}", "weights": args.weights, "T": T, "H": H,
                   "I": I, "chunks": chunks},
        "tflops": round(flops / (ms_step * 1e-3) / 1e12, 1),
        "frac_peak_mfma": round(flops / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "algorithmic_gbs": round((wbytes + 4 * T * H) / (ms_step * 1e-3) / 1e9, 1),
        "stage_ms": {n: round(v, 5) for n, v in stage_ms.items()},
        "stage_ms_how": (f"HIP events around every stage of {n_breakdown} further steps after the "
                         "timed region; inside it only gate/up carries events (roofline)"),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_info

        import oracle as O
        from moe_inputs import bf16_bits
        print(f"[bench] timed loop done ({ms_step:.3f} ms/step); CPU oracle baseline next",
              file=sys.stderr, flush=True)
        n = min(args.cpu_sample_tokens or 64, T)
        hb = [bf16_bits(w) for w in (wg, wu, wd)]     # host copies (not timed)
        if fp8:  # the oracle's own E4M3 encoding, dequantised per chunk (not timed)
            deq = lambda m: O.dequantize_rows(*O.quantize_rows(m))
            Ic = I // chunks
            hb = [deq(hb[0]), deq(hb[1]),
                  np.concatenate([deq(np.ascontiguousarray(hb[2][:, c * Ic:(c + 1) * Ic]))
                                  for c in range(chunks)], axis=1)]
        xb = bf16_bits(x[:n])
        t0 = time.perf_counter()
        O.dense_mlp(xb, *hb)
        dt = time.perf_counter() - t0
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        out["cpu_baseline"] = {"value": round(n / dt, 3), "unit": "tokens/s", "cores": threads,
                               "kind": "oracle",
                               "sample": f"first {n} tokens of the batch through the FP64 oracle's dense "
                                         f"layer (weights staged in host memory beforehand), {dt:.1f} s"}
    print(json.dumps(out), flush=True)


def attention_cpu_baseline(args, u, ws_cpu, glob):
    from threadpoolctl import threadpool_info

    import oracle as O
    from moe_inputs import bf16_bits

    n = min(args.cpu_sample_tokens or 2048, ATTN_T)
    ub = bf16_bits(u[:n])
    wb = [bf16_bits(w) for w in ws_cpu]
    t0 = time.perf_counter()
    O.attention_sublayer(ub, *wb, glob, window=ATTN_WINDOW)
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {"value": round(n / dt, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"a whole {n}-token sequence (the first {n} tokens of the input) through "
                      f"the FP64 oracle's attention sublayer, {dt:.1f} s; its attention part "
                      f"per token is {'smaller than at 8192 tokens' if glob else 'the same as at 8192 tokens past the first 512'}"}


def cpu_baseline(args, shape, x, wr, wg, wu, wd, off, routing=None):
    """The FP64 CPU oracle timed on a bounded, evenly spread sample of the
    batch (whole block: router, selection, experts, combine), with the
    sampled tokens' expert weights staged in host memory beforehand.  With
    the device's routing and output of the same batch (`routing`: y, ids,
    weights) it also reports their parity: the oracle's routing of every
    token (ids as sets, exclusions below the 1e-6 margin, weight error) and
    the sampled outputs (rel-L2, max-abs / RMS)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle as O
    from moe_inputs import bf16_bits

    n = args.cpu_sample_tokens or {"decode": 64, "tiny": 128}.get(shape.name, 16)
    if args.weights == "fp8" and not args.cpu_sample_tokens:
        n = 8  # the oracle's host-side E4M3 encoding of each touched expert is slow
    n = min(n, shape.T)
    toks = np.unique(np.linspace(0, shape.T - 1, n).round().astype(np.int64))
    xall = bf16_bits(x)
    xb = xall[toks]
    wrb = bf16_bits(wr)
    offn = None if off is None else off.cpu().numpy()
    # stage the sampled tokens' expert weights in host memory (not timed)
    z = O.router_logits(xb, wrb, offn)
    ids, _, _, _ = O.group_limited_topk(O.sigmoid(z), shape.groups, shape.topk_groups, shape.k,
                                        shape.scale)
    host = {int(e): (bf16_bits(wg[e]), bf16_bits(wu[e]), bf16_bits(wd[e])) for e in np.unique(ids)}
    if args.weights == "fp8":  # the oracle's own E4M3 encoding, dequantised (not timed)
        host = {e: tuple(O.dequantize_rows(*O.quantize_rows(m)) for m in ws) for e, ws in host.items()}
    t0 = time.perf_counter()
    ref = O.moe_block(xb, wrb, lambda e: host[e], shape.groups, shape.topk_groups, shape.k,
                      shape.scale, offn)
    dt = time.perf_counter() - t0
    del host
    blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        affinity = os.cpu_count()
    res = {"value": round(toks.size / dt, 3), "unit": "tokens/s", "cores": blas, "kind": "oracle",
           "affinity_cores": affinity, "blas_threads": blas,
           "sample": f"{toks.size} evenly spread tokens of the {shape.name} batch (T={shape.T}), "
                     f"whole block in FP64 ({len(np.unique(ids))} experts' weights staged in host "
                     f"memory beforehand), {dt:.1f} s"}
    if routing is not None:
        res["parity"] = oracle_parity(shape, xall, wrb, offn, routing, toks, ref)
    return res


def oracle_parity(shape, xall, wrb, offn, routing, toks, ref):
    """Parity of the device's routing (every token) and output (the sampled
    tokens) against the oracle, with the acceptance rule of the tests:
    tokens whose oracle margin is below 1e-6 are excluded and reported."""
    import numpy as np

    import oracle as O
    from moe_inputs import bf16_bits

    y_gpu, ids_gpu, w_gpu = routing
    s = O.sigmoid(O.router_logits(xall, wrb, offn))
    ids_o, w_o, m_g, m_e = O.group_limited_topk(s, shape.groups, shape.topk_groups, shape.k,
                                                shape.scale)
    keep = np.minimum(m_g, m_e) >= 1e-6
    ids_g = ids_gpu.cpu().numpy().astype(np.int64)
    w_g = w_gpu.cpu().numpy().astype(np.float64)
    same = (np.sort(ids_g, 1) == np.sort(ids_o, 1)).all(1)
    # the device's weights against the oracle's scores at the device's own ids
    sel = np.take_along_axis(s, ids_g, axis=1)
    w_err = np.abs(w_g - shape.scale * sel / sel.sum(1, keepdims=True))
    ks = keep[toks]
    yg = O.bf16_bits_to_f64(bf16_bits(y_gpu))[toks][ks]
    yo = ref["y"][ks]
    rms = float(np.sqrt(np.mean(yo ** 2))) if yo.size else 0.0
    return {"tokens": int(ids_g.shape[0]),
            "excluded_below_margin": int((~keep).sum()),
            "excluded_tokens": np.nonzero(~keep)[0].tolist()[:64],
            "kept_tokens_with_other_ids": int((~same & keep).sum()),
            "excluded_tokens_with_other_ids": int((~same & ~keep).sum()),
            "max_weight_err": float(w_err.max()),
            "sampled_tokens": int(ks.sum()),
            "sampled_rel_l2": float(np.linalg.norm(yg - yo) / max(np.linalg.norm(yo), 1e-300)),
            "sampled_max_abs_over_rms": float(np.abs(yg - yo).max() / max(rms, 1e-300))
            if yo.size else None,
            "bar": "ids as sets on kept tokens; rel-L2 <= 5e-3; max-abs <= 2e-2 RMS"}


if __name__ == "__main__":
    main()
