#!/usr/bin/env python3
"""Benchmark of the fused MoE layer on one MI355X.

Headline workload: the Mixtral-shaped bf16 decode layer (E=8 experts, top-2,
H=4096, I=14336) at the token counts M = 1, 4, 16, 32, 63.  One step is one
fused forward (routing, align, gate/up product with SiLU*up, down product
with the weighted combine, finalize) at each M of the sweep, on seeded
synthetic inputs already resident in HBM.

value = expert-weight bytes of the experts that received tokens, summed over
the sweep, divided by the step time (GB/s).  Per-M span, per-stage times
(HIP events recorded by the library around each launch on the stream) and
the roofline of the dominant kernel (the gate/up product) are reported on
the same JSON line, with the CPU oracle timed on a bounded sample of the
same workload.

Other workloads (--config qwen3|deepseek|prefill|tiny) print the same line
for that layer; they are measurement aids, not the headline.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
FP8_PEAK_TFLOPS = 5000.0       # dense fp8 MFMA
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA
METRIC = "fused-MoE layer µs + weight HBM GB/s (frac of peak) at M=1..64; prefill TFLOP/s"


def log(msg: str):
    sys.stderr.write("[bench] %s\n" % msg)
    sys.stderr.flush()


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="mixtral", choices=["mixtral", "qwen3", "deepseek", "prefill", "tiny"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0, help="budget of the CPU oracle sample")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this layer is built and timed on a single MI355X; "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        return 2

    import torch
    import moe_layer_align_amd as moe
    from synth import CONFIGS, gen_logits, gen_weights, gen_x

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    moe.load()  # fails loudly when the HIP library is missing
    dev = torch.device("cuda:0")
    cfg = CONFIGS[args.config]
    fp8 = cfg.dtype == "fp8"
    esz = 1 if fp8 else 2
    log("generating %s weights on the GPU" % cfg.name)
    w13, w2, s13, s2 = gen_weights(cfg, 0, device=dev)
    s13_t = torch.tensor([s13], device=dev) if fp8 else None
    s2_t = torch.tensor([s2], device=dev) if fp8 else None

    calls = []
    for M in cfg.ms:
        x = gen_x(cfg.H, M, 0, sub=M).to(dev)
        lg = gen_logits(cfg, M, 0, sub=M).to(dev)
        ws = torch.empty(moe.workspace_size(M, cfg.E, cfg.H, cfg.I, cfg.k, cfg.dtype), dtype=torch.uint8, device=dev)
        y = torch.empty(M, cfg.H, dtype=torch.bfloat16, device=dev)
        counts = torch.empty(cfg.E, dtype=torch.int32, device=dev)
        calls.append(dict(M=M, x=x, lg=lg, ws=ws, y=y, counts=counts))

    stream = torch.cuda.current_stream()

    def run(c, events=None):
        moe.fused_forward(c["x"], c["lg"], w13, w2, cfg.k, cfg.dtype, s13_t, s2_t, out=c["y"], workspace=c["ws"],
                          expert_counts=c["counts"], stream=stream, events=events)

    # active experts from the layer's own routing, for the byte and flop accounting
    for c in calls:
        run(c)
    torch.cuda.synchronize()
    for c in calls:
        cnt = c["counts"].cpu()
        c["active"] = int((cnt > 0).sum())
        c["w_bytes"] = c["active"] * 3 * cfg.H * cfg.I * esz
        c["g1_bytes"] = c["active"] * 2 * cfg.H * cfg.I * esz
        c["flops"] = 6.0 * c["M"] * cfg.k * cfg.H * cfg.I

    log("warmup %d steps" % args.warmup)
    for _ in range(args.warmup):
        for c in calls:
            run(c)
    torch.cuda.synchronize()

    ns = moe.NUM_STAGES
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(2 * ns)] for _ in calls] for _ in range(args.steps)]
    for step in evs:  # materialise the hipEvent_t handles
        for per_call in step:
            for e in per_call:
                e.record(stream)
    torch.cuda.synchronize()
    handles = [[[e.cuda_event for e in per_call] for per_call in step] for step in evs]

    log("timing %d steps" % args.steps)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for s in range(args.steps):
        for j, c in enumerate(calls):
            run(c, handles[s][j])
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps

    per_m = []
    g1_ms_sum = 0.0
    g1_bytes_sum = 0.0
    for j, c in enumerate(calls):
        span = [evs[s][j][0].elapsed_time(evs[s][j][2 * ns - 1]) for s in range(args.steps)]
        stage = [[evs[s][j][2 * q].elapsed_time(evs[s][j][2 * q + 1]) for s in range(args.steps)] for q in range(ns)]
        g1_ms_sum += sum(stage[2])
        g1_bytes_sum += c["g1_bytes"] * args.steps
        us = statistics.median(span) * 1e3
        entry = dict(M=c["M"], us=round(us, 2), active_experts=c["active"], weight_bytes=c["w_bytes"],
                     gbps=round(c["w_bytes"] / us / 1e3, 1), hbm_frac=round(c["w_bytes"] / us / 1e3 / HBM_PEAK_GBS, 4),
                     tflops=round(c["flops"] / us / 1e6, 2))
        for q, name in enumerate(moe.STAGE_NAMES):
            entry["%s_us" % name] = round(statistics.median(stage[q]) * 1e3, 2)
        per_m.append(entry)

    total_bytes = sum(c["w_bytes"] for c in calls)
    total_flops = sum(c["flops"] for c in calls)
    if cfg.name == "prefill":
        value = total_flops / (ms_per_step * 1e-3) / 1e12
        unit = "TFLOP/s"
        g1_flops = 4.0 * calls[0]["M"] * cfg.k * cfg.H * cfg.I * args.steps
        ach = g1_flops / (g1_ms_sum * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=round(ach, 1), peak=FP8_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(ach / FP8_PEAK_TFLOPS, 4), traffic=None)
    else:
        value = total_bytes / (ms_per_step * 1e-3) / 1e9
        unit = "GB/s"
        ach = g1_bytes_sum / (g1_ms_sum * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(ach / HBM_PEAK_GBS, 4), traffic=None)
    roof["kernel"] = "gemm1_decode_kernel (gate/up product + SiLU*up)"

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, calls, (w13, w2, s13, s2), args.cpu_seconds, unit)

    ms_str = ",".join(str(m) for m in cfg.ms)
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f8e4m3" if fp8 else "bf16",
        "data": "synthetic: seeded N(0,1) hidden states, N(0,1/fan_in) expert weights, router logits per workload",
        "config": {
            "workload": "%s-shaped %s layer E=%d top-%d H=%d I=%d, M in {%s}" % (cfg.name, cfg.dtype, cfg.E, cfg.k,
                                                                               cfg.H, cfg.I, ms_str),
            "E": cfg.E, "top_k": cfg.k, "H": cfg.H, "I": cfg.I, "M_sweep": list(cfg.ms), "router_logits": cfg.logits,
        },
        "per_m": per_m,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def cpu_baseline(cfg, calls, weights, budget_s, unit):
    """The CPU oracle on the same inputs, as many sweep points as fit the budget."""
    import torch
    import oracle

    w13, w2, s13, s2 = weights
    log("cpu baseline: copying weights to the host")
    w13h, w2h = w13.cpu(), w2.cpu()
    done, secs, work = [], 0.0, 0.0
    for c in sorted(calls, key=lambda c: c["M"]):
        x = c["x"].cpu()
        lg = c["lg"].cpu()
        # expected cost from the last measured rate; stop before the budget is exceeded
        if done and secs / work * (c["w_bytes"] if unit == "GB/s" else c["flops"]) + secs > budget_s:
            break
        log("cpu baseline: oracle at M=%d" % c["M"])
        t0 = time.perf_counter()
        oracle.layer(x, lg, w13h, w2h, cfg.k, cfg.dtype, s13, s2)
        secs += time.perf_counter() - t0
        work += c["w_bytes"] if unit == "GB/s" else c["flops"]
        done.append(c["M"])
    val = work / secs / (1e9 if unit == "GB/s" else 1e12)
    return {"value": round(val, 4), "unit": unit, "cores": oracle.num_threads(), "kind": "oracle",
            "seconds": round(secs, 2),
            "sample": "full layer (all tokens) at M in {%s} of the sweep; weights already in host memory"
                      % ",".join(str(m) for m in done)}


if __name__ == "__main__":
    sys.exit(main())
