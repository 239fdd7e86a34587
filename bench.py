#!/usr/bin/env python3
"""Benchmark of the fused MoE layer on one MI355X.

Headline workload: the Mixtral-shaped bf16 decode layer (E=8 experts, top-2,
H=4096, I=14336) at the token counts M = 1, 4, 16, 32, 63.  One step is one
fused forward (routing, align, gate/up product with SiLU*up, down product
with the weighted combine, finalize) at each M of the sweep, on seeded
synthetic inputs already resident in HBM.

Cold cache: before every layer call a 1 GiB buffer is read (summed), which
evicts the 256 MB Infinity Cache and the L2s with clean lines, so no expert
weight is served from a cache filled by the previous call.  (A write flush
would leave the caches full of dirty lines whose write-back then competes
with the layer's reads, which no real model step does: the previous layers
mostly read weights.)  The layer's time is the span
between HIP events recorded on the launch stream right before its first
kernel and right after its last one, with no event in between (each adds a
few microseconds); the flush is outside the span.

value = expert-weight bytes of the experts that received tokens, summed over
the sweep, divided by the summed layer spans (GB/s); for the prefill
workload, real-pair flops 6*M*k*H*I over the span (TFLOP/s).  The roofline
object covers the dominant kernel (the gate/up product): its algorithmic
bytes (or flops) over its launch durations, from HIP events around that
launch in a second timed pass of the same steps.  The CPU oracle is timed on
a bounded sample of the same workload.

The default run then times the other workloads the metric names, each with
its own roofline object and CPU baseline, under "workloads": the fp8
prefill layer (E=128, top-8, H=4096, I=1536, M=4096; TFLOP/s against the
fp8 MFMA peak), the Qwen3-shaped fp8 sweep and the DeepSeek-V3-shaped fp8
sweep (GB/s against HBM).  --config X times workload X alone and prints its
line with X as the headline.
"""
from __future__ import annotations

import argparse
import hashlib
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
FLUSH_BYTES = 1 << 30

# HBM bytes per launch of the gate/up product, from rocprofv3 FETCH_SIZE and
# WRITE_SIZE runs of this script (scaled by the reading of a 1 GiB copy), and
# the SHA-256 of the kernel sources they were taken on.  The figure is
# reported only while those sources are unchanged.
DECODE_SOURCES = ("moe_layer_align_amd/csrc/gemm_decode.h", "moe_layer_align_amd/csrc/layer_small.h",
                  "moe_layer_align_amd/csrc/route_align.h", "moe_layer_align_amd/csrc/moe_device.h")
SINGLE_SOURCES = ("moe_layer_align_amd/csrc/layer_small.h", "moe_layer_align_amd/csrc/gemm_decode.h",
                  "moe_layer_align_amd/csrc/route_align.h", "moe_layer_align_amd/csrc/moe_device.h")
PREFILL_SOURCES = ("moe_layer_align_amd/csrc/gemm_prefill.h", "moe_layer_align_amd/csrc/moe_device.h")
TRAFFIC = {
    "mixtral": {"src_sha256": "6f5c6fbb7854f74b5824eaab3d58e3a4d7a0fd3d985fff56850075a58ead077a",
                "bytes_per_launch": 1511736166},
    "qwen3": {"src_sha256": "6f5c6fbb7854f74b5824eaab3d58e3a4d7a0fd3d985fff56850075a58ead077a",
              "bytes_per_launch": 240921788},
    "deepseek": {"src_sha256": "6f5c6fbb7854f74b5824eaab3d58e3a4d7a0fd3d985fff56850075a58ead077a",
                 "bytes_per_launch": 3292697022},
    "prefill": {"src_sha256": "03c79ae18bdf7882c8bb719695f3be451b6ed688155ea513e78d2fa19b851177",
                "bytes_per_launch": 3019611436},
}


def log(msg: str):
    sys.stderr.write("[bench] %s\n" % msg)
    sys.stderr.flush()


def kernel_sources_sha256(sources) -> str:
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default=None, choices=["mixtral", "qwen3", "deepseek", "prefill", "tiny"],
                    help="time this workload only (default: the Mixtral headline, then the prefill, Qwen3 and "
                         "DeepSeek workloads under 'workloads')")
    ap.add_argument("--no-flush", action="store_true", help="hot-cache numbers: skip the cache flush before each call")
    ap.add_argument("--router-gemm", action="store_true",
                    help="the layer computes its router logits from the hidden states and N(0,1/H) router "
                         "weights [E,H] (inside the timed span) instead of taking the workload's logits")
    ap.add_argument("--per-channel", action="store_true",
                    help="fp8 workloads: one weight scale per weight row instead of one per tensor")
    ap.add_argument("--per-expert", action="store_true",
                    help="fp8 workloads: one weight scale per expert instead of one per tensor")
    ap.add_argument("--shared", type=int, default=0, metavar="S",
                    help="S shared experts (every token also passes through them, weight one)")
    ap.add_argument("--single-launch", action="store_true",
                    help="tiny token counts (at most 16 tokens and 64 pairs) run as one launch (tuning "
                         "single_launch = 1) instead of the default multi-launch path")
    ap.add_argument("--down", choices=["auto", "token", "expert"], default="auto",
                    help="down product of layers with at most 64 pairs: auto (default: per token, with the "
                         "combine in the same launch), token (required), expert (per-expert down product and a "
                         "separate finalize)")
    ap.add_argument("--routing", choices=["auto", "separate"], default="auto",
                    help="tiny layers (at most 16 tokens and 64 pairs, per-token down product): auto (default: "
                         "the routing and sort-and-pad inside the gate/up launch, the layer in two launches, "
                         "where that fits) or separate (routing launches of their own)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0, help="budget of the CPU oracle sample")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB a few times (reference reading for "
                         "the FETCH_SIZE/WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this layer is built and timed on a single MI355X; "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        return 2

    import torch
    import moe_layer_align_amd as moe

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.calibrate_copy:
        return calibrate_copy(args.calibrate_copy)
    moe.load()  # fails loudly when the HIP library is missing
    if (args.per_channel or args.per_expert) and args.config in (None, "mixtral", "tiny"):
        print("--per-channel and --per-expert apply to the fp8 workloads: give --config qwen3|deepseek|prefill",
              file=sys.stderr)
        return 2
    peaks = achieved_peaks()
    if args.config is not None:
        line = measure(args.config, args)
    else:
        line = measure("mixtral", args)
        extra = {}
        for name in ("prefill", "qwen3", "deepseek"):
            sub = measure(name, args, cpu_seconds=args.cpu_seconds / 2)
            extra[name] = dict(value=sub["metric_value"], **{key: sub[key] for key in (
                "unit", "ms_per_step", "dtype", "config", "per_m", "roofline", "cpu_baseline")})
            torch.cuda.empty_cache()
        line["workloads"] = extra
    for key in ("metric_value",):
        line.pop(key, None)
    line["achieved_peaks"] = peaks
    for roof in [line["roofline"]] + [w["roofline"] for w in line.get("workloads", {}).values()]:
        for r in (roof, roof.get("other_kernel")):
            if r:
                # the fp8 product's operands are real data: the random-operand ceiling
                ceil = peaks["hbm_read_gbs"] if r["bound"] == "hbm" else peaks["fp8_mfma_random_operands_tflops"]
                r["frac_of_achieved_peak"] = round(r["achieved"] / ceil, 4) if (
                    r["bound"] == "hbm" or r["peak"] == FP8_PEAK_TFLOPS) else None
    print(json.dumps(line), flush=True)
    return 0


def achieved_peaks(reps: int = 5) -> dict:
    """What this GPU delivers, from the probes of libmoe_probes.so, timed
    with HIP events on the launch stream: the read bandwidth of a 4 GiB
    streaming read (16 times the last-level cache, so HBM) and the issue
    rate of independent 32x32x64 fp8 MFMAs on all compute units; the best of
    `reps` calls each."""
    import torch
    from moe_layer_align_amd import probes

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    nbytes = 4 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    grid_r = 8192
    sink = torch.empty(grid_r, dtype=torch.int32, device=dev)
    grid_m, iters = 512, 2000
    out = torch.empty(grid_m * 16, dtype=torch.float32, device=dev)

    def best(fn):
        fn()  # warm
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            b.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        return min(ts)

    t_read = best(lambda: probes.hbm_read(buf, sink, grid_r, stream))
    t_mfma = best(lambda: probes.mfma_fp8_loop(out, grid_m, iters, False, stream))
    torch.cuda.synchronize()
    if not torch.all(out == 64.0 * iters):
        raise RuntimeError("MFMA probe returned wrong sums")
    t_mfma_rand = best(lambda: probes.mfma_fp8_loop(out, grid_m, iters, True, stream))
    flops = grid_m * 4 * iters * 4 * 2.0 * 32 * 32 * 64
    res = dict(hbm_read_gbs=round(nbytes / t_read / 1e9, 1), fp8_mfma_tflops=round(flops / t_mfma / 1e12, 1),
               fp8_mfma_random_operands_tflops=round(flops / t_mfma_rand / 1e12, 1),
               how="best of %d: streaming read of 4 GiB by %d workgroups; %d workgroups x 4 waves x %d rounds of "
                   "4 independent 32x32x64 fp8 MFMAs (libmoe_probes.so), operands 1.0 and pseudo-random"
                   % (reps, grid_r, grid_m, iters))
    log("achieved peaks: %s" % res)
    del buf
    torch.cuda.empty_cache()
    return res


def measure(config: str, args, cpu_seconds=None) -> dict:
    """Time one workload's sweep; returns its JSON line (as a dict)."""
    import torch
    import moe_layer_align_amd as moe
    from synth import (CONFIGS, gen_logits, gen_router_weights, gen_weights, gen_weights_per_channel,
                       gen_weights_per_expert, gen_x)

    dev = torch.device("cuda:0")
    cfg = CONFIGS[config]
    fp8 = cfg.dtype == "fp8"
    esz = 1 if fp8 else 2
    log("generating %s weights on the GPU" % cfg.name)
    if args.per_channel and args.per_expert or args.shared < 0:
        raise SystemExit("give at most one of --per-channel and --per-expert, and --shared >= 0")
    S = args.shared
    per_channel = args.per_channel and fp8
    per_expert = args.per_expert and fp8
    ES, KS = cfg.E + S, cfg.k + S  # experts and slots per token with the shared experts
    if per_channel or per_expert:
        gen = gen_weights_per_channel if per_channel else gen_weights_per_expert
        w13, w2, s13_t, s2_t = gen(cfg, 0, device=dev, E=ES)
        s13, s2 = s13_t, s2_t
    else:
        w13, w2, s13, s2 = gen_weights(cfg, 0, device=dev, E=ES)
        s13_t = torch.tensor([s13], device=dev) if fp8 else None
        s2_t = torch.tensor([s2], device=dev) if fp8 else None

    calls = []
    for M in cfg.ms:
        x = gen_x(cfg.H, M, 0, sub=M).to(dev)
        lg = gen_logits(cfg, M, 0, sub=M).to(dev)
        ws = torch.empty(moe.workspace_size(M, ES, cfg.H, cfg.I, KS, cfg.dtype), dtype=torch.uint8, device=dev)
        y = torch.empty(M, cfg.H, dtype=torch.bfloat16, device=dev)
        counts = torch.empty(ES, dtype=torch.int32, device=dev)
        calls.append(dict(M=M, x=x, lg=lg, ws=ws, y=y, counts=counts))

    stream = torch.cuda.current_stream()
    flush_buf = None if args.no_flush else torch.ones(FLUSH_BYTES // 4, dtype=torch.int32, device=dev)

    router_w = gen_router_weights(cfg.E, cfg.H, 0, device=dev) if args.router_gemm else None

    down = {"auto": 0, "token": 1, "expert": -1}[args.down]
    small = lambda M: M <= 16 and M * KS <= 64 and cfg.E <= 256
    tok_ok = lambda M: M * KS <= 64
    tuning_for = {M: moe.Tuning(single_launch=1 if (args.single_launch and small(M)) else 0,
                                down_per_token=down if (down != 1 or tok_ok(M)) else 0,
                                routing_in_gate_up=-1 if args.routing == "separate" else 0) for M in cfg.ms}

    mode = 1 if per_channel else 2 if per_expert else 0
    for c in calls:  # the launch sequence each call takes, from the library's own plan
        c["path"] = moe.fused_path(c["M"], cfg.E, cfg.H, cfg.I, cfg.k, cfg.dtype, n_shared=S, weight_scale_mode=mode,
                                   router_w=args.router_gemm, tuning=tuning_for[c["M"]])

    def run(c, events=None):
        moe.fused_forward(c["x"], None if args.router_gemm else c["lg"], w13, w2, cfg.k, cfg.dtype, s13_t, s2_t,
                          out=c["y"], workspace=c["ws"], expert_counts=c["counts"], stream=stream, events=events,
                          router_w=router_w, n_shared=S, tuning=tuning_for[c["M"]])

    def flush(i):
        if flush_buf is not None:
            flush_buf.sum()

    # active experts from the layer's own routing, for the byte and flop accounting
    for c in calls:
        run(c)
    torch.cuda.synchronize()
    for c in calls:
        cnt = c["counts"].cpu()
        c["active"] = int((cnt > 0).sum())
        c["w_bytes"] = c["active"] * 3 * cfg.H * cfg.I * esz
        c["g1_bytes"] = c["active"] * 2 * cfg.H * cfg.I * esz
        c["flops"] = 6.0 * c["M"] * KS * cfg.H * cfg.I
        c["g1_flops"] = 4.0 * c["M"] * KS * cfg.H * cfg.I

    log("warmup %d steps" % args.warmup)
    for s in range(args.warmup):
        for c in calls:
            flush(s)
            run(c)
    torch.cuda.synchronize()

    # Two timed passes of the same steps.  Pass A times the layer: events only
    # at its start and end (slots 0 and 9 of the library's stage events; an
    # event recorded between two kernels adds a few microseconds to the span).
    # Pass B times the dominant kernel for the roofline: events only around
    # the gate/up launch (slots 4 and 5).
    ns = moe.NUM_STAGES

    def timed_pass(slots, label):
        evs = [[{i: torch.cuda.Event(enable_timing=True) for i in slots} for _ in calls] for _ in range(args.steps)]
        for step in evs:  # materialise the hipEvent_t handles
            for per_call in step:
                for e in per_call.values():
                    e.record(stream)
        torch.cuda.synchronize()
        handles = [[[per_call[i].cuda_event if i in per_call else None for i in range(2 * ns)] for per_call in step]
                   for step in evs]
        log("timing %d steps (%s)" % (args.steps, label))
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        for s in range(args.steps):
            for j, c in enumerate(calls):
                flush(s + j)
                run(c, handles[s][j])
        t1.record(stream)
        torch.cuda.synchronize()

        def between(a, b):
            return [[evs[s][j][a].elapsed_time(evs[s][j][b]) for s in range(args.steps)] for j in range(len(calls))]
        return between, t0.elapsed_time(t1)

    between, wall_ms = timed_pass((0, 2 * ns - 1), "layer spans")
    span_ms = between(0, 2 * ns - 1)
    # Pass B: the launches of the dominant kernels.  A call that takes the
    # multi-launch or the two-launch path runs its gate/up launch between
    # events 4 and 5; one that takes the single-launch layer runs that one
    # kernel between events 0 and 1 (the library then records events 1..9
    # back to back after it).
    between, _ = timed_pass((0, 1, 4, 5), "dominant-kernel launches")
    first_ms, g1_ms = between(0, 1), between(4, 5)
    for j, c in enumerate(calls):
        c["single"] = c["path"] == "single_launch"
        c["kern_ms"] = first_ms[j] if c["single"] else g1_ms[j]
    layer_ms_per_step = sum(sum(v) for v in span_ms) / args.steps

    # Per-stage breakdown, outside the timed region (all ten events per call).
    log("per-stage breakdown")
    n_prof = min(args.steps, 10)
    stage_ms = []
    for j, c in enumerate(calls):
        per = []
        for s in range(n_prof):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2 * ns)]
            flush(s)
            run(c, _materialise(e, stream))
            per.append(e)
        torch.cuda.synchronize()
        stage_ms.append([statistics.median(p[2 * q].elapsed_time(p[2 * q + 1]) for p in per) for q in range(ns)])

    per_m = []
    for j, c in enumerate(calls):
        us = statistics.median(span_ms[j]) * 1e3
        kern_us = statistics.median(c["kern_ms"]) * 1e3
        entry = dict(M=c["M"], us=round(us, 2), active_experts=c["active"], weight_bytes=c["w_bytes"],
                     gbps=round(c["w_bytes"] / us / 1e3, 1), hbm_frac=round(c["w_bytes"] / us / 1e3 / HBM_PEAK_GBS, 4),
                     tflops=round(c["flops"] / us / 1e6, 2), path=c["path"])
        if c["single"]:
            entry["single_launch_kernel_us"] = round(kern_us, 2)
        else:
            entry["gate_up_gbps"] = round(c["g1_bytes"] / kern_us / 1e3, 1)
        for q, name in enumerate(moe.STAGE_NAMES):
            entry["%s_us" % name] = round(stage_ms[j][q] * 1e3, 2)
        per_m.append(entry)

    total_bytes = sum(c["w_bytes"] for c in calls)
    total_flops = sum(c["flops"] for c in calls)
    if cfg.name == "prefill":
        value = total_flops / (layer_ms_per_step * 1e-3) / 1e12
        unit = "TFLOP/s"
    else:
        value = total_bytes / (layer_ms_per_step * 1e-3) / 1e9
        unit = "GB/s"

    # Roofline of the kernel that takes the most time over the sweep: the
    # gate/up product of the multi-launch calls (algorithmic bytes: W13 of the
    # experts with tokens; prefill: 4*M*k*H*I flops) or the single-launch
    # layer (bytes: W13 and W2 of those experts); the other kind, when the
    # sweep has both, is reported beside it.
    def roofline(single: bool):
        sel = [c for c in calls if c["single"] == single]
        if not sel:
            return None
        kern_ms = sum(sum(c["kern_ms"]) for c in sel)
        n = args.steps * len(sel)
        if cfg.name == "prefill":
            ach = sum(c["g1_flops"] for c in sel) * args.steps / (kern_ms * 1e-3) / 1e12
            r = dict(bound="mfma", achieved=round(ach, 1), peak=FP8_PEAK_TFLOPS if fp8 else BF16_PEAK_TFLOPS,
                     unit="TFLOP/s")
        else:
            work = sum((c["w_bytes"] if single else c["g1_bytes"]) for c in sel)
            ach = work * args.steps / (kern_ms * 1e-3) / 1e9
            r = dict(bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s")
        r["frac"] = round(ach / r["peak"], 4)
        tr = TRAFFIC.get(cfg.name + ("_single" if single else ""))
        srcs = PREFILL_SOURCES if cfg.name == "prefill" else (SINGLE_SOURCES if single else DECODE_SOURCES)
        # the counters were taken on the default inputs (cold cache, given
        # logits, per-tensor scales) of these kernel sources
        r["traffic"] = tr["bytes_per_launch"] if (tr and tr["src_sha256"] == kernel_sources_sha256(srcs)
                                                  and not (args.no_flush or per_channel or per_expert
                                                           or args.shared or args.router_gemm)) else None
        r["traffic_unit"] = "bytes per launch (HBM, rocprofv3 FETCH_SIZE+WRITE_SIZE)"
        ms_of = lambda paths: ",".join(str(c["M"]) for c in sel if c["path"] in paths)
        two, dec = ms_of(("two_launches",)), ms_of(("decode", "decode_token_down"))
        r["kernel"] = ("prefill_gemm_kernel<0, *> (tiled gate/up product + SiLU*up)" if cfg.name == "prefill"
                       else "layer1_kernel (the whole layer in one cooperative launch) at M = %s"
                       % ",".join(str(c["M"]) for c in sel) if single
                       else "; ".join(x for x in (
                           "tiny_gate_up_kernel (routing, sort-and-pad and the gate/up product + SiLU*up in one "
                           "launch) at M = %s" % two if two else "",
                           "gate/up product + SiLU*up (gemm1_decode_kernel, or gemm1_stream_kernel for fp8 layers "
                           "whose plan takes the long-stream variant) at M = %s" % dec if dec else "") if x))
        r["avg_launch_us"] = round(kern_ms * 1e3 / n, 2)
        r["launches"] = n
        r["kernel_ms_total"] = kern_ms
        return r

    roofs = [r for r in (roofline(False), roofline(True)) if r is not None]
    roofs.sort(key=lambda r: -r["kernel_ms_total"])
    for r in roofs:
        del r["kernel_ms_total"]
    roof = roofs[0]
    if len(roofs) > 1:
        roof["other_kernel"] = roofs[1]

    cpu = None
    if not args.no_cpu_baseline and not args.router_gemm:  # the oracle sample takes the workload's logits
        cpu = cpu_baseline(cfg, calls, (w13, w2, s13, s2), cpu_seconds or args.cpu_seconds, unit, n_shared=S,
                           min_s=min(10.0, cpu_seconds or args.cpu_seconds))

    ms_str = ",".join(str(m) for m in cfg.ms)
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(layer_ms_per_step, 4),
        "wall_ms_per_step": round(wall_ms / args.steps, 4),
        "cache": "hot" if args.no_flush else "cold (1 GiB read before each call, outside the layer span)",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f8e4m3" if fp8 else "bf16",
        "data": "synthetic: seeded N(0,1) hidden states, N(0,1/fan_in) expert weights, router logits per workload",
        "config": {
            "workload": "%s-shaped %s layer E=%d top-%d H=%d I=%d%s, M in {%s}" % (
                cfg.name, cfg.dtype, cfg.E, cfg.k, cfg.H, cfg.I, " +%d shared" % S if S else "", ms_str),
            "E": cfg.E, "top_k": cfg.k, "H": cfg.H, "I": cfg.I, "M_sweep": list(cfg.ms), "router_logits": cfg.logits,
            "weight_scales": ("per channel" if per_channel else "per expert" if per_expert
                              else "per tensor") if fp8 else None,
            "shared_experts": S,
            "logits_source": "computed in the layer from router weights" if args.router_gemm else "given",
            "single_launch": "at M <= 16 with at most 64 pairs" if args.single_launch else "off",
            "routing": {"auto": "in the gate/up launch where the layer fits two launches",
                        "separate": "launches of its own"}[args.routing],
            "paths": {str(c["M"]): c["path"] for c in calls},
            "down_product": {"auto": "per token with the combine at <= 64 pairs, else per expert + finalize",
                             "token": "per token with the combine where it fits",
                             "expert": "per expert + finalize"}[args.down],
        },
        "per_m": per_m,
        "roofline": roof,
        "cpu_baseline": cpu,
        "metric_value": round(value, 2),
    }
    del w13, w2, calls, flush_buf
    return line


def _materialise(events, stream):
    """hipEvent_t handles of fresh torch events (torch creates them lazily)."""
    for e in events:
        e.record(stream)
    return [e.cuda_event for e in events]


def calibrate_copy(mib: int) -> int:
    """A plain copy of known size: under rocprofv3 --pmc its FETCH_SIZE and
    WRITE_SIZE readings per dispatch, divided by the bytes it must move,
    give the factor that turns those counters into HBM bytes."""
    import torch
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n, "dispatches": 5}), flush=True)
    return 0


def cpu_baseline(cfg, calls, weights, budget_s, unit, min_s=10.0, n_shared=0):
    """The CPU oracle on the same inputs, timed on a bounded sample.

    The oracle evaluates every (token, expert) pair with dense loops, so its
    time is proportional to the number of pairs it evaluates.  For each point
    of the sweep (smallest M first) it runs the whole layer when that fits the
    remaining budget, else an evenly spaced subset of the tokens, and its rate
    is extrapolated to all M*k pairs of that point.  Short sweeps are repeated
    until about min_s seconds have been spent.
    """
    import oracle

    w13, w2, s13, s2 = weights
    kk = cfg.k + n_shared  # pairs per token
    log("cpu baseline: copying weights to the host")
    w13h, w2h = w13.cpu(), w2.cpu()
    work_sum, secs_sum, spent, parts, rounds = 0.0, 0.0, 0.0, [], 0
    sec_per_pair = None
    while rounds == 0 or (spent < min(min_s, budget_s) and all(p.endswith(":all") for p in parts)):
        rounds += 1
        ordered = sorted(calls, key=lambda c: c["M"])
        for idx, c in enumerate(ordered):
            M = c["M"]
            # the budget left is shared by the points of this pass not yet run
            left = budget_s / len(calls) if sec_per_pair is None else (budget_s - spent) / (len(ordered) - idx)
            n_tok = M if sec_per_pair is None else int(max(1, min(M, left / (sec_per_pair * kk))))
            if sec_per_pair is None and M * kk > 256:
                n_tok = max(1, 256 // kk)  # probe the rate first
            toks = sorted({int(round(i * (M - 1) / max(n_tok - 1, 1))) for i in range(n_tok)}) if n_tok < M else None
            log("cpu baseline: oracle at M=%d on %s tokens" % (M, M if toks is None else len(toks)))
            x, lg = c["x"].cpu(), c["lg"].cpu()
            t0 = time.perf_counter()
            oracle.layer(x, lg, w13h, w2h, cfg.k, cfg.dtype, s13, s2, tokens=toks,
                         all_pairs_h=False if toks is not None else None, n_shared=n_shared)
            dt = time.perf_counter() - t0
            spent += dt
            n_pairs = (M if toks is None else len(toks)) * kk
            sec_per_pair = dt / n_pairs
            work_sum += c["w_bytes"] if unit == "GB/s" else c["flops"]
            secs_sum += sec_per_pair * M * kk
            if rounds == 1:
                parts.append("M=%d:%s" % (M, "all" if toks is None else "%d/%d tokens" % (len(toks), M)))
            if spent > budget_s:
                break
        if spent > budget_s:
            break
    val = work_sum / secs_sum / (1e9 if unit == "GB/s" else 1e12)
    return {"value": round(val, 4), "unit": unit, "cores": oracle.num_threads(), "kind": "oracle",
            "seconds": round(spent, 2),
            "sample": "oracle (scalar fp64, OpenMP) on the same seeded inputs, weights in host memory; "
                      "points %s, %d pass(es); a token subset is extrapolated by pairs to the full layer"
                      % (", ".join(parts), rounds)}


if __name__ == "__main__":
    sys.exit(main())
