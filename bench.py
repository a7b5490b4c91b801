#!/usr/bin/env python3
"""Benchmark of the MI355X MegaMoE per-rank layer forward (one GPU).

A step is one pass of the whole path over one batch of received rows:
stage (BF16 -> e4m3 1x128 quantisation + route check) -> compaction ->
FC1 (+ SwiGLU + 1x128 requant) -> FC2 -> weighted combine to BF16.  Inputs
are synthetic and already resident in HBM when timing starts.

Headline workload: the DeepSeek-V3-like one-GPU share (H=7168, I=2048, 32
local experts, top-8, balanced block-permutation routing, T=4096 tokens).
The same JSON line also carries the token-sweep points where the targets
sit (T=8 and 64: weight-streaming, HBM-bound; T=512: between the two regimes, HBM-bound
by FLOP per byte; T=8192 and 32768: MFMA-bound),
each timed the same way, with its own roofline (bound chosen by the step's
FLOP per algorithmic byte against the machine balance) and a sampled CPU
baseline (the float64 oracle on this host).

Prints one JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer TFLOP/s + % FP8 MFMA peak (HBM GB/s small T), 32 experts, T=8..32768"
FP8_PEAK_TFLOPS = 5000.0  # MI355X dense FP8 MFMA (no sparsity)
HBM_PEAK_GBS = 8000.0     # MI355X HBM3E
BALANCE = FP8_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)  # FLOP per byte (625)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def row_bytes(n, mx):
    """Bytes of one staged activation row of n elements: e4m3 + 1x128 float32
    scales, or (MXFP8 x BF16) two e4m3 term planes + one exponent word per 32."""
    return 2 * n + n // 8 if mx else n + n // 32


def weight_bytes(shape, counts, mx, which=("w13", "w2")):
    H, I = shape.hidden, shape.intermediate
    touched = int(sum(1 for c in counts if c > 0))
    per = 0
    if "w13" in which:
        per += 2 * I * H * (1 + 1 / 32) if mx else 2 * I * H + 4 * (2 * I // 128) * (H // 128)
    if "w2" in which:
        per += H * I * (1 + 1 / 32) if mx else H * I + 4 * (H // 128) * (I // 128)
    return touched * per


def workload_bytes(shape, counts, tokens, with_stage=True, mx=False):
    """Algorithmic HBM bytes of one step: the touched experts' weights, the
    staged rows read by FC1, the FC1 output written and read, the BF16 FC2
    rows written and read, the BF16 output, 16 bytes of routing metadata per
    route, and the staging (BF16 read, staged row written)."""
    H, I = shape.hidden, shape.intermediate
    R = int(sum(counts))
    x = tokens * row_bytes(H, mx)
    h = 2 * R * row_bytes(I, mx)
    y = 2 * R * H * 2
    out = tokens * H * 2
    meta = R * 16
    stage = (2 * tokens * H + tokens * row_bytes(H, mx)) if with_stage else 0
    return weight_bytes(shape, counts, mx) + x + h + y + out + meta + stage


def fc1_bytes(shape, counts, tokens, mx=False):
    """Algorithmic HBM bytes of one FC1 launch: W13 of the touched experts
    (with its scales), the staged rows it reads, the h rows it writes."""
    R = int(sum(counts))
    return weight_bytes(shape, counts, mx, ("w13",)) + tokens * row_bytes(shape.hidden, mx) + \
        R * row_bytes(shape.intermediate, mx)


def fc1_flops(R, H, I):
    return 4.0 * R * H * I


# HBM bytes per FC1 launch from the committed FETCH_SIZE / WRITE_SIZE counter
# passes.  The figure is valid only for the kernel source it was taken on: the
# file records a hash of the sources that decide the FC1 kernel and its launch.
COUNTER_FILE = os.path.join(ROOT, "profiles", "fc1_dsv3_T4096_hbm_counters.txt")
COUNTER_SOURCES = ["mixture_experts_ffn_route_amd/csrc/moe_gemm_fp8.hip",
                   "mixture_experts_ffn_route_amd/csrc/moe_gemm_fp8_body.inc",
                   "mixture_experts_ffn_route_amd/csrc/moe_gemm_fp8_pp.inc",
                   "mixture_experts_ffn_route_amd/csrc/moe_gemm_fp8_stream.inc",
                   "mixture_experts_ffn_route_amd/csrc/moe_device.h",
                   "mixture_experts_ffn_route_amd/csrc/moe_store_dev.h",
                   "mixture_experts_ffn_route_amd/csrc/moe_host.cpp",
                   "mixture_experts_ffn_route_amd/csrc/moe_api.cpp"]


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for rel in COUNTER_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload):
    """FC1 HBM bytes per launch from the counter file, or None when absent,
    taken on another workload, or taken on a different kernel source."""
    try:
        with open(COUNTER_FILE) as f:
            kv = dict(ln.split(":", 1) for ln in f.read().splitlines() if ":" in ln and not ln.startswith(" "))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("source_hash") != kernel_source_hash() or kv.get("workload") != workload:
        return None
    try:
        return int(kv["fc1_hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return 1


def run_cpu_baseline(inp, sample_tokens, tokens):
    """The float64 oracle, as it stands, on the first `sample_tokens` tokens
    of the workload (full forward: staging, weight decode, both GEMMs,
    combine)."""
    from oracle import moe_ref

    S = min(sample_tokens, tokens)
    t0 = time.perf_counter()
    args = (inp.x_bf16[:S], inp.topk_idx[:S], inp.topk_w[:S], inp.w13, inp.w13_scale, inp.w2, inp.w2_scale)
    if inp.weight_format.startswith("mxfp8"):
        moe_ref.forward_mx(*args, elem="e5m2" if inp.weight_format == "mxfp8_e5m2" else "e4m3")
    else:
        moe_ref.forward_fp8(*args)
    dt = time.perf_counter() - t0
    R = S * inp.shape.top_k
    flops = 6.0 * R * inp.shape.hidden * inp.shape.intermediate
    cores = min(blas_threads(), len(os.sched_getaffinity(0)))
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"first {S} of {tokens} tokens of the same workload (full forward incl. staging and weight "
                      f"decode), {dt:.1f} s"}


def slot_timer_report(args, base, flags, mx):
    """Cycles per K-block of each phase of the 256-token GEMM kernel's two
    slots, per GEMM and wave group (moe_debug_slot_timers), and the share of
    the tile epilogue, over `steps` forwards of the headline workload after
    the usual settle and warm-up.  The timed build reads a cycle counter at
    every phase boundary, so its step time is a little longer than the plain
    build's."""
    import torch

    from mixture_experts_ffn_route_amd import _lib as L
    from mixture_experts_ffn_route_amd.harness import make_layer, to_device
    from synthetic import MoEShape, make_layer_inputs

    tokens = args.tokens or base.tokens
    shape = MoEShape(tokens, base.hidden, base.intermediate, base.experts, base.top_k, base.routing)
    dev = to_device(make_layer_inputs(shape, seed=args.seed, weight_format=args.weights))
    layer = make_layer(shape, dev, mx=mx, flags=flags, expected_m=args.expected_m)
    out = torch.empty((tokens, shape.hidden), dtype=torch.bfloat16, device="cuda")

    def step():
        layer.stage(dev.x, dev.topk_idx, dev.topk_w, out=out)
        layer.forward()

    t0 = time.perf_counter()
    while time.perf_counter() - t0 < args.settle_s:
        step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    L.moe_debug_slot_timers()  # clears the counters
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / args.steps * 1e3
    w = L.moe_debug_slot_timers()
    names = ["load_dma_issue", "load_lds_and_records", "load_barrier", "mfma_slot_issue", "own_load_wait",
             "mfma_barrier", "epilogue"]
    rep = {"workload": f"{args.config} T={tokens}", "tactic": layer.tactic()["block_m"], "steps": args.steps,
           "ms_per_step": round(ms, 4), "unit": "cycles per K-block per wave (epilogue: share of the kernel)"}
    for g, gemm in ((0, "fc1"), (16, "fc2")):
        for grp in range(2):
            d = w[g + grp * 8: g + grp * 8 + 8]
            kblocks = d[7]
            if kblocks == 0:
                continue
            row = {n: round(d[i] / kblocks, 1) for i, n in enumerate(names[:6])}
            row["k_block_total"] = round(sum(d[:6]) / kblocks, 1)
            row["epilogue_share"] = round(d[6] / max(sum(d[:7]), 1), 4)
            rep[f"{gemm}_group{grp}"] = row
    print(json.dumps(rep), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-s", type=float, default=0.4,
                    help="untimed steps run for at least this long before the warm-up steps: the GPU "
                         "reaches its steady clock only after some 25 steps of this workload")
    ap.add_argument("--config", default="dsv3", choices=["tiny", "small", "dsv3", "skewed"])
    ap.add_argument("--tokens", type=int, default=None, help="override T of the headline workload")
    ap.add_argument("--points", default="8,64,512,8192,32768",
                    help="extra token counts of the same shape timed into the JSON line ('' for none)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--weights", default="fp8_block", choices=["fp8_block", "mxfp8", "mxfp8_e5m2"],
                    help="fp8_block: e4m3 + 128x128 scales, e4m3 1x128 activations; "
                         "mxfp8 / mxfp8_e5m2: e4m3 / e5m2 + E8M0 per 32 weights x BF16 activations")
    ap.add_argument("--ffn", default="two", choices=["two", "persistent"],
                    help="two: FC1 and FC2 launches; persistent: one launch, FC2 tiles start as their rows are ready")
    ap.add_argument("--combine", default="separate", choices=["separate", "fused"],
                    help="separate: combine kernel after FC2; fused: last-arriver combine inside FC2")
    ap.add_argument("--cpu-sample", type=int, default=2048,
                    help="tokens of the headline workload for the CPU oracle baseline (0: no CPU baselines)")
    ap.add_argument("--cpu-point-sample", type=int, default=64, help="tokens per extra point for its CPU baseline")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run one device-to-device copy of this many MiB (reference for HBM byte counters)")
    ap.add_argument("--no-stream", action="store_true",
                    help="run FC2 at 64-token tiles on the LDS-ring kernel too (MOE_FLAG_NO_STREAM)")
    ap.add_argument("--stream-fc1", action="store_true",
                    help="run FC1 at 64-token tiles on the streaming kernel (MOE_FLAG_STREAM_FC1)")
    ap.add_argument("--expected-m", type=int, default=None,
                    help="expected rows per expert, which picks the token tile (default: T*K/E)")
    ap.add_argument("--sweep", default="", help="comma-separated token counts; extra lines to --sweep-out")
    ap.add_argument("--sweep-out", default="bench_sweep.jsonl", help="file the sweep lines are appended to")
    ap.add_argument("--slot-timers", action="store_true",
                    help="diagnostic: load the library built with slot timers (build.py --slot-timers), run the "
                         "headline workload and print the 256-token GEMMs' cycles per K-block and phase instead "
                         "of the bench line")
    args = ap.parse_args()
    if args.slot_timers:
        os.environ["MOE_SLOT_TIMERS"] = "1"

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the layer; the library runs on one GPU, and the "
              "expert-parallel exchange between GPUs is out of its scope.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from mixture_experts_ffn_route_amd import _lib as L
    from mixture_experts_ffn_route_amd.harness import make_layer, to_device
    from synthetic import CONFIGS, MoEShape, make_layer_inputs
    from synthetic.workloads import LayerInputs, make_activations, make_routing

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    base = CONFIGS[args.config]
    mx = ("e5m2" if args.weights == "mxfp8_e5m2" else "e4m3") if args.weights.startswith("mxfp8") else False
    # The MXFP8 x BF16 path issues two FP8 MFMAs per K-block (hi and lo
    # activation terms), so its ceiling in layer FLOPs is half the FP8 peak.
    peak = FP8_PEAK_TFLOPS / 2 if mx else FP8_PEAK_TFLOPS
    flags = L.MOE_FLAG_CHECK_ROUTES | (L.MOE_FLAG_FUSED_COMBINE if args.combine == "fused" else 0)
    if args.no_stream:
        flags |= L.MOE_FLAG_NO_STREAM
    if args.stream_fc1:
        flags |= L.MOE_FLAG_STREAM_FC1
    persistent = args.ffn == "persistent"
    if persistent:
        flags |= L.MOE_FLAG_PERSISTENT_FFN

    cache = {}

    if args.slot_timers:
        slot_timer_report(args, base, flags, mx)
        return

    def inputs_for(shape):
        """Seeded inputs of one token count; the expert weights (which do not
        depend on T) are generated once and shared by every point."""
        if "w" not in cache:
            inp = make_layer_inputs(shape, seed=args.seed, weight_format=args.weights)
            cache["w"] = (inp.w13, inp.w13_scale, inp.w2, inp.w2_scale)
            return inp
        idx, w = make_routing(shape, args.seed)
        x = make_activations(shape.tokens, shape.hidden, args.seed)
        return LayerInputs(shape, args.weights, x, idx, w, *cache["w"])

    def measure(tokens, steps, warmup, cpu_sample):
        """One workload: settle + warm-up, `steps` timed steps (mean), then
        the same number of steps each bracketed by events (p50, min), then
        FC1's own time (events around FC1 only) and a per-kernel breakdown
        (events around every kernel, untimed pass)."""
        shape = MoEShape(tokens, base.hidden, base.intermediate, base.experts, base.top_k, base.routing)
        t0 = time.perf_counter()
        inp = inputs_for(shape)
        log(f"[bench] generated T={tokens} inputs in {time.perf_counter() - t0:.1f}s")
        dev = to_device(inp)
        layer = make_layer(shape, dev, mx=mx, flags=flags, expected_m=args.expected_m)
        out = torch.empty((tokens, shape.hidden), dtype=torch.bfloat16, device="cuda")

        def step():
            layer.stage(dev.x, dev.topk_idx, dev.topk_w, out=out)
            layer.forward()

        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while True:  # clock settle
            for _ in range(5):
                step()
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= args.settle_s:
                break
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        mean_s = (time.perf_counter() - t0) / steps
        # per-step times: one event record per step (a few us of stream time
        # each, so p50 and min sit slightly above the event-free mean)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record()
        for i in range(steps):
            step()
            ev[i + 1].record()
        torch.cuda.synchronize()
        per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
        # FC1's own time: HIP events the library records around each FC1
        # launch on its launch stream
        layer.profile(True, kernels=("fc1",))
        for _ in range(steps):
            step()
        fc1 = layer.profile_read()["fc1"]
        layer.profile(True)
        for _ in range(min(steps, 10)):
            step()
        prof = layer.profile_read()
        layer.profile(False)
        status = layer.status()
        counts = layer.region("counts", torch.int32, (shape.experts,)).cpu().numpy()
        R = int(counts.sum())
        H, I = shape.hidden, shape.intermediate
        flops = 6.0 * R * H * I
        B = workload_bytes(shape, counts, tokens, mx=mx)
        fc1_s = fc1[0] / max(fc1[1], 1) / 1e3
        fc1_b = fc1_bytes(shape, counts, tokens, mx=mx)
        fc1_f = fc1_flops(R, H, I) if not persistent else flops
        # the roofline that bounds the step: MFMA above the machine balance
        if flops / B >= BALANCE:
            roof = {"bound": "mfma", "achieved": round(fc1_f / fc1_s / 1e12, 2), "peak": peak, "unit": "TFLOP/s"}
        else:
            roof = {"bound": "hbm", "achieved": round(fc1_b / fc1_s / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s"}
        roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
        rec = {
            "tokens": tokens, "routes": R, "status": status,
            "ms_per_step": round(mean_s * 1e3, 4),
            "ms_per_step_p50": round(per[len(per) // 2], 4), "ms_per_step_min": round(per[0], 4),
            "tflops": round(flops / mean_s / 1e12, 2), "pct_mfma_peak": round(100 * flops / mean_s / 1e12 / peak, 2),
            "gbs_algorithmic": round(B / mean_s / 1e9, 1),
            "pct_hbm_peak": round(100 * B / mean_s / 1e9 / HBM_PEAK_GBS, 2),
            "flop_per_byte": round(flops / B, 1),
            "fc1_ms": round(fc1_s * 1e3, 4), "fc1_roofline": roof,
            "kernel_avg_ms": {k: round(v[0] / max(v[1], 1), 4) for k, v in prof.items()},
            "tactic": layer.tactic()["block_m"], "stream_depth": [layer.tactic()["stream_depth_fc1"], layer.tactic()["stream_depth_fc2"]],
        }
        log(f"[bench] T={tokens} {json.dumps(rec)}")
        if cpu_sample > 0:
            log(f"[bench] CPU oracle baseline on {min(cpu_sample, tokens)} tokens ...")
            rec["cpu_baseline"] = run_cpu_baseline(inp, cpu_sample, tokens)
            log(f"[bench] cpu baseline {rec['cpu_baseline']}")
        layer.close()
        del layer, dev, out
        torch.cuda.empty_cache()
        return shape, rec

    for T in [int(t) for t in args.sweep.split(",") if t]:
        _, rec = measure(T, max(5, args.steps // 2), args.warmup, 0)
        rec.update({"weights": args.weights, "combine": args.combine, "ffn": args.ffn})
        log("[sweep]", json.dumps(rec))
        os.makedirs(os.path.dirname(args.sweep_out) or ".", exist_ok=True)
        with open(args.sweep_out, "a") as f:
            f.write(json.dumps(rec) + "\n")

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy of {n} bytes done")
        del src, dst

    T = args.tokens or base.tokens
    shape, head = measure(T, args.steps, args.warmup, args.cpu_sample)
    points = []
    for Tp in [int(t) for t in args.points.split(",") if t]:
        if Tp == T:
            continue
        _, rec = measure(Tp, args.steps, args.warmup, args.cpu_point_sample if args.cpu_sample > 0 else 0)
        points.append(rec)

    H, I = shape.hidden, shape.intermediate
    workload = (f"{args.config} T={T} H={H} I={I} E={shape.experts} K={shape.top_k} routing={shape.routing}"
                + (f" weights=mxfp8_{mx} activations=bf16" if mx else ""))
    roof = dict(head["fc1_roofline"])
    roof["kernel"] = ("fc1 (MX-scaled FP8 grouped GEMM, two activation terms + SwiGLU + bf16 split)" if mx
                      else "fc1+fc2 persistent (FP8 grouped GEMMs, one launch)" if persistent
                      else "fc1 (FP8 grouped GEMM + SwiGLU + 1x128 requant)")
    roof["traffic"] = stored_traffic(workload)
    roof["kernel_source_hash"] = kernel_source_hash()
    line = {
        "metric": METRIC,
        "value": head["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"bf16 x mxfp8_{mx}" if mx else "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": workload, "tokens": T, "routes": head["routes"], "combine": args.combine,
                   "ffn": args.ffn, "ms_per_step_p50": head["ms_per_step_p50"],
                   "ms_per_step_min": head["ms_per_step_min"], "hbm_gbs_algorithmic": head["gbs_algorithmic"],
                   "pct_mfma_peak": head["pct_mfma_peak"], "kernel_avg_ms": head["kernel_avg_ms"],
                   "settle_s": args.settle_s},
        "roofline": roof,
        "cpu_baseline": head.get("cpu_baseline"),
        "points": points,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
