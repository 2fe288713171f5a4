#!/usr/bin/env python3
"""Benchmark of the fused MoE expert-FFN forward on one MI355X.

A step is one call of the whole hot path (routing, L1 GEMM + SwiGLU/clamp/
re-quantisation, L2 GEMM, combine) on one batch of synthetic DeepSeek-V3
shaped input (H=7168, I=2048, E=256, k=8, e4m3 activations x e2m1 weights
with e8m0 1x32 scales).  Inputs are resident in HBM before timing starts.

Prints ONE JSON line: headline workload T=8192 with Zipf(1.2) routing and
10% empty experts (MFMA-bound: useful TFLOP/s and fraction of the dense FP8
MFMA peak), plus the T=128 weight-streaming workload (HBM-bound: fraction of
the 8 TB/s HBM peak) under "secondary", the roofline of the kernel and the
CPU oracle timed on a bounded token sample.  The pre-dispatch activation
quantisation (bf16 x of the headline shape -> e4m3 + e8m0) is timed under
"quantize" (HBM-bound), the gate + top-k router of the same shape under
"router".
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

METRIC = "µs/call + useful TFLOP/s (frac of MFMA/HBM peak), DeepSeek-shape MoE at T=128/8192"
PEAK_FP8_TFLOPS = 5000.0     # MI355X dense FP8 MFMA (FP8 x FP4 issues at the FP8 rate on gfx950)
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCES = ("mixture_experts_ffn_histogram_amd/csrc/moe_ffn_kernel.hip",
                  "mixture_experts_ffn_histogram_amd/csrc/moe_ffn_device.h",
                  "mixture_experts_ffn_histogram_amd/csrc/moe_ffn_kernel.h",
                  "mixture_experts_ffn_histogram_amd/csrc/moe_ffn_layout.h",
                  "mixture_experts_ffn_histogram_amd/csrc/moe_ffn_api.cpp")


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(p, active_experts: int) -> int:
    """Bytes one call must move at least: the weights (+scales) of every expert
    that receives a token, x (+scales), topk, and y (bf16)."""
    H, I, T, k = p["H"], p["I"], p["T"], p["k"]
    per_expert = 2 * I * (H // 2) + 2 * I * (H // 32) + H * (I // 2) + H * (I // 32)
    per_token = H + H // 32 + k * 8 + H * 2
    return active_experts * per_expert + T * per_token


def traffic_from_profiles(workload: str):
    """Measured HBM bytes per launch, when a counter summary for this exact kernel source exists.

    The summary (profiles/moe_ffn_kernel_<workload>_traffic.md) holds the lines
    `kernel_hash: <hash>` and `hbm_bytes_per_launch: <bytes>`."""
    path = os.path.join(ROOT, "profiles", f"moe_ffn_kernel_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith((" ", "|", "#")):
                key, _, val = line.partition(":")
                fields[key.strip()] = val.strip()
    if fields.get("kernel_hash") != kernel_hash():
        return None
    try:
        return int(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def run_workload(name: str, steps: int, warmup: int, threads: int, log):
    import numpy as np
    import torch

    import mixture_experts_ffn_histogram_amd as mf
    from mixture_experts_ffn_histogram_amd import synth

    cfg = synth.CONFIGS[name]
    t0 = time.time()
    p = synth.make_problem(cfg, threads=threads)
    log(f"[bench] {name}: inputs generated in {time.time() - t0:.1f}s")
    dev = torch.device("cuda:0")
    d = {n: torch.from_numpy(np.ascontiguousarray(p[n])).to(dev)
         for n in ("x", "x_sf", "topk_idx", "topk_weights", "w1", "w1_sf", "w2", "w2_sf")}
    T, H, I, E, k = p["T"], p["H"], p["I"], p["E"], p["k"]
    m = mf.MoeFFN(T, H, I, E, k, p["recipe"], device=dev)
    y = torch.empty((T, H), dtype=torch.int16, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    # weight transforms, once per set of weights (outside the timed calls)
    km = mf.kmajor_weight_scales(d["w1_sf"], d["w2_sf"], E, H, I) if p["recipe"] == mf.RECIPE_FP8_FP4 else (None, None)
    wt = mf.tiled_weights(d["w1"], d["w2"], E, H, I) if p["recipe"] == mf.RECIPE_FP8_FP4 else (None, None)

    def call():
        m(num_tokens=T, x=d["x"], x_sf=d["x_sf"], topk_idx=d["topk_idx"], topk_weights=d["topk_weights"],
          w1=d["w1"], w1_sf=d["w1_sf"], w2=d["w2"], w2_sf=d["w2_sf"], w1_sf_kmajor=km[0], w2_sf_kmajor=km[1],
          w1_tiled=wt[0], w2_tiled=wt[1],
          y=y, y_dtype=mf.Y_BF16,
          activation_clamp=cfg.clamp, status=status, stream=stream)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    if int(status.item()) != 0:
        raise RuntimeError(f"device status {int(status.item())}")
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(steps):
        call()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    if int(status.item()) != 0:
        raise RuntimeError(f"device status {int(status.item())}")
    idx = p["topk_idx"]
    valid = (idx >= 0) & (idx < E)
    R = int(valid.sum())
    active = int(len(np.unique(idx[valid])))
    flops = 6.0 * R * H * I
    abytes = algorithmic_bytes(p, active)
    log(f"[bench] {name}: {ms * 1e3:.1f} us/call, R={R}, active experts={active}")
    return {"p": p, "cfg": cfg, "ms": ms, "R": R, "active": active, "flops": flops, "bytes": abytes}


def run_quantize(T: int, H: int, steps: int, warmup: int, log):
    """Pre-dispatch activation quantisation (bf16 [T, H] -> e4m3 + e8m0 per 1x32), HBM-bound."""
    import numpy as np
    import torch

    import mixture_experts_ffn_histogram_amd as mf
    from mixture_experts_ffn_histogram_amd import synth

    dev = torch.device("cuda:0")
    x = torch.from_numpy(synth.activations_bf16(T, H, seed=T).view(np.int16)).to(dev)
    q = torch.empty((T, H), dtype=torch.uint8, device=dev)
    sf = torch.empty((T, H // 32), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        mf.quantize_activations(x, q, sf, stream)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(steps):
        mf.quantize_activations(x, q, sf, stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    nbytes = T * H * 2 + T * H + T * (H // 32)
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"[bench] quantize T={T} H={H}: {ms * 1e3:.1f} us/call, {gbs:.0f} GB/s")
    return {"workload": f"quantize_bf16_to_e4m3_T{T}_H{H}", "us_per_call": round(ms * 1e3, 2),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None, "kernel": "quantize_act_kernel",
                         "work_per_launch": f"{nbytes} algorithmic bytes (2 B read + 1 B + 1/32 B written "
                                            "per element)"}}


def run_router(T: int, H: int, E: int, k: int, steps: int, warmup: int, log):
    """Gate + top-k (softmax router) on the headline shape; the logits GEMM streams x once."""
    import numpy as np
    import torch

    import mixture_experts_ffn_histogram_amd as mf
    from mixture_experts_ffn_histogram_amd import synth

    dev = torch.device("cuda:0")
    x = torch.from_numpy(synth.activations_bf16(T, H, seed=T).view(np.int16)).to(dev)
    wg = torch.from_numpy(synth.router_weights_bf16(E, H, seed=E).view(np.int16)).to(dev)
    logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        mf.route_topk(x, wg, logits, idx, w, stream)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(steps):
        mf.route_topk(x, wg, logits, idx, w, stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    nbytes = T * H * 2 + E * H * 2 + T * k * 8
    gbs = nbytes / (ms * 1e-3) / 1e9
    tflops = 2.0 * T * E * H / (ms * 1e-3) / 1e12
    log(f"[bench] router T={T} H={H} E={E} k={k}: {ms * 1e3:.1f} us/call, {gbs:.0f} GB/s, {tflops:.0f} TFLOP/s")
    return {"workload": f"router_softmax_top{k}_T{T}_H{H}_E{E}", "us_per_call": round(ms * 1e3, 2),
            "useful_tflops": round(tflops, 1),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                         "kernel": "router_logits_kernel + router_topk_kernel",
                         "work_per_launch": f"{nbytes} algorithmic bytes (x, gate weights, top-k outputs)"}}


def cpu_baseline(p, clamp: float, target_s: float, log):
    """The CPU oracle as it stands, per-token path, on a bounded token sample."""
    import numpy as np

    import oracle
    T = p["T"]
    rng = np.random.default_rng(0)
    n = 2
    while True:
        toks = sorted(rng.choice(T, size=min(n, T), replace=False).tolist())
        t0 = time.time()
        oracle.forward_tokens(p, toks, False, clamp)
        dt = time.time() - t0
        if dt >= target_s or n >= T:
            break
        n = min(T, max(n * 2, int(n * target_s / max(dt, 1e-3) * 1.1)))
    idx = p["topk_idx"][toks]
    valid = (idx >= 0) & (idx < p["E"])
    flops = 6.0 * float(valid.sum()) * p["H"] * p["I"]
    log(f"[bench] oracle: {len(toks)} tokens in {dt:.1f}s on {oracle.num_threads()} threads")
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{len(toks)} of {T} tokens (all their top-k slots), per-token oracle path, "
                      f"{dt:.1f} s; whole call extrapolated to {dt * T / len(toks) * 1e6:.0f} us",
            "us_per_call_extrapolated": dt * T / len(toks) * 1e6}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="deepseek_fp8xfp4_T8192_zipf")
    ap.add_argument("--secondary", default="deepseek_fp8xfp4_T128")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-quantize", action="store_true",
                    help="skip the timings of the steps before the forward (quantisation, router)")
    ap.add_argument("--threads", type=int, default=min(16, os.cpu_count() or 8))
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (read + write) a few times, for scaling the "
                         "FETCH_SIZE / WRITE_SIZE counters of a profiler pass")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path (asked for {max(args.gpus, world)} "
              "GPUs). Run with --gpus 1.", file=sys.stderr)
        return 2

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    import torch
    assert torch.cuda.is_available(), "bench.py needs an MI355X"
    torch.cuda.set_device(0)

    if args.copy_calibration:
        n = args.copy_calibration << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 3}), flush=True)
        return 0

    main_r = run_workload(args.workload, args.steps, args.warmup, args.threads, log)
    p = main_r["p"]
    tflops = main_r["flops"] / (main_r["ms"] * 1e-3) / 1e12
    traffic = traffic_from_profiles(args.workload)
    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_r["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3 x e2m1 (e8m0 1x32 scales), fp32 accumulate, bf16 y",
        "data": "synthetic",
        "config": {"workload": args.workload, "T": p["T"], "H": p["H"], "I": p["I"], "E": p["E"], "k": p["k"],
                   "routing": main_r["cfg"].routing, "routed_rows": main_r["R"],
                   "active_experts": main_r["active"]},
        "us_per_call": round(main_r["ms"] * 1e3, 1),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_FP8_TFLOPS, 4), "traffic": traffic,
                     "kernel": "moe_ffn_kernel<2,128>",
                     "work_per_launch": f"{main_r['flops']:.4e} useful flop = 6 * R * H * I"},
    }
    if args.secondary and args.secondary != "none":
        sec = run_workload(args.secondary, args.steps, args.warmup, args.threads, log)
        gbs = sec["bytes"] / (sec["ms"] * 1e-3) / 1e9
        out["secondary"] = {
            "workload": args.secondary, "us_per_call": round(sec["ms"] * 1e3, 1),
            "useful_tflops": round(sec["flops"] / (sec["ms"] * 1e-3) / 1e12, 2),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic_from_profiles(args.secondary),
                         "kernel": "moe_ffn_kernel<2,16>",
                         "work_per_launch": f"{sec['bytes']} algorithmic bytes ({sec['active']} active experts)"}}
    if not args.no_quantize:
        out["quantize"] = run_quantize(p["T"], p["H"], args.steps, args.warmup, log)
        out["router"] = run_router(p["T"], p["H"], p["E"], p["k"], args.steps, args.warmup, log)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(p, main_r["cfg"].clamp, args.cpu_seconds, log)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
