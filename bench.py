#!/usr/bin/env python3
"""Benchmark of the fused MoE expert-FFN forward on one MI355X.

A step is one call of the whole hot path (routing, L1 GEMM + SwiGLU/clamp/
re-quantisation, L2 GEMM, combine) on one batch of synthetic DeepSeek-V3
shaped input (H=7168, I=2048, E=256, k=8, e4m3 activations x e2m1 weights
with e8m0 1x32 scales).  Inputs are resident in HBM before timing starts;
the weights are held once, in the TILED layout.

Prints ONE JSON line: the headline workload T=8192 with Zipf(1.2) routing and
10% empty experts (MFMA-bound: useful TFLOP/s and fraction of the dense FP8
and MXFP4 MFMA peaks), the kernel's roofline and the CPU oracle timed on a
bounded token sample; beside it the T=128 weight-streaming workload
("secondary", HBM-bound), reserve 0 against reserve 2 at T=8192, T=32768,
the T=8192 call with row-major weights, the BF16 T=64 and FP8 x FP8 T=512
workloads, the pre-dispatch activation quantisation ("quantize") and the
gate + top-k router ("router") of the headline shape.
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
PEAK_MXFP4_TFLOPS = 10100.0  # MI355X dense MXFP4 MFMA
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
    w = {0: 2.0, 1: 1.0, 2: 0.5, 3: 1.0}[p["recipe"]]                  # weight bytes per element
    sf = {0: 0.0, 1: 1 / 32, 2: 1 / 32, 3: 4 / (128 * 128)}[p["recipe"]]  # weight scale bytes per element
    xe = {0: 2.0, 1: 1.0, 2: 1.0, 3: 1.0}[p["recipe"]] + {0: 0.0, 1: 1 / 32, 2: 1 / 32, 3: 4 / 128}[p["recipe"]]
    per_expert = int(3 * I * H * (w + sf))
    per_token = int(H * xe) + k * 8 + H * 2
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


class Workload:
    """One workload's inputs on the device and a forward call enqueuing it.

    The e2m1 weights are held once, in the TILED layout (the production layout),
    unless layout says otherwise; the row-major device copy used to prepare them
    is freed before any timing."""

    def __init__(self, name: str, threads: int, log, layout=None, weights=None, weight_copies: int = 1,
                 device_weights=None):
        import numpy as np
        import torch

        import mixture_experts_ffn_histogram_amd as mf
        from mixture_experts_ffn_histogram_amd import synth

        self.cfg = cfg = synth.CONFIGS[name]
        t0 = time.time()
        p = synth.make_problem(cfg, threads=threads, weights=weights)
        log(f"[bench] {name}: inputs generated in {time.time() - t0:.1f}s")
        self.p = p
        dev = torch.device("cuda:0")
        T, H, I, E, k = p["T"], p["H"], p["I"], p["E"], p["k"]
        if layout is None:
            layout = mf.WEIGHTS_TILED if p["recipe"] == mf.RECIPE_FP8_FP4 else mf.WEIGHTS_ROW_MAJOR
        self.layout = layout
        up = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        self.d = {n: up(p[n]) for n in ("topk_idx", "topk_weights")}
        if p.get("x_bf16") is not None:   # x quantised on the fly: the quantiser runs inside every timed step
            self.x_bf16 = torch.from_numpy(np.ascontiguousarray(p["x_bf16"]).view(np.int16)).to(dev)
            self.d["x"] = torch.empty((T, H), dtype=torch.uint8, device=dev)
            self.d["x_sf"] = torch.empty((T, H // 32), dtype=torch.uint8, device=dev)
        else:
            self.x_bf16 = None
            self.d["x"], self.d["x_sf"] = up(p["x"]), up(p["x_sf"])
        # weight_copies > 1: identical copies used in turn, so that consecutive calls cannot find the
        # weights in the 256 MB Infinity Cache
        self.wsets = [] if device_weights is None else [device_weights]
        for _ in range(weight_copies if device_weights is None else 0):
            w = [up(p[n]) for n in ("w1", "w1_sf", "w2", "w2_sf")]
            if layout == mf.WEIGHTS_TILED:
                w = list(mf.tile_weights(*w, E, H, I))
                torch.cuda.synchronize()
            self.wsets.append(w)
        self.m = mf.MoeFFN(T, H, I, E, k, p["recipe"], device=dev, weight_layout=layout)
        self.y = torch.empty((T, H), dtype=torch.int16, device=dev)
        self.status = torch.zeros(1, dtype=torch.int32, device=dev)
        self.stream = torch.cuda.current_stream()
        self.calls = 0
        idx = p["topk_idx"]
        valid = (idx >= 0) & (idx < E)
        self.R = int(valid.sum())
        self.active = int(len(np.unique(idx[valid])))
        self.flops = 6.0 * self.R * H * I
        self.bytes = algorithmic_bytes(p, self.active)

    def call(self, reserved_cus: int = -1):
        import mixture_experts_ffn_histogram_amd as mf
        d, w = self.d, self.wsets[self.calls % len(self.wsets)]
        self.calls += 1
        if self.x_bf16 is not None:
            mf.quantize_activations(self.x_bf16, d["x"], d["x_sf"], self.stream)
        self.m(num_tokens=self.p["T"], x=d["x"], x_sf=d["x_sf"], topk_idx=d["topk_idx"],
               topk_weights=d["topk_weights"], w1=w[0], w1_sf=w[1], w2=w[2], w2_sf=w[3], y=self.y,
               y_dtype=mf.Y_BF16, activation_clamp=self.cfg.clamp, status=self.status, stream=self.stream,
               reserved_cus=reserved_cus)

    def check(self):
        if int(self.status.item()) != 0:
            raise RuntimeError(f"device status {int(self.status.item())}")

    def time(self, steps: int, warmup: int, reserved_cus: int = -1) -> float:
        """ms per call: `warmup` untimed calls, then `steps` calls between HIP events recorded on the
        stream the calls are enqueued on (synchronised on both sides)."""
        import torch
        for _ in range(warmup):
            self.call(reserved_cus)
        torch.cuda.synchronize()
        self.check()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(self.stream)
        for _ in range(steps):
            self.call(reserved_cus)
        ev1.record(self.stream)
        torch.cuda.synchronize()
        self.check()
        return ev0.elapsed_time(ev1) / steps

    def free(self):
        import torch
        self.d = self.wsets = self.m = self.y = None
        torch.cuda.synchronize()
        torch.cuda.empty_cache()


def run_workload(name: str, steps: int, warmup: int, threads: int, log, **kw):
    w = Workload(name, threads, log, **kw)
    ms = w.time(steps, warmup)
    log(f"[bench] {name}: {ms * 1e3:.1f} us/call, R={w.R}, active experts={w.active}")
    return w, ms


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
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": f"{len(toks)} of {T} tokens (all their top-k slots), per-token oracle path, "
                      f"{dt:.1f} s; whole call extrapolated to {dt * T / len(toks) * 1e6:.0f} us",
            "us_per_call_extrapolated": dt * T / len(toks) * 1e6}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="deepseek_fp8xfp4_T8192_zipf")
    ap.add_argument("--secondary", default="deepseek_fp8xfp4_T128")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-quantize", action="store_true",
                    help="skip the timings of the steps before the forward (quantisation, router)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other workloads (C1, C2, T=32768, row-major layout, reserve A/B)")
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

    import mixture_experts_ffn_histogram_amd as mf
    from mixture_experts_ffn_histogram_amd import synth

    if args.copy_calibration:
        n = args.copy_calibration << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 3}), flush=True)
        return 0

    # ---- headline: the MFMA-bound workload, weights held once in the TILED layout
    main_w, ms = run_workload(args.workload, args.steps, args.warmup, args.threads, log)
    p = main_w.p
    tflops = main_w.flops / (ms * 1e-3) / 1e12
    traffic = traffic_from_profiles(args.workload)
    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3 x e2m1 (e8m0 1x32 scales), fp32 accumulate, bf16 y",
        "data": "synthetic",
        "config": {"workload": args.workload, "T": p["T"], "H": p["H"], "I": p["I"], "E": p["E"], "k": p["k"],
                   "routing": main_w.cfg.routing, "routed_rows": main_w.R, "active_experts": main_w.active,
                   "weight_layout": "tiled (the one device copy of the weights)"},
        "us_per_call": round(ms * 1e3, 1),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_FP8_TFLOPS, 4),
                     "peak_mxfp4": PEAK_MXFP4_TFLOPS, "frac_mxfp4": round(tflops / PEAK_MXFP4_TFLOPS, 4),
                     "traffic": traffic, "kernel": "moe_ffn_kernel<2,128,true>",
                     "work_per_launch": f"{main_w.flops:.4e} useful flop = 6 * R * H * I"},
    }
    if not args.no_extra:
        # the pages' kernel check: reserve 0 against reserve 2, 100 calls each, interleaved in 5 rounds
        r0 = r2 = 0.0
        for _ in range(5):
            r0 += main_w.time(20, 2, reserved_cus=0)
            r2 += main_w.time(20, 2, reserved_cus=2)
        out["reserve_ab"] = {"workload": args.workload, "calls_each": 100,
                             "reserve0_us_per_call": round(r0 / 5 * 1e3, 1),
                             "reserve2_us_per_call": round(r2 / 5 * 1e3, 1)}
        log(f"[bench] reserve 0 / 2: {r0 / 5 * 1e3:.1f} / {r2 / 5 * 1e3:.1f} us/call")
        # T=32768 (same shapes; the headline's device weights)
        c5 = Workload("deepseek_fp8xfp4_T32768_zipf", args.threads, log, weights=synth.weights_of(p),
                      device_weights=main_w.wsets[0])
        ms5 = c5.time(5, 2)
        t5 = c5.flops / (ms5 * 1e-3) / 1e12
        out["T32768"] = {"workload": "deepseek_fp8xfp4_T32768_zipf", "timed_calls": 5,
                         "us_per_call": round(ms5 * 1e3, 1), "useful_tflops": round(t5, 1),
                         "frac_fp8_peak": round(t5 / PEAK_FP8_TFLOPS, 4),
                         "frac_mxfp4_peak": round(t5 / PEAK_MXFP4_TFLOPS, 4), "routed_rows": c5.R,
                         "weights": "the T=8192 workload's (same shapes)"}
        log(f"[bench] T=32768: {ms5 * 1e3:.1f} us/call, {t5:.0f} TFLOP/s")
        c5.wsets = None
        c5.free()
    host_w = synth.weights_of(p)
    main_w.free()
    if not args.no_extra:
        # the same call with the weights row-major (the canonical layout; 64-row token blocks)
        rm = Workload(args.workload, args.threads, log, layout=mf.WEIGHTS_ROW_MAJOR, weights=host_w)
        msr = rm.time(args.steps, args.warmup)
        tr = rm.flops / (msr * 1e-3) / 1e12
        out["row_major_layout"] = {"workload": args.workload, "us_per_call": round(msr * 1e3, 1),
                                   "useful_tflops": round(tr, 1), "frac_fp8_peak": round(tr / PEAK_FP8_TFLOPS, 4)}
        log(f"[bench] {args.workload} row-major weights: {msr * 1e3:.1f} us/call")
        rm.free()
    del host_w
    if args.secondary and args.secondary != "none":
        sec, mss = run_workload(args.secondary, args.steps, args.warmup, args.threads, log)
        gbs = sec.bytes / (mss * 1e-3) / 1e9
        out["secondary"] = {
            "workload": args.secondary, "us_per_call": round(mss * 1e3, 1),
            "useful_tflops": round(sec.flops / (mss * 1e-3) / 1e12, 2),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic_from_profiles(args.secondary),
                         "kernel": "moe_ffn_kernel<2,16,true>",
                         "work_per_launch": f"{sec.bytes} algorithmic bytes ({sec.active} active experts)"}}
        sec.free()
    if not args.no_extra:
        c1 = Workload("bf16_T64_H256_I128_E8_k2", args.threads, log)
        ms1 = c1.time(100, 10)
        out["C1_bf16_T64"] = {"workload": "bf16_T64_H256_I128_E8_k2", "us_per_call": round(ms1 * 1e3, 2),
                              "useful_tflops": round(c1.flops / (ms1 * 1e-3) / 1e12, 3),
                              "bound": "launch latency (25 MFLOP, 1.7 MB)"}
        log(f"[bench] C1: {ms1 * 1e3:.1f} us/call")
        c1.free()
        # two weight copies in turn: 2 x 311 MB do not fit the 256 MB Infinity Cache
        c2 = Workload("fp8xfp8_T512_H2048_I768_E64_k6", args.threads, log, weight_copies=2)
        ms2 = c2.time(100, 10)
        xb, c2.x_bf16 = c2.x_bf16, None       # x already quantised: the forward alone
        ms2f = c2.time(100, 10)
        c2.x_bf16 = xb
        gb2 = c2.bytes / (ms2f * 1e-3) / 1e9
        out["C2_fp8xfp8_T512"] = {"workload": "fp8xfp8_T512_H2048_I768_E64_k6",
                                  "us_per_call_quantise_and_forward": round(ms2 * 1e3, 2),
                                  "us_per_call_forward": round(ms2f * 1e3, 2),
                                  "useful_tflops": round(c2.flops / (ms2f * 1e-3) / 1e12, 1),
                                  "roofline": {"bound": "hbm", "achieved": round(gb2, 1), "peak": PEAK_HBM_GBS,
                                               "unit": "GB/s", "frac": round(gb2 / PEAK_HBM_GBS, 4),
                                               "work_per_launch": f"{c2.bytes} algorithmic bytes"},
                                  "weights": "2 copies used in turn (not cache-resident)"}
        log(f"[bench] C2: {ms2 * 1e3:.1f} us/call quantise + forward, {ms2f * 1e3:.1f} forward, "
            f"{gb2:.0f} GB/s")
        c2.free()
        # the (1, 128, 128) recipe with fp32 scales at the same shape (two weight copies in turn)
        b8 = Workload("fp8block128_T512_H2048_I768_E64_k6", args.threads, log, weight_copies=2)
        msb = b8.time(100, 10)
        gbb = b8.bytes / (msb * 1e-3) / 1e9
        out["block128_fp32_scales_T512"] = {
            "workload": "fp8block128_T512_H2048_I768_E64_k6", "us_per_call": round(msb * 1e3, 2),
            "useful_tflops": round(b8.flops / (msb * 1e-3) / 1e12, 1),
            "roofline": {"bound": "hbm", "achieved": round(gbb, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbb / PEAK_HBM_GBS, 4), "work_per_launch": f"{b8.bytes} algorithmic bytes"},
            "weights": "2 copies used in turn (not cache-resident)"}
        log(f"[bench] (1,128,128) T=512: {msb * 1e3:.1f} us/call, {gbb:.0f} GB/s")
        b8.free()
    if not args.no_quantize:
        out["quantize"] = run_quantize(p["T"], p["H"], args.steps, args.warmup, log)
        out["router"] = run_router(p["T"], p["H"], p["E"], p["k"], args.steps, args.warmup, log)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(p, main_w.cfg.clamp, args.cpu_seconds, log)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
