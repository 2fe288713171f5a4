"""Shared helpers of the GPU parity tests: upload a synthetic problem, run the
HIP forward through the C ABI binding, and compare with the CPU oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import mixture_experts_ffn_histogram_amd as mf
import oracle
from mixture_experts_ffn_histogram_amd import synth

# Bounds on y, relative to RMS(y_ref) over the call's rows.
TOL_FP8 = 2e-2
TOL_BF16 = 5e-3


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def _t(a, dev):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(dev)


def upload(p: dict, dev="cuda") -> dict:
    return {n: _t(p[n], dev) for n in ("x", "x_sf", "topk_idx", "topk_weights", "w1", "w1_sf", "w2", "w2_sf")}


def upload_inputs(p: dict, d: dict) -> None:
    """Copy fresh x / topk of `p` into the existing device tensors of `d` (graph replay)."""
    for n in ("x", "x_sf", "topk_idx", "topk_weights"):
        if p[n] is None:
            continue
        a = np.ascontiguousarray(p[n])
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        d[n].copy_(torch.from_numpy(a))


class Runner:
    """One problem shape, its workspace and output buffers on the device."""

    def __init__(self, p: dict, max_tokens: int | None = None, y_fp32: bool | None = None, kmajor: bool = True):
        self.p = p
        self.T = p["T"]
        self.max_tokens = self.T if max_tokens is None else max_tokens
        self.y_fp32 = p["y_fp32"] if y_fp32 is None else y_fp32
        self.m = mf.MoeFFN(self.max_tokens, p["H"], p["I"], p["E"], p["k"], p["recipe"])
        self.d = upload(p)
        H, E, k = p["H"], p["E"], p["k"]
        # K-major weight-scale copies and tiled weights (the 128-row tiles need them; other tiles
        # ignore them)
        self.km = (None, None)
        self.wt = (None, None)
        if kmajor and p["recipe"] == mf.RECIPE_FP8_FP4:
            self.km = mf.kmajor_weight_scales(self.d["w1_sf"], self.d["w2_sf"], E, H, p["I"])
            self.wt = mf.tiled_weights(self.d["w1"], self.d["w2"], E, H, p["I"])
        self.y = torch.empty((max(self.max_tokens, 1), H), dtype=torch.float32 if self.y_fp32 else torch.int16,
                             device="cuda")
        self.counts = torch.empty(E, dtype=torch.int32, device="cuda")
        self.offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
        nslots = max(self.max_tokens * k, 1)
        self.r2s = torch.empty(nslots, dtype=torch.int32, device="cuda")
        self.s2r = torch.empty(nslots, dtype=torch.int32, device="cuda")
        self.status = torch.zeros(1, dtype=torch.int32, device="cuda")

    def run(self, num_tokens: int | None = None, clamp: float | None = None, reserved_cus: int = -1,
            max_cus: int = 0, stream=None, sentinel: bool = True):
        T = self.T if num_tokens is None else num_tokens
        if sentinel:
            self.y.fill_(-12345)
            self.r2s.fill_(-7)
            self.s2r.fill_(-7)
        d = self.d
        mf.forward(self.m.problem, self.m.workspace, num_tokens=T, x=d["x"], x_sf=d["x_sf"],
                   topk_idx=d["topk_idx"], topk_weights=d["topk_weights"], w1=d["w1"], w1_sf=d["w1_sf"],
                   w2=d["w2"], w2_sf=d["w2_sf"], y=self.y,
                   y_dtype=mf.Y_FP32 if self.y_fp32 else mf.Y_BF16,
                   activation_clamp=self.p["clamp"] if clamp is None else clamp,
                   reserved_cus=reserved_cus, max_cus=max_cus, expert_counts=self.counts,
                   expert_offsets=self.offsets, row_to_slot=self.r2s, slot_to_row=self.s2r,
                   status=self.status, stream=stream, w1_sf_kmajor=self.km[0], w2_sf_kmajor=self.km[1],
                   w1_tiled=self.wt[0], w2_tiled=self.wt[1])

    def y_float(self, T=None) -> np.ndarray:
        T = self.T if T is None else T
        y = self.y[:T].cpu().numpy()
        if self.y_fp32:
            return y.astype(np.float64)
        return oracle.bf16_bits_to_f32(y.view(np.uint16)).astype(np.float64)

    def tables(self, T=None):
        T = self.T if T is None else T
        k = self.p["k"]
        off = self.offsets.cpu().numpy()
        R = int(off[-1])
        return (self.counts.cpu().numpy(), off, self.r2s[:R].cpu().numpy(), self.s2r[:T * k].cpu().numpy())


def oracle_y(p: dict, y_fp32: bool, clamp: float, tokens=None) -> np.ndarray:
    if tokens is None:
        y = oracle.forward(p, y_fp32, clamp)["y"]
    else:
        y, _ = oracle.forward_tokens(p, tokens, y_fp32, clamp)
    if y_fp32:
        return y.astype(np.float64)
    return oracle.bf16_bits_to_f32(y).astype(np.float64)


def rel_err(y_gpu: np.ndarray, y_ref: np.ndarray) -> tuple[float, float]:
    rms = float(np.sqrt(np.mean(y_ref ** 2))) if y_ref.size else 0.0
    err = float(np.max(np.abs(y_gpu - y_ref))) if y_ref.size else 0.0
    return err / rms if rms > 0 else err, rms


def tol_for(recipe: int) -> float:
    return TOL_BF16 if recipe == synth.RECIPE_BF16 else TOL_FP8


# Rounding-decision band for the parity checks: the scaled FP8 MFMA sums each
# 128-element step with reduced internal precision (measured on gfx950: at
# most 2^-11.5 of the largest product of the step), so the kernel's L1 outputs
# differ from the exact ones by ~1e-5 of the row's RMS.  A code whose exact
# activation lies within RHO * RMS(L1 row) * sensitivity of a rounding
# midpoint may legitimately land on either neighbour; the oracle turns this
# band into a per-element allowance on y.  RHO is ~7x the largest distance
# to the midpoint observed at a flipped code.
RHO = 2.0 ** -12


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of the bf16 grid at |v| (8 significant bits; subnormal floor 2^-133)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.ldexp(1.0, (np.maximum(e, -126) - 7).astype(np.int32)), np.ldexp(1.0, -133))


def oracle_y_band(p: dict, y_fp32: bool, clamp: float, tokens=None):
    """Oracle y and the per-element allowance: the re-quantisation band and,
    for a bf16 y, one bf16 step at the value (the kernel's fp32 sum and the
    exact one may straddle a bf16 rounding midpoint)."""
    toks = list(range(p["T"])) if tokens is None else list(tokens)
    y, allow, _ = oracle.forward_tokens_band(p, toks, y_fp32, clamp, RHO)
    yf = y.astype(np.float64) if y_fp32 else oracle.bf16_bits_to_f32(y).astype(np.float64)
    if not y_fp32:
        allow = allow + bf16_ulp(yf)
    return yf, allow


def assert_y_parity(y_gpu: np.ndarray, y_ref: np.ndarray, allow: np.ndarray, tol: float, what: str = ""):
    rms = float(np.sqrt(np.mean(y_ref ** 2))) if y_ref.size else 0.0
    d = np.abs(y_gpu - y_ref)
    bound = tol * rms + allow
    raw = float(d.max() / rms) if rms > 0 else 0.0
    over = int((d > tol * rms).sum())
    log(f"  {what} max|dy|/rms = {raw:.3e}  elements beyond {tol:g} rms: {over} (all within their allowance: "
        f"{bool(np.all(d <= bound))})  max allowance/rms = {float(allow.max() / rms) if rms > 0 else 0:.3e}")
    assert np.all(d <= bound), f"{what}: {int((d > bound).sum())} elements outside tol*rms + allowance"
    return raw


def assert_h_decisions(run: "Runner", p: dict, rows, clamp: float):
    """GPU re-quantised activations (workspace h / h_sf) against the oracle's, row by row."""
    if p["recipe"] == synth.RECIPE_BF16:
        return 0
    v = run.m.view()
    ws = run.m.workspace
    off = run.offsets.cpu().numpy()
    r2s = run.r2s[: int(off[-1])].cpu().numpy()
    I = p["I"]
    dec = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    flips = 0
    for r in rows:
        r = int(r)
        e = int(np.searchsorted(off, r, side="right") - 1)
        t = int(r2s[r]) // p["k"]
        row = oracle.ffn_row(p, t, e, clamp, rho=RHO)
        hb = ws[v.h + r * v.h_row_bytes: v.h + (r + 1) * v.h_row_bytes].cpu().numpy()
        sfb = ws[v.h_sf + r * v.h_sf_row_bytes: v.h_sf + (r + 1) * v.h_sf_row_bytes].cpu().numpy()
        g_val = dec[hb] * np.repeat(np.ldexp(1.0, sfb.astype(np.int32) - 127), 32)
        diff = np.abs(g_val - row["hq"])
        bad = diff > row["delta"]
        assert not bad.any(), f"row {r}: {int(bad.sum())} codes outside the band (first at {np.where(bad)[0][:5]})"
        flips += int((diff > 0).sum())
    return flips


def check_tables(run: "Runner", p: dict, T: int) -> None:
    """Routing outputs of the last call equal the oracle's bit for bit."""
    idx = p["topk_idx"][:T]
    counts, offsets, r2s, s2r, _ = oracle.route(idx, p["E"])
    g_counts, g_off, g_r2s, g_s2r = run.tables(T)
    assert np.array_equal(g_counts, counts)
    assert np.array_equal(g_off, offsets)
    assert np.array_equal(g_r2s, r2s)
    assert np.array_equal(g_s2r, s2r)
