"""Shared helpers of the GPU parity tests: upload a synthetic problem, run the
HIP forward through the C ABI binding, and compare with the CPU oracle."""
from __future__ import annotations

import json
import os
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

    def __init__(self, p: dict, max_tokens: int | None = None, y_fp32: bool | None = None, layout: int | None = None):
        """layout: the weights' storage layout on the device (default: TILED for the e2m1 recipe, the
        production layout, else row-major); the device then holds that one copy of the weights."""
        self.p = p
        self.T = p["T"]
        self.max_tokens = self.T if max_tokens is None else max_tokens
        self.y_fp32 = p["y_fp32"] if y_fp32 is None else y_fp32
        if layout is None:
            layout = mf.WEIGHTS_TILED if p["recipe"] == mf.RECIPE_FP8_FP4 else mf.WEIGHTS_ROW_MAJOR
        self.layout = layout
        self.m = mf.MoeFFN(self.max_tokens, p["H"], p["I"], p["E"], p["k"], p["recipe"], weight_layout=layout)
        self.d = upload(p)
        if p.get("x") is None and p.get("x_bf16") is not None:  # quantised on the fly (quantize_on_the_fly)
            self.d["x"] = torch.empty((p["T"], p["H"]), dtype=torch.uint8, device="cuda")
            self.d["x_sf"] = torch.empty((p["T"], p["H"] // 32), dtype=torch.uint8, device="cuda")
        H, E, k = p["H"], p["E"], p["k"]
        if layout == mf.WEIGHTS_TILED:
            d = self.d
            d["w1"], d["w1_sf"], d["w2"], d["w2_sf"] = mf.tile_weights(d["w1"], d["w1_sf"], d["w2"], d["w2_sf"],
                                                                       E, H, p["I"])
            torch.cuda.synchronize()
        self.y = torch.empty((max(self.max_tokens, 1), H), dtype=torch.float32 if self.y_fp32 else torch.int16,
                             device="cuda")
        self.y32 = self.y if self.y_fp32 else None   # fp32 y of the parity runs (allocated on first use)
        self.counts = torch.empty(E, dtype=torch.int32, device="cuda")
        self.offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
        nslots = max(self.max_tokens * k, 1)
        self.r2s = torch.empty(nslots, dtype=torch.int32, device="cuda")
        self.s2r = torch.empty(nslots, dtype=torch.int32, device="cuda")
        self.status = torch.zeros(1, dtype=torch.int32, device="cuda")

    def run(self, num_tokens: int | None = None, clamp: float | None = None, reserved_cus: int = -1,
            max_cus: int = 0, stream=None, sentinel: bool = True, y32: bool = False):
        """One forward call.  y32: write an fp32 y into self.y32 instead of self.y."""
        T = self.T if num_tokens is None else num_tokens
        if y32 and self.y32 is None:
            self.y32 = torch.empty((max(self.max_tokens, 1), self.p["H"]), dtype=torch.float32, device="cuda")
        y = self.y32 if y32 else self.y
        if sentinel:
            y.fill_(-12345)
            self.r2s.fill_(-7)
            self.s2r.fill_(-7)
        d = self.d
        mf.forward(self.m.problem, self.m.workspace, num_tokens=T, x=d["x"], x_sf=d["x_sf"],
                   topk_idx=d["topk_idx"], topk_weights=d["topk_weights"], w1=d["w1"], w1_sf=d["w1_sf"],
                   w2=d["w2"], w2_sf=d["w2_sf"], y=y,
                   y_dtype=mf.Y_FP32 if (y32 or self.y_fp32) else mf.Y_BF16,
                   activation_clamp=self.p["clamp"] if clamp is None else clamp,
                   reserved_cus=reserved_cus, max_cus=max_cus, expert_counts=self.counts,
                   expert_offsets=self.offsets, row_to_slot=self.r2s, slot_to_row=self.s2r,
                   status=self.status, stream=stream)

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


def quantize_on_the_fly(p: dict, run: "Runner") -> None:
    """x given as bf16 (p["x_bf16"]): the GPU's pre-dispatch quantiser fills the
    runner's device x / x_sf, the oracle's quantiser fills p["x"] / p["x_sf"]
    (the oracle's inputs); the two must agree bit for bit."""
    xb = torch.from_numpy(np.ascontiguousarray(p["x_bf16"]).view(np.int16)).cuda()
    mf.quantize_activations(xb, run.d["x"], run.d["x_sf"])
    q, sf = oracle.quantize_act(p["x_bf16"])
    torch.cuda.synchronize()
    assert np.array_equal(run.d["x"].cpu().numpy(), q), "quantised x differs from the oracle's"
    assert np.array_equal(run.d["x_sf"].cpu().numpy(), sf), "x scales differ from the oracle's"
    p["x"], p["x_sf"] = q, sf


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


# Rounding-decision band of the re-quantisation.  The scaled FP8 MFMA sums
# each 128-element K step with reduced internal precision: measured on gfx950,
# the step result is off by at most 2^-11.5 of the step's largest |product|.
# The oracle's band (oracle/moe_oracle.c, requant_band) bounds every L1
# output's error by RHO times the sum over the steps of their largest
# |product| (plus the fp32 accumulation), carries it through the clamp and
# SwiGLU, and marks each activation that may legitimately be re-quantised to
# another code with the largest change it can take.  RHO = 2^-10.5 is twice
# the measured step error.
RHO = 2.0 ** -10.5

_E4M3 = None
_E2M1 = None


def _codec_tables():
    """Value of every e4m3 byte and every e2m1 nibble, from the oracle's codecs
    (pinned exhaustively against torch's format casts)."""
    global _E4M3, _E2M1
    if _E4M3 is None:
        _E4M3 = np.array([oracle.dec_e4m3(b) for b in range(256)], np.float64)
        _E2M1 = np.array([oracle.dec_e2m1(n) for n in range(16)], np.float64)
    return _E4M3, _E2M1


def w2_abs_cols(p: dict, e: int, cols: np.ndarray) -> np.ndarray:
    """|W2(e, n, i)| for all n < H and i in cols, dequantised: [H, len(cols)] float64."""
    e4, e2 = _codec_tables()
    cols = np.asarray(cols, np.int64)
    if p["recipe"] == synth.RECIPE_FP8_B128:   # fp32 factor per 128 x 128 block
        scale = np.repeat(p["w2_sf"][e][:, cols // 128].astype(np.float64), 128, axis=0)
        return np.abs(e4[p["w2"][e][:, cols]] * scale)
    scale = np.ldexp(1.0, p["w2_sf"][e][:, cols // 32].astype(np.int32) - 127)
    if p["recipe"] == synth.RECIPE_FP8_FP4:
        b = p["w2"][e][:, cols // 2]
        nib = np.where(cols % 2 == 0, b & 15, b >> 4)
        v = e2[nib]
    else:
        v = e4[p["w2"][e][:, cols]]
    return np.abs(v * scale)


def workspace_h_rows(run: "Runner", rows) -> tuple[np.ndarray, np.ndarray]:
    """Re-quantised activation rows of the last call, read from the workspace:
    e4m3 codes [n, I] and e8m0 scales [n, I/32]."""
    v = run.m.view()
    ws = run.m.workspace
    r = torch.as_tensor(np.asarray(rows, np.int64), device=ws.device)
    hb, sb = int(v.h_row_bytes), int(v.h_sf_row_bytes)
    ci = v.h + r[:, None] * hb + torch.arange(hb, device=ws.device)[None, :]
    si = v.h_sf + r[:, None] * sb + torch.arange(sb, device=ws.device)[None, :]
    return ws[ci].cpu().numpy(), ws[si].cpu().numpy()


def h_values(p: dict, codes: np.ndarray, sfs: np.ndarray) -> np.ndarray:
    """Values of one re-quantised row from its e4m3 codes and its scales (e8m0 per 1x32, or one fp32
    factor per 1x128 for the (1, 128, 128) recipe)."""
    e4, _ = _codec_tables()
    if p["recipe"] == synth.RECIPE_FP8_B128:
        return e4[codes] * np.repeat(np.ascontiguousarray(sfs).view(np.float32).astype(np.float64), 128)
    return e4[codes] * np.repeat(np.ldexp(1.0, sfs.astype(np.int32) - 127), 32)


def _b128_codes(h: np.ndarray) -> np.ndarray:
    """e4m3 code values of a row re-quantised with one fp32 factor per 128
    values: s = max(amax / 448, 2^-126), and the largest value is 448 * s."""
    b = h.reshape(-1, 128)
    s = np.maximum(np.abs(b).max(axis=1, keepdims=True) / 448.0, 2.0 ** -126)
    return (b / s).reshape(-1)


def round_bf16(v: np.ndarray) -> np.ndarray:
    """Values rounded to bf16 (8 significant bits, round half to even; subnormal spacing 2^-133;
    no overflow handling: the values here are far from bf16's range limits)."""
    v = np.asarray(v, np.float64)
    _, e = np.frexp(v)                                   # |v| = m 2^e, m in [0.5, 1)
    sp = np.ldexp(1.0, np.maximum(e, -125) - 8)          # spacing at |v|
    return np.rint(v / sp) * sp                          # rint: ties to even; v / sp and the product are exact


def o_rounding_bound(ox: np.ndarray, dev: np.ndarray) -> np.ndarray:
    """How far bf16(g) can lie from bf16(ox) for any g with |g - ox| <= dev (bf16 rounding is
    monotone, so the ends of the interval give the extremes)."""
    r = round_bf16(ox)
    return np.maximum(np.abs(round_bf16(ox + dev) - r), np.abs(round_bf16(ox - dev) - r))


def scan_flips(p: dict, toks, s2r: np.ndarray, codes: np.ndarray, sfs: np.ndarray, hq: np.ndarray,
               delta: np.ndarray, ox: np.ndarray, oeps: np.ndarray) -> tuple[np.ndarray, dict]:
    """Compare the GPU's re-quantised rows with the oracle's, for every valid
    slot of the listed tokens (codes / sfs row n belongs to the n-th valid slot
    in (token, slot) order).  Every value that differs must lie inside the
    oracle's band (|h_gpu - h_ref| <= delta), else the test fails.  Returns the
    allowance on y that the differing values and the rounding of each slot's
    L2 result to bf16 can cause,
        allow[q, n] = sum_j |w[t, j]| * o_rounding_bound(ox_j[n], dev_j[n]),
        dev_j[n] = oeps_j[n] + sum_i |h_gpu - h_ref|_i * |W2(e_j, n, i)|:
    the GPU's L2 sum lies within dev_j of the exact one ox_j (the oracle's
    contraction-error bound plus the flips' effect, the latter summed per
    expert as one product of |W2(e)| with the rows' differences), and both
    sides round their sum to bf16.  Also returns counts: rows,
    re-quantisation flips (an e4m3 code that changed) and
    the 32-element blocks holding one.  With e8m0 scales a changed code shows
    as a value more than 2^-16 apart, finer than any e4m3 step; with one fp32
    factor per 128 values the factor's last bits move every value of a block,
    so there the codes are compared: the block's largest value always holds
    code 448, which gives the factor back exactly (code * s / s is exact)."""
    k, H, E = p["k"], p["H"], p["E"]
    idx, w = p["topk_idx"], p["topk_weights"]
    allow = np.zeros((len(toks), H), np.float64)
    per_expert = {}
    flip_dev = {}
    flips = blocks = nrows = scale_moved = 0
    scale_rel = 0.0
    n = 0
    for q, t in enumerate(toks):
        for j in range(k):
            e = int(idx[t, j])
            if not (0 <= e < E):
                continue
            assert s2r[t * k + j] >= 0
            g = h_values(p, codes[n], sfs[n])
            d = g - hq[q, j]
            bad = np.abs(d) > delta[q, j]
            assert not bad.any(), (f"token {t} slot {j} (expert {e}): {int(bad.sum())} re-quantised values outside "
                                   f"the rounding-decision band, first at i={np.where(bad)[0][:5]}")
            if np.any(d):
                per_expert.setdefault(e, []).append((q, j, np.abs(d)))
            if p["recipe"] == synth.RECIPE_FP8_B128:
                flip = _b128_codes(g) != _b128_codes(hq[q, j])
                sg = np.abs(g.reshape(-1, 128)).max(axis=1)
                sr = np.abs(hq[q, j].reshape(-1, 128)).max(axis=1)
                rel = np.abs(sg - sr) / np.maximum(sr, 2.0 ** -126)
                scale_moved += int((rel > 2.0 ** -16).sum())
                scale_rel = max(scale_rel, float(rel.max()))
            else:
                flip = np.abs(d) > np.abs(hq[q, j]) * 2.0 ** -16
            flips += int(flip.sum())
            blocks += int(np.unique(np.nonzero(flip)[0] // 32).size)
            nrows += 1
            n += 1
    for e, items in per_expert.items():
        D = np.stack([a for _, _, a in items], axis=1)                # [I, rows]
        cols = np.nonzero(D.any(axis=1))[0]
        contrib = w2_abs_cols(p, e, cols) @ D[cols]                    # [H, rows]
        for c, (q, j, _) in enumerate(items):
            flip_dev[(q, j)] = contrib[:, c]
    for q, t in enumerate(toks):
        for j in range(k):
            if not (0 <= int(idx[t, j]) < E):
                continue
            dev = oeps[q, j] + flip_dev[(q, j)] if (q, j) in flip_dev else oeps[q, j]
            allow[q] += abs(float(w[t, j])) * o_rounding_bound(ox[q, j], dev)
    stats = {"rows": nrows, "flips": flips, "flip_blocks": blocks}
    if p["recipe"] == synth.RECIPE_FP8_B128:
        stats.update(scale_moved_blocks=scale_moved, max_scale_rel=scale_rel)
    return allow, stats


def _record(stats: dict) -> None:
    path = os.environ.get("MOE_FFN_PARITY_LOG")
    if path:
        with open(path, "a") as fh:
            fh.write(json.dumps(stats) + "\n")


def collect_gpu(run: "Runner", p: dict, toks, num_tokens: int | None = None, clamp: float | None = None,
                stream=None) -> dict:
    """Run the call twice on the device (fp32 y, then bf16 y when the runner's y
    is bf16) and bring back what the parity check needs: fp32 / bf16 y rows of
    the listed tokens, the re-quantised rows of their valid slots (workspace h /
    h_sf), slot_to_row, the status of both calls and whether the bf16 y is
    bitwise the round-to-nearest-even of the fp32 y over all T rows."""
    T = p["T"] if num_tokens is None else num_tokens
    clamp = p["clamp"] if clamp is None else clamp
    k = p["k"]
    sync = (lambda: stream.synchronize()) if stream is not None else torch.cuda.synchronize
    run.run(num_tokens=T, clamp=clamp, y32=True, stream=stream)
    sync()
    out = {"status32": int(run.status.item())}
    s2r = run.s2r[: T * k].cpu().numpy()
    rows = [int(s2r[t * k + j]) for t in toks for j in range(k) if 0 <= p["topk_idx"][t, j] < p["E"]]
    out["s2r"] = s2r
    out["codes"], out["sfs"] = workspace_h_rows(run, rows) if rows else (None, None)
    ti = torch.as_tensor(np.asarray(toks, np.int64), device=run.y.device)
    out["y32"] = run.y32[ti].cpu().numpy().astype(np.float64)
    if not run.y_fp32:
        run.run(num_tokens=T, clamp=clamp, stream=stream)
        sync()
        out["status16"] = int(run.status.item())
        out["bf16_is_rounding"] = bool(torch.equal(run.y[:T].view(torch.bfloat16), run.y32[:T].to(torch.bfloat16)))
        out["y16"] = run.y[ti].view(torch.bfloat16).float().cpu().numpy().astype(np.float64)
    return out


def check_collected(p: dict, toks, col: dict, what: str, clamp: float | None = None, status: int = 0) -> dict:
    """The oracle side of fp8_parity, on what collect_gpu brought back."""
    clamp = p["clamp"] if clamp is None else clamp
    assert col["status32"] == status, f"{what}: device status {col['status32']}"
    log(f"  {what}: oracle on {len(toks)} tokens")
    ref32, hq, delta, ox, oeps, _ = oracle.forward_tokens_rows(p, toks, True, clamp, RHO)
    ref32 = ref32.astype(np.float64)
    allow, fl = scan_flips(p, toks, col["s2r"], col["codes"], col["sfs"], hq, delta, ox, oeps)
    rms = float(np.sqrt(np.mean(ref32 ** 2))) if ref32.size else 0.0
    d = np.abs(col["y32"] - ref32)
    raw = float(d.max() / rms) if rms > 0 else 0.0
    over = int((d > TOL_FP8 * rms).sum())
    outside = int((d > TOL_FP8 * rms + allow).sum())
    stats = {"what": what, "tokens": len(toks), "rows": fl["rows"], "flips": fl["flips"],
             "flip_blocks": fl["flip_blocks"], "raw_fp32": raw, "beyond_tol_fp32": over,
             "max_allow_over_rms": float(allow.max() / rms) if rms > 0 else 0.0, "elements": int(d.size)}
    for key in ("scale_moved_blocks", "max_scale_rel"):
        if key in fl:
            stats[key] = fl[key]
    if "y16" in col:
        assert col["status16"] == status, f"{what}: device status {col['status16']} (bf16 y)"
        assert col["bf16_is_rounding"], f"{what}: bf16 y is not the rounding of the fp32 y"
        ref16 = torch.from_numpy(ref32.astype(np.float32)).to(torch.bfloat16).float().numpy().astype(np.float64)
        rms16 = float(np.sqrt(np.mean(ref16 ** 2))) if ref16.size else 0.0
        d16 = np.abs(col["y16"] - ref16)
        stats.update(raw_bf16=float(d16.max() / rms16) if rms16 > 0 else 0.0,
                     beyond_tol_bf16=int((d16 > TOL_FP8 * rms16).sum()), differing_bf16=int((d16 > 0).sum()))
    log(f"  {what}: fp32 y max|dy|/rms = {raw:.3e}, beyond {TOL_FP8:g} rms: {over}/{d.size}; "
        f"{fl['flips']} flipped codes in {fl['flip_blocks']} blocks of {fl['rows']} rows "
        f"(max allowance/rms {stats['max_allow_over_rms']:.2e})"
        + (f"; {fl['scale_moved_blocks']} 128-blocks whose scale moved by more than 2^-16 "
           f"(max {fl['max_scale_rel']:.2e})" if "scale_moved_blocks" in fl else "")
        + (f"; bf16 y max|dy|/rms = {stats['raw_bf16']:.3e}, beyond: {stats['beyond_tol_bf16']}, "
           f"differing: {stats['differing_bf16']}" if "raw_bf16" in stats else ""))
    _record(stats)
    assert outside == 0, f"{what}: {outside} y elements outside {TOL_FP8:g} rms + the rounding decisions' allowance"
    return stats


def fp8_parity(run: "Runner", p: dict, what: str, tokens=None, clamp: float | None = None,
               num_tokens: int | None = None, status: int = 0) -> dict:
    """Parity of an FP8-recipe call (the GPU call runs here, twice: fp32 y, then bf16 y).

    * y in fp32: |y_gpu - y_ref| <= TOL_FP8 * RMS(y_ref) + allow per element,
      y_ref the oracle's fp32 y, allow the effect of the re-quantisation flips
      the GPU actually made (scan_flips), each flip checked to lie inside the
      oracle's band.  The raw max|dy| / RMS and the elements beyond the plain
      bound are recorded.
    * y in bf16: bitwise the round-to-nearest-even of the GPU's fp32 y (the
      same fp32 sums, one rounding); its distance to the bf16 rounding of the
      oracle's fp32 y is reported, not asserted.
    `p` describes the call's inputs (its first num_tokens rows are the call's tokens)."""
    T = p["T"] if num_tokens is None else num_tokens
    toks = list(range(T)) if tokens is None else sorted(set(int(t) for t in tokens))
    col = collect_gpu(run, p, toks, T, clamp)
    return check_collected(p, toks, col, what, clamp, status)


def check_tile_rows(run: "Runner", p: dict, rows, what: str, clamp: float | None = None) -> dict:
    """Routed rows of the last call (e.g. one whole token block of an expert,
    i.e. every tile of both GEMM phases that touches it) against the oracle's
    per-row intermediates: each re-quantised value equals the oracle's or lies
    inside its rounding-decision band, and each bf16 L2 output row o satisfies
    |o_gpu - o_ref| <= 2e-2 RMS(o_ref) + o_rounding_bound(o_exact, o_eps +
    the effect of that row's flips)."""
    import concurrent.futures as cf
    clamp = p["clamp"] if clamp is None else clamp
    e4, _ = _codec_tables()
    k = p["k"]
    off = run.offsets.cpu().numpy()
    r2s = run.r2s[: int(off[-1])].cpu().numpy()
    rows = [int(r) for r in rows]
    codes, sfs = workspace_h_rows(run, rows)
    v = run.m.view()
    ws = run.m.workspace
    H = p["H"]
    ri = torch.as_tensor(np.asarray(rows, np.int64), device=ws.device)
    assert int(v.o_row_bytes) == 2 * H, "the e4m3 recipes keep each slot's L2 result in bf16"
    oi = v.o + ri[:, None] * v.o_row_bytes + torch.arange(2 * H, device=ws.device)[None, :]
    o_gpu = ws[oi].view(torch.bfloat16).float().cpu().numpy().astype(np.float64)
    ex = [int(np.searchsorted(off, r, side="right") - 1) for r in rows]

    def one(i):
        return oracle.ffn_row(p, int(r2s[rows[i]]) // k, ex[i], clamp, rho=RHO)

    with cf.ThreadPoolExecutor(min(16, os.cpu_count() or 8)) as pool:
        refs = list(pool.map(one, range(len(rows))))
    o_ref = np.stack([r["o"] for r in refs]).astype(np.float64)
    rms = float(np.sqrt(np.mean(o_ref ** 2)))
    flips = 0
    worst = 0.0
    for i, ref in enumerate(refs):
        g = h_values(p, codes[i], sfs[i])
        d = g - ref["hq"]
        bad = np.abs(d) > ref["delta"]
        assert not bad.any(), f"{what}: row {rows[i]}: {int(bad.sum())} codes outside the band"
        nz = np.nonzero(d)[0]
        dev = ref["o_eps"] + (w2_abs_cols(p, ex[i], nz) @ np.abs(d[nz]) if nz.size else 0.0)
        allow = o_rounding_bound(ref["o_exact"], dev)
        flips += int(nz.size)
        do = np.abs(o_gpu[i] - o_ref[i])
        worst = max(worst, float(do.max() / rms))
        assert np.all(do <= TOL_FP8 * rms + allow), f"{what}: row {rows[i]}: o outside tolerance"
    log(f"  {what}: {len(rows)} rows, {flips} flipped codes, o max|do|/rms = {worst:.3e}")
    _record({"what": what, "rows": len(rows), "flips": flips, "raw_o": worst})
    return {"rows": len(rows), "flips": flips, "raw_o": worst}


def sample_tokens(p: dict, n: int, seed: int, rare_all: bool = True):
    """First and last token, every token of the rarest non-empty expert (two
    when rare_all is False), two of the busiest, then random tokens up to n.
    Returns (tokens, rarest expert, its row count)."""
    T, E = p["T"], p["E"]
    idx = p["topk_idx"]
    rng = np.random.default_rng(seed)
    counts = np.bincount(idx[(idx >= 0) & (idx < E)], minlength=E)
    busiest = int(np.argmax(counts))
    rare = int(np.argmin(np.where(counts > 0, counts, 1 << 30)))
    toks = {0, T - 1}
    hit = np.where((idx == rare).any(axis=1))[0]
    toks.update(int(t) for t in (hit if rare_all else hit[:2]))
    toks.update(int(t) for t in np.where((idx == busiest).any(axis=1))[0][:2])
    while len(toks) < n:
        toks.add(int(rng.integers(T)))
    return sorted(toks), rare, int(counts[rare])


def check_tables(run: "Runner", p: dict, T: int) -> None:
    """Routing outputs of the last call equal the oracle's bit for bit."""
    idx = p["topk_idx"][:T]
    counts, offsets, r2s, s2r, _ = oracle.route(idx, p["E"])
    g_counts, g_off, g_r2s, g_s2r = run.tables(T)
    assert np.array_equal(g_counts, counts)
    assert np.array_equal(g_off, offsets)
    assert np.array_equal(g_r2s, r2s)
    assert np.array_equal(g_s2r, s2r)
