"""CPU oracle for the fused MoE expert-FFN forward (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The GPU library never imports, links or calls
it.  It wraps ``moe_oracle.c`` (plain C, double accumulation) through ctypes.

Parity status of each function is recorded next to it; every function here
is pinned by ``tests/test_oracle_pins.py`` (codecs against torch's format
casts and brute-force nearest search, the scale rule by its defining
inequalities, routing by a brute-force sort, the GEMMs by exact rational
arithmetic, the activation by torch's silu, the whole forward by the dense
special case and by invariants).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")

RECIPE_BF16 = 0
RECIPE_FP8_FP8 = 1
RECIPE_FP8_FP4 = 2
RECIPE_FP8_B128 = 3   # e4m3 x e4m3, fp32 scales per 1 x 128 (activations) and 128 x 128 (weights)

OK = 0
BAD_EXPERT_INDEX = 1


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
               "-Wall", "-Wextra", _SRC, "-o", _LIB, "-lm"]
        subprocess.run(cmd, check=True)
    return _LIB


class _Problem(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int64), ("hidden", ctypes.c_int64),
                ("intermediate", ctypes.c_int64), ("num_experts", ctypes.c_int64),
                ("top_k", ctypes.c_int64), ("recipe", ctypes.c_int32),
                ("y_fp32", ctypes.c_int32), ("activation_clamp", ctypes.c_float),
                ("pad_", ctypes.c_int32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        d, u8, u16, i64, f32, P = (ctypes.c_double, ctypes.c_uint8, ctypes.c_uint16,
                                    ctypes.c_int64, ctypes.c_float, ctypes.c_void_p)
        for name, res, args in [
            ("oracle_dec_e4m3", d, [u8]), ("oracle_dec_e2m1", d, [u8]),
            ("oracle_dec_e8m0", d, [u8]), ("oracle_dec_bf16", d, [u16]),
            ("oracle_round_e4m3_sat", d, [d]), ("oracle_enc_e4m3", u8, [d]),
            ("oracle_round_bf16", d, [d]), ("oracle_enc_bf16", u16, [d]),
            ("oracle_scale_exp", ctypes.c_int, [d]), ("oracle_swiglu", f32, [f32, f32, f32]),
            ("oracle_route", ctypes.c_int, [P, i64, i64, i64, P, P, P, P]),
            ("oracle_forward", ctypes.c_int, [P] + [P] * 14),
            ("oracle_forward_tokens", ctypes.c_int, [P] + [P] * 8 + [P, i64, P]),
            ("oracle_forward_tokens_band", ctypes.c_int, [P] + [P] * 8 + [P, i64, P, d, P]),
            ("oracle_forward_tokens_rows", ctypes.c_int, [P] + [P] * 8 + [P, i64, P, d, P, P, P, P]),
            ("oracle_ffn_row", ctypes.c_int, [P, P, P, i64, i64, P, P, P, P, P, P, P, P, P, P, d, P, P, P]),
            ("oracle_num_threads", ctypes.c_int, []),
            ("oracle_quantize_act", ctypes.c_int, [P, i64, i64, P, P]),
            ("oracle_route_topk", ctypes.c_int, [P, P, i64, i64, i64, i64, P, P, P]),
        ]:
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _ptr(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return ctypes.c_void_p(a.ctypes.data)


def _problem(T, H, I, E, k, recipe, y_fp32, clamp):
    return _Problem(int(T), int(H), int(I), int(E), int(k), int(recipe), int(y_fp32), float(clamp), 0)


# ---- scalar codecs (pinned exhaustively / by sweep) ----
def dec_e4m3(b): return lib().oracle_dec_e4m3(int(b))
def dec_e2m1(n): return lib().oracle_dec_e2m1(int(n))
def dec_e8m0(b): return lib().oracle_dec_e8m0(int(b))
def dec_bf16(b): return lib().oracle_dec_bf16(int(b))
def round_e4m3_sat(v): return lib().oracle_round_e4m3_sat(float(v))
def enc_e4m3(v): return lib().oracle_enc_e4m3(float(v))
def round_bf16(v): return lib().oracle_round_bf16(float(v))
def enc_bf16(v): return lib().oracle_enc_bf16(float(v))
def scale_exp(amax): return lib().oracle_scale_exp(float(amax))
def swiglu(g, u, clamp): return lib().oracle_swiglu(float(g), float(u), float(clamp))
def num_threads(): return lib().oracle_num_threads()


def route(topk_idx: np.ndarray, num_experts: int):
    """Routing tables: counts[E], offsets[E+1], row_to_slot[R], slot_to_row[T*k], status."""
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    T, k = idx.shape
    counts = np.zeros(num_experts, np.int32)
    offsets = np.zeros(num_experts + 1, np.int32)
    r2s = np.full(max(T * k, 1), -7, np.int32)
    s2r = np.full(max(T * k, 1), -7, np.int32)
    rc = lib().oracle_route(_ptr(idx), T, k, num_experts, _ptr(counts), _ptr(offsets), _ptr(r2s), _ptr(s2r))
    if rc < 0:
        raise RuntimeError(f"oracle_route failed: {rc}")
    R = int(offsets[-1])
    return counts, offsets, r2s[:R].copy(), s2r[:T * k].copy(), rc


def _args(p):
    return [np.ascontiguousarray(p[n]) if p.get(n) is not None else None
            for n in ("x", "x_sf", "topk_idx", "topk_weights", "w1", "w1_sf", "w2", "w2_sf")]


def forward(p: dict, y_fp32: bool, clamp: float, want_tables: bool = False, want_o: bool = False):
    """Full routed forward.  ``p`` holds the problem arrays (see the synth module).

    Returns y (float32 array, or uint16 bf16 bits when y_fp32 is False) and,
    on request, the routing tables and the per-row L2 outputs (float32 arrays; bf16 values for the
    e4m3 recipes).
    """
    T, H, I, E, k, recipe = p["T"], p["H"], p["I"], p["E"], p["k"], p["recipe"]
    x, x_sf, idx, w, w1, w1_sf, w2, w2_sf = _args(p)
    y = np.zeros((T, H), np.float32 if y_fp32 else np.uint16)
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    r2s = np.zeros(max(T * k, 1), np.int32)
    s2r = np.zeros(max(T * k, 1), np.int32)
    o = np.zeros((max(T * k, 1), H), np.float32) if want_o else None
    prob = _problem(T, H, I, E, k, recipe, y_fp32, clamp)
    rc = lib().oracle_forward(ctypes.byref(prob), _ptr(x), _ptr(x_sf), _ptr(idx), _ptr(w),
                              _ptr(w1), _ptr(w1_sf), _ptr(w2), _ptr(w2_sf), _ptr(y),
                              _ptr(counts), _ptr(offsets), _ptr(r2s), _ptr(s2r), _ptr(o))
    if rc < 0:
        raise RuntimeError(f"oracle_forward failed: {rc}")
    out = {"y": y, "status": rc}
    if want_tables:
        R = int(offsets[-1])
        out.update(counts=counts, offsets=offsets, row_to_slot=r2s[:R].copy(), slot_to_row=s2r[:T * k].copy())
    if want_o:
        out["o"] = o[: int(offsets[-1])]
    return out


def forward_tokens(p: dict, tokens, y_fp32: bool, clamp: float):
    """Per-token forward for the listed tokens (no routing tables)."""
    T, H, I, E, k, recipe = p["T"], p["H"], p["I"], p["E"], p["k"], p["recipe"]
    x, x_sf, idx, w, w1, w1_sf, w2, w2_sf = _args(p)
    toks = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
    y = np.zeros((len(toks), H), np.float32 if y_fp32 else np.uint16)
    prob = _problem(T, H, I, E, k, recipe, y_fp32, clamp)
    rc = lib().oracle_forward_tokens(ctypes.byref(prob), _ptr(x), _ptr(x_sf), _ptr(idx), _ptr(w),
                                     _ptr(w1), _ptr(w1_sf), _ptr(w2), _ptr(w2_sf),
                                     _ptr(toks), len(toks), _ptr(y))
    if rc < 0:
        raise RuntimeError(f"oracle_forward_tokens failed: {rc}")
    return y, rc


def forward_tokens_band(p: dict, tokens, y_fp32: bool, clamp: float, rho: float):
    """Per-token forward plus the allowance of re-quantisation decisions within band rho.

    Returns (y_rows, allow_rows, status): allow_rows[q, n] bounds how far y can
    move when an implementation whose L1 result differs from the exact one by
    a relative rho picks the other grid point (or block exponent) for elements
    that lie that close to a rounding boundary.
    """
    T, H, I, E, k, recipe = p["T"], p["H"], p["I"], p["E"], p["k"], p["recipe"]
    x, x_sf, idx, w, w1, w1_sf, w2, w2_sf = _args(p)
    toks = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
    y = np.zeros((len(toks), H), np.float32 if y_fp32 else np.uint16)
    allow = np.zeros((len(toks), H), np.float64)
    prob = _problem(T, H, I, E, k, recipe, y_fp32, clamp)
    rc = lib().oracle_forward_tokens_band(ctypes.byref(prob), _ptr(x), _ptr(x_sf), _ptr(idx), _ptr(w),
                                          _ptr(w1), _ptr(w1_sf), _ptr(w2), _ptr(w2_sf),
                                          _ptr(toks), len(toks), _ptr(y), float(rho), _ptr(allow))
    if rc < 0:
        raise RuntimeError(f"oracle_forward_tokens_band failed: {rc}")
    return y, allow, rc


def forward_tokens_rows(p: dict, tokens, y_fp32: bool, clamp: float, rho: float):
    """Per-token forward of the listed tokens that also returns, for every slot
    j of listed token q, the re-quantised activation values of that routed row
    (hq[q, j, :]) and the rounding-decision band of each for `rho`
    (delta[q, j, :]), the row's exact L2 sums before their rounding to the
    per-slot output type (ox[q, j, :]) and the contraction-error bound of each
    (oeps[q, j, :], zero for the BF16 recipe); masked slots keep NaN rows.
    Returns (y_rows, hq, delta, ox, oeps, status)."""
    T, H, I, E, k, recipe = p["T"], p["H"], p["I"], p["E"], p["k"], p["recipe"]
    x, x_sf, idx, w, w1, w1_sf, w2, w2_sf = _args(p)
    toks = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
    y = np.zeros((len(toks), H), np.float32 if y_fp32 else np.uint16)
    hq = np.full((len(toks), k, I), np.nan, np.float64)
    delta = np.full((len(toks), k, I), np.nan, np.float64)
    ox = np.full((len(toks), k, H), np.nan, np.float64)
    oeps = np.full((len(toks), k, H), np.nan, np.float64)
    prob = _problem(T, H, I, E, k, recipe, y_fp32, clamp)
    rc = lib().oracle_forward_tokens_rows(ctypes.byref(prob), _ptr(x), _ptr(x_sf), _ptr(idx), _ptr(w),
                                          _ptr(w1), _ptr(w1_sf), _ptr(w2), _ptr(w2_sf),
                                          _ptr(toks), len(toks), _ptr(y), float(rho), _ptr(hq), _ptr(delta),
                                          _ptr(ox), _ptr(oeps))
    if rc < 0:
        raise RuntimeError(f"oracle_forward_tokens_rows failed: {rc}")
    return y, hq, delta, ox, oeps, rc


def ffn_row(p: dict, t: int, e: int, clamp: float, rho: float = 0.0):
    """Intermediates of one routed row: L1 output, activation, re-quantised h, h codes/scales, L2 output
    (fp32 for the BF16 recipe, bf16 values for the e4m3 recipes), its exact sums before that rounding
    and their contraction-error bound for `rho`, and the rounding-decision band of each re-quantised
    element for `rho`."""
    T, H, I, E, k, recipe = p["T"], p["H"], p["I"], p["E"], p["k"], p["recipe"]
    x, x_sf, idx, w, w1, w1_sf, w2, w2_sf = _args(p)
    c = np.zeros(2 * I, np.float32)
    h = np.zeros(I, np.float32)
    hq = np.zeros(I, np.float64)
    codes = np.zeros(I, np.uint16 if recipe == RECIPE_BF16 else np.uint8)
    hsf = np.zeros(I // 32, np.uint8)
    o = np.zeros(H, np.float32)
    delta = np.zeros(I, np.float64)
    ox = np.zeros(H, np.float64)
    oeps = np.zeros(H, np.float64)
    prob = _problem(T, H, I, E, k, recipe, 1, clamp)
    rc = lib().oracle_ffn_row(ctypes.byref(prob), _ptr(x), _ptr(x_sf), int(t), int(e),
                              _ptr(w1), _ptr(w1_sf), _ptr(w2), _ptr(w2_sf),
                              _ptr(c), _ptr(h), _ptr(hq), _ptr(codes), _ptr(hsf), _ptr(o),
                              float(rho), _ptr(delta), _ptr(ox), _ptr(oeps))
    if rc < 0:
        raise RuntimeError(f"oracle_ffn_row failed: {rc}")
    if recipe == RECIPE_FP8_B128:   # one fp32 scale per 1 x 128 block
        hsf = hsf.view(np.float32)
    return {"c": c, "h": h, "hq": hq, "h_codes": codes, "h_sf": hsf, "o": o, "delta": delta, "o_exact": ox,
            "o_eps": oeps}


def quantize_act(x_bits: np.ndarray):
    """Pre-dispatch quantisation of bf16 activations (uint16 bit patterns [T, H], H % 32 == 0):
    returns (e4m3 codes uint8 [T, H], e8m0 scales uint8 [T, H/32])."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    T, H = x.shape
    codes = np.zeros((T, H), np.uint8)
    sf = np.zeros((T, H // 32), np.uint8)
    rc = lib().oracle_quantize_act(_ptr(x), int(T), int(H), _ptr(codes), _ptr(sf))
    if rc < 0:
        raise RuntimeError(f"oracle_quantize_act failed: {rc}")
    return codes, sf


def route_topk(x_bits: np.ndarray, wg_bits: np.ndarray, k: int):
    """Softmax router: x [T, H] and Wg [E, H] bf16 bit patterns -> (logits float64 [T, E],
    topk_idx int32 [T, k], topk_weights float32 [T, k])."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    wg = np.ascontiguousarray(wg_bits, dtype=np.uint16)
    T, H = x.shape
    E = wg.shape[0]
    assert wg.shape[1] == H
    logits = np.zeros((T, E), np.float64)
    idx = np.zeros((T, k), np.int32)
    w = np.zeros((T, k), np.float32)
    rc = lib().oracle_route_topk(_ptr(x), _ptr(wg), int(T), int(H), int(E), int(k), _ptr(logits), _ptr(idx), _ptr(w))
    if rc < 0:
        raise RuntimeError(f"oracle_route_topk failed: {rc}")
    return logits, idx, w


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)
