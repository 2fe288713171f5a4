"""Seeded synthetic inputs for the fused MoE expert-FFN forward.

This module draws data only: random codes, scale bytes, routing choices and
routing weights.  It implements none of the forward's arithmetic; element
codes are produced by torch's own format casts (e4m3, bf16) or drawn directly
from a fixed distribution over the 16 E2M1 codes.  Both the GPU tests and the
CPU oracle consume the same arrays.

Recipe (what each tensor looks like):
  * e4m3 tensors (x, FP8 weights): per 1x32 block a scale byte 127 + b + j
    with j in {-1, 0, +1} (probabilities 1/4, 1/2, 1/4); codes = e4m3 cast of N(0, 64^2) clipped to
    +-448, so that code * 2^(b + j) has roughly the target spread
    (b = round(log2(sigma / 64)); sigma = 1 for x, 1/sqrt(fan_in) for weights).
  * E2M1 weights: magnitude index m in 0..7 (values 0, .5, 1, 1.5, 2, 3, 4, 6)
    drawn with probabilities FP4_MAG_PROBS, uniform sign; scale byte per
    block 127 + round(log2(sigma / FP4_STD)) + j, j as for e4m3.
  * bf16 tensors: bf16 cast of N(0, sigma^2).
  * the (1, 128, 128) recipe: e4m3 codes as above; one fp32 scale per
    1 x 128 activation block, 2^u / 64 (u uniform in [-1, 1]), and per
    128 x 128 weight block, sigma / 64 * 2^u (u uniform in [-1/2, 1/2]).
  * x of a config with x_bf16 set (the FP8 x FP8 workload): bf16 N(0, 1),
    quantised on the fly by the pre-dispatch quantiser (e4m3 + e8m0 1x32).
  * routing "softmax": logits N(0,1) [T,E] -> softmax -> top-k (descending)
    -> weights renormalised over the k picks.
  * routing "uniform": k distinct experts per token, uniformly at random;
    weights softmax of k N(0,1) draws.
  * routing "zipf": floor(0.1 E) experts forced empty; the others get
    popularity p ~ rank^-s (s = 1.2) under a random ranking; each token picks
    k distinct experts by Gumbel-top-k on log p; weights softmax of k N(0,1).
"""
from __future__ import annotations

import concurrent.futures as _cf
import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch

RECIPE_BF16 = 0
RECIPE_FP8_FP8 = 1
RECIPE_FP8_FP4 = 2
RECIPE_FP8_B128 = 3
RECIPE_NAMES = {RECIPE_BF16: "bf16", RECIPE_FP8_FP8: "fp8xfp8", RECIPE_FP8_FP4: "fp8xfp4",
                RECIPE_FP8_B128: "fp8_block128"}

# Probability of each E2M1 magnitude index (0, .5, 1, 1.5, 2, 3, 4, 6).
FP4_MAG_PROBS = np.array([0.10, 0.19, 0.18, 0.16, 0.13, 0.15, 0.07, 0.02])
_FP4_MAG_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
FP4_STD = float(np.sqrt((FP4_MAG_PROBS * _FP4_MAG_VALUES ** 2).sum()))


@dataclass(frozen=True)
class Config:
    name: str
    recipe: int
    T: int
    H: int
    I: int
    E: int
    k: int
    routing: str            # "softmax" | "uniform" | "zipf"
    seed: int
    clamp: float = 7.0
    y_fp32: bool = False
    zipf_s: float = 1.2
    empty_frac: float = 0.1
    x_bf16: bool = False    # x drawn as bf16 N(0, 1), to be quantised by the pre-dispatch quantiser
    extra: dict = field(default_factory=dict, compare=False)

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


# The five workloads, and one of the (1, 128, 128) recipe.  Names state what they are.
CONFIGS = {
    "bf16_T64_H256_I128_E8_k2": Config("bf16_T64_H256_I128_E8_k2", RECIPE_BF16, 64, 256, 128, 8, 2,
                                       "softmax", 101, y_fp32=True),
    "fp8xfp8_T512_H2048_I768_E64_k6": Config("fp8xfp8_T512_H2048_I768_E64_k6", RECIPE_FP8_FP8, 512, 2048, 768,
                                             64, 6, "uniform", 202, x_bf16=True),
    "deepseek_fp8xfp4_T128": Config("deepseek_fp8xfp4_T128", RECIPE_FP8_FP4, 128, 7168, 2048, 256, 8,
                                    "softmax", 303),
    "deepseek_fp8xfp4_T8192_zipf": Config("deepseek_fp8xfp4_T8192_zipf", RECIPE_FP8_FP4, 8192, 7168, 2048, 256, 8,
                                          "zipf", 404),
    "deepseek_fp8xfp4_T32768_zipf": Config("deepseek_fp8xfp4_T32768_zipf", RECIPE_FP8_FP4, 32768, 7168, 2048, 256,
                                           8, "zipf", 505),
    # the (1, 128, 128) fp32-scale recipe at the FP8 x FP8 workload's shape
    "fp8block128_T512_H2048_I768_E64_k6": Config("fp8block128_T512_H2048_I768_E64_k6", RECIPE_FP8_B128, 512, 2048,
                                                 768, 64, 6, "uniform", 606),
}

# tensor ids for seed derivation
_TID = {"x": 1, "x_sf": 2, "route": 3, "w1": 4, "w1_sf": 5, "w2": 6, "w2_sf": 7}


def _rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def _e4m3_codes(rng: np.random.Generator, shape) -> np.ndarray:
    v = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(64.0)
    np.clip(v, -448.0, 448.0, out=v)
    return torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _bf16_bits(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    v = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(sigma)
    return torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


_JITTER = np.array([-1, 0, 1, 0], np.int16)   # two random bits -> -1, 0, +1 with probabilities 1/4, 1/2, 1/4


def _scale_bytes(rng: np.random.Generator, shape, base_exp: int) -> np.ndarray:
    n = int(np.prod(shape))
    u = rng.bit_generator.random_raw((n + 7) // 8).view(np.uint8)[:n]
    return (127 + base_exp + _JITTER[u & 3]).astype(np.uint8).reshape(shape)


def _fp4_byte_table() -> np.ndarray:
    """uint16 random -> one byte holding two E2M1 codes drawn from FP4_MAG_PROBS."""
    cdf = np.cumsum(FP4_MAG_PROBS)
    u = (np.arange(128) + 0.5) / 128.0
    mag = np.searchsorted(cdf, u, side="right").clip(0, 7)         # 7 random bits -> magnitude index
    # E2M1 code of magnitude index m is m itself (exponent/mantissa bits in order); bit 3 is the sign
    nib = np.concatenate([mag, mag | 8]).astype(np.uint8)           # 8th random bit -> sign
    lo = nib[np.arange(65536) & 255]
    hi = nib[np.arange(65536) >> 8]
    return (lo | (hi << 4)).astype(np.uint8)


_FP4_TABLE = None


def _fp4_packed(rng: np.random.Generator, shape_bytes) -> np.ndarray:
    global _FP4_TABLE
    if _FP4_TABLE is None:
        _FP4_TABLE = _fp4_byte_table()
    n = int(np.prod(shape_bytes))
    u = rng.bit_generator.random_raw((n + 3) // 4).view(np.uint16)[:n]
    return _FP4_TABLE[u].reshape(shape_bytes)


def _weights(cfg: Config, which: str, rows: int, K: int, threads: int):
    """Weights [E, rows, K] (K = contraction) in the recipe's storage format."""
    E = cfg.E
    sigma = 1.0 / math.sqrt(K)
    tid, tid_sf = _TID[which], _TID[which + "_sf"]
    if cfg.recipe == RECIPE_BF16:
        w = np.empty((E, rows, K), np.uint16)
        sf = None
    elif cfg.recipe == RECIPE_FP8_B128:
        w = np.empty((E, rows, K), np.uint8)
        sf = np.empty((E, rows // 128, K // 128), np.float32)
    elif cfg.recipe == RECIPE_FP8_FP8:
        w = np.empty((E, rows, K), np.uint8)
        sf = np.empty((E, rows, K // 32), np.uint8)
    else:
        w = np.empty((E, rows, K // 2), np.uint8)
        sf = np.empty((E, rows, K // 32), np.uint8)

    def one(e):
        rng = _rng(cfg.seed, tid, e)
        if cfg.recipe == RECIPE_BF16:
            w[e] = _bf16_bits(rng, (rows, K), sigma)
            return
        rs = _rng(cfg.seed, tid_sf, e)
        if cfg.recipe == RECIPE_FP8_B128:
            w[e] = _e4m3_codes(rng, (rows, K))
            sf[e] = (sigma / 64.0 * np.exp2(rs.uniform(-0.5, 0.5, size=(rows // 128, K // 128)))).astype(np.float32)
        elif cfg.recipe == RECIPE_FP8_FP8:
            w[e] = _e4m3_codes(rng, (rows, K))
            sf[e] = _scale_bytes(rs, (rows, K // 32), int(round(math.log2(sigma / 64.0))))
        else:
            w[e] = _fp4_packed(rng, (rows, K // 2))
            sf[e] = _scale_bytes(rs, (rows, K // 32), int(round(math.log2(sigma / FP4_STD))))

    if threads > 1 and E > 1:
        with _cf.ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, range(E)))
    else:
        for e in range(E):
            one(e)
    return w, sf


def _softmax_rows(z: np.ndarray) -> np.ndarray:
    return torch.softmax(torch.from_numpy(np.ascontiguousarray(z, dtype=np.float32)), dim=-1).numpy()


def routing(cfg: Config, T: int | None = None):
    """topk_idx [T,k] int32 and topk_weights [T,k] float32 for the config's routing law."""
    T = cfg.T if T is None else T
    E, k = cfg.E, cfg.k
    rng = _rng(cfg.seed, _TID["route"], T)
    if cfg.routing == "softmax":
        logits = rng.standard_normal(size=(T, E), dtype=np.float32)
        probs = torch.softmax(torch.from_numpy(logits), dim=-1)
        top = torch.topk(probs, k, dim=-1, largest=True, sorted=True)
        w = top.values / top.values.sum(dim=-1, keepdim=True)
        return top.indices.numpy().astype(np.int32), w.numpy().astype(np.float32)
    if cfg.routing == "uniform":
        keys = rng.random(size=(T, E))
        idx = np.argsort(keys, axis=1, kind="stable")[:, :k].astype(np.int32)
        w = _softmax_rows(rng.standard_normal(size=(T, k), dtype=np.float32))
        return idx, w.astype(np.float32)
    if cfg.routing == "zipf":
        n_empty = int(math.floor(cfg.empty_frac * E))
        perm = rng.permutation(E)
        active = perm[n_empty:]                      # perm[:n_empty] are forced empty
        ranks = np.arange(1, len(active) + 1, dtype=np.float64)
        logp = -cfg.zipf_s * np.log(ranks)            # popularity of active[i] ~ (i+1)^-s
        g = rng.gumbel(size=(T, len(active)))
        scores = logp[None, :] + g
        pick = np.argpartition(-scores, k - 1, axis=1)[:, :k]
        order = np.take_along_axis(scores, pick, axis=1).argsort(axis=1)[:, ::-1]
        pick = np.take_along_axis(pick, order, axis=1)
        idx = active[pick].astype(np.int32)
        w = _softmax_rows(rng.standard_normal(size=(T, k), dtype=np.float32))
        return idx, w.astype(np.float32)
    raise ValueError(f"unknown routing {cfg.routing!r}")


def activations(cfg: Config, T: int | None = None):
    """x [T,H] codes and x_sf [T,H/32] (None for bf16; both None when the
    config draws bf16 x for on-the-fly quantisation: see x_bf16_of)."""
    T = cfg.T if T is None else T
    H = cfg.H
    rng = _rng(cfg.seed, _TID["x"], T)
    if cfg.recipe == RECIPE_BF16:
        return _bf16_bits(rng, (T, H), 1.0), None
    if cfg.x_bf16:
        return None, None
    x = _e4m3_codes(rng, (T, H))
    if cfg.recipe == RECIPE_FP8_B128:
        u = _rng(cfg.seed, _TID["x_sf"], T).uniform(-1.0, 1.0, size=(T, H // 128))
        return x, (np.exp2(u) / 64.0).astype(np.float32)
    x_sf = _scale_bytes(_rng(cfg.seed, _TID["x_sf"], T), (T, H // 32), int(round(math.log2(1.0 / 64.0))))
    return x, x_sf


def x_bf16_of(cfg: Config, T: int | None = None) -> np.ndarray:
    """x ~ N(0, 1) as bf16 bit patterns [T, H] (configs whose x is quantised on the fly)."""
    T = cfg.T if T is None else T
    return _bf16_bits(_rng(cfg.seed, _TID["x"], T, 16), (T, cfg.H), 1.0)


def activations_bf16(T: int, H: int, seed: int) -> np.ndarray:
    """bf16 activations [T, H] (uint16 bit patterns) for the pre-dispatch quantisation:
    N(0, 1) rows times a per-token log-normal gain (sigma 1), with one element
    in 500 boosted 16x (outlier channels), so blocks span a wide range of scales."""
    rng = _rng(seed, _TID["x"], T, H)
    v = rng.standard_normal(size=(T, H), dtype=np.float32)
    v *= np.exp(rng.standard_normal(size=(T, 1))).astype(np.float32)
    v[rng.random(size=(T, H)) < 0.002] *= np.float32(16.0)
    return torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def router_weights_bf16(E: int, H: int, seed: int) -> np.ndarray:
    """Router (gate) weights Wg [E, H] as bf16 bit patterns, N(0, 1/H): with N(0, 1)
    activations the logits are about N(0, 1) (the configs' softmax-top-k routing)."""
    return _bf16_bits(_rng(seed, 101, E, H), (E, H), 1.0 / math.sqrt(H))


def make_problem(cfg: Config, T: int | None = None, threads: int = 8, weights=None) -> dict:
    """All inputs of one forward call as numpy arrays (plus the dims)."""
    T = cfg.T if T is None else T
    x, x_sf = activations(cfg, T)
    idx, w = routing(cfg, T)
    if weights is None:
        w1, w1_sf = _weights(cfg, "w1", 2 * cfg.I, cfg.H, threads)
        w2, w2_sf = _weights(cfg, "w2", cfg.H, cfg.I, threads)
    else:
        w1, w1_sf, w2, w2_sf = weights
    return {"name": cfg.name, "T": T, "H": cfg.H, "I": cfg.I, "E": cfg.E, "k": cfg.k, "recipe": cfg.recipe,
            "x": x, "x_sf": x_sf, "x_bf16": x_bf16_of(cfg, T) if cfg.x_bf16 else None,
            "topk_idx": idx, "topk_weights": w,
            "w1": w1, "w1_sf": w1_sf, "w2": w2, "w2_sf": w2_sf,
            "clamp": cfg.clamp, "y_fp32": cfg.y_fp32}


def weights_of(p: dict):
    return p["w1"], p["w1_sf"], p["w2"], p["w2_sf"]


def with_inputs(p: dict, cfg: Config, seed: int) -> dict:
    """Same weights, fresh x / topk drawn from another seed (for replay checks)."""
    c2 = cfg.with_(seed=seed)
    x, x_sf = activations(c2, p["T"])
    idx, w = routing(c2, p["T"])
    q = dict(p)
    q.update(x=x, x_sf=x_sf, x_bf16=x_bf16_of(c2, p["T"]) if c2.x_bf16 else None, topk_idx=idx, topk_weights=w)
    return q
