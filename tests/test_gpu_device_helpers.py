"""The forward's device helpers against the oracle's encoders and their definitions (MI355X only).

The L1 epilogues and the pre-dispatch quantiser write their e4m3 codes with
the hardware pack conversion (`e4m3x4` in the device helpers).  Its codes
must be the oracle's (its round-to-nearest-even saturating rounding, then its
encoder) for every
value the kernels can hand it: every e4m3 value, every midpoint between
neighbouring values and the floats next to it, fp32 denormals, magnitudes in
(448, 464] (the fp32-scale recipe's quotient can pass 448 by an ulp), and
random values over the whole range, uniform and log-uniform.

The L2 epilogues round each slot's result to bf16 with the other pack
conversion (`bf16x2`): its bits must be the oracle's round-to-nearest-even
bf16 for every bf16 value, every midpoint between neighbours and the floats
next to it, fp32 denormals and random finite values below 2^127 (the
results are far from overflow; NaN is not an input).

The L1 epilogues take each 1x32 block's largest magnitude over the four
16-lane rows of a wave with the gfx950 lane-swap moves (`max_over_rows`):
every lane must get the largest of lanes l, l^16, l^32 and l^48.

The block's e8m0 exponent (`block_scale_exp`, read off the fp32 bits with
selects, no branches) must be the oracle's scale rule for every largest
magnitude a block can have: zero, fp32 denormals, each boundary 448 * 2^E of
the clamped range and the floats next to it, mantissas next to 1.75, the
largest finite float, NaN (exponent 0), and random values over the range.
(+infinity is outside: no block of finite products reaches it.)"""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


def conversion_inputs() -> np.ndarray:
    pos = sorted({oracle.dec_e4m3(c) for c in range(0x7F)})           # 0 .. 448, finite codes
    vals = [v for p in pos for v in (p, -p)]
    for a, b in zip(pos[:-1], pos[1:]):
        mid = np.float32(0.5 * (a + b))                                # exact: neighbours differ in 4 bits
        for m in (mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1e30))):
            vals += [float(m), -float(m)]
    vals += list(np.arange(1, 65, dtype=np.uint32).view(np.float32) * 1)   # fp32 denormals
    vals += [448.0 + 0.5 * k for k in range(1, 33)] + [-(448.0 + 0.5 * k) for k in range(1, 33)]
    vals.append(float(np.nextafter(np.float32(448), np.float32(1e30))))
    rng = np.random.default_rng(2024)
    uni = rng.uniform(-448.0, 448.0, 100_000).astype(np.float32)
    log = (np.exp2(rng.uniform(-30.0, 8.7, 100_000)) * rng.choice([-1.0, 1.0], 100_000)).astype(np.float32)
    v = np.concatenate([np.asarray(vals, np.float32), uni, log])
    pad = (-v.size) % 4
    return np.concatenate([v, np.zeros(pad, np.float32)])


def test_e4m3x4_matches_oracle_encoder():
    path = os.path.join(HERE, "native", "libmoe_helpers.so")
    if not os.path.exists(path):
        pytest.fail(f"{path} is missing: build it with mixture_experts_ffn_histogram_amd/build.py build_test_helpers()")
    lib = ctypes.CDLL(path)
    lib.moe_test_e4m3x4.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.moe_test_e4m3x4.restype = ctypes.c_int
    v = conversion_inputs()
    n4 = v.size // 4
    x = torch.from_numpy(v).cuda()
    out = torch.zeros(n4, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    assert lib.moe_test_e4m3x4(x.data_ptr(), out.data_ptr(), n4, stream.cuda_stream) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint8)                             # byte j of dword i = value 4 i + j
    ref = np.fromiter((oracle.enc_e4m3(oracle.round_e4m3_sat(float(a))) for a in v), np.uint8, count=v.size)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, (f"{bad.size} of {v.size} codes differ, first: "
                           + ", ".join(f"{v[i]!r}: gpu 0x{got[i]:02x} oracle 0x{ref[i]:02x}" for i in bad[:6]))


def bf16_inputs() -> np.ndarray:
    bits = np.arange(0x0000, 0x7F80, dtype=np.uint32)                       # every finite non-negative bf16
    vals = (bits << 16).view(np.float32)
    vals = vals[vals < np.float32(2.0 ** 127)]
    nxt = ((bits + 1) << 16).view(np.float32)[: vals.size]
    mid = vals + (nxt - vals) / np.float32(2)                                # exact: 9 significant bits
    mid = mid[np.isfinite(mid)]
    near = np.concatenate([np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(np.inf))])
    den = np.arange(1, 4097, dtype=np.uint32).view(np.float32)               # fp32 denormals
    rng = np.random.default_rng(77)
    rnd = rng.integers(0, 0x7F000000, 200_000, dtype=np.uint32).view(np.float32)
    v = np.concatenate([vals, mid, near, den, rnd])
    v = np.concatenate([v, -v]).astype(np.float32)
    return np.concatenate([v, np.zeros(v.size % 2, np.float32)])


def test_bf16x2_matches_oracle_rounding():
    path = os.path.join(HERE, "native", "libmoe_helpers.so")
    if not os.path.exists(path):
        pytest.fail(f"{path} is missing: build it with mixture_experts_ffn_histogram_amd/build.py build_test_helpers()")
    lib = ctypes.CDLL(path)
    lib.moe_test_bf16x2.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.moe_test_bf16x2.restype = ctypes.c_int
    v = bf16_inputs()
    n2 = v.size // 2
    x = torch.from_numpy(v).cuda()
    out = torch.zeros(n2, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    assert lib.moe_test_bf16x2(x.data_ptr(), out.data_ptr(), n2, stream.cuda_stream) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)                               # half j of dword i = value 2 i + j
    ref = np.fromiter((oracle.enc_bf16(oracle.round_bf16(float(a))) for a in v), np.uint16, count=v.size)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, (f"{bad.size} of {v.size} values differ, first: "
                           + ", ".join(f"{v[i]!r}: gpu 0x{got[i]:04x} oracle 0x{ref[i]:04x}" for i in bad[:6]))


def test_max_over_rows_is_the_four_lane_max():
    path = os.path.join(HERE, "native", "libmoe_helpers.so")
    if not os.path.exists(path):
        pytest.fail(f"{path} is missing: build it with mixture_experts_ffn_histogram_amd/build.py build_test_helpers()")
    lib = ctypes.CDLL(path)
    lib.moe_test_max_over_rows.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.moe_test_max_over_rows.restype = ctypes.c_int
    rng = np.random.default_rng(9)
    v = rng.normal(0.0, 10.0, 256 * 64).astype(np.float32)
    v[::7] = np.abs(v[::7])                                   # ties and signs mixed
    v[5::64] = v[5 ^ 16::64]
    x = torch.from_numpy(v).cuda()
    out = torch.zeros_like(x)
    assert lib.moe_test_max_over_rows(x.data_ptr(), out.data_ptr(), v.size, torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    w = v.reshape(-1, 64)
    lanes = np.arange(64)
    ref = np.maximum.reduce([w[:, lanes ^ d] for d in (0, 16, 32, 48)])
    assert np.array_equal(out.cpu().numpy().reshape(-1, 64), ref)


def test_block_scale_exp_matches_oracle_rule():
    path = os.path.join(HERE, "native", "libmoe_helpers.so")
    if not os.path.exists(path):
        pytest.fail(f"{path} is missing: build it with mixture_experts_ffn_histogram_amd/build.py build_test_helpers()")
    lib = ctypes.CDLL(path)
    lib.moe_test_block_scale_exp.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.moe_test_block_scale_exp.restype = ctypes.c_int
    f32 = np.float32
    vals = [0.0, -0.0, float("nan"), float(np.finfo(f32).max), float(np.finfo(f32).tiny)]
    vals += list(np.arange(1, 65, dtype=np.uint32).view(f32))                  # smallest denormals
    vals += list((np.uint32(0x007FFFFF) - np.arange(64, dtype=np.uint32)).view(f32))  # largest denormals
    for E in range(-140, 120):                                                  # 448 * 2^119 is the last finite one
        b = f32(np.ldexp(448.0, E))                                              # 448 * 2^E (denormal below -133)
        if b == 0:
            continue
        vals += [float(b), float(np.nextafter(b, f32(0))), float(np.nextafter(b, f32(np.inf)))]
    for p in range(-126, 127, 3):                                               # mantissas next to 1.75
        m = f32(np.ldexp(1.75, p))
        vals += [float(np.nextafter(m, f32(0))), float(m), float(np.nextafter(m, f32(np.inf)))]
    rng = np.random.default_rng(77)
    vals += list(np.exp2(rng.uniform(-149.0, 127.9, 50_000)).astype(f32))
    v = np.asarray(vals, f32)
    x = torch.from_numpy(v).cuda()
    out = torch.zeros(v.size, dtype=torch.int32, device="cuda")
    assert lib.moe_test_block_scale_exp(x.data_ptr(), out.data_ptr(), v.size, torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = np.array([oracle.scale_exp(float(a)) for a in v], np.int32)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, (f"{bad.size} of {v.size} differ, first: "
                           + ", ".join(f"{v[i]!r}: gpu {got[i]} oracle {ref[i]}" for i in bad[:6]))
