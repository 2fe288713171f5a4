"""Pins of the oracle's pre-dispatch activation quantisation (no GPU needed).

bf16 activations -> e4m3 codes + one e8m0 scale per 1x32 block.  The oracle
is checked against torch's e4m3 cast, a brute-force nearest search over the
whole e4m3 grid, the scale rule's defining inequalities, blocks built from
known codes (which must come back unchanged), and the special blocks (zeros,
signed zeros, bf16 subnormals, the largest bf16).
"""
import numpy as np
import torch

import oracle
from mixture_experts_ffn_histogram_amd import synth

E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
FINITE_CODES = np.array([c for c in range(256) if not np.isnan(E4M3[c])])


def bits_to_f64(bits):
    return oracle.bf16_bits_to_f32(bits).astype(np.float64)


def f32_to_bf16_bits(a):
    """Round-to-nearest-even fp32 -> bf16 bit patterns (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def test_scale_rule_inequalities_and_torch_cast():
    x = synth.activations_bf16(40, 1024, seed=7)
    codes, sf = oracle.quantize_act(x)
    v = bits_to_f64(x).reshape(40, 32, 32)
    amax = np.abs(v).max(axis=2)
    E = sf.astype(np.int64) - 127
    assert (amax > 0).all()
    # smallest power of two that clips nothing
    assert (amax <= 448.0 * np.exp2(E.astype(np.float64))).all()
    assert (amax > 448.0 * np.exp2(E.astype(np.float64) - 1)).all()
    # codes: torch's round-to-nearest-even e4m3 cast of the exactly scaled values
    scaled = torch.from_numpy((v * np.exp2(-E.astype(np.float64))[:, :, None]).reshape(40, 1024))
    ref = scaled.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)


def test_codes_are_the_nearest_grid_point_by_brute_force():
    rng = np.random.default_rng(3)
    x = f32_to_bf16_bits(rng.standard_normal((4, 64)).astype(np.float32) * np.float32(3.0))
    codes, sf = oracle.quantize_act(x)
    v = bits_to_f64(x)
    for t in range(4):
        for i in range(64):
            E = int(sf[t, i // 32]) - 127
            s = v[t, i] * 2.0 ** -E
            d = np.abs(E4M3[FINITE_CODES] - s)
            best = FINITE_CODES[d == d.min()]
            if len(best) > 1:  # tie: the even mantissa (lowest code bit 0); zero keeps the input's sign
                best = best[(best & 1) == 0]
            if E4M3[best[0]] == 0.0:
                best = np.array([0x80 if np.signbit(s) else 0x00])
            assert codes[t, i] == best[0], (t, i, s)


def test_blocks_built_from_codes_round_trip():
    # each block: codes drawn from the whole grid with the block max fixed at
    # 448 or 256 (so the scale rule must pick exactly E), times 2^E
    rng = np.random.default_rng(11)
    T, nb = 6, 8
    want_codes = rng.choice(FINITE_CODES, size=(T, nb, 32))
    want_E = rng.integers(-100, 100, size=(T, nb))
    want_codes[:, :, 5] = np.where(rng.random((T, nb)) < 0.5, 0x7E, 0x78)  # 448 or 256
    want_codes[:, :, 5] |= (rng.random((T, nb)) < 0.5).astype(np.int64) << 7
    vals = E4M3[want_codes] * np.exp2(want_E.astype(np.float64))[:, :, None]
    x = f32_to_bf16_bits(vals.astype(np.float32).reshape(T, nb * 32))
    assert np.array_equal(bits_to_f64(x), vals.reshape(T, nb * 32))  # exact in bf16
    codes, sf = oracle.quantize_act(x)
    assert np.array_equal(sf.astype(np.int64) - 127, want_E)
    # -0 comes back as code 0x80, +0 as 0x00: compare values and signs
    got = E4M3[codes.reshape(T, nb, 32)]
    assert np.array_equal(got, E4M3[want_codes])
    assert np.array_equal(np.signbit(got), np.signbit(E4M3[want_codes]))


def test_special_blocks():
    H = 32 * 5
    x = np.zeros((1, H), np.uint16)
    x[0, 32:64] = 0x8000                               # block 1: all -0
    x[0, 64:96] = np.arange(1, 33, dtype=np.uint16)    # block 2: bf16 subnormals m * 2^-133
    x[0, 96] = 0x7F7F                                  # block 3: largest finite bf16 and small values
    x[0, 97:128] = f32_to_bf16_bits(np.linspace(-1.0, 1.0, 31, dtype=np.float32))
    x[0, 128:160] = f32_to_bf16_bits(np.full(32, -1e-3, np.float32))  # block 4: constant negative
    codes, sf = oracle.quantize_act(x)
    assert sf[0, 0] == 127 and (codes[0, :32] == 0).all()
    assert sf[0, 1] == 127 and (codes[0, 32:64] == 0x80).all()
    # subnormals: amax = 32 * 2^-133 is far below 448 * 2^-127 -> E clamps at -127;
    # the scaled values m * 2^-6 round like torch's e4m3 cast (exact for m < 16)
    assert sf[0, 2] == 0
    ref = torch.from_numpy(np.arange(1, 33) * 2.0 ** -6).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes[0, 64:96], ref)
    assert np.array_equal(E4M3[codes[0, 64:80]], np.arange(1, 17) * 2.0 ** -6)
    # largest bf16, 1.9921875 * 2^127 = 255 * 2^120: E = 120 (255 <= 448, 127.5 < 224 would
    # allow no smaller E), and 255 rounds to the e4m3 neighbour 256 (grid 16 in [128, 256))
    assert sf[0, 3] == 127 + 120
    assert E4M3[codes[0, 96]] == 256.0
    # constant block: every element is exactly the block max after scaling
    E4 = int(sf[0, 4]) - 127
    assert np.all(E4M3[codes[0, 128:160]] == E4M3[codes[0, 128]])
    assert abs(E4M3[codes[0, 128]] * 2.0 ** E4 - bits_to_f64(x[0, 128:129])[0]) <= 2.0 ** (E4 + 4)


def test_rows_are_independent_and_T0():
    x = synth.activations_bf16(9, 256, seed=5)
    c_all, s_all = oracle.quantize_act(x)
    for t in (0, 4, 8):
        c1, s1 = oracle.quantize_act(x[t:t + 1])
        assert np.array_equal(c1[0], c_all[t]) and np.array_equal(s1[0], s_all[t])
    c0, s0 = oracle.quantize_act(np.zeros((0, 256), np.uint16))
    assert c0.shape == (0, 256) and s0.shape == (0, 8)
