"""Pins of the oracle's softmax router (gate GEMM -> top-k -> renormalised weights), no GPU.

The logits are checked against torch's float64 matmul of the decoded bf16
operands, the selection against a brute-force sort by (descending logit,
ascending expert id), the weights against torch's softmax over the selected
logits, and the tie rule against experts with identical gate rows.
"""
import numpy as np
import torch

import oracle
from mixture_experts_ffn_histogram_amd import synth


def dec(bits):
    return torch.from_numpy(oracle.bf16_bits_to_f32(bits).astype(np.float64))


def test_logits_selection_and_weights():
    T, H, E, k = 24, 512, 64, 6
    x = synth.activations_bf16(T, H, seed=21)
    wg = synth.router_weights_bf16(E, H, seed=22)
    logits, idx, w = oracle.route_topk(x, wg, k)
    ref = (dec(x) @ dec(wg).T).numpy()
    mag = (dec(x).abs() @ dec(wg).abs().T).numpy()
    assert np.all(np.abs(logits - ref) <= 1e-12 * mag + 1e-300)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-logits[t, e], e))[:k]
        assert list(idx[t]) == order
        sm = torch.softmax(torch.from_numpy(logits[t, order]), dim=0).to(torch.float32).numpy()
        assert np.array_equal(w[t], sm) or np.max(np.abs(w[t] - sm)) <= 2 ** -24
        assert abs(float(w[t].astype(np.float64).sum()) - 1.0) <= k * 2 ** -24
        assert np.all(np.diff(w[t]) <= 0)


def test_ties_take_the_lower_expert_id_and_permutation():
    T, H, E, k = 8, 128, 16, 4
    x = synth.activations_bf16(T, H, seed=3)
    wg = synth.router_weights_bf16(E, H, seed=4)
    wg[9] = wg[2]    # experts 2 and 9 always tie
    wg[12] = wg[5]
    logits, idx, w = oracle.route_topk(x, wg, k)
    for t in range(T):
        s = list(idx[t])
        for a, b in ((2, 9), (5, 12)):
            if a in s and b in s:
                assert s.index(a) + 1 == s.index(b)       # adjacent, lower id first
                assert w[t, s.index(a)] == w[t, s.index(b)]
            else:
                assert b not in s                          # the higher id is never chosen alone
    # relabelling the experts relabels the choice (no ties among the rest here)
    perm = np.random.default_rng(5).permutation(E)
    wg2 = synth.router_weights_bf16(E, H, seed=6)
    l1, i1, w1 = oracle.route_topk(x, wg2, k)
    l2, i2, w2 = oracle.route_topk(x, wg2[perm], k)   # new expert j is old expert perm[j]
    assert np.array_equal(perm[i2], i1)
    assert np.array_equal(w1, w2)
