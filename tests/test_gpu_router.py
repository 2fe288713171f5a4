"""Gate + top-k on the GPU (through the C ABI) against the CPU oracle.

The GPU sums the logits in fp32 on the MFMA, the oracle in double, so the
logits agree within the fp32 accumulation bound and the selection is compared
where it is unique: with delta = that bound for the token, every expert the
GPU ranks above another must not be more than 2*delta below it in the exact
logits, and no expert left out may be more than 2*delta above a chosen one.
When the top k+1 exact logits are separated by more than 2*delta this forces
the oracle's exact choice and order.  The weights are compared with the
oracle's formula applied to the GPU's choice."""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_histogram_amd as mf
import oracle
from mixture_experts_ffn_histogram_amd import synth

from gpu_common import log

pytestmark = pytest.mark.gpu

# fp32 accumulation of K/32 MFMA partial sums: each addition rounds once, so
# |error| <= (K/32) * 2^-24 * sum|x*w| <= 2^-16 * sum|x*w| for K <= 8192.
REL = 2.0 ** -16


def run_gpu(x, wg, k):
    dev = torch.device("cuda:0")
    T, H = x.shape
    E = wg.shape[0]
    xd = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev)
    wd = torch.from_numpy(np.ascontiguousarray(wg).view(np.int16)).to(dev)
    logits = torch.full((T, E), float("nan"), dtype=torch.float32, device=dev)
    idx = torch.full((T, k), -7, dtype=torch.int32, device=dev)
    w = torch.full((T, k), float("nan"), dtype=torch.float32, device=dev)
    mf.route_topk(xd, wd, logits, idx, w)
    torch.cuda.synchronize()
    return logits.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()


def check(x, wg, k, gl, gi, gw):
    rl, ri, rw = oracle.route_topk(x, wg, k)
    xf = oracle.bf16_bits_to_f32(x).astype(np.float64)
    wf = oracle.bf16_bits_to_f32(wg).astype(np.float64)
    delta = REL * (np.abs(xf) @ np.abs(wf).T)                      # [T, E] bound per logit
    assert np.all(np.abs(gl.astype(np.float64) - rl) <= delta), "logits outside the fp32 bound"
    T, E = rl.shape
    ambiguous = 0
    for t in range(T):
        d = 2.0 * delta[t].max()
        sel = list(gi[t])
        assert len(set(sel)) == k and all(0 <= e < E for e in sel), (t, sel)
        ls = rl[t, sel]
        # ranked order consistent with the exact logits up to 2*delta
        for i in range(k):
            assert np.all(ls[i] >= ls[i + 1:] - d), (t, sel)
        rest = np.setdiff1d(np.arange(E), sel)
        if len(rest):
            assert rl[t, rest].max() <= ls.min() + d, (t, sel)
        if list(ri[t]) != sel:
            ambiguous += 1
            top = np.sort(rl[t])[::-1][:k + 1]
            assert np.min(np.diff(top[::-1])) <= d, (t, "differs from the oracle although the choice is unique")
        # weights: the oracle's formula on the GPU's choice
        ex = np.exp(ls - ls.max())
        wr = ex / ex.sum()
        assert np.all(np.abs(gw[t].astype(np.float64) - wr) <= 2.0 * d + 4e-7), (t, gw[t], wr)
    return ambiguous


@pytest.mark.parametrize("T,H,E,k", [(64, 256, 8, 2), (512, 2048, 64, 6), (128, 7168, 256, 8),
                                     (300, 384, 40, 5), (37, 128, 18, 3), (1, 64, 512, 64), (129, 640, 16, 16),
                                     # more than 256 experts (32 logits per top-k lane), ragged E, many tokens
                                     (300, 256, 300, 8), (130, 192, 512, 33),
                                     # k = 1 (weight exactly 1) and k = E (every expert, full order)
                                     (200, 256, 20, 1), (70, 128, 24, 24)])
def test_router_matches_oracle(T, H, E, k):
    log(f"router T={T} H={H} E={E} k={k}")
    x = synth.activations_bf16(T, H, seed=T + H)
    wg = synth.router_weights_bf16(E, H, seed=E)
    gl, gi, gw = run_gpu(x, wg, k)
    amb = check(x, wg, k, gl, gi, gw)
    log(f"  tokens whose choice differs inside the fp32 band: {amb}")


def test_router_ties_take_the_lower_id():
    T, H, E, k = 96, 256, 32, 4
    x = synth.activations_bf16(T, H, seed=1)
    wg = synth.router_weights_bf16(E, H, seed=2)
    wg[17] = wg[3]
    wg[30] = wg[3]
    gl, gi, gw = run_gpu(x, wg, k)
    assert np.array_equal(gl[:, 17], gl[:, 3]) and np.array_equal(gl[:, 30], gl[:, 3])
    for t in range(T):
        s = list(gi[t])
        pos = [s.index(e) for e in (3, 17, 30) if e in s]
        assert pos == sorted(pos) and (not pos or pos == list(range(pos[0], pos[0] + len(pos))))
        assert (17 not in s or 3 in s) and (30 not in s or 17 in s)
    check(x, wg, k, gl, gi, gw)


def test_router_full_size_sampled():
    # DeepSeek-V3 router shape at the T=8192 workload: all tokens on the GPU,
    # 512 sampled tokens against the oracle (rows are independent)
    T, H, E, k = 8192, 7168, 256, 8
    log(f"router full size T={T} H={H} E={E} k={k}")
    x = synth.activations_bf16(T, H, seed=8192)
    wg = synth.router_weights_bf16(E, H, seed=256)
    gl, gi, gw = run_gpu(x, wg, k)
    rows = np.sort(np.random.default_rng(0).choice(T, 512, replace=False))
    amb = check(x[rows], wg, k, gl[rows], gi[rows], gw[rows])
    log(f"  sampled tokens whose choice differs inside the fp32 band: {amb}")


def test_router_T0_and_errors():
    dev = torch.device("cuda:0")
    z = lambda *s, dt=torch.float32: torch.zeros(s, dtype=dt, device=dev)
    mf.route_topk(z(0, 64, dt=torch.int16), z(8, 64, dt=torch.int16), z(0, 8), z(0, 2, dt=torch.int32), z(0, 2))
    L = mf.lib()
    assert L.moe_ffn_route_topk(None, None, 4, 96, 8, 2, None, None, None, None) == mf.ERR_UNSUPPORTED
    assert L.moe_ffn_route_topk(None, None, 4, 64, 8, 9, None, None, None, None) == mf.ERR_INVALID_ARG
    assert L.moe_ffn_route_topk(None, None, 4, 64, 8, 2, None, None, None, None) == mf.ERR_INVALID_ARG
