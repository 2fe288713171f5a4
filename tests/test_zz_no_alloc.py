"""The entry point that allocates nothing (moe_ffn_forward_noalloc) against
moe_ffn_forward on the same inputs, through the C ABI (MI355X only).

Two calls in a row on the library's static workspace, the second with a
smaller input, each compared with the ordinary forward on a workspace of its
own: y (fp32 and bf16), the routing tables and the status must be bitwise
equal.  Calls run on a stream of their own (no allocation happens inside the
no-alloc call; the test allocates its buffers beforehand)."""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_histogram_amd as mf
from mixture_experts_ffn_histogram_amd import synth
from gpu_common import Runner, log

pytestmark = pytest.mark.gpu


def _noalloc(run: Runner, T: int, y, y_dtype, counts, offsets, r2s, s2r, status):
    d = run.d
    mf.forward_noalloc(run.m.problem, num_tokens=T, x=d["x"], x_sf=d["x_sf"], topk_idx=d["topk_idx"],
                       topk_weights=d["topk_weights"], w1=d["w1"], w1_sf=d["w1_sf"], w2=d["w2"], w2_sf=d["w2_sf"],
                       y=y, y_dtype=y_dtype, activation_clamp=run.p["clamp"], expert_counts=counts,
                       expert_offsets=offsets, row_to_slot=r2s, slot_to_row=s2r, status=status)


@pytest.mark.parametrize("recipe,H,I,E,k,T1,T2", [
    (synth.RECIPE_FP8_FP4, 1024, 512, 16, 4, 700, 90),     # 128-row tiles, then 32-row wave tiles
    (synth.RECIPE_FP8_FP8, 512, 256, 8, 2, 300, 17),
    (synth.RECIPE_BF16, 256, 128, 8, 2, 64, 5),
])
def test_noalloc_matches_forward_on_two_calls(recipe, H, I, E, k, T1, T2):
    cfg = synth.Config(f"noalloc_r{recipe}", recipe, T1, H, I, E, k, "softmax", 41 + recipe)
    p = synth.make_problem(cfg, threads=8)
    run = Runner(p)   # max_tokens = T1
    dev = torch.device("cuda:0")
    y_dtype = mf.Y_FP32 if run.y_fp32 else mf.Y_BF16
    y = torch.empty_like(run.y)
    counts = torch.empty_like(run.counts)
    offsets = torch.empty_like(run.offsets)
    r2s = torch.empty_like(run.r2s)
    s2r = torch.empty_like(run.s2r)
    status = torch.full((1,), -1, dtype=torch.int32, device=dev)
    for T in (T1, T2):
        log(f"no-alloc recipe {recipe}: T={T} of {T1}")
        run.run(num_tokens=T)
        y.fill_(-12345)
        r2s.fill_(-7)
        s2r.fill_(-7)
        status.fill_(-1)
        _noalloc(run, T, y, y_dtype, counts, offsets, r2s, s2r, status)
        torch.cuda.synchronize()
        assert int(run.status.item()) == 0 and int(status.item()) == 0
        assert torch.equal(y, run.y), f"T={T}: y differs from moe_ffn_forward"
        assert torch.equal(counts, run.counts) and torch.equal(offsets, run.offsets)
        R = int(offsets[-1].item())
        assert torch.equal(r2s[:R], run.r2s[:R]) and torch.equal(s2r[:T * k], run.s2r[:T * k])
        assert bool((y[T:] == -12345).all())
