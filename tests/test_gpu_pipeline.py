"""The three calls chained on the GPU: router -> pre-dispatch quantisation ->
fused forward, from bf16 activations to y, against the oracle chain.

Every intermediate the GPU hands on is checked before the next step uses it:
the top-k choice where it is unique (the router test's criterion), the codes
and scales bit for bit, then y of the forward fed with the GPU's own routing
and codes against the oracle forward on the same inputs (gpu_common.fp8_parity)."""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_histogram_amd as mf
import oracle
from mixture_experts_ffn_histogram_amd import synth

from gpu_common import Runner, fp8_parity, log
from test_gpu_router import check as check_router

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,H,I,E,k", [(64, 512, 256, 16, 4), (300, 1024, 512, 32, 8)])
def test_router_quantize_forward_chain(T, H, I, E, k):
    log(f"pipeline T={T} H={H} I={I} E={E} k={k}")
    dev = torch.device("cuda:0")
    xb = synth.activations_bf16(T, H, seed=T + 1)
    wg = synth.router_weights_bf16(E, H, seed=E + 1)
    xd = torch.from_numpy(xb.view(np.int16)).to(dev)
    wd = torch.from_numpy(wg.view(np.int16)).to(dev)
    logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    q = torch.empty((T, H), dtype=torch.uint8, device=dev)
    sf = torch.empty((T, H // 32), dtype=torch.uint8, device=dev)
    mf.route_topk(xd, wd, logits, idx, w)
    mf.quantize_activations(xd, q, sf)
    torch.cuda.synchronize()
    gi, gw = idx.cpu().numpy(), w.cpu().numpy()
    check_router(xb, wg, k, logits.cpu().numpy(), gi, gw)
    rq, rsf = oracle.quantize_act(xb)
    assert np.array_equal(q.cpu().numpy(), rq) and np.array_equal(sf.cpu().numpy(), rsf)

    # the forward on the GPU's routing and codes (weights: the seeded e2m1 set of this shape)
    cfg = synth.Config(f"pipeline_T{T}", synth.RECIPE_FP8_FP4, T, H, I, E, k, "softmax", T + 2)
    p = synth.make_problem(cfg, threads=8)
    p.update(x=rq, x_sf=rsf, topk_idx=np.ascontiguousarray(gi), topk_weights=np.ascontiguousarray(gw))
    run = Runner(p)
    fp8_parity(run, p, f"pipeline T={T}")
