"""GPU parity of the (1, 128, 128) recipe with fp32 scale factors (MI355X only).

e4m3 activations and weights with one fp32 scale per 1 x 128 activation block
and per 128 x 128 weight block, h re-quantised per 1 x 128 block ("SM90
MegaMoE dev log", Phase-1 entry: the wrapper's recipe (1, 128, 128) with the
float SF path).  Routing bit-exact; y through gpu_common.fp8_parity (fp32 y
within 2e-2 RMS plus the effect of the GPU's in-band re-quantisation
differences, every one checked against the oracle's band; bf16 y the rounding
of the fp32 y); bitwise determinism across grid sizes."""
import numpy as np
import pytest
import torch

from mixture_experts_ffn_histogram_amd import synth
from gpu_common import Runner, check_tables, fp8_parity, log

pytestmark = pytest.mark.gpu

B128 = synth.RECIPE_FP8_B128


@pytest.mark.parametrize("T,H,I,E,k,routing", [
    (77, 384, 256, 5, 3, "softmax"),        # ragged token blocks, 3 / 2 K stages
    (300, 1024, 512, 8, 4, "softmax"),      # several 64-row blocks per expert
    (512, 2048, 768, 64, 6, "uniform"),     # the FP8 x FP8 workload's shape
    (128, 7168, 2048, 16, 8, "softmax"),    # DeepSeek dims, 16 experts
])
def test_block128_parity(T, H, I, E, k, routing):
    cfg = synth.Config(f"b128_T{T}_H{H}_I{I}_E{E}_k{k}", B128, T, H, I, E, k, routing, T + H)
    p = synth.make_problem(cfg, threads=16)
    log(f"(1,128,128) T={T} H={H} I={I} E={E} k={k}")
    run = Runner(p)
    run.run()
    torch.cuda.synchronize()
    assert int(run.status.item()) == 0
    check_tables(run, p, T)
    fp8_parity(run, p, f"(1,128,128) T={T} H={H} I={I} E={E} k={k}")


def test_block128_clamp_and_grid_invariance():
    cfg = synth.Config("b128_clamp", B128, 96, 512, 256, 6, 2, "softmax", 3)
    p = synth.make_problem(cfg, threads=8)
    p["x_sf"] = (p["x_sf"] * np.float32(16.0)).astype(np.float32)   # |L1| >> 7: the clamp engages
    run = Runner(p)
    for c in (7.0, 0.0):
        fp8_parity(run, p, f"(1,128,128) clamp {c}", clamp=c)
    outs = []
    for reserve, cap in [(2, 0), (0, 0), (2, 40), (200, 0)]:
        run.run(reserved_cus=reserve, max_cus=cap)
        torch.cuda.synchronize()
        assert int(run.status.item()) == 0
        outs.append(run.y.clone())
    for o in outs[1:]:
        assert torch.equal(o, outs[0])
