"""Side-stream liveness of the persistent grid (MI355X only).

The scenario of the sglang "Reserve SMs for DeepGEMM MegaMoE grid barriers"
change: another stream holds a few CUs while the MoE call runs.  A helper
kernel takes whole CUs (all 160 KB of their LDS) for 400 ms on a side stream:
2 workgroups (two CUs on two XCDs) or 7 (one CU on seven XCDs; workgroups
are dispatched round-robin over the XCDs).  With the default reserve of 2 the MoE call must
finish, with status OK and the same y as an unobstructed call, while the
helper still runs.  With reserve 0 the outcome is reported (live, blocked
until the helper ends, or timed out): the kernel's two-workgroups-per-CU
footprint is meant to keep it live as well.
"""
import ctypes
import os
import time

import numpy as np
import pytest
import torch

from mixture_experts_ffn_histogram_amd import synth
from gpu_common import Runner, log

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def _side_lib():
    path = os.path.join(HERE, "native", "libmoe_side.so")
    if not os.path.exists(path):
        pytest.fail(f"{path} is missing: run __graft_entry__.build()")
    L = ctypes.CDLL(path)
    L.side_start.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_void_p)]
    L.side_running.argtypes = [ctypes.c_void_p]
    L.side_finish.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_uint32)]
    return L


@pytest.mark.parametrize("blocks", [2, 7])
def test_side_stream_liveness(blocks):
    L = _side_lib()
    cfg = synth.Config("live_fp8xfp4", synth.RECIPE_FP8_FP4, 2048, 1024, 512, 16, 4, "uniform", 9)
    p = synth.make_problem(cfg, threads=8)
    run = Runner(p)
    # a non-blocking stream: the legacy null stream would wait for the helper
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run.run(reserved_cus=2, stream=s)
    s.synchronize()
    assert int(run.status.item()) == 0
    y_ref = run.y.clone()

    results = {}
    for reserve in (2, 0):
        h = ctypes.c_void_p()
        rc = L.side_start(blocks, 400, ctypes.byref(h))
        assert rc == 0, f"side_start failed ({rc})"
        time.sleep(0.02)  # let the helper become resident
        t0 = time.time()
        with torch.cuda.stream(s):
            run.run(reserved_cus=reserve, stream=s)
        s.synchronize()
        dt = time.time() - t0
        still = L.side_running(h)
        xcc = (ctypes.c_uint32 * 7)()
        done = L.side_finish(h, xcc)
        st = int(run.status.item())
        results[reserve] = (dt, still, st)
        log(f"helper on {blocks} CUs (XCDs {list(xcc)[:blocks]}), reserve {reserve}: "
            f"MoE call {dt * 1e3:.1f} ms, helper still running at completion: {still == 1}, status {st}, "
            f"helper workgroups done {done}")
        assert done == blocks
        if reserve == 2:
            assert st == 0, "reserve 2 must complete normally"
            assert still == 1, "the call with reserve 2 waited for the side stream"
            assert torch.equal(run.y, y_ref), "y differs from the unobstructed call"
        else:
            assert st in (0, 2), f"unexpected status {st} with reserve 0"
            if st == 0:
                assert torch.equal(run.y, y_ref)
