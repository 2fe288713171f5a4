"""One side-stream liveness scenario in a fresh process (run by test_gpu_liveness.py).

HIP maps streams onto a few hardware queues (four by default).  Two streams
that share a queue execute in order, so a MoE call queued behind the helper
kernel would wait for it whatever the kernel's footprint.  In a fresh process
the helper's stream and the MoE stream, created one after the other, get
queues of their own; inside a long test session they may not.

Usage: python liveness_case.py BLOCKS.  Prints one JSON line per reserve.
"""
import ctypes
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import torch  # noqa: E402

from mixture_experts_ffn_histogram_amd import synth  # noqa: E402
from gpu_common import Runner  # noqa: E402


def main(blocks: int) -> int:
    path = os.path.join(HERE, "native", "libmoe_side.so")
    L = ctypes.CDLL(path)
    L.side_start.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_void_p)]
    L.side_running.argtypes = [ctypes.c_void_p]
    L.side_finish.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_uint32)]
    torch.cuda.set_device(0)
    cfg = synth.Config("live_fp8xfp4", synth.RECIPE_FP8_FP4, 2048, 1024, 512, 16, 4, "uniform", 9)
    p = synth.make_problem(cfg, threads=8)
    run = Runner(p)
    s = torch.cuda.Stream()  # non-blocking: the legacy null stream would wait for the helper
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run.run(reserved_cus=2, stream=s)
    s.synchronize()
    if int(run.status.item()) != 0:
        print(json.dumps({"error": f"unobstructed call status {int(run.status.item())}"}), flush=True)
        return 1
    y_ref = run.y.clone()
    for reserve in (2, 0):
        h = ctypes.c_void_p()
        rc = L.side_start(blocks, 400, ctypes.byref(h))
        if rc != 0:
            print(json.dumps({"error": f"side_start failed ({rc})"}), flush=True)
            return 1
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
        print(json.dumps({"reserve": reserve, "ms": dt * 1e3, "helper_running": int(still), "status": st,
                          "helper_done": int(done), "xcc": list(xcc)[:blocks],
                          "y_equal": bool(torch.equal(run.y, y_ref)) if st == 0 else None}), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main(int(sys.argv[1])))
