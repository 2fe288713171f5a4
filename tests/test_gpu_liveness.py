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
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("blocks", [2, 7])
def test_side_stream_liveness(blocks):
    # The scenario runs in a fresh process (liveness_case.py): streams created
    # earlier in a long session may make the helper's stream and the MoE
    # stream share a hardware queue, which serialises them regardless of the
    # kernel.
    lib = os.path.join(HERE, "native", "libmoe_side.so")
    if not os.path.exists(lib):
        pytest.fail(f"{lib} is missing: run __graft_entry__.build()")
    print(f"liveness scenario: helper on {blocks} CUs", flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(HERE, "liveness_case.py"), str(blocks)],
                       capture_output=True, text=True, timeout=240)
    lines = [json.loads(x) for x in r.stdout.splitlines() if x.startswith("{")]
    assert r.returncode == 0 and len(lines) == 2, f"scenario failed (rc {r.returncode}): {r.stdout[-2000:]} {r.stderr[-2000:]}"
    for res in lines:
        print(f"helper on {blocks} CUs (XCDs {res['xcc']}), reserve {res['reserve']}: MoE call {res['ms']:.1f} ms, "
              f"helper still running at completion: {res['helper_running'] == 1}, status {res['status']}", flush=True)
        assert res["helper_done"] == blocks
        if res["reserve"] == 2:
            assert res["status"] == 0, "reserve 2 must complete normally"
            assert res["helper_running"] == 1, "the call with reserve 2 waited for the side stream"
            assert res["y_equal"], "y differs from the unobstructed call"
        else:
            assert res["status"] in (0, 2), f"unexpected status {res['status']} with reserve 0"
            if res["status"] == 0:
                assert res["y_equal"]
