"""GPU parity of the HIP forward against the CPU oracle (MI355X only).

Routing outputs must match bit for bit.  y: BF16 recipe within 5e-3 RMS(y_ref)
(fp32 y); FP8 recipes (gpu_common.fp8_parity): the fp32 y within 2e-2
RMS(y_ref) plus the effect of the re-quantisation flips the GPU actually made
(every flipped code checked against the oracle's rounding-decision band), and
the bf16 y bitwise the rounding of the fp32 y.  Every call goes through the C
ABI (moe_ffn_forward) via the Python binding.
"""
import numpy as np
import pytest
import torch

import oracle
from mixture_experts_ffn_histogram_amd import synth
from gpu_common import (Runner, check_tables, fp8_parity, log, oracle_y, quantize_on_the_fly, rel_err,
                        upload_inputs)

pytestmark = pytest.mark.gpu


def _check_tables(run: Runner, p: dict, T: int):
    check_tables(run, p, T)


def _small_cfg(recipe, T, H, I, E, k, routing="softmax", seed=7, y_fp32=False):
    return synth.Config(f"r{recipe}_T{T}_H{H}_I{I}_E{E}_k{k}", recipe, T, H, I, E, k, routing, seed, y_fp32=y_fp32)


@pytest.mark.parametrize("T", [0, 8, 48, 192, 1000, 1500])
def test_routing_bitexact_with_masks(T):
    cfg = _small_cfg(synth.RECIPE_FP8_FP4, max(T, 1), 256, 128, 16, 4, "uniform", seed=31)
    p = synth.make_problem(cfg, T=max(T, 1), threads=4)
    if T:
        rng = np.random.default_rng(T)
        p["topk_idx"][rng.random(p["topk_idx"].shape) < 0.1] = -1
    p["T"] = max(T, 1)
    log(f"routing T={T}")
    run = Runner(p)
    run.run(num_tokens=T)
    torch.cuda.synchronize()
    assert int(run.status.item()) == 0
    _check_tables(run, p, T)
    if T == 0:
        assert int(run.counts.sum().item()) == 0
        assert bool((run.y == -12345).all())


@pytest.mark.parametrize("y_fp32", [True, False])
def test_bf16_recipe_full(y_fp32):
    cfg = synth.CONFIGS["bf16_T64_H256_I128_E8_k2"]
    p = synth.make_problem(cfg, threads=4)
    log(f"bf16 T64 y_fp32={y_fp32}")
    run = Runner(p, y_fp32=y_fp32)
    run.run()
    torch.cuda.synchronize()
    _check_tables(run, p, p["T"])
    ref = oracle_y(p, y_fp32, p["clamp"])
    got = run.y_float()
    err, rms = rel_err(got, ref)
    log(f"  max|dy|/rms = {err:.3e}")
    if y_fp32:
        assert err <= 5e-3
    else:
        # one bf16 rounding step of y may flip on either side
        assert np.all(np.abs(got - ref) <= 5e-3 * rms + np.abs(ref) * 2.0 ** -8)


def test_fp8xfp8_config_full():
    # x ~ N(0, 1) quantised on the fly: GPU quantiser for the call, oracle quantiser for the oracle
    cfg = synth.CONFIGS["fp8xfp8_T512_H2048_I768_E64_k6"]
    p = synth.make_problem(cfg, threads=8)
    log("fp8xfp8 T512 full")
    run = Runner(p)
    quantize_on_the_fly(p, run)
    run.run()
    torch.cuda.synchronize()
    assert int(run.status.item()) == 0
    _check_tables(run, p, p["T"])
    fp8_parity(run, p, "fp8xfp8 T512 (C2)")


TILED, ROW_MAJOR = 1, 0


@pytest.mark.parametrize("T,E,k,layout", [(64, 32, 8, TILED), (96, 32, 8, TILED), (40, 8, 4, TILED),
                                           (333, 8, 3, TILED), (1000, 4, 2, TILED), (2048, 8, 4, TILED),
                                           (64, 32, 8, ROW_MAJOR), (96, 32, 8, ROW_MAJOR), (333, 8, 3, ROW_MAJOR),
                                           (2048, 8, 4, ROW_MAJOR)])
def test_fp8xfp4_reduced_full(T, E, k, layout):
    # spans token-block sizes 16..128 (average rows per expert 16 .. 1024) and ragged tails, with the
    # weights in the TILED layout (every tile kind, the 128-row one included) or row-major
    cfg = _small_cfg(synth.RECIPE_FP8_FP4, T, 1024, 512, E, k, "softmax", seed=T + E)
    p = synth.make_problem(cfg, threads=8)
    log(f"fp8xfp4 reduced T={T} E={E} k={k} layout={layout}")
    run = Runner(p, layout=layout)
    run.run()
    torch.cuda.synchronize()
    assert int(run.status.item()) == 0
    _check_tables(run, p, T)
    fp8_parity(run, p, f"fp8xfp4 T={T} E={E} k={k} layout={layout}")


@pytest.mark.parametrize("bm", [128, 64, 32, 16])
@pytest.mark.parametrize("T,H,I,E,k", [
    (300, 384, 128, 4, 2),    # K stages: L1 3, L2 1 (no steady loop); odd H/128: half-empty last L2 block
    (257, 1152, 640, 2, 1),   # L1 9 stages, L2 5 (two trailing stages; last scale groups of 1 stage); ragged
    (520, 1024, 512, 3, 3),   # several full 128-row blocks per expert
])
def test_fp8xfp4_block128_shapes(T, H, I, E, k, bm, monkeypatch):
    # ragged K-stage counts (partial last scale group of the TILED layout) on every tile kind
    monkeypatch.setenv("MOE_FFN_BLOCK_M", str(bm))
    cfg = _small_cfg(synth.RECIPE_FP8_FP4, T, H, I, E, k, "softmax", seed=T + H)
    p = synth.make_problem(cfg, threads=8)
    log(f"block {bm}: T={T} H={H} I={I} E={E} k={k}")
    run = Runner(p)
    run.run()
    torch.cuda.synchronize()
    assert int(run.status.item()) == 0
    _check_tables(run, p, T)
    fp8_parity(run, p, f"block {bm} T={T} H={H} I={I}")


def test_deepseek_T128_all_tokens():
    # the whole call at the DeepSeek shape (C3): all 128 tokens, all 1024 routed rows' codes
    cfg = synth.CONFIGS["deepseek_fp8xfp4_T128"]
    p = synth.make_problem(cfg, threads=16)
    log("deepseek T128 (full shape), all tokens")
    run = Runner(p)
    run.run()
    torch.cuda.synchronize()
    assert int(run.status.item()) == 0
    _check_tables(run, p, p["T"])
    fp8_parity(run, p, "deepseek T128 (C3)")


def test_deterministic_and_grid_size_invariant():
    cfg = _small_cfg(synth.RECIPE_FP8_FP4, 700, 1024, 512, 16, 6, "uniform", seed=5)
    p = synth.make_problem(cfg, threads=8)
    run = Runner(p)
    outs = []
    for reserve, cap in [(2, 0), (2, 0), (0, 0), (64, 0), (2, 40), (200, 0)]:
        log(f"determinism reserve={reserve} cap={cap}")
        run.run(reserved_cus=reserve, max_cus=cap)
        torch.cuda.synchronize()
        assert int(run.status.item()) == 0
        outs.append(run.y.clone())
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


def test_bad_expert_index_reported_and_masked():
    cfg = _small_cfg(synth.RECIPE_FP8_FP8, 64, 256, 128, 8, 2, "uniform", seed=3)
    p = synth.make_problem(cfg, threads=4)
    p["topk_idx"][5, 1] = 9
    p["topk_idx"][7, 0] = -4
    run = Runner(p)
    run.run()
    torch.cuda.synchronize()
    assert int(run.status.item()) == 1
    q = dict(p, topk_idx=p["topk_idx"].copy())
    q["topk_idx"][(q["topk_idx"] < -1) | (q["topk_idx"] >= 8)] = -1
    _check_tables(run, q, 64)
    fp8_parity(run, q, "bad index", status=1)
    # the next call on the same workspace is clean
    p2 = dict(q)
    run.p = p2
    upload_inputs(p2, run.d)
    run.run()
    torch.cuda.synchronize()
    assert int(run.status.item()) == 0


def test_num_tokens_below_capacity_leaves_tail_rows():
    cfg = _small_cfg(synth.RECIPE_FP8_FP4, 200, 512, 256, 8, 2, "softmax", seed=11)
    p = synth.make_problem(cfg, threads=4)
    run = Runner(p)
    q = dict(p, T=77, x=p["x"][:77], x_sf=p["x_sf"][:77], topk_idx=p["topk_idx"][:77],
             topk_weights=p["topk_weights"][:77])
    fp8_parity(run, q, "T=77 of 200", num_tokens=77)
    assert bool((run.y[77:] == -12345).all()) and bool((run.y32[77:] == -12345).all())
    _check_tables(run, q, 77)


def test_clamp_engaged_and_off():
    cfg = _small_cfg(synth.RECIPE_FP8_FP4, 64, 512, 256, 8, 2, "softmax", seed=13)
    p = synth.make_problem(cfg, threads=4)
    p["x_sf"] = (p["x_sf"].astype(np.int32) + 4).astype(np.uint8)  # x scaled by 16: |L1| >> 7
    run = Runner(p)
    for c in (7.0, 0.0):
        log(f"clamp {c}")
        fp8_parity(run, p, f"clamp {c}", clamp=c)


def test_graph_replay_changed_inputs_matches_eager():
    cfg = _small_cfg(synth.RECIPE_FP8_FP4, 256, 1024, 512, 16, 4, "softmax", seed=21)
    p = synth.make_problem(cfg, threads=8)
    run = Runner(p)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run.run(stream=s, sentinel=False)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run.run(stream=torch.cuda.current_stream(), sentinel=False)
    for r in range(6):
        q = synth.with_inputs(p, cfg, seed=1000 + r)
        if r == 3:
            q["topk_idx"][::3, 1] = -1
        upload_inputs(q, run.d)
        run.y.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        y_graph = run.y.clone()
        st = int(run.status.item())
        run.p = q
        run.run(sentinel=False)
        torch.cuda.synchronize()
        log(f"replay {r}: status {st}")
        assert st == 0
        assert torch.equal(y_graph, run.y), f"replay {r} differs from eager"
        _check_tables(run, q, q["T"])
        fp8_parity(run, q, f"replay {r}")


def tiled_scales_reference(src: np.ndarray) -> np.ndarray:
    """The TILED scale layout written out: per expert and 16-row block, groups of four K stages,
    each group [16 rows][n stages][4 blocks] (n = stages left, at most 4)."""
    E, rows, kb = src.shape
    nk = kb // 4
    out = np.empty(E * rows * kb, np.uint8)
    for e in range(E):
        for b in range(rows // 16):
            for G in range((nk + 3) // 4):
                n = min(4, nk - 4 * G)
                base = e * rows * kb + (b * nk + 4 * G) * 64
                out[base: base + 64 * n] = src[e, 16 * b: 16 * b + 16, 16 * G: 16 * G + 4 * n].reshape(-1)
    return out


@pytest.mark.parametrize("E,rows,kb", [(3, 16, 4), (2, 256, 12), (2, 48, 20), (1, 32, 36), (2, 4096, 224),
                                       (1, 7168, 64)])
def test_transform_weight_scales_bitexact(E, rows, kb):
    import mixture_experts_ffn_histogram_amd as mf
    rng = np.random.default_rng(rows + kb)
    src = rng.integers(0, 256, size=(E, rows, kb), dtype=np.uint8)
    s = torch.from_numpy(src).cuda()
    d = torch.full((E, rows, kb), 0xA5, dtype=torch.uint8, device="cuda")
    log(f"scale transform E={E} rows={rows} kb={kb}")
    mf.transform_weight_scales(s, d, E, rows, kb)
    torch.cuda.synchronize()
    assert np.array_equal(d.cpu().numpy().reshape(-1), tiled_scales_reference(src))


@pytest.mark.parametrize("E,rows,kbytes", [(3, 16, 64), (2, 48, 192), (2, 4096, 3584), (1, 7168, 1024)])
def test_transform_weights_bitexact(E, rows, kbytes):
    import mixture_experts_ffn_histogram_amd as mf
    rng = np.random.default_rng(rows + kbytes)
    src = rng.integers(0, 256, size=(E, rows, kbytes), dtype=np.uint8)
    s = torch.from_numpy(src).cuda()
    d = torch.full((E, rows, kbytes), 0xA5, dtype=torch.uint8, device="cuda")
    log(f"weight transform E={E} rows={rows} kbytes={kbytes}")
    mf.transform_weights(s, d, E, rows, kbytes)
    torch.cuda.synchronize()
    # [e][b][r][s][g][c] -> [e][b][s][g][r][c]: 16-row blocks, 64-byte stages, lane g*16 + r
    ref = src.reshape(E, rows // 16, 16, kbytes // 64, 4, 16).transpose(0, 1, 3, 4, 2, 5)
    assert np.array_equal(d.cpu().numpy().reshape(-1), np.ascontiguousarray(ref).reshape(-1))


def test_large_call_row_major_uses_64_row_tiles(monkeypatch):
    # the 128-row tiles read the TILED layout; a row-major call asking for them runs on 64-row
    # tiles and must give the same answer
    monkeypatch.setenv("MOE_FFN_BLOCK_M", "128")
    cfg = _small_cfg(synth.RECIPE_FP8_FP4, 520, 1024, 512, 3, 3, "softmax", seed=5)
    p = synth.make_problem(cfg, threads=8)
    log("block 128 requested, row-major weights")
    run = Runner(p, layout=ROW_MAJOR)
    fp8_parity(run, p, "row-major (64-row tiles)")
    y64 = run.y.clone()
    run_t = Runner(p, layout=TILED)
    fp8_parity(run_t, p, "TILED (128-row tiles)")
    log(f"  64-row vs 128-row tiles: {int((y64 != run_t.y).sum())} of {y64.numel()} y elements differ in the last bit")


# Control-block words (32-bit) of the workspace: bar[0..5], exit_count 6,
# tile_next 7, tile_next2 8, abort 9, status 10, xq 11..26, verdict 27, pad 28..63;
# then the barrier group counters, one 128-byte line per group (words 64, 96, ..., 288).
@pytest.mark.parametrize("word,value", [(6, 5), (6, 1 << 30), (2, 1), (9, 1), (27, 1), (50, 7), (64, 3), (96, 1),
                                        (300, 2)])
def test_dirty_workspace_reported_without_waiting(word, value):
    import time
    cfg = _small_cfg(synth.RECIPE_FP8_FP4, 64, 256, 128, 8, 2, "softmax", seed=17)
    p = synth.make_problem(cfg, threads=4)
    run = Runner(p)
    run.run()
    torch.cuda.synchronize()
    assert int(run.status.item()) == 0
    y_ref = run.y.clone()
    ctrl = run.m.workspace[:1280].view(torch.int32)
    ctrl[word] = value
    torch.cuda.synchronize()
    log(f"dirty control word {word} = {value}")
    for _ in range(2):   # the block stays dirty until the caller zeroes it
        t0 = time.time()
        run.run()
        torch.cuda.synchronize()
        dt = time.time() - t0
        assert int(run.status.item()) == 3, f"status {int(run.status.item())}"
        assert dt < 0.5, f"dirty call took {dt:.2f} s (a wait ran into its timeout)"
    run.m.workspace.zero_()
    run.run()
    torch.cuda.synchronize()
    assert int(run.status.item()) == 0
    assert torch.equal(run.y, y_ref)
    assert not bool(run.m.workspace[:1280].any()), "a clean call must leave the control block zeroed"
