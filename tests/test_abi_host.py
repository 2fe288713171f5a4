"""Host-side checks of the C ABI (no GPU needed, no compute calls).

The library must load and export every function include/moe_ffn.h declares;
the launch-size rule must follow the CU-reserve arithmetic of the sglang
"Reserve SMs for DeepGEMM MegaMoE grid barriers" change (physical CUs minus
the reserve, at least 2, capped, rounded down to even); argument checks must
fail with the documented codes before touching a device.
"""
import ctypes
import os
import re

import pytest

import mixture_experts_ffn_histogram_amd as mf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    text = open(os.path.join(ROOT, "include", "moe_ffn.h")).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(moe_ffn_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_function():
    names = _header_functions()
    assert set(names) == set(mf.EXPORTS), names
    lib = mf.lib()
    for n in names:
        assert hasattr(lib, n), n


@pytest.mark.parametrize("phys,reserve,cap,expect", [
    (256, 2, 0, 254),      # default reserve on MI355X
    (256, 0, 0, 256),      # reserve disabled
    (256, -3, 0, 256),     # negative reserve counts as 0
    (256, 3, 0, 252),      # odd result rounded down to even
    (255, 0, 0, 254),
    (256, 256, 0, 2),      # excessive reserve keeps 2
    (256, 1000, 0, 2),
    (256, 2, 100, 100),    # cap below the limit
    (256, 2, 101, 100),    # odd cap rounded down
    (256, 2, 300, 254),    # cap above the limit has no effect
    (256, 2, 1, 2),        # never below 2
    (8, 2, 0, 6),
])
def test_launch_size_rule(phys, reserve, cap, expect):
    assert mf.launch_size(phys, reserve, cap) == expect


def test_workspace_size_depends_on_problem_only_and_grows_with_tokens():
    sizes = [mf.get_workspace_size(mf.make_problem(t, 7168, 2048, 256, 8, mf.RECIPE_FP8_FP4))
             for t in (0, 1, 128, 8192)]
    assert sizes == sorted(sizes) and sizes[0] > 0
    v = mf.get_workspace_view(mf.make_problem(128, 7168, 2048, 256, 8, mf.RECIPE_FP8_FP4))
    # per routed row: e4m3 h codes, one e8m0 byte per 32, and the L2 result in bf16
    assert v.h_row_bytes == 2048 and v.h_sf_row_bytes == 64 and v.o_row_bytes == 7168 * 2
    assert v.h % 256 == 0 and v.h_sf % 256 == 0 and v.o % 256 == 0
    assert v.o + 128 * 8 * 7168 * 2 <= sizes[2]
    vb = mf.get_workspace_view(mf.make_problem(64, 256, 128, 8, 2, mf.RECIPE_BF16))
    assert vb.h_row_bytes == 256 and vb.h_sf_row_bytes == 0 and vb.o_row_bytes == 256 * 4   # fp32 L2 result


def test_token_alignment_and_strerror():
    for r in (mf.RECIPE_BF16, mf.RECIPE_FP8_FP8, mf.RECIPE_FP8_FP4, mf.RECIPE_FP8_BLOCK128):
        assert mf.get_token_alignment(r) == 1
    with pytest.raises(mf.MoeFFNError):
        mf.get_token_alignment(7)
    for code in (mf.OK, mf.ERR_INVALID_ARG, mf.ERR_UNSUPPORTED, mf.ERR_WORKSPACE_TOO_SMALL, mf.ERR_HIP,
                 mf.STATUS_BAD_EXPERT_INDEX, mf.STATUS_TIMEOUT, mf.STATUS_DIRTY_WORKSPACE):
        assert mf.strerror(code) and mf.strerror(code) != "unknown code"


@pytest.mark.parametrize("dims,code", [
    ((16, 100, 128, 8, 2, mf.RECIPE_FP8_FP4), mf.ERR_UNSUPPORTED),   # H not a multiple of 128
    ((16, 256, 96, 8, 2, mf.RECIPE_FP8_FP8), mf.ERR_UNSUPPORTED),    # I not a multiple of 128
    ((16, 256, 128, 513, 2, mf.RECIPE_FP8_FP4), mf.ERR_UNSUPPORTED),  # too many experts
    ((16, 256, 128, 8, 65, mf.RECIPE_FP8_FP4), mf.ERR_UNSUPPORTED),   # top-k too large
    ((-1, 256, 128, 8, 2, mf.RECIPE_FP8_FP4), mf.ERR_INVALID_ARG),
    ((16, 256, 128, 0, 2, mf.RECIPE_FP8_FP4), mf.ERR_INVALID_ARG),
    ((16, 256, 128, 8, 2, 4), mf.ERR_INVALID_ARG),                                    # no such recipe
    ((16, 192, 128, 8, 2, mf.RECIPE_FP8_BLOCK128), mf.ERR_UNSUPPORTED),               # H not a multiple of 128
    ((16, 256, 128, 8, 2, mf.RECIPE_FP8_BLOCK128, mf.WEIGHTS_TILED), mf.ERR_UNSUPPORTED),
    ((16, 256, 128, 8, 2, mf.RECIPE_FP8_FP4, 2), mf.ERR_INVALID_ARG),               # no such weight layout
    ((16, 256, 128, 8, 2, mf.RECIPE_BF16, mf.WEIGHTS_TILED), mf.ERR_UNSUPPORTED),   # TILED holds e2m1 only
    ((16, 256, 128, 8, 2, mf.RECIPE_FP8_FP8, mf.WEIGHTS_TILED), mf.ERR_UNSUPPORTED),
])
def test_problem_validation(dims, code):
    with pytest.raises(mf.MoeFFNError) as ei:
        mf.get_workspace_size(mf.make_problem(*dims))
    assert ei.value.code == code


def test_tiled_layout_problem_has_the_same_workspace():
    a = mf.get_workspace_size(mf.make_problem(8192, 7168, 2048, 256, 8, mf.RECIPE_FP8_FP4, mf.WEIGHTS_ROW_MAJOR))
    b = mf.get_workspace_size(mf.make_problem(8192, 7168, 2048, 256, 8, mf.RECIPE_FP8_FP4, mf.WEIGHTS_TILED))
    assert a == b


# Byte ranges the tiles address with 32-bit offsets must stay below 2^31:
# x rows (max_tokens * H * elem), h rows ((max_tokens * k + 128) * I * elem)
# and one expert's W1 (2I * H * weight bytes).  Each case sits on one side of
# one of these limits.
@pytest.mark.parametrize("dims,ok", [
    # DeepSeek shape: the h rows bind first, (T*8 + 128) * 2048 < 2^31 <=> T <= 131055
    ((131055, 7168, 2048, 256, 8, mf.RECIPE_FP8_FP4), True),
    ((131056, 7168, 2048, 256, 8, mf.RECIPE_FP8_FP4), False),
    # x rows bind: BF16 x, T * 4096 * 2 < 2^31 <=> T <= 262143
    ((262143, 4096, 64, 8, 1, mf.RECIPE_BF16), True),
    ((262144, 4096, 64, 8, 1, mf.RECIPE_BF16), False),
    # e4m3 x: T * 8192 < 2^31 <=> T <= 262143
    ((262143, 8192, 128, 8, 1, mf.RECIPE_FP8_FP8), True),
    ((262144, 8192, 128, 8, 1, mf.RECIPE_FP8_FP8), False),
    # h rows of BF16: (T*2 + 128) * 8192 * 2 < 2^31 <=> T <= 65471
    ((65471, 256, 8192, 8, 2, mf.RECIPE_BF16), True),
    ((65472, 256, 8192, 8, 2, mf.RECIPE_BF16), False),
    # one expert's W1: e2m1 I * H, e4m3 2 * I * H, bf16 4 * I * H bytes
    ((16, 65536, 32640, 8, 2, mf.RECIPE_FP8_FP4), True),
    ((16, 65536, 32768, 8, 2, mf.RECIPE_FP8_FP4), False),
    ((16, 32768, 32640, 8, 2, mf.RECIPE_FP8_FP8), True),
    ((16, 32768, 32768, 8, 2, mf.RECIPE_FP8_FP8), False),
    ((16, 16384, 32704, 8, 2, mf.RECIPE_BF16), True),
    ((16, 16384, 32768, 8, 2, mf.RECIPE_BF16), False),
])
def test_problem_32bit_offset_limits(dims, ok):
    prob = mf.make_problem(*dims)
    if ok:
        assert mf.get_workspace_size(prob) > 0
    else:
        with pytest.raises(mf.MoeFFNError) as ei:
            mf.get_workspace_size(prob)
        assert ei.value.code == mf.ERR_UNSUPPORTED


def _args(**kw):
    a = mf.Args()
    a.num_tokens = kw.get("num_tokens", 4)
    for n in ("x", "x_sf", "topk_idx", "topk_weights", "w1", "w1_sf", "w2", "w2_sf", "y"):
        setattr(a, n, kw.get(n, 4096))   # aligned non-null sentinels; never dereferenced on these paths
    a.y_dtype = kw.get("y_dtype", mf.Y_BF16)
    a.activation_clamp = 7.0
    a.reserved_cus = -1
    return a


@pytest.mark.parametrize("change,code", [
    ({"num_tokens": 17}, mf.ERR_INVALID_ARG),          # above max_tokens
    ({"num_tokens": -1}, mf.ERR_INVALID_ARG),
    ({"x": None}, mf.ERR_INVALID_ARG),
    ({"w1": 4100}, mf.ERR_INVALID_ARG),                # misaligned
    ({"y_dtype": 5}, mf.ERR_INVALID_ARG),
])
def test_forward_argument_checks_fail_before_any_device_work(change, code):
    prob = mf.make_problem(16, 256, 128, 8, 2, mf.RECIPE_FP8_FP4)
    a = _args(**change)
    ws = ctypes.c_void_p(1 << 20)
    rc = mf.lib().moe_ffn_forward(ctypes.byref(prob), ctypes.byref(a), ws, ctypes.c_size_t(1 << 40), None)
    assert rc == code


def test_forward_rejects_small_workspace():
    prob = mf.make_problem(16, 256, 128, 8, 2, mf.RECIPE_FP8_FP4)
    a = _args()
    need = mf.get_workspace_size(prob)
    rc = mf.lib().moe_ffn_forward(ctypes.byref(prob), ctypes.byref(a), ctypes.c_void_p(1 << 20),
                                  ctypes.c_size_t(need - 1), None)
    assert rc == mf.ERR_WORKSPACE_TOO_SMALL


@pytest.mark.parametrize("kw,code", [
    (dict(src=None), mf.ERR_INVALID_ARG),
    (dict(dst=None), mf.ERR_INVALID_ARG),
    (dict(rows=24), mf.ERR_INVALID_ARG),       # rows not a multiple of 16
    (dict(kb=6), mf.ERR_INVALID_ARG),          # k_blocks not a multiple of 4 (whole 128-element stages)
    (dict(kb=0), mf.ERR_INVALID_ARG),
    (dict(E=0), mf.ERR_INVALID_ARG),
    (dict(dst=4098), mf.ERR_INVALID_ARG),      # dst not 4-byte aligned
    (dict(src=4097), mf.ERR_INVALID_ARG),      # src not 4-byte aligned
])
def test_transform_weight_scales_argument_checks(kw, code):
    a = dict(src=4096, dst=8192, E=2, rows=16, kb=4)
    a.update(kw)
    rc = mf.lib().moe_ffn_transform_weight_scales(
        None if a["src"] is None else ctypes.c_void_p(a["src"]), None if a["dst"] is None else ctypes.c_void_p(a["dst"]),
        a["E"], a["rows"], a["kb"], None)
    assert rc == code


@pytest.mark.parametrize("kw,code", [
    (dict(H=48), mf.ERR_UNSUPPORTED),          # hidden not a multiple of 32
    (dict(H=0), mf.ERR_INVALID_ARG),
    (dict(T=-1), mf.ERR_INVALID_ARG),
    (dict(T=0, x=None, q=None, sf=None), mf.OK),  # no-op, no device work
    (dict(x=None), mf.ERR_INVALID_ARG),
    (dict(sf=None), mf.ERR_INVALID_ARG),
    (dict(x=4104), mf.ERR_INVALID_ARG),        # x not 16-byte aligned
    (dict(q=4100), mf.ERR_INVALID_ARG),        # codes not 8-byte aligned
])
def test_quantize_activations_argument_checks(kw, code):
    a = dict(x=4096, T=4, H=64, q=8192, sf=12288)
    a.update(kw)
    p = lambda v: None if v is None else ctypes.c_void_p(v)
    rc = mf.lib().moe_ffn_quantize_activations(p(a["x"]), a["T"], a["H"], p(a["q"]), p(a["sf"]), None)
    assert rc == code


@pytest.mark.parametrize("kw,code", [
    (dict(H=96), mf.ERR_UNSUPPORTED),          # hidden not a multiple of 64
    (dict(E=513), mf.ERR_UNSUPPORTED),
    (dict(E=0), mf.ERR_INVALID_ARG),
    (dict(k=0), mf.ERR_INVALID_ARG),
    (dict(k=9), mf.ERR_INVALID_ARG),           # top_k > num_experts
    (dict(E=128, k=65), mf.ERR_INVALID_ARG),   # top_k > 64
    (dict(T=-1), mf.ERR_INVALID_ARG),
    (dict(T=0, x=None, w=None, l=None, i=None, p=None), mf.OK),
    (dict(l=None), mf.ERR_INVALID_ARG),
    (dict(x=4104), mf.ERR_INVALID_ARG),        # x not 16-byte aligned
    (dict(i=4098), mf.ERR_INVALID_ARG),        # topk_idx not 4-byte aligned
])
def test_route_topk_argument_checks(kw, code):
    a = dict(x=4096, w=8192, T=4, H=64, E=8, k=2, l=12288, i=16384, p=20480)
    a.update(kw)
    p = lambda v: None if v is None else ctypes.c_void_p(v)
    rc = mf.lib().moe_ffn_route_topk(p(a["x"]), p(a["w"]), a["T"], a["H"], a["E"], a["k"], p(a["l"]), p(a["i"]),
                                     p(a["p"]), None)
    assert rc == code


@pytest.mark.parametrize("kw,code", [
    (dict(src=None), mf.ERR_INVALID_ARG),
    (dict(rows=24), mf.ERR_INVALID_ARG),       # rows not a multiple of 16
    (dict(kb=96), mf.ERR_INVALID_ARG),         # k_bytes not a multiple of 64
    (dict(E=0), mf.ERR_INVALID_ARG),
    (dict(dst=8200), mf.ERR_INVALID_ARG),      # dst not 16-byte aligned
])
def test_transform_weights_argument_checks(kw, code):
    a = dict(src=4096, dst=8192, E=2, rows=32, kb=128)
    a.update(kw)
    p = lambda v: None if v is None else ctypes.c_void_p(v)
    rc = mf.lib().moe_ffn_transform_weights(p(a["src"]), p(a["dst"]), a["E"], a["rows"], a["kb"], None)
    assert rc == code


def test_forward_noalloc_rejects_problems_beyond_its_scratch():
    # checked before any device work: the DeepSeek shape at 8192 tokens needs ~2 GB
    prob = mf.make_problem(8192, 7168, 2048, 256, 8, mf.RECIPE_FP8_FP4, mf.WEIGHTS_TILED)
    assert mf.get_workspace_size(prob) > mf.NOALLOC_MAX_WORKSPACE
    rc = mf.lib().moe_ffn_forward_noalloc(ctypes.byref(prob), ctypes.byref(_args()), None)
    assert rc == mf.ERR_WORKSPACE_TOO_SMALL
    # the DeepSeek shape at 128 tokens fits
    small = mf.make_problem(128, 7168, 2048, 256, 8, mf.RECIPE_FP8_FP4, mf.WEIGHTS_TILED)
    assert mf.get_workspace_size(small) <= mf.NOALLOC_MAX_WORKSPACE
    bad = mf.make_problem(16, 256, 128, 0, 2, mf.RECIPE_FP8_FP4)
    assert mf.lib().moe_ffn_forward_noalloc(ctypes.byref(bad), ctypes.byref(_args()), None) == mf.ERR_INVALID_ARG
