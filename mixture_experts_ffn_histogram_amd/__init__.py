"""MI355X (gfx950) fused MoE expert-FFN forward: Python binding of libmoe_ffn.so.

The names mirror the C ABI in ``include/moe_ffn.h``; every function only
marshals arguments (torch tensors -> device pointers) and calls the library.
There is no CPU or PyTorch fallback: if the HIP library is missing, loading
it raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_ffn.so")

RECIPE_BF16 = 0
RECIPE_FP8_FP8 = 1
RECIPE_FP8_FP4 = 2
RECIPE_FP8_BLOCK128 = 3
WEIGHTS_ROW_MAJOR = 0
WEIGHTS_TILED = 1
Y_BF16 = 0
Y_FP32 = 1

OK = 0
ERR_INVALID_ARG = -1
ERR_UNSUPPORTED = -2
ERR_WORKSPACE_TOO_SMALL = -3
ERR_HIP = -4
STATUS_OK = 0
STATUS_BAD_EXPERT_INDEX = 1
STATUS_TIMEOUT = 2
STATUS_DIRTY_WORKSPACE = 3


class Problem(ctypes.Structure):
    _fields_ = [("max_tokens", ctypes.c_int64), ("hidden", ctypes.c_int64),
                ("intermediate", ctypes.c_int64), ("num_experts", ctypes.c_int64),
                ("top_k", ctypes.c_int64), ("recipe", ctypes.c_int32), ("weight_layout", ctypes.c_int32)]


class Args(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int64),
                ("x", ctypes.c_void_p), ("x_sf", ctypes.c_void_p),
                ("topk_idx", ctypes.c_void_p), ("topk_weights", ctypes.c_void_p),
                ("w1", ctypes.c_void_p), ("w1_sf", ctypes.c_void_p),
                ("w2", ctypes.c_void_p), ("w2_sf", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("y_dtype", ctypes.c_int32),
                ("activation_clamp", ctypes.c_float),
                ("reserved_cus", ctypes.c_int32), ("max_cus", ctypes.c_int32),
                ("expert_counts", ctypes.c_void_p), ("expert_offsets", ctypes.c_void_p),
                ("row_to_slot", ctypes.c_void_p), ("slot_to_row", ctypes.c_void_p),
                ("status", ctypes.c_void_p)]


class WorkspaceView(ctypes.Structure):
    _fields_ = [("h", ctypes.c_size_t), ("h_sf", ctypes.c_size_t), ("o", ctypes.c_size_t),
                ("h_row_bytes", ctypes.c_int64), ("h_sf_row_bytes", ctypes.c_int64),
                ("o_row_bytes", ctypes.c_int64)]


EXPORTS = ("moe_ffn_get_workspace_size", "moe_ffn_get_token_alignment", "moe_ffn_forward",
           "moe_ffn_strerror", "moe_ffn_launch_size", "moe_ffn_get_workspace_view",
           "moe_ffn_transform_weight_scales", "moe_ffn_quantize_activations", "moe_ffn_route_topk",
           "moe_ffn_transform_weights", "moe_ffn_forward_noalloc")
NOALLOC_MAX_WORKSPACE = 64 << 20

_lib = None


def lib():
    """Load libmoe_ffn.so (raises OSError when it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise OSError(f"{LIB_PATH} is missing: build it with mixture_experts_ffn_histogram_amd/build.py "
                          "(the forward has no fallback path)")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        L.moe_ffn_get_workspace_size.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(ctypes.c_size_t)]
        L.moe_ffn_get_workspace_size.restype = ctypes.c_int
        L.moe_ffn_get_token_alignment.argtypes = [ctypes.c_int32, ctypes.POINTER(ctypes.c_int64)]
        L.moe_ffn_get_token_alignment.restype = ctypes.c_int
        L.moe_ffn_forward.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(Args), P, ctypes.c_size_t, P]
        L.moe_ffn_forward.restype = ctypes.c_int
        L.moe_ffn_strerror.argtypes = [ctypes.c_int]
        L.moe_ffn_strerror.restype = ctypes.c_char_p
        L.moe_ffn_launch_size.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
        L.moe_ffn_launch_size.restype = ctypes.c_int
        L.moe_ffn_get_workspace_view.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(WorkspaceView)]
        L.moe_ffn_get_workspace_view.restype = ctypes.c_int
        L.moe_ffn_transform_weight_scales.argtypes = [P, P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, P]
        L.moe_ffn_transform_weight_scales.restype = ctypes.c_int
        L.moe_ffn_quantize_activations.argtypes = [P, ctypes.c_int64, ctypes.c_int64, P, P, P]
        L.moe_ffn_quantize_activations.restype = ctypes.c_int
        L.moe_ffn_route_topk.argtypes = [P, P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                         P, P, P, P]
        L.moe_ffn_route_topk.restype = ctypes.c_int
        L.moe_ffn_transform_weights.argtypes = [P, P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, P]
        L.moe_ffn_transform_weights.restype = ctypes.c_int
        L.moe_ffn_forward_noalloc.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(Args), P]
        L.moe_ffn_forward_noalloc.restype = ctypes.c_int
        _lib = L
    return _lib


class MoeFFNError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {strerror(code)} ({code})")
        self.code = code


def _check(code: int, what: str) -> int:
    if code != OK:
        raise MoeFFNError(code, what)
    return code


def make_problem(max_tokens: int, hidden: int, intermediate: int, num_experts: int, top_k: int,
                 recipe: int, weight_layout: int = WEIGHTS_ROW_MAJOR) -> Problem:
    return Problem(int(max_tokens), int(hidden), int(intermediate), int(num_experts), int(top_k), int(recipe),
                   int(weight_layout))


def get_workspace_size(problem: Problem) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_ffn_get_workspace_size(ctypes.byref(problem), ctypes.byref(n)), "moe_ffn_get_workspace_size")
    return int(n.value)


def get_token_alignment(recipe: int) -> int:
    a = ctypes.c_int64(0)
    _check(lib().moe_ffn_get_token_alignment(int(recipe), ctypes.byref(a)), "moe_ffn_get_token_alignment")
    return int(a.value)


def get_workspace_view(problem: Problem) -> WorkspaceView:
    v = WorkspaceView()
    _check(lib().moe_ffn_get_workspace_view(ctypes.byref(problem), ctypes.byref(v)), "moe_ffn_get_workspace_view")
    return v


def strerror(code: int) -> str:
    return lib().moe_ffn_strerror(int(code)).decode()


def launch_size(physical_cus: int, reserved_cus: int, max_cus: int = 0) -> int:
    return int(lib().moe_ffn_launch_size(int(physical_cus), int(reserved_cus), int(max_cus)))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def transform_weight_scales(src, dst, num_experts: int, rows: int, k_blocks: int, stream=None) -> None:
    """Enqueue moe_ffn_transform_weight_scales: row-major e8m0 scales [E, rows, k_blocks] -> the TILED
    layout (uint8 device tensors)."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    rc = lib().moe_ffn_transform_weight_scales(_ptr(src), _ptr(dst), int(num_experts), int(rows), int(k_blocks),
                                               ctypes.c_void_p(stream.cuda_stream))
    _check(rc, "moe_ffn_transform_weight_scales")


def quantize_activations(x_bf16, x_e4m3, x_sf, stream=None) -> None:
    """Enqueue moe_ffn_quantize_activations: bf16 x [T, H] (int16 or bfloat16 device tensor) ->
    e4m3 codes x_e4m3 [T, H] and e8m0 scales x_sf [T, H/32] (uint8 device tensors)."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    T, H = int(x_bf16.shape[0]), int(x_bf16.shape[1])
    assert x_bf16.is_contiguous() and x_e4m3.is_contiguous() and x_sf.is_contiguous()
    assert x_bf16.element_size() == 2 and tuple(x_e4m3.shape) == (T, H) and x_sf.numel() == T * (H // 32)
    rc = lib().moe_ffn_quantize_activations(_ptr(x_bf16), T, H, _ptr(x_e4m3), _ptr(x_sf),
                                            ctypes.c_void_p(stream.cuda_stream))
    _check(rc, "moe_ffn_quantize_activations")


def route_topk(x_bf16, w_gate_bf16, logits, topk_idx, topk_weights, stream=None) -> None:
    """Enqueue moe_ffn_route_topk: x [T, H] and w_gate [E, H] bf16 (int16 or bfloat16 device
    tensors) -> logits fp32 [T, E], topk_idx int32 [T, k], topk_weights fp32 [T, k]."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    T, H = int(x_bf16.shape[0]), int(x_bf16.shape[1])
    E, k = int(w_gate_bf16.shape[0]), int(topk_idx.shape[1])
    for a in (x_bf16, w_gate_bf16, logits, topk_idx, topk_weights):
        assert a.is_contiguous()
    assert x_bf16.element_size() == 2 and w_gate_bf16.element_size() == 2 and int(w_gate_bf16.shape[1]) == H
    assert tuple(logits.shape) == (T, E) and logits.dtype == torch.float32
    assert tuple(topk_idx.shape) == (T, k) and topk_idx.dtype == torch.int32
    assert tuple(topk_weights.shape) == (T, k) and topk_weights.dtype == torch.float32
    rc = lib().moe_ffn_route_topk(_ptr(x_bf16), _ptr(w_gate_bf16), T, H, E, k, _ptr(logits), _ptr(topk_idx),
                                  _ptr(topk_weights), ctypes.c_void_p(stream.cuda_stream))
    _check(rc, "moe_ffn_route_topk")


def transform_weights(src, dst, num_experts: int, rows: int, k_bytes: int, stream=None) -> None:
    """Enqueue moe_ffn_transform_weights: tiled copy of packed e2m1 weights (uint8 device tensors)."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    rc = lib().moe_ffn_transform_weights(_ptr(src), _ptr(dst), int(num_experts), int(rows), int(k_bytes),
                                         ctypes.c_void_p(stream.cuda_stream))
    _check(rc, "moe_ffn_transform_weights")


def tile_weights(w1, w1_sf, w2, w2_sf, num_experts: int, hidden: int, intermediate: int, stream=None):
    """The e2m1 weights and their scales in the TILED layout (four new device tensors, same shapes
    and sizes as the row-major ones): the storage a problem with weight_layout=WEIGHTS_TILED takes."""
    import torch
    w1t, w2t = torch.empty_like(w1), torch.empty_like(w2)
    s1t, s2t = torch.empty_like(w1_sf), torch.empty_like(w2_sf)
    transform_weights(w1, w1t, num_experts, 2 * intermediate, hidden // 2, stream)
    transform_weights(w2, w2t, num_experts, hidden, intermediate // 2, stream)
    transform_weight_scales(w1_sf, s1t, num_experts, 2 * intermediate, hidden // 32, stream)
    transform_weight_scales(w2_sf, s2t, num_experts, hidden, intermediate // 32, stream)
    return w1t, s1t, w2t, s2t


def _args(num_tokens, x, x_sf, topk_idx, topk_weights, w1, w1_sf, w2, w2_sf, y, y_dtype, activation_clamp,
          reserved_cus, max_cus, expert_counts, expert_offsets, row_to_slot, slot_to_row, status) -> Args:
    return Args(int(num_tokens), _ptr(x), _ptr(x_sf), _ptr(topk_idx), _ptr(topk_weights),
                _ptr(w1), _ptr(w1_sf), _ptr(w2), _ptr(w2_sf), _ptr(y), int(y_dtype), float(activation_clamp),
                int(reserved_cus), int(max_cus), _ptr(expert_counts), _ptr(expert_offsets),
                _ptr(row_to_slot), _ptr(slot_to_row), _ptr(status))


def forward_noalloc(problem: Problem, *, num_tokens: int, x, x_sf, topk_idx, topk_weights,
                    w1, w1_sf, w2, w2_sf, y, y_dtype: int, activation_clamp: float,
                    reserved_cus: int = -1, max_cus: int = 0, expert_counts=None, expert_offsets=None,
                    row_to_slot=None, slot_to_row=None, status=None, stream=None) -> None:
    """Enqueue moe_ffn_forward_noalloc: the forward on the library's own static workspace (at most
    NOALLOC_MAX_WORKSPACE bytes; calls overlapping on one GPU race)."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    a = _args(num_tokens, x, x_sf, topk_idx, topk_weights, w1, w1_sf, w2, w2_sf, y, y_dtype, activation_clamp,
              reserved_cus, max_cus, expert_counts, expert_offsets, row_to_slot, slot_to_row, status)
    _check(lib().moe_ffn_forward_noalloc(ctypes.byref(problem), ctypes.byref(a), ctypes.c_void_p(stream.cuda_stream)),
           "moe_ffn_forward_noalloc")


def forward(problem: Problem, workspace, *, num_tokens: int, x, x_sf, topk_idx, topk_weights,
            w1, w1_sf, w2, w2_sf, y, y_dtype: int, activation_clamp: float,
            reserved_cus: int = -1, max_cus: int = 0, expert_counts=None, expert_offsets=None,
            row_to_slot=None, slot_to_row=None, status=None, stream=None) -> None:
    """Enqueue moe_ffn_forward on `stream` (default: torch's current stream).

    All tensors are device tensors laid out as include/moe_ffn.h states; the
    workspace is a uint8 device tensor of at least get_workspace_size() bytes,
    zero-filled once after allocation.
    """
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    a = _args(num_tokens, x, x_sf, topk_idx, topk_weights, w1, w1_sf, w2, w2_sf, y, y_dtype, activation_clamp,
              reserved_cus, max_cus, expert_counts, expert_offsets, row_to_slot, slot_to_row, status)
    rc = lib().moe_ffn_forward(ctypes.byref(problem), ctypes.byref(a), ctypes.c_void_p(workspace.data_ptr()),
                               ctypes.c_size_t(workspace.numel() * workspace.element_size()),
                               ctypes.c_void_p(stream.cuda_stream))
    _check(rc, "moe_ffn_forward")


class MoeFFN:
    """Owns a problem description and its zero-initialised workspace."""

    def __init__(self, max_tokens, hidden, intermediate, num_experts, top_k, recipe, device="cuda",
                 weight_layout=WEIGHTS_ROW_MAJOR):
        import torch
        self.problem = make_problem(max_tokens, hidden, intermediate, num_experts, top_k, recipe, weight_layout)
        self.workspace_bytes = get_workspace_size(self.problem)
        self.workspace = torch.zeros(self.workspace_bytes, dtype=torch.uint8, device=device)
        self.recipe = recipe

    def __call__(self, **kw) -> None:
        forward(self.problem, self.workspace, **kw)

    def view(self):
        return get_workspace_view(self.problem)
