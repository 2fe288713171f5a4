"""Pre-dispatch activation quantisation on the GPU (through the C ABI) against
the CPU oracle: codes and scales must be bit-identical."""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_histogram_amd as mf
import oracle
from mixture_experts_ffn_histogram_amd import synth

from gpu_common import log

pytestmark = pytest.mark.gpu


def run_gpu(x_bits: np.ndarray):
    T, H = x_bits.shape
    dev = torch.device("cuda:0")
    x = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).to(dev)
    q = torch.full((T, H), 0xAB, dtype=torch.uint8, device=dev)
    sf = torch.full((T, H // 32), 0xAB, dtype=torch.uint8, device=dev)
    mf.quantize_activations(x, q, sf)
    torch.cuda.synchronize()
    return q.cpu().numpy(), sf.cpu().numpy()


@pytest.mark.parametrize("T,H", [(1, 32), (3, 96), (37, 7168), (128, 7168), (300, 2048), (5, 544), (1000, 160)])
def test_quantize_matches_oracle(T, H):
    log(f"quantize T={T} H={H}")
    x = synth.activations_bf16(T, H, seed=T * 7 + H)
    q, sf = run_gpu(x)
    rq, rsf = oracle.quantize_act(x)
    assert np.array_equal(sf, rsf)
    assert np.array_equal(q, rq)


def test_quantize_special_values():
    # zeros, -0, bf16 subnormals, the largest finite bf16, ties of the e4m3
    # grid, tiny values next to large ones (underflow to signed zero)
    H = 32 * 8
    x = np.zeros((2, H), np.uint16)
    x[0, 32:64] = 0x8000
    x[0, 64:96] = np.arange(1, 33, dtype=np.uint16)
    x[0, 96] = 0x7F7F
    x[0, 97:128] = 0xFF7F
    x[0, 128:160] = np.arange(0x3F80, 0x3FA0, dtype=np.uint16)      # 1.0 .. in bf16 steps (ties at 3 bits)
    x[0, 160:192] = np.arange(0xBF80, 0xBFA0, dtype=np.uint16)
    x[0, 192] = 0x4380                                              # 256 next to tiny values
    x[0, 193:224] = np.arange(0x0080, 0x009F, dtype=np.uint16) | 0x8000
    x[0, 224:256] = 0x0001                                          # smallest subnormal, constant
    x[1] = synth.activations_bf16(1, H, seed=99)[0]
    log("quantize special values")
    q, sf = run_gpu(x)
    rq, rsf = oracle.quantize_act(x)
    assert np.array_equal(sf, rsf)
    assert np.array_equal(q, rq)


def test_quantize_T0_and_errors():
    dev = torch.device("cuda:0")
    x = torch.zeros((0, 64), dtype=torch.int16, device=dev)
    q = torch.zeros((0, 64), dtype=torch.uint8, device=dev)
    sf = torch.zeros((0, 2), dtype=torch.uint8, device=dev)
    mf.quantize_activations(x, q, sf)  # no-op
    L = mf.lib()
    assert L.moe_ffn_quantize_activations(None, 4, 48, None, None, None) == mf.ERR_UNSUPPORTED
    assert L.moe_ffn_quantize_activations(None, 4, 64, None, None, None) == mf.ERR_INVALID_ARG
    assert L.moe_ffn_quantize_activations(None, -1, 64, None, None, None) == mf.ERR_INVALID_ARG


def test_quantize_full_size_feeds_the_forward_layout():
    # the DeepSeek-V3 activation shape of the T=8192 workload
    T, H = 8192, 7168
    log(f"quantize full size T={T} H={H}")
    x = synth.activations_bf16(T, H, seed=8192)
    q, sf = run_gpu(x)
    rq, rsf = oracle.quantize_act(x)
    assert np.array_equal(sf, rsf)
    assert np.array_equal(q, rq)
