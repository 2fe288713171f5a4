// Pre-dispatch activation quantisation for the e4m3 recipes: bf16 x -> e4m3
// codes + one e8m0 scale per 1x32 block along the hidden dimension.
//
// The pages place this step right before the fused forward (sglang PR
// "[Blackwell] Reserve SMs for DeepGEMM MegaMoE grid barriers": Fix section,
// pre-dispatch keeps the process-wide setting; its digest, key-code section:
// the buffer fetch and pre-dispatch quantisation precede the kernel call) but
// do not state its arithmetic.  It uses the rule the forward applies when it
// re-quantises the activation: the block's scale is the smallest power of two
// 2^E with amax <= 448 * 2^E (clamped to [-127, 127], E = 0 for an all-zero
// block) and each element is rounded to nearest even in E4M3FN after the
// exact scaling by 2^-E.
//
// Bandwidth-bound: a lane takes 8 consecutive elements (one 16-byte load),
// 4 lanes form a 1x32 block (amax by two lane exchanges), and a wave covers
// 512 elements per step.  Because H is a multiple of 32, blocks never cross
// rows, so the tensor is treated as one flat sequence of blocks and the
// scale of block b is byte b of x_sf ([T, H/32] row-major).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_ffn_device.h"

namespace moeffn {

constexpr int kQuantThreads = 256;
constexpr int kQuantUnroll = 2;  // 512-element steps in flight per wave (2, 4 and 8 measured: 2 is fastest)

__global__ __launch_bounds__(kQuantThreads) void quantize_act_kernel(const uint16_t* __restrict__ x,
                                                                     uint8_t* __restrict__ q,
                                                                     uint8_t* __restrict__ sf, int64_t n_elems) {
  const int lane = threadIdx.x & 63;
  const int64_t nsteps = (n_elems + 511) / 512;
  const int64_t wave = (int64_t)blockIdx.x * (kQuantThreads / 64) + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (kQuantThreads / 64);
  for (int64_t s0 = wave * kQuantUnroll; s0 < nsteps; s0 += nwaves * kQuantUnroll) {
    v4i v[kQuantUnroll];
    bool in[kQuantUnroll];
#pragma unroll
    for (int u = 0; u < kQuantUnroll; u++) {
      const int64_t e0 = (s0 + u) * 512 + (int64_t)lane * 8;
      in[u] = e0 < n_elems;  // n_elems is a multiple of 32: a lane's 8 elements are all in or all out
      v[u] = in[u] ? ldg16(x + e0) : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kQuantUnroll; u++) {
      const int64_t e0 = (s0 + u) * 512 + (int64_t)lane * 8;
      float f[8];
#pragma unroll
      for (int d = 0; d < 4; d++) {
        const uint32_t w = (uint32_t)v[u][d];
        f[2 * d] = __uint_as_float(w << 16);
        f[2 * d + 1] = __uint_as_float(w & 0xFFFF0000u);
      }
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 8; i++) amax = __builtin_fmaxf(amax, __builtin_fabsf(f[i]));
      amax = __builtin_fmaxf(amax, __shfl_xor(amax, 1, 64));
      amax = __builtin_fmaxf(amax, __shfl_xor(amax, 2, 64));
      const int E = block_scale_exp(amax);
      float g[8];
#pragma unroll
      for (int i = 0; i < 8; i++) g[i] = __builtin_amdgcn_ldexpf(f[i], -E);  // |g| <= 448 by the choice of E
      const uint32_t lo = e4m3x4(g[0], g[1], g[2], g[3]);
      const uint32_t hi = e4m3x4(g[4], g[5], g[6], g[7]);
      if (in[u]) {
        stg8(q + e0, lo, hi);
        if ((lane & 3) == 0) stg1(sf + (e0 >> 5), (uint8_t)(E + 127));
      }
    }
  }
}

hipError_t launch_quantize_act(const uint16_t* x, uint8_t* q, uint8_t* sf, int64_t n_elems, hipStream_t stream) {
  const int64_t nsteps = (n_elems + 511) / 512;
  const int64_t waves = (nsteps + kQuantUnroll - 1) / kQuantUnroll;
  int64_t blocks = (waves + (kQuantThreads / 64) - 1) / (kQuantThreads / 64);
  if (blocks > 16384) blocks = 16384;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(quantize_act_kernel, dim3((unsigned)blocks), dim3(kQuantThreads), 0, stream, x, q, sf, n_elems);
  return hipGetLastError();
}

}  // namespace moeffn
