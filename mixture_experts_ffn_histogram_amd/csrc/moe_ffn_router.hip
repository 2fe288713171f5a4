// Gate and top-k: the softmax router that produces topk_idx / topk_weights
// for the fused forward.  The sglang page "[Blackwell] Reserve SMs for
// DeepGEMM MegaMoE grid barriers" (Fix section) runs gate computation and
// top-k selection before the MegaMoE call; the pages give no formula, and
// the reading is a softmax router: logits = x . Wg^T (bf16 inputs, fp32
// accumulation), the k largest logits of a token in descending order (equal
// logits: lower expert id first), weights = softmax over the selected logits
// (the top-k probabilities renormalised to sum 1).
//
// Two kernels.  router_logits_kernel: a dense bf16 GEMM on
// v_mfma_f32_16x16x32_bf16; a workgroup computes 128 tokens x 64 experts
// (4 waves x 32 tokens); both operands are staged through LDS (see below).
// The gate rows are the A operand, so a lane holds 4 consecutive experts of
// one token and stores them as one 16-byte piece of the logits row.
// router_topk_kernel: one wave per token, k rounds of a wave-wide (value
// desc, id asc) maximum, then the renormalised softmax of the chosen logits
// in fp32.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "moe_ffn_device.h"

namespace moeffn {

typedef __bf16 v8bf_r __attribute__((ext_vector_type(8)));

constexpr int kRouterTok = 128;                               // tokens per workgroup (4 waves x 32)
constexpr int kRouterExp = 64;                               // experts per workgroup (4 blocks of 16)
constexpr int kRouterStage = (kRouterExp + kRouterTok) * 128;  // one 64-element K step: 24 KB

// Logits tile: 64 gate rows x 128 token rows, both staged through a 3-buffer
// LDS ring by buffer loads that write LDS directly (fill instruction q holds
// rows 8q..8q+7 of the stage: q < 8 gate rows, q >= 8 token rows; lane l
// reads row 8q + l/8, 16-byte chunk (l%8) ^ f, f = 4(q&1) + l/16, so each
// quad of lanes reads one 64-byte segment and the operand reads are free of
// LDS bank conflicts), two K steps ahead, one workgroup barrier per step.
// The waits are explicit (vmcnt before the barrier, issue order pinned by
// scheduling barriers) and each ring buffer is its own LDS object.
__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ wg,
                                                            float* __restrict__ logits, int T, int H, int E) {
  __shared__ __attribute__((aligned(16))) uint8_t ring0[kRouterStage];
  __shared__ __attribute__((aligned(16))) uint8_t ring1[kRouterStage];
  __shared__ __attribute__((aligned(16))) uint8_t ring2[kRouterStage];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int t0 = blockIdx.x * kRouterTok;
  const int e0 = blockIdx.y * kRouterExp;
  const int nblk = min(4, (E - e0 + 15) / 16);  // 16-expert blocks holding an expert < E
  const int nks = H / 64;

  // fills of this wave: instructions q = 6 * wave + i (rows past the end read the last row)
  const rsrc_t rA = make_rsrc(wg, (uint32_t)E * (uint32_t)H * 2u);
  const rsrc_t rB = make_rsrc(x, (uint32_t)T * (uint32_t)H * 2u);
  uint32_t voff[6];
#pragma unroll
  for (int i = 0; i < 6; i++) {
    const int q = 6 * wave + i;
    const int rr = (q < 8 ? 8 * q : 8 * (q - 8)) + (lane >> 3);
    const int row = q < 8 ? min(e0 + rr, E - 1) : min(t0 + rr, T - 1);
    voff[i] = (uint32_t)row * (uint32_t)H * 2u + (uint32_t)(((lane & 7) ^ (4 * (q & 1) + (lane >> 4))) * 16);
  }
  auto dma = [&](int s, uint8_t* buf) {
#pragma unroll
    for (int i = 0; i < 6; i++) {
      const int q = 6 * wave + i;
      buf_load_lds16(q < 8 ? rA : rB, buf + q * 1024, s < nks ? voff[i] : kBufDead, (uint32_t)s * 128u);
    }
  };
  // operand of MFMA h for 16-row block b of a region: row r16, chunk 4h + g
  const uint32_t rd0 = (uint32_t)((r16 >> 3) * 1024 + (r16 & 7) * 128);
  uint32_t rdc[2];
#pragma unroll
  for (int h = 0; h < 2; h++) rdc[h] = rd0 + (uint32_t)((((4 * h + g) ^ (r16 >> 1))) * 16);

  v4f acc[4][2];
#pragma unroll
  for (int j = 0; j < 4; j++)
#pragma unroll
    for (int t = 0; t < 2; t++) acc[j][t] = v4f{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const uint8_t* buf) {
#pragma unroll
    for (int h = 0; h < 2; h++) {
      v4i bo[2];
#pragma unroll
      for (int t = 0; t < 2; t++) bo[t] = *(const v4i*)(buf + 8 * 1024 + (2 * wave + t) * 2048 + rdc[h]);
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const v4i ao = *(const v4i*)(buf + j * 2048 + rdc[h]);
#pragma unroll
        for (int t = 0; t < 2; t++)
          acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf_r, ao),
                                                              __builtin_bit_cast(v8bf_r, bo[t]), acc[j][t], 0, 0, 0);
      }
    }
  };

  dma(0, ring0);
  __builtin_amdgcn_sched_barrier(0);
  dma(1, ring1);
  __builtin_amdgcn_sched_barrier(0);
  int s0 = 0;
  for (; s0 + 3 <= nks; s0 += 3) {
    MOEFFN_WAIT_VMCNT(6);  // this wave's fill of step s0 has landed (step s0+1's 6 fills may be in flight)
    __builtin_amdgcn_s_barrier();
    dma(s0 + 2, ring2);
    __builtin_amdgcn_sched_barrier(0);
    compute(ring0);
    __builtin_amdgcn_sched_barrier(0);
    MOEFFN_WAIT_VMCNT(6);
    __builtin_amdgcn_s_barrier();
    dma(s0 + 3, ring0);
    __builtin_amdgcn_sched_barrier(0);
    compute(ring1);
    __builtin_amdgcn_sched_barrier(0);
    MOEFFN_WAIT_VMCNT(6);
    __builtin_amdgcn_s_barrier();
    dma(s0 + 4, ring1);
    __builtin_amdgcn_sched_barrier(0);
    compute(ring2);
    __builtin_amdgcn_sched_barrier(0);
  }
  // nks % 3 trailing steps, already in flight in ring0 / ring1
  if (s0 < nks) {
    MOEFFN_WAIT_VMCNT(0);
    __builtin_amdgcn_s_barrier();
    compute(ring0);
  }
  if (s0 + 1 < nks) {
    MOEFFN_WAIT_VMCNT(0);
    __builtin_amdgcn_s_barrier();
    compute(ring1);
  }
  MOEFFN_WAIT_VMCNT(0);  // no fill outlives the workgroup

  // lane (c = r16, g) holds experts e0 + 16j + 4g .. +3 of token t0 + 32 wave + 16t + c
#pragma unroll
  for (int t = 0; t < 2; t++) {
    const int tok = t0 + 32 * wave + 16 * t + r16;
    if (tok >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      if (j >= nblk) continue;
      const int e = e0 + 16 * j + 4 * g;
      float* dst = logits + (size_t)tok * E + e;
      if ((E & 3) == 0 && e + 4 <= E) {
        stg16f(dst, acc[j][t]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; i++)
          if (e + i < E) dst[i] = acc[j][t][i];
      }
    }
  }
}

constexpr int kTopkMaxPerLane = 8;  // E <= 512

__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ logits, int32_t* __restrict__ idx,
                                                          float* __restrict__ wts, int T, int E, int k) {
  const int lane = threadIdx.x & 63;
  const int nw = gridDim.x * 4;
  for (int t = blockIdx.x * 4 + (threadIdx.x >> 6); t < T; t += nw) {
    float v[kTopkMaxPerLane];
#pragma unroll
    for (int q = 0; q < kTopkMaxPerLane; q++) {
      const int e = lane + 64 * q;
      v[q] = e < E ? logits[(size_t)t * E + e] : -INFINITY;
    }
    uint32_t taken = 0;
    int my_e = 0;
    float my_v = -INFINITY, vmax = 0.f;
    for (int j = 0; j < k; j++) {
      float bv = -INFINITY;
      int be = 0x7FFFFFFF;
#pragma unroll
      for (int q = 0; q < kTopkMaxPerLane; q++) {
        const int e = lane + 64 * q;
        if (e < E && !((taken >> q) & 1u) && (v[q] > bv || (v[q] == bv && e < be))) {
          bv = v[q];
          be = e;
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off, 64);
        const int oe = __shfl_xor(be, off, 64);
        if (ov > bv || (ov == bv && oe < be)) {
          bv = ov;
          be = oe;
        }
      }
      if ((be & 63) == lane) taken |= 1u << (be >> 6);
      if (j == 0) vmax = bv;
      if (lane == j) {
        my_e = be;
        my_v = bv;
      }
    }
    const float ex = lane < k ? expf(my_v - vmax) : 0.f;
    float den = ex;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) den += __shfl_xor(den, off, 64);
    if (lane < k) {
      idx[(size_t)t * k + lane] = my_e;
      wts[(size_t)t * k + lane] = ex / den;
    }
  }
}

hipError_t launch_router(const uint16_t* x, const uint16_t* wg, float* logits, int32_t* idx, float* wts, int T, int H,
                         int E, int k, hipStream_t stream) {
  const dim3 g1((unsigned)((T + kRouterTok - 1) / kRouterTok), (unsigned)((E + kRouterExp - 1) / kRouterExp));
  hipLaunchKernelGGL(router_logits_kernel, g1, dim3(256), 0, stream, x, wg, logits, T, H, E);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int blocks = (T + 3) / 4;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(router_topk_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, logits, idx, wts, T, E, k);
  return hipGetLastError();
}

}  // namespace moeffn
