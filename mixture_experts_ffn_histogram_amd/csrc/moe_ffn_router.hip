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
// with 8 waves (4 groups of 32 tokens x 2 halves of K, all sharing the 64
// gate rows through the vector L1; the two K halves are added in a fixed
// order through LDS, so the result is deterministic).  The gate rows are the
// A operand, so a lane holds 4 consecutive experts of one token and stores
// them as one 16-byte piece of the logits row.  Both operands are read
// K-contiguous, 64 bytes per quad of lanes, two 64-element K steps ahead.  router_topk_kernel: one wave per
// token, k rounds of a wave-wide (value desc, id asc) maximum, then the
// renormalised softmax of the chosen logits in fp32.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "moe_ffn_device.h"

namespace moeffn {

typedef __bf16 v8bf_r __attribute__((ext_vector_type(8)));

constexpr int kRouterTok = 128;   // tokens per workgroup (4 token groups x 32)
constexpr int kRouterExp = 64;    // experts per workgroup (4 blocks of 16)
constexpr int kRouterThreads = 512;  // 8 waves: 4 token groups x 2 halves of K

__global__ __launch_bounds__(kRouterThreads) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                                       const uint16_t* __restrict__ wg,
                                                                       float* __restrict__ logits, int T, int H,
                                                                       int E) {
  __shared__ v4f red[4][8][64];  // K-half 1 partials of each token group: [group][j*2+t][lane]
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tg = wave & 3, kh = wave >> 2;
  const int r16 = lane & 15, g = lane >> 4;
  const int t0 = blockIdx.x * kRouterTok + tg * 32;
  const int e0 = blockIdx.y * kRouterExp;
  const int nblk = min(4, (E - e0 + 15) / 16);  // 16-expert blocks holding an expert < E

  // Loads read one 64-byte segment per quad of lanes (the texture unit
  // spends a cycle per distinct segment a quad touches): load h of a 16-row
  // block gives lane 16G + 4A + U row 4A + G, 16-byte chunk 4h + U.  A 4x4
  // lane transpose (ds_bpermute, swapping lane bits 0-1 with 4-5) then puts
  // row r, chunk 4h + g in lane (r, g): MFMA h's operand, K elements
  // 32h + 8g .. +7, the same order for A and B.  Rows past the end read the
  // last row; their results are not stored.
  const int rq = (lane & 12) | (lane >> 4);                   // row of the block this lane loads
  const int cq = (lane & 3) * 8;                              // its element offset in a 32-element half
  const int src = (((lane & 3) << 4) | (lane & 12) | (lane >> 4)) * 4;
  const uint16_t* ap[4];
  const uint16_t* bp[2];
#pragma unroll
  for (int j = 0; j < 4; j++) ap[j] = wg + (size_t)min(e0 + 16 * j + rq, E - 1) * H + cq;
#pragma unroll
  for (int t = 0; t < 2; t++) bp[t] = x + (size_t)min(t0 + 16 * t + rq, T - 1) * H + cq;

  v4f acc[4][2];
#pragma unroll
  for (int j = 0; j < 4; j++)
#pragma unroll
    for (int t = 0; t < 2; t++) acc[j][t] = v4f{0.f, 0.f, 0.f, 0.f};
  v4i a[3][4][2], b[3][2][2];
  auto load = [&](int buf, int ks) {
    const size_t k0 = (size_t)ks * 64;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      a[buf][j][0] = ldg16(ap[j] + k0);
      a[buf][j][1] = ldg16(ap[j] + k0 + 32);
    }
#pragma unroll
    for (int t = 0; t < 2; t++) {
      b[buf][t][0] = ldg16(bp[t] + k0);
      b[buf][t][1] = ldg16(bp[t] + k0 + 32);
    }
  };
  auto tr = [&](const v4i& v) {
    v4i r;
#pragma unroll
    for (int c = 0; c < 4; c++) r[c] = __builtin_amdgcn_ds_bpermute(src, v[c]);
    return r;
  };
  auto compute = [&](int buf) {
#pragma unroll
    for (int h = 0; h < 2; h++) {
      v4i bo[2];
#pragma unroll
      for (int t = 0; t < 2; t++) bo[t] = tr(b[buf][t][h]);
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const v4i ao = tr(a[buf][j][h]);
#pragma unroll
        for (int t = 0; t < 2; t++)
          acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf_r, ao),
                                                              __builtin_bit_cast(v8bf_r, bo[t]), acc[j][t], 0, 0, 0);
      }
    }
  };
  // this wave's half of the K steps, two steps in flight ahead of the one in
  // use; loads past the half re-read its last step (never used), so the
  // steady loop carries no branch
  const int nks = H / 64;
  const int kb = (nks * kh) / 2, n = (nks * (kh + 1)) / 2 - kb;
  if (n > 0) {
    auto step = [&](int s) { return kb + min(s, n - 1); };
    load(0, step(0));
    load(1, step(1));
    int s = 0;
    // scheduling barriers keep each step's loads ahead of the MFMAs that do
    // not need them: a step waits only for its own buffer, two steps old
    for (; s + 3 <= n; s += 3) {
      load(2, step(s + 2));
      __builtin_amdgcn_sched_barrier(0);
      compute(0);
      __builtin_amdgcn_sched_barrier(0);
      load(0, step(s + 3));
      __builtin_amdgcn_sched_barrier(0);
      compute(1);
      __builtin_amdgcn_sched_barrier(0);
      load(1, step(s + 4));
      __builtin_amdgcn_sched_barrier(0);
      compute(2);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (s < n) compute(0);
    if (s + 1 < n) compute(1);
  }

  // logits = K-half 0 + K-half 1, in this order
  if (kh == 1) {
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int t = 0; t < 2; t++) red[tg][j * 2 + t][lane] = acc[j][t];
  }
  __syncthreads();
  if (kh == 1 || t0 >= T) return;
  // lane (c = r16, g) holds experts e0 + 16j + 4g .. +3 of token t0 + 16t + c
#pragma unroll
  for (int t = 0; t < 2; t++) {
    const int tok = t0 + 16 * t + r16;
    if (tok >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      if (j >= nblk) continue;
      const v4f o = red[tg][j * 2 + t][lane];
      const v4f v = v4f{acc[j][t][0] + o[0], acc[j][t][1] + o[1], acc[j][t][2] + o[2], acc[j][t][3] + o[3]};
      const int e = e0 + 16 * j + 4 * g;
      float* dst = logits + (size_t)tok * E + e;
      if ((E & 3) == 0 && e + 4 <= E) {
        stg16f(dst, v);
      } else {
#pragma unroll
        for (int i = 0; i < 4; i++)
          if (e + i < E) dst[i] = v[i];
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
  hipLaunchKernelGGL(router_logits_kernel, g1, dim3(kRouterThreads), 0, stream, x, wg, logits, T, H, E);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int blocks = (T + 3) / 4;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(router_topk_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, logits, idx, wts, T, E, k);
  return hipGetLastError();
}

}  // namespace moeffn
