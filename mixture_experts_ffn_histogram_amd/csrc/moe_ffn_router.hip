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
// with 8 waves (two per SIMD, so one hides the other's waits) of 32 tokens x
// 32 experts each (square wave tiles read the fewest LDS bytes per MFMA);
// both operands are staged through LDS (see below).
// The gate rows are the A operand, so a lane holds 4 consecutive experts of
// one token and stores them as one 16-byte piece of the logits row.
// router_topk_kernel: 16 lanes per token, k rounds of a (value desc, id
// asc) maximum over the row, then the renormalised softmax of the chosen
// logits in fp32.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "moe_ffn_device.h"

namespace moeffn {

typedef __bf16 v8bf_r __attribute__((ext_vector_type(8)));

constexpr int kRouterTok = 128;                               // tokens per workgroup
constexpr int kRouterExp = 64;                               // experts per workgroup (4 blocks of 16)
constexpr int kRouterWaves = 8;                              // 4 token quarters x 2 expert halves
constexpr int kRouterThreads = 64 * kRouterWaves;
constexpr int kRouterStage = (kRouterExp + kRouterTok) * 128;  // one 64-element K step: 24 KB
constexpr int kRouterFills = (kRouterExp + kRouterTok) / 8 / kRouterWaves;  // 8-row fill instructions per wave
static_assert(kRouterFills * kRouterWaves * 8 == kRouterExp + kRouterTok && kRouterTok == 4 * 32 &&
                  kRouterExp == 2 * 32 && kRouterWaves == 8,
              "fills and 32 x 32 wave tiles must divide evenly over the waves");

// Logits tile: 64 gate rows x 128 token rows, both staged through a 3-buffer
// LDS ring by buffer loads that write LDS directly (fill instruction q holds
// rows 8q..8q+7 of the stage: q < 8 gate rows, q >= 8 token rows; lane l
// reads row 8q + l/8, 16-byte chunk (l%8) ^ f, f = 4(q&1) + l/16, so each
// quad of lanes reads one 64-byte segment and the operand reads are free of
// LDS bank conflicts), two K steps ahead, one workgroup barrier per step.
// The waits are explicit (vmcnt before the barrier, issue order pinned by
// scheduling barriers) and each ring buffer is its own LDS object.
__global__ __launch_bounds__(kRouterThreads) void router_logits_kernel(const uint16_t* __restrict__ x,
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

  // fills of this wave: instructions q = kRouterFills * wave + i (rows past the end read the last row)
  const rsrc_t rA = make_rsrc(wg, (uint32_t)E * (uint32_t)H * 2u);
  const rsrc_t rB = make_rsrc(x, (uint32_t)T * (uint32_t)H * 2u);
  uint32_t voff[kRouterFills];
#pragma unroll
  for (int i = 0; i < kRouterFills; i++) {
    const int q = kRouterFills * wave + i;
    const int rr = (q < 8 ? 8 * q : 8 * (q - 8)) + (lane >> 3);
    const int row = q < 8 ? min(e0 + rr, E - 1) : min(t0 + rr, T - 1);
    voff[i] = (uint32_t)row * (uint32_t)H * 2u + (uint32_t)(((lane & 7) ^ (4 * (q & 1) + (lane >> 4))) * 16);
  }
  auto dma = [&](int s, uint8_t* buf) {
#pragma unroll
    for (int i = 0; i < kRouterFills; i++) {
      const int q = kRouterFills * wave + i;
      buf_load_lds16(q < 8 ? rA : rB, buf + q * 1024, s < nks ? voff[i] : kBufDead, (uint32_t)s * 128u);
    }
  };
  // operand of MFMA h for 16-row block b of a region: row r16, chunk 4h + g
  const uint32_t rd0 = (uint32_t)((r16 >> 3) * 1024 + (r16 & 7) * 128);
  uint32_t rdc[2];
#pragma unroll
  for (int h = 0; h < 2; h++) rdc[h] = rd0 + (uint32_t)((((4 * h + g) ^ (r16 >> 1))) * 16);

  // wave tile: token 16-blocks 2 tq, 2 tq + 1 and expert 16-blocks 2 eh, 2 eh + 1
  const int tq = wave & 3, eh = wave >> 2;
  v4f acc[2][2];
#pragma unroll
  for (int j = 0; j < 2; j++)
#pragma unroll
    for (int t = 0; t < 2; t++) acc[j][t] = v4f{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const uint8_t* buf) {
#pragma unroll
    for (int h = 0; h < 2; h++) {
      v4i ao[2], bo[2];
#pragma unroll
      for (int t = 0; t < 2; t++) bo[t] = *(const v4i*)(buf + 8 * 1024 + (2 * tq + t) * 2048 + rdc[h]);
#pragma unroll
      for (int j = 0; j < 2; j++) ao[j] = *(const v4i*)(buf + (2 * eh + j) * 2048 + rdc[h]);
#pragma unroll
      for (int j = 0; j < 2; j++)
#pragma unroll
        for (int t = 0; t < 2; t++)
          acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf_r, ao[j]),
                                                              __builtin_bit_cast(v8bf_r, bo[t]), acc[j][t], 0, 0, 0);
    }
  };

  dma(0, ring0);
  __builtin_amdgcn_sched_barrier(0);
  dma(1, ring1);
  __builtin_amdgcn_sched_barrier(0);
  int s0 = 0;
  for (; s0 + 3 <= nks; s0 += 3) {
    MOEFFN_WAIT_VMCNT(kRouterFills);  // this wave's fill of step s0 has landed (step s0+1's may be in flight)
    __builtin_amdgcn_s_barrier();
    dma(s0 + 2, ring2);
    __builtin_amdgcn_sched_barrier(0);
    compute(ring0);
    __builtin_amdgcn_sched_barrier(0);
    MOEFFN_WAIT_VMCNT(kRouterFills);
    __builtin_amdgcn_s_barrier();
    dma(s0 + 3, ring0);
    __builtin_amdgcn_sched_barrier(0);
    compute(ring1);
    __builtin_amdgcn_sched_barrier(0);
    MOEFFN_WAIT_VMCNT(kRouterFills);
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

  // lane (c = r16, g) holds experts e0 + 16 (2 eh + j) + 4g .. +3 of token t0 + 32 tq + 16t + c
#pragma unroll
  for (int t = 0; t < 2; t++) {
    const int tok = t0 + 32 * tq + 16 * t + r16;
    if (tok >= T) continue;
#pragma unroll
    for (int j = 0; j < 2; j++) {
      if (2 * eh + j >= nblk) continue;
      const int e = e0 + 16 * (2 * eh + j) + 4 * g;
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

// Order-preserving integer key of an fp32 logit (a larger float gives a
// larger signed key; -inf maps above INT32_MIN, which marks "not a candidate").
// Adding +0 turns -0 into +0, so the two zeros compare equal as they do in fp32.
__device__ __forceinline__ int topk_key(float f) {
  const int b = __float_as_int(f + 0.0f);
  return b >= 0 ? b : b ^ 0x7FFFFFFF;
}
__device__ __forceinline__ float topk_val(int key) { return __int_as_float(key >= 0 ? key : key ^ 0x7FFFFFFF); }

// (key desc, id asc) maximum of a lane and its DPP partner.  CTRL: quad_perm
// [1,0,3,2] (0xB1), quad_perm [2,3,0,1] (0x4E), row_half_mirror (0x141),
// row_mirror (0x140).
template <int CTRL>
__device__ __forceinline__ void topk_merge(int& bk, int& be) {
  const int ok = __builtin_amdgcn_mov_dpp(bk, CTRL, 0xF, 0xF, false);
  const int oe = __builtin_amdgcn_mov_dpp(be, CTRL, 0xF, 0xF, false);
  const bool take = (ok > bk) | ((ok == bk) & (oe < be));
  bk = take ? ok : bk;
  be = take ? oe : be;
}

// Sum over the 16 lanes of a row (the same butterfly in every lane, so every
// lane ends with the same bits).
__device__ __forceinline__ float row16_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false));
  return v;
}

// Top-k: 16 lanes per token (4 tokens per wave).  Lane r holds the keys of
// experts r, r + 16, ... (NPL of them, E <= 16 * NPL); each of the k rounds
// takes the lane-local best and reduces it over the 16-lane row with DPP
// moves (quad swaps, then the half-row and row mirrors), comparing (logit
// desc, id asc), so equal logits give the lower expert id and the order does
// not depend on the schedule.  The winner's key is then retired to INT32_MIN.
// Selects only, no branches, in the k rounds.
template <int NPL>
__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ logits, int32_t* __restrict__ idx,
                                                          float* __restrict__ wts, int T, int E, int k) {
  constexpr int kNone = INT32_MIN;
  const int lane = threadIdx.x & 63, r = lane & 15;
  const int nw = gridDim.x * 4;
  for (int tb = blockIdx.x * 4 + (threadIdx.x >> 6); tb * 4 < T; tb += nw) {
    const int t = tb * 4 + (lane >> 4);
    const bool tok = t < T;
    const float* row = logits + (size_t)(tok ? t : T - 1) * E;  // clamped: every load in bounds, no branches
    int key[NPL];
#pragma unroll
    for (int q = 0; q < NPL; q++) {
      const int e = r + 16 * q;
      const float x = row[e < E ? e : E - 1];
      key[q] = e < E ? topk_key(tok ? x : 0.f) : kNone;
    }
    int my_e[4] = {0, 0, 0, 0};
    int my_k[4] = {kNone, kNone, kNone, kNone};
    int kmax = 0;
    for (int j = 0; j < k; j++) {
      int bk = kNone, be = 0x7FFFFFFF;
#pragma unroll
      for (int q = 0; q < NPL; q++) {
        const bool take = key[q] > bk;  // q ascending: an equal key keeps the lower id
        bk = take ? key[q] : bk;
        be = take ? r + 16 * q : be;
      }
      topk_merge<0xB1>(bk, be);
      topk_merge<0x4E>(bk, be);
      topk_merge<0x141>(bk, be);
      topk_merge<0x140>(bk, be);
#pragma unroll
      for (int q = 0; q < NPL; q++) key[q] = (be == r + 16 * q) ? kNone : key[q];
      kmax = j == 0 ? bk : kmax;
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const bool mine = j == 16 * u + r;
        my_e[u] = mine ? be : my_e[u];
        my_k[u] = mine ? bk : my_k[u];
      }
    }
    const float vmax = topk_val(kmax);
    float ex[4], part = 0.f;
#pragma unroll
    for (int u = 0; u < 4; u++) {
      ex[u] = (16 * u + r < k) ? expf(topk_val(my_k[u]) - vmax) : 0.f;
      part += ex[u];
    }
    const float den = row16_sum(part);
    if (tok) {
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const int jj = 16 * u + r;
        if (jj < k) {
          idx[(size_t)t * k + jj] = my_e[u];
          wts[(size_t)t * k + jj] = ex[u] / den;
        }
      }
    }
  }
}

hipError_t launch_router(const uint16_t* x, const uint16_t* wg, float* logits, int32_t* idx, float* wts, int T, int H,
                         int E, int k, hipStream_t stream) {
  const dim3 g1((unsigned)((T + kRouterTok - 1) / kRouterTok), (unsigned)((E + kRouterExp - 1) / kRouterExp));
  hipLaunchKernelGGL(router_logits_kernel, g1, dim3(kRouterThreads), 0, stream, x, wg, logits, T, H, E);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int blocks = (T + 15) / 16;  // 16 tokens per workgroup
  if (blocks > 4096) blocks = 4096;
  if (E <= 256)
    hipLaunchKernelGGL(router_topk_kernel<16>, dim3((unsigned)blocks), dim3(256), 0, stream, logits, idx, wts, T, E, k);
  else
    hipLaunchKernelGGL(router_topk_kernel<32>, dim3((unsigned)blocks), dim3(256), 0, stream, logits, idx, wts, T, E, k);
  return hipGetLastError();
}

}  // namespace moeffn
