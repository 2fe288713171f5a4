// Persistent fused MoE expert-FFN forward for gfx950 (MI355X).
//
// One launch of G workgroups (G = CUs - reserve, even) runs the whole call:
//   R1  per-chunk expert histogram of topk_idx; zero the readiness counters
//   --  grid barrier 0
//   R2  per-expert column scan over the chunk histograms -> counts[e]
//   --  grid barrier 1
//   R3  offsets = exclusive scan of counts (every workgroup, in LDS); stable
//       scatter: row_to_slot / slot_to_row, ascending slot inside an expert
//   --  grid barrier 2
//   T   tile loop over a global queue: all L1 tiles (gather x rows, scaled
//       MFMA, fused SwiGLU + clamp + 1x32 e8m0 re-quantisation -> h), then
//       all L2 tiles (each waits on the readiness counter of its token
//       block, scaled MFMA -> fp32 o per routed row)
//   --  grid barrier 3
//   C   combine: y[t] = sum over valid slots j (ascending) of w[t,j] o[row]
//   X   the last workgroup out re-zeroes the control block.
// The stages follow the method of the MegaMoE pages: dispatch (expert count,
// source token / top-k index write: SM90 MegaMoE dev log, Phase 2), L1 GEMM,
// activation with clamp and re-quantisation into l2_acts / l2_acts_sf (dev
// log, Phase 1 buffer views; sglang PR digest, key code), L2 GEMM, combine
// ("[Bugfix] Reset MegaMoE combine readiness ...": every readiness state is
// reset per call, nothing is keyed on a launch id).
//
// GEMM tiles: weights are the MFMA A operand (rows = output features), tokens
// the B operand (columns), so a lane holds 4 consecutive features of one
// token: the gate and up values of a feature meet in the same lane and the
// 1x32 amax along the intermediate dimension is an in-lane max plus two
// cross-lane steps.  Each wave owns 64 weight rows and streams them straight
// from HBM into a register ring (no reuse, so no LDS); the BM tokens of the
// tile are shared by the 4 waves through a double-buffered LDS stage.
//
// Scaled MFMA operand layout (v_mfma_scale_f32_16x16x128_f8f6f4; measured):
// lane l serves row/column l%16 and lane group g = l/16.  An e2m1 operand
// holds K elements g*32 .. g*32+31 (16 bytes, element 2j in the low nibble);
// an e4m3 operand holds K elements g*16..g*16+15 in bytes 0-15 and
// 64+g*16 .. 64+g*16+15 in bytes 16-31.  The e8m0 scale of 32-block b of a
// row/column comes from lane row + 16*b (byte selected by opsel), so lane
// (row, g) supplies the scale of block g.
#include "moe_ffn_device.h"
#include "moe_ffn_kernel.h"

namespace moeffn {

enum { ST_OK = 0, ST_BAD_EXPERT_INDEX = 1, ST_TIMEOUT = 2, ST_DIRTY = 3 };

template <int RECIPE, int BM>
struct Cfg {
  static constexpr bool kBF16 = RECIPE == 0;
  static constexpr bool kW4 = RECIPE == 2;
  static constexpr int KS = kBF16 ? 64 : 128;        // K elements per stage (128 bytes of a token row)
  static constexpr int ADW = kW4 ? 4 : 8;            // dwords of A per lane per 16-row block per stage
  static constexpr int NTB = BM / 16;                // 16-token blocks
  static constexpr int P = BM <= 32 ? 4 : 2;         // A register ring depth (stages in flight)
  static constexpr int BSTAGE = BM * 128;            // bytes of B per stage
  static constexpr int BUNITS = BM * 8;              // 16-byte pieces of B per stage
  static constexpr int BPT = (BUNITS + kThreads - 1) / kThreads;
  static constexpr bool kStream = BM == 16;          // weights used once: non-temporal loads
};

struct Shared {
  int off[kMaxExperts + 1];     // expert row offsets
  int mbo[kMaxExperts + 1];     // expert token-block offsets
  int cnt[kMaxExperts];         // expert counts / histogram scratch
  int wcnt[4][kMaxExperts];     // per-wave running counters of the scatter
  int scan[4];
  int flag;
  uint32_t tile;
};

template <int BM>
struct SharedB {
  uint8_t b[2][BM * 128] __attribute__((aligned(16)));
  uint32_t bsf[2][BM];
  const uint8_t* brow[BM];
  const uint8_t* bsfrow[BM];
};

// ---------------------------------------------------------------------------
// status / abort
// ---------------------------------------------------------------------------
__device__ __forceinline__ void raise_status(const KParams& p, int code, bool fatal) {
  int expected = 0;
  __hip_atomic_compare_exchange_strong(&p.ctrl->status, &expected, code, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  if (fatal) st_relaxed(&p.ctrl->abort, 1u);
}

// Whole-grid barrier `id`: every workgroup arrives once per call.  The wait
// is bounded: on timeout the call is aborted with ST_TIMEOUT.  Returns false
// when the call is aborted.
__device__ bool grid_barrier(const KParams& p, int id, Shared& sh) {
  fence_release();
  __syncthreads();
  if (threadIdx.x == 0) {
    int ok = 1;
    add_release(&p.ctrl->bar[id], 1u);
    const uint64_t t0 = now_ticks();
    while (ld_relaxed(&p.ctrl->bar[id]) < gridDim.x) {
      if (ld_relaxed(&p.ctrl->abort)) { ok = 0; break; }
      if (now_ticks() - t0 > p.timeout_ticks) { raise_status(p, ST_TIMEOUT, true); ok = 0; break; }
      __builtin_amdgcn_s_sleep(2);
    }
    if (ld_relaxed(&p.ctrl->abort)) ok = 0;
    sh.flag = ok;
  }
  __syncthreads();
  fence_acquire();
  const int ok = sh.flag;
  __syncthreads();
  return ok != 0;
}

// ---------------------------------------------------------------------------
// R1: chunk histograms
// ---------------------------------------------------------------------------
__device__ void phase_histogram(const KParams& p, Shared& sh, int S, int C, int nready) {
  const int tid = threadIdx.x;
  int bad = 0;
  for (int c = blockIdx.x; c < C; c += gridDim.x) {
    for (int e = tid; e < p.E; e += kThreads) sh.cnt[e] = 0;
    __syncthreads();
    const int beg = c * (int)p.chunk_slots;
    const int end = min(S, beg + (int)p.chunk_slots);
    for (int s = beg + tid; s < end; s += kThreads) {
      const int e = p.idx[s];
      if ((unsigned)e < (unsigned)p.E) atomicAdd(&sh.cnt[e], 1);
      else if (e != -1) bad = 1;
    }
    __syncthreads();
    for (int e = tid; e < p.E; e += kThreads) p.hist[(size_t)c * p.E + e] = sh.cnt[e];
    __syncthreads();
  }
  for (int i = blockIdx.x * kThreads + tid; i < nready; i += gridDim.x * kThreads) p.ready[i] = 0u;
  if (bad) raise_status(p, ST_BAD_EXPERT_INDEX, false);
}

// ---------------------------------------------------------------------------
// R2: column scan over chunks for each expert
// ---------------------------------------------------------------------------
__device__ void phase_column_scan(const KParams& p, Shared& sh, int C) {
  const int tid = threadIdx.x;
  for (int e = blockIdx.x; e < p.E; e += gridDim.x) {
    const int v = tid < C ? p.hist[(size_t)tid * p.E + e] : 0;
    int total;
    const int pre = block_excl_scan(v, sh.scan, &total);
    if (tid < C) p.hist[(size_t)tid * p.E + e] = pre;
    if (tid == 0) p.counts[e] = total;
  }
}

// Exclusive scan of src[0..E) into dst[0..E], dst[E] = total (E <= 512).
__device__ void table_scan(const int* src, int* dst, int E, Shared& sh) {
  const int tid = threadIdx.x;
  const int a0 = 2 * tid < E ? src[2 * tid] : 0;
  const int a1 = 2 * tid + 1 < E ? src[2 * tid + 1] : 0;
  int total;
  const int pre = block_excl_scan(a0 + a1, sh.scan, &total);
  if (2 * tid < E) dst[2 * tid] = pre;
  if (2 * tid + 1 < E) dst[2 * tid + 1] = pre + a0;
  if (tid == 0) dst[E] = total;
  __syncthreads();
}

// Routing tables in LDS: counts, row offsets, token-block offsets.
__device__ void load_tables(const KParams& p, Shared& sh, int bm) {
  const int tid = threadIdx.x;
  for (int e = tid; e < p.E; e += kThreads) sh.cnt[e] = p.counts[e];
  __syncthreads();
  table_scan(sh.cnt, sh.off, p.E, sh);
  // token blocks per expert, reusing wcnt[0] as scratch
  for (int e = tid; e < p.E; e += kThreads) sh.wcnt[0][e] = (sh.cnt[e] + bm - 1) / bm;
  __syncthreads();
  table_scan(sh.wcnt[0], sh.mbo, p.E, sh);
}

// ---------------------------------------------------------------------------
// R3: stable scatter.  Slot order inside an expert = ascending slot index.
// Each chunk is split into 4 contiguous quarters, one per wave; a wave walks
// its quarter 64 slots at a time, ranking lanes with equal expert id by a
// ballot match, and keeps a running count per expert in LDS.
// ---------------------------------------------------------------------------
__device__ void phase_scatter(const KParams& p, Shared& sh, int S, int C) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = p.E;
  if (blockIdx.x == 0) {
    for (int e = tid; e <= E; e += kThreads) {
      p.offsets[e] = sh.off[e];
      if (p.out_offsets) p.out_offsets[e] = sh.off[e];
      if (e < E && p.out_counts) p.out_counts[e] = sh.cnt[e];
    }
  }
  const int NB = E > 1 ? 32 - __clz(E - 1) : 0;
  const uint64_t lt = (1ull << lane) - 1ull;
  const int quarter = (int)p.chunk_slots / 4;
  for (int c = blockIdx.x; c < C; c += gridDim.x) {
    const int wbeg = c * (int)p.chunk_slots + wave * quarter;
    const int wend = min(S, wbeg + quarter);
    for (int e = lane; e < E; e += 64) sh.wcnt[wave][e] = 0;
    __syncthreads();
    for (int s0 = wbeg; s0 < wend; s0 += 64) {
      const int s = s0 + lane;
      const int raw = s < wend ? p.idx[s] : -1;
      const bool valid = (unsigned)raw < (unsigned)E;
      const int e = valid ? raw : 0;
      uint64_t m = __ballot(valid);
      for (int b = 0; b < NB; b++) {
        const bool bit = (e >> b) & 1;
        const uint64_t bb = __ballot(valid && bit);
        m &= bit ? bb : ~bb;
      }
      if (valid && __popcll(m & lt) == 0) sh.wcnt[wave][e] += __popcll(m);
    }
    __syncthreads();
    for (int e = tid; e < E; e += kThreads) {
      int run = sh.off[e] + p.hist[(size_t)c * E + e];
      for (int w = 0; w < 4; w++) {
        const int t = sh.wcnt[w][e];
        sh.wcnt[w][e] = run;
        run += t;
      }
    }
    __syncthreads();
    for (int s0 = wbeg; s0 < wend; s0 += 64) {
      const int s = s0 + lane;
      const bool inr = s < wend;
      const int raw = inr ? p.idx[s] : -1;
      const bool valid = (unsigned)raw < (unsigned)E;
      const int e = valid ? raw : 0;
      uint64_t m = __ballot(valid);
      for (int b = 0; b < NB; b++) {
        const bool bit = (e >> b) & 1;
        const uint64_t bb = __ballot(valid && bit);
        m &= bit ? bb : ~bb;
      }
      const int rank = __popcll(m & lt);
      const int base = valid ? sh.wcnt[wave][e] : 0;
      if (valid && rank == 0) sh.wcnt[wave][e] = base + __popcll(m);
      if (valid) {
        const int row = base + rank;
        p.r2s[row] = s;
        p.s2r[s] = row;
        if (p.out_r2s) p.out_r2s[row] = s;
        if (p.out_s2r) p.out_s2r[s] = row;
      } else if (inr) {
        p.s2r[s] = -1;
        if (p.out_s2r) p.out_s2r[s] = -1;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// GEMM tile
// ---------------------------------------------------------------------------
template <bool NT>
__device__ __forceinline__ v4i load16(const uint8_t* ptr) {
  if constexpr (NT) return __builtin_nontemporal_load((const v4i*)ptr);
  else return *(const v4i*)ptr;
}

// One tile: expert e, token block mb (BM routed rows), feature block nb.
// L1: 4 waves x (32 gate + 32 up rows) = 128 intermediate features;
// L2: 4 waves x 64 rows = 256 hidden outputs.
template <int RECIPE, int BM>
__device__ void gemm_tile(const KParams& p, Shared& sh, SharedB<BM>& sb, bool l1, int e, int mb, int nb) {
  using C = Cfg<RECIPE, BM>;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, r16 = lane & 15;
  const int H = p.H, I = p.I;
  const int row0 = sh.off[e] + mb * BM;
  const int nrows = min(BM, sh.cnt[e] - mb * BM);
  const int K = l1 ? H : I;
  const int nk = K / C::KS;
  const size_t wrow_bytes = C::kW4 ? (size_t)K / 2 : (C::kBF16 ? (size_t)K * 2 : (size_t)K);
  const size_t wsf_row = (size_t)K / 32;

  // B rows of the tile: gathered x rows (L1) or consecutive h rows (L2)
  if (tid < BM) {
    const int m = tid;
    if (l1) {
      const int slot = p.r2s[row0 + (m < nrows ? m : 0)];
      const size_t tok = (size_t)(slot / p.k);
      sb.brow[m] = p.x + tok * (size_t)H * (C::kBF16 ? 2 : 1);
      sb.bsfrow[m] = C::kBF16 ? nullptr : p.x_sf + tok * (size_t)(H / 32);
    } else {
      const size_t r = (size_t)(row0 + m);  // rows past the expert stay inside the padded h buffer
      sb.brow[m] = p.h + r * (size_t)I * (C::kBF16 ? 2 : 1);
      sb.bsfrow[m] = C::kBF16 ? nullptr : p.h_sf + r * (size_t)(I / 32);
    }
  }

  // A rows owned by this wave
  int arow[4];
  bool active;
  const uint8_t* W;
  const uint8_t* Wsf;
  if (l1) {
    const int i0 = nb * 128 + wave * 32;
    active = i0 < I;
    arow[0] = i0; arow[1] = i0 + 16; arow[2] = I + i0; arow[3] = I + i0 + 16;
    W = p.w1 + (size_t)e * 2 * I * wrow_bytes;
    Wsf = C::kBF16 ? nullptr : p.w1_sf + (size_t)e * 2 * I * wsf_row;
  } else {
    const int n0 = nb * 256 + wave * 64;
    active = n0 < H;
    arow[0] = n0; arow[1] = n0 + 16; arow[2] = n0 + 32; arow[3] = n0 + 48;
    W = p.w2 + (size_t)e * H * wrow_bytes;
    Wsf = C::kBF16 ? nullptr : p.w2_sf + (size_t)e * H * wsf_row;
  }
  const uint8_t* aptr[4];
  const uint8_t* sptr[4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const size_t r = (size_t)(active ? arow[j] + r16 : 0);
    size_t lane_off;
    if constexpr (C::kW4) lane_off = (size_t)g * 16;          // e2m1: elements g*32..g*32+31
    else if constexpr (C::kBF16) lane_off = (size_t)g * 32;   // bf16: elements g*16..g*16+15
    else lane_off = (size_t)g * 16;                           // e4m3: bytes g*16 and 64+g*16
    aptr[j] = W + r * wrow_bytes + lane_off;
    sptr[j] = C::kBF16 ? nullptr : Wsf + r * wsf_row;
  }
  __syncthreads();  // brow / bsfrow visible

  v4f acc[4][C::NTB];
#pragma unroll
  for (int j = 0; j < 4; j++)
#pragma unroll
    for (int t = 0; t < C::NTB; t++) acc[j][t] = v4f{0.f, 0.f, 0.f, 0.f};

  v4i ar[C::P][4][C::ADW / 4];
  uint32_t sar[C::P][4];
  v4i br[2][C::BPT];
  uint32_t bsr[2];

  auto load_a = [&](int slot, int ks) {
    if (!active) return;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const size_t kb = (size_t)ks * 128;  // 128 bytes of a bf16 row per stage, 64 of e2m1, 128 of e4m3
      if constexpr (C::kW4) {
        ar[slot][j][0] = load16<C::kStream>(aptr[j] + (size_t)ks * 64);
      } else if constexpr (C::kBF16) {
        ar[slot][j][0] = load16<C::kStream>(aptr[j] + kb);
        ar[slot][j][1] = load16<C::kStream>(aptr[j] + kb + 16);
      } else {
        ar[slot][j][0] = load16<C::kStream>(aptr[j] + kb);
        ar[slot][j][1] = load16<C::kStream>(aptr[j] + kb + 64);
      }
      if constexpr (!C::kBF16) sar[slot][j] = *(const uint32_t*)(sptr[j] + (size_t)ks * 4);
    }
  };
  auto load_b = [&](int slot, int ks) {
#pragma unroll
    for (int u = 0; u < C::BPT; u++) {
      const int unit = tid + u * kThreads;
      if (unit < C::BUNITS) br[slot][u] = *(const v4i*)(sb.brow[unit >> 3] + (size_t)ks * 128 + (unit & 7) * 16);
    }
    if constexpr (!C::kBF16) {
      if (tid < BM) bsr[slot] = *(const uint32_t*)(sb.bsfrow[tid] + (size_t)ks * 4);
    }
  };
  auto store_b = [&](int slot, int buf) {
#pragma unroll
    for (int u = 0; u < C::BPT; u++) {
      const int unit = tid + u * kThreads;
      if (unit < C::BUNITS) {
        const int m = unit >> 3, q = unit & 7;
        const int half = C::kBF16 ? (q & 1) : (q >> 2);
        const int gg = C::kBF16 ? (q >> 1) : (q & 3);
        const int dst = (((m >> 4) * 2 + half) * 64 + gg * 16 + (m & 15)) * 16;
        *(v4i*)(&sb.b[buf][dst]) = br[slot][u];
      }
    }
    if constexpr (!C::kBF16) {
      if (tid < BM) sb.bsf[buf][tid] = bsr[slot];
    }
  };
  auto compute = [&](int slot, int buf) {
    if (!active) return;
#pragma unroll
    for (int t = 0; t < C::NTB; t++) {
      const v4i b0 = *(const v4i*)(&sb.b[buf][((t * 2 + 0) * 64 + lane) * 16]);
      const v4i b1 = *(const v4i*)(&sb.b[buf][((t * 2 + 1) * 64 + lane) * 16]);
      if constexpr (C::kBF16) {
#pragma unroll
        for (int j = 0; j < 4; j++) {
          acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, ar[slot][j][0]),
                                                              __builtin_bit_cast(v8bf, b0), acc[j][t], 0, 0, 0);
          acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, ar[slot][j][1]),
                                                              __builtin_bit_cast(v8bf, b1), acc[j][t], 0, 0, 0);
        }
      } else {
        const v8i bb = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        const int sbv = (int)(sb.bsf[buf][t * 16 + r16] >> (8 * g));
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const int sav = (int)(sar[slot][j] >> (8 * g));
          if constexpr (C::kW4) {
            const v8i aa = {ar[slot][j][0][0], ar[slot][j][0][1], ar[slot][j][0][2], ar[slot][j][0][3], 0, 0, 0, 0};
            acc[j][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aa, bb, acc[j][t], 4, 0, 0, sav, 0, sbv);
          } else {
            const v8i aa = {ar[slot][j][0][0], ar[slot][j][0][1], ar[slot][j][0][2], ar[slot][j][0][3],
                            ar[slot][j][1][0], ar[slot][j][1][1], ar[slot][j][1][2], ar[slot][j][1][3]};
            acc[j][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aa, bb, acc[j][t], 0, 0, 0, sav, 0, sbv);
          }
        }
      }
    }
  };

  // Pipeline: A ring P stages ahead; B two stages ahead in registers, one in LDS.
#pragma unroll
  for (int s = 0; s < C::P; s++)
    if (s < nk) load_a(s, s);
  load_b(0, 0);
  if (nk > 1) load_b(1, 1);
  store_b(0, 0);
  for (int ks0 = 0; ks0 < nk; ks0 += C::P) {
#pragma unroll
    for (int s = 0; s < C::P; s++) {
      const int ks = ks0 + s;
      if (ks < nk) {
        if (ks + 2 < nk) load_b(s & 1, ks + 2);
        __syncthreads();
        compute(s, s & 1);
        if (ks + C::P < nk) load_a(s, ks + C::P);
        if (ks + 1 < nk) store_b((s + 1) & 1, (s + 1) & 1);
      }
    }
  }
  __syncthreads();  // every wave is done with the B stages before the next tile refills them

  if (!active) return;
  if (l1) {
    const int i0 = nb * 128 + wave * 32;
#pragma unroll
    for (int t = 0; t < C::NTB; t++) {
      const int m = t * 16 + r16;
      float hv[8];
#pragma unroll
      for (int hh = 0; hh < 2; hh++)
#pragma unroll
        for (int j = 0; j < 4; j++) hv[hh * 4 + j] = swiglu(acc[hh][t][j], acc[2 + hh][t][j], p.clamp_on, p.clamp);
      const size_t row = (size_t)(row0 + m);
      if constexpr (C::kBF16) {
        if (m < nrows) {
#pragma unroll
          for (int hh = 0; hh < 2; hh++) {
            const uint32_t lo = f32_to_bf16(hv[hh * 4 + 0]) | (f32_to_bf16(hv[hh * 4 + 1]) << 16);
            const uint32_t hi = f32_to_bf16(hv[hh * 4 + 2]) | (f32_to_bf16(hv[hh * 4 + 3]) << 16);
            uint2* dst = (uint2*)(p.h + (row * I + (size_t)(i0 + hh * 16 + 4 * g)) * 2);
            *dst = make_uint2(lo, hi);
          }
        }
      } else {
        float amax = 0.f;
#pragma unroll
        for (int j = 0; j < 8; j++) amax = __builtin_fmaxf(amax, __builtin_fabsf(hv[j]));
        amax = __builtin_fmaxf(amax, __shfl_xor(amax, 16, 64));
        amax = __builtin_fmaxf(amax, __shfl_xor(amax, 32, 64));
        const int E = block_scale_exp(amax);
        if (m < nrows) {
#pragma unroll
          for (int hh = 0; hh < 2; hh++) {
            uint32_t word = 0;
#pragma unroll
            for (int j = 0; j < 4; j++) word |= f32_to_e4m3(__builtin_amdgcn_ldexpf(hv[hh * 4 + j], -E)) << (8 * j);
            *(uint32_t*)(p.h + row * I + (size_t)(i0 + hh * 16 + 4 * g)) = word;
          }
          if (g == 0) p.h_sf[row * (size_t)(I / 32) + (size_t)(i0 / 32)] = (uint8_t)(E + 127);
        }
      }
    }
  } else {
#pragma unroll
    for (int t = 0; t < C::NTB; t++) {
      const int m = t * 16 + r16;
      if (m < nrows) {
        const size_t row = (size_t)(row0 + m);
#pragma unroll
        for (int j = 0; j < 4; j++) *(v4f*)(p.o + row * H + (size_t)(arow[j] + 4 * g)) = acc[j][t];
      }
    }
  }
}

// Largest e in [0, E) with mbo[e] * nb <= t (t < mbo[E] * nb).
__device__ __forceinline__ int find_expert(const int* mbo, int E, int nb, int t) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (mbo[mid] * nb <= t) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

template <int RECIPE, int BM>
__device__ bool phase_tiles(const KParams& p, Shared& sh, SharedB<BM>& sb) {
  const int tid = threadIdx.x;
  const int E = p.E;
  const int nmb = sh.mbo[E];
  const int NB1 = (p.I + 127) / 128;
  const int NB2 = (p.H + 255) / 256;
  const int n1 = nmb * NB1, n2 = nmb * NB2;
  for (;;) {
    if (tid == 0) {
      uint32_t t = 0xFFFFFFFFu;
      if (!ld_relaxed(&p.ctrl->abort))
        t = __hip_atomic_fetch_add(&p.ctrl->tile_next, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sh.tile = t;
    }
    __syncthreads();
    const uint32_t t = sh.tile;
    __syncthreads();
    if (t == 0xFFFFFFFFu) return false;
    if (t >= (uint32_t)(n1 + n2)) return true;
    const bool l1 = t < (uint32_t)n1;
    const int tt = l1 ? (int)t : (int)t - n1;
    const int NB = l1 ? NB1 : NB2;
    const int e = find_expert(sh.mbo, E, NB, tt);
    const int nmb_e = sh.mbo[e + 1] - sh.mbo[e];
    const int loc = tt - sh.mbo[e] * NB;
    const int nb = loc / nmb_e, mb = loc % nmb_e;
    const int gmb = sh.mbo[e] + mb;
    if (!l1) {
      // wait until every L1 tile of this token block has published its h rows
      if (tid == 0) {
        int ok = 1;
        const uint64_t t0 = now_ticks();
        while (ld_relaxed(&p.ready[gmb]) < (uint32_t)NB1) {
          if (ld_relaxed(&p.ctrl->abort)) { ok = 0; break; }
          if (now_ticks() - t0 > p.timeout_ticks) { raise_status(p, ST_TIMEOUT, true); ok = 0; break; }
          __builtin_amdgcn_s_sleep(1);
        }
        sh.flag = ok;
      }
      __syncthreads();
      fence_acquire();
      const int ok = sh.flag;
      __syncthreads();
      if (!ok) return false;
    }
    gemm_tile<RECIPE, BM>(p, sh, sb, l1, e, mb, nb);
    if (l1) {
      fence_release();
      __syncthreads();
      if (tid == 0) add_release(&p.ready[gmb], 1u);
    }
  }
}

// ---------------------------------------------------------------------------
// C: combine.  Work unit = (token, 1024-wide slice of H).
// ---------------------------------------------------------------------------
__device__ void phase_combine(const KParams& p) {
  const int tid = threadIdx.x;
  const int H = p.H, k = p.k;
  const int nch = (H + 1023) / 1024;
  const int units = p.T * nch;
  for (int u = blockIdx.x; u < units; u += gridDim.x) {
    const int t = u / nch;
    const int hcol = (u - t * nch) * 1024 + tid * 4;
    if (hcol >= H) continue;
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < k; j0 += 8) {
      v4f ov[8];
      float wv[8];
      bool vv[8];
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const int jj = j0 + j;
        const int row = jj < k ? p.s2r[(size_t)t * k + jj] : -1;
        vv[j] = row >= 0;
        wv[j] = vv[j] ? p.tw[(size_t)t * k + jj] : 0.f;
        ov[j] = vv[j] ? *(const v4f*)(p.o + (size_t)row * H + hcol) : v4f{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int j = 0; j < 8; j++) {
        if (vv[j]) {
          acc[0] = __builtin_fmaf(wv[j], ov[j][0], acc[0]);
          acc[1] = __builtin_fmaf(wv[j], ov[j][1], acc[1]);
          acc[2] = __builtin_fmaf(wv[j], ov[j][2], acc[2]);
          acc[3] = __builtin_fmaf(wv[j], ov[j][3], acc[3]);
        }
      }
    }
    if (p.y_fp32) {
      *(v4f*)((float*)p.y + (size_t)t * H + hcol) = acc;
    } else {
      const uint32_t lo = f32_to_bf16(acc[0]) | (f32_to_bf16(acc[1]) << 16);
      const uint32_t hi = f32_to_bf16(acc[2]) | (f32_to_bf16(acc[3]) << 16);
      *(uint2*)((uint16_t*)p.y + (size_t)t * H + hcol) = make_uint2(lo, hi);
    }
  }
}

// ---------------------------------------------------------------------------
// The persistent kernel.  __launch_bounds__(256, 2): registers and LDS sized
// so that two workgroups fit on one CU, which keeps the grid co-resident when
// another stream holds a few CUs of an XCD.
// ---------------------------------------------------------------------------
template <int RECIPE, int BM>
__global__ __launch_bounds__(kThreads, 2) void moe_ffn_kernel(KParams p) {
  __shared__ Shared sh;
  __shared__ SharedB<BM> sb;
  const int tid = threadIdx.x;
  const int S = p.T * p.k;
  const int C = (S + (int)p.chunk_slots - 1) / (int)p.chunk_slots;
  const int nready = (S + BM - 1) / BM + p.E;

  if (tid == 0) {
    int dirty = 0;
    if (ld_relaxed(&p.ctrl->exit_count) != 0u && ld_relaxed(&p.ctrl->abort) == 0u) {
      dirty = 1;
      raise_status(p, ST_DIRTY, true);
      if (p.out_status) *p.out_status = ST_DIRTY;
    }
    sh.flag = dirty;
  }
  __syncthreads();
  const int dirty = sh.flag;
  __syncthreads();

  if (!dirty) {
    phase_histogram(p, sh, S, C, nready);
    if (!grid_barrier(p, 0, sh)) goto done;
    phase_column_scan(p, sh, C);
    if (!grid_barrier(p, 1, sh)) goto done;
    load_tables(p, sh, BM);
    phase_scatter(p, sh, S, C);
    if (!grid_barrier(p, 2, sh)) goto done;
    if (!phase_tiles<RECIPE, BM>(p, sh, sb)) goto done;
    if (!grid_barrier(p, 3, sh)) goto done;
    phase_combine(p);
  }
done:
  fence_release();
  __syncthreads();
  if (tid == 0) {
    const uint32_t old = add_acq_rel(&p.ctrl->exit_count, 1u);
    if (old == gridDim.x - 1 && !dirty) {
      // last workgroup out: every other workgroup is past its last access
      const int st = __hip_atomic_load(&p.ctrl->status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (p.out_status) *p.out_status = st;
      for (int i = 0; i < kNumBarriers; i++) st_relaxed(&p.ctrl->bar[i], 0u);
      st_relaxed(&p.ctrl->tile_next, 0u);
      st_relaxed(&p.ctrl->abort, 0u);
      __hip_atomic_store(&p.ctrl->status, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      st_release(&p.ctrl->exit_count, 0u);
    }
  }
}

int max_block_m(int recipe) { return recipe == 2 ? 128 : 64; }

template <int RECIPE, int BM>
static hipError_t launch_one(int grid, const KParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((moe_ffn_kernel<RECIPE, BM>), dim3(grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int RECIPE>
static hipError_t launch_recipe(int bm, int grid, const KParams& p, hipStream_t stream) {
  switch (bm) {
    case 16: return launch_one<RECIPE, 16>(grid, p, stream);
    case 32: return launch_one<RECIPE, 32>(grid, p, stream);
    case 64: return launch_one<RECIPE, 64>(grid, p, stream);
    case 128:
      if constexpr (RECIPE == 2) return launch_one<RECIPE, 128>(grid, p, stream);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_forward(int recipe, int bm, int grid, const KParams& p, hipStream_t stream) {
  switch (recipe) {
    case 0: return launch_recipe<0>(bm, grid, p, stream);
    case 1: return launch_recipe<1>(bm, grid, p, stream);
    case 2: return launch_recipe<2>(bm, grid, p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moeffn
