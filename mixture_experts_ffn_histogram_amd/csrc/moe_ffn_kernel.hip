// Persistent fused MoE expert-FFN forward for gfx950 (MI355X).
//
// One launch of G workgroups (G = CUs - reserve, even) runs the whole call.
// Routing, small calls (T*k <= kLocalRouteSlots): every workgroup builds the
// routing tables of the whole call in its own LDS (histogram, prefix sums,
// stable ranks); workgroup 0 publishes them.  Large calls:
//   R1  per-chunk expert histogram of topk_idx (one chunk per workgroup at
//       most)                                                -- grid barrier 0
//   R2  every workgroup reads the whole per-chunk histogram: expert totals,
//       prefix sums in LDS, the first row of each expert in its own chunk;
//       stable scatter of its chunk                          -- grid barrier 1
// Then, for every call:
//   L1  tile queue of L1 tiles: gathered x rows x W1 on scaled MFMA, fused
//       SwiGLU + clamp + 1x32 e8m0 re-quantisation -> h      -- grid barrier 2
//   L2  tile queue of L2 tiles: h x W2 -> o per routed row (bf16; fp32 for the BF16
//       recipe)                                               -- grid barrier 3
//   C   combine: y[t] = sum over valid slots j (ascending) of w[t,j] o[row]
//   X   the last workgroup out re-zeroes the control block.
// The stages follow the method of the MegaMoE pages: dispatch (expert count,
// source token / top-k index write: SM90 MegaMoE dev log, Phase 2), L1 GEMM,
// activation with clamp and re-quantisation into l2_acts / l2_acts_sf (dev
// log, Phase 1 buffer views; sglang PR digest, key code), L2 GEMM, combine.
// Every counter is reset per call and nothing is keyed on a launch id
// ("[Bugfix] Reset MegaMoE combine readiness for CUDA graph replay").
//
// Hand-offs between workgroups use whole-grid barriers only.  The 8 XCDs of
// MI355X have separate L2 caches, so publishing data to another workgroup
// needs an agent-scope release (a write-back of the XCD's L2) and consuming
// it an acquire (an invalidate); per-tile hand-offs (one release per L1 tile,
// one acquire per L2 tile) measured slower than one barrier between the
// phases, whose cost is the imbalance of the last L1 tiles.
//
// GEMM tiles: weights are the MFMA A operand (rows = output features), tokens
// the B operand (columns), so a lane holds 4 consecutive features of one
// token: the gate and up values of a feature meet in the same lane and the
// 1x32 amax along the intermediate dimension is an in-lane max plus two
// cross-lane steps.  Token blocks of 16/32 rows (few rows per expert) use
// wave tiles: every wave claims its own tile and streams weights and token
// rows through a register ring.  Token blocks of 64/128 rows use workgroup
// tiles: 4 waves x 64 weight rows share the token rows through LDS.
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
constexpr uint32_t kQueueClosed = 0x80000000u;
enum { BAR_HIST = 0, BAR_SCATTER = 1, BAR_L1 = 2, BAR_L2 = 3 };

template <int RECIPE, int BM>
struct Cfg {
  static constexpr bool kBF16 = RECIPE == 0;
  static constexpr bool kW4 = RECIPE == 2;
  static constexpr bool kB128 = RECIPE == 3;          // fp32 scales per 1x128 / 128x128 block
  static constexpr int KS = kBF16 ? 64 : 128;        // K elements per stage (128 bytes of a token row)
  static constexpr int ADW = kW4 ? 4 : 8;            // dwords of A per lane per 16-row block per stage
  static constexpr int NTB = BM / 16;                // 16-token blocks
  static constexpr int P = 2;                        // A register ring depth (stages in flight)
  static constexpr int PB = BM <= 32 ? 2 : 1;        // B register prefetch depth (stages)
  static constexpr int BSTAGE = BM * 128;            // bytes of B per stage
  static constexpr int BUNITS = BM * 8;              // 16-byte pieces of B per stage
  static constexpr int BPT = (BUNITS + kThreads - 1) / kThreads;
  static constexpr bool kStream = false;             // non-temporal weight loads (measured slower)
};

struct Shared {
  int off[kMaxExperts + 1];     // expert row offsets
  int mbo[kMaxExperts + 1];     // expert token-block offsets
  int cnt[kMaxExperts];         // expert counts / histogram scratch
  int pfx[kMaxExperts];         // rows of each expert in the routing chunks before this workgroup's
  int scan[4];
  int flag;
  uint32_t tile;
};

// Routing scratch in LDS: per-wave running counters of the scatter and, for a
// small call, the row -> slot table of the whole call.  The 128-row tile
// kernel keeps the counters inside its first ring buffer and has no table
// (its calls always route through the workspace).
typedef int WaveCounters[4][kMaxExperts];

template <int BM>
struct SharedB {
  uint8_t b[2][BM * 128] __attribute__((aligned(16)));
  uint32_t bsf[2][BM];
  uint32_t boff[BM];     // byte offset of token row m of the tile (x row for L1, h row for L2)
  uint32_t bsfoff[BM];   // byte offset of its scale row
};

// Four consecutive values of a routed row's L2 result (element index idx of
// the [rows][H] buffer): fp32 for the BF16 recipe; bf16, rounded to nearest
// even, for the e4m3 recipes (the output type; the combine sums in fp32).
template <int RECIPE>
__device__ __forceinline__ void store_o4(const KParams& p, size_t idx, const v4f& v) {
  if constexpr (RECIPE == 0) {
    stg16f((float*)p.o + idx, v);
  } else {
    stg8((uint16_t*)p.o + idx, bf16x2(v[0], v[1]), bf16x2(v[2], v[3]));
  }
}

// Slot of routed row `row`: from LDS for a small call, else from the workspace.
__device__ __forceinline__ int route_slot(const KParams& p, const int* lr2s, bool local, int row) {
  return local ? lr2s[row] : (int)ldg4(p.r2s + row);
}

// ---------------------------------------------------------------------------
// status / abort
// ---------------------------------------------------------------------------
__device__ __forceinline__ void raise_status(const KParams& p, int code, bool fatal) {
  int expected = 0;
  __hip_atomic_compare_exchange_strong(&p.ctrl->status, &expected, code, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  if (fatal) {
    st_relaxed(&p.ctrl->abort, 1u);
    st_relaxed(&p.ctrl->tile_next, kQueueClosed);   // every later claim lands past the last tile
    st_relaxed(&p.ctrl->tile_next2, kQueueClosed);
    for (int l = 0; l < 2; l++)
      for (int r = 0; r < 8; r++) st_relaxed(&p.ctrl->xq[l][r], kQueueClosed);
  }
}

// Whole-grid barrier `id`, the seq-th barrier of the call (from 0): every
// workgroup arrives once per call, in two levels.  A workgroup counts itself
// in its group's counter (group = blockIdx % 8, each counter on a 128-byte
// line of its own, so the arrivals spread over 8 counters instead of queueing
// G deep on one); the last workgroup of a group counts the group in the root
// counter bar[id]; every workgroup waits until all groups are in.  A group
// counter accumulates over the call's barriers: barrier seq is complete for a
// group of n workgroups when it reaches (seq + 1) * n.  The wait is bounded:
// on timeout the call is aborted with ST_TIMEOUT.  Returns false when the
// call is aborted.
__device__ bool grid_barrier(const KParams& p, int id, int seq, Shared& sh) {
  fence_release();
  __syncthreads();
  if (threadIdx.x == 0) {
    int ok = 1;
    const uint32_t G = gridDim.x, grp = blockIdx.x % kBarGroups;
    const uint32_t gsize = (G - grp + kBarGroups - 1) / kBarGroups;
    const uint32_t groups = G < (uint32_t)kBarGroups ? G : (uint32_t)kBarGroups;
    const uint32_t old = add_acq_rel(p.bars + grp * kBarLineWords, 1u);
    if (old == (uint32_t)(seq + 1) * gsize - 1u) add_release(&p.ctrl->bar[id], 1u);
    const uint64_t t0 = now_ticks();
    while (ld_relaxed(&p.ctrl->bar[id]) < groups) {
      if (ld_relaxed(&p.ctrl->abort)) { ok = 0; break; }
      if (now_ticks() - t0 > p.timeout_ticks) { raise_status(p, ST_TIMEOUT, true); ok = 0; break; }
      __builtin_amdgcn_s_sleep(1);
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

// Entry check of the per-call state.  Every word of the control block and of
// the barrier group counters must be zero when a call starts (the workspace
// is zeroed once after allocation and every call leaves them zeroed).  Workgroup 0 reads all of it before any
// workgroup of this call writes to it -- the others wait for its verdict --
// so the check never sees this call's own counters.  A dirty block is
// reported once (out_status = DIRTY_WORKSPACE), marked aborted so that no
// wait of this call can block, and otherwise left as found: every workgroup
// then skips all work, barriers and the exit reset, and later calls stay
// dirty until the caller zeroes the workspace.  Returns the verdict (a wait
// that runs out counts as not clean and raises TIMEOUT).
constexpr uint32_t kVerdictClean = 1u, kVerdictDirty = 2u;

__device__ uint32_t entry_verdict(const KParams& p, Shared& sh) {
  const int tid = threadIdx.x;
  uint32_t* words = reinterpret_cast<uint32_t*>(p.ctrl);
  if (blockIdx.x == 0) {
    uint32_t w = tid < kCtrlWords ? ld_relaxed(words + tid) : 0u;
    for (int i = tid; i < kBarGroups * kBarLineWords; i += kThreads) w |= ld_relaxed(p.bars + i);
    const int nonzero = __syncthreads_or(w != 0u);
    if (tid == 0) {
      if (nonzero) {
        st_relaxed(&p.ctrl->abort, 1u);
        st_relaxed(&p.ctrl->verdict, kVerdictDirty);
        if (p.out_status) *p.out_status = ST_DIRTY;
      } else {
        st_relaxed(&p.ctrl->verdict, kVerdictClean);
      }
    }
    return nonzero ? kVerdictDirty : kVerdictClean;
  }
  if (tid == 0) {
    uint32_t v;
    const uint64_t t0 = now_ticks();
    while ((v = ld_relaxed(&p.ctrl->verdict)) == 0u) {
      if (now_ticks() - t0 > p.timeout_ticks) {
        raise_status(p, ST_TIMEOUT, true);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    sh.tile = v;
  }
  __syncthreads();
  const uint32_t v = sh.tile;
  __syncthreads();
  return v;
}

// ---------------------------------------------------------------------------
// Routing
// ---------------------------------------------------------------------------
// R1 (large calls): per-chunk histograms, chunk c = slots [c * cs, (c + 1) * cs).
__device__ void phase_histogram(const KParams& p, Shared& sh, int S, int C, int cs) {
  const int tid = threadIdx.x;
  int bad = 0;
  for (int c = blockIdx.x; c < C; c += gridDim.x) {
    for (int e = tid; e < p.E; e += kThreads) sh.cnt[e] = 0;
    __syncthreads();
    const int beg = c * cs;
    const int end = min(S, beg + cs);
    for (int s = beg + tid; s < end; s += kThreads) {
      const int e = p.idx[s];
      if ((unsigned)e < (unsigned)p.E) atomicAdd(&sh.cnt[e], 1);
      else if (e != -1) bad = 1;
    }
    __syncthreads();
    for (int e = tid; e < p.E; e += kThreads) p.hist[(size_t)c * p.E + e] = sh.cnt[e];
    __syncthreads();
  }
  if (bad) raise_status(p, ST_BAD_EXPERT_INDEX, false);
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

// Row offsets and token-block offsets of the experts from sh.cnt.
__device__ void build_tables(const KParams& p, Shared& sh, WaveCounters& wcnt, int bm) {
  const int tid = threadIdx.x;
  table_scan(sh.cnt, sh.off, p.E, sh);
  for (int e = tid; e < p.E; e += kThreads) wcnt[0][e] = (sh.cnt[e] + bm - 1) / bm;
  __syncthreads();
  table_scan(wcnt[0], sh.mbo, p.E, sh);
}

// Counts and offsets to the workspace and the optional outputs.
__device__ void publish_tables(const KParams& p, const Shared& sh) {
  for (int e = threadIdx.x; e <= p.E; e += kThreads) {
    p.offsets[e] = sh.off[e];
    if (p.out_offsets) p.out_offsets[e] = sh.off[e];
    if (e < p.E) {
      p.counts[e] = sh.cnt[e];
      if (p.out_counts) p.out_counts[e] = sh.cnt[e];
    }
  }
}

// Stable scatter of the slots [beg, end): slot order inside an expert is the
// ascending slot index.  The range is split into 4 contiguous quarters, one
// per wave; a wave walks its quarter 64 slots at a time, ranking lanes with
// equal expert id by a ballot match, and keeps a running count per expert in
// LDS.  The first row of expert e in this range is off[e] + (prefix ? prefix[e] : 0).
// Rows go to the LDS table `lds_r2s` and/or, when `to_global`, to the
// workspace and the optional outputs.
__device__ void scatter_range(const KParams& p, Shared& sh, WaveCounters& wcnt, int beg, int end, const int* prefix,
                              int* lds_r2s, bool to_global) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = p.E;
  const int NB = E > 1 ? 32 - __clz(E - 1) : 0;
  const uint64_t lt = (1ull << lane) - 1ull;
  const int quarter = ((end - beg + 3) / 4 + 63) / 64 * 64;
  const int wbeg = beg + wave * quarter;
  const int wend = min(end, wbeg + quarter);
  for (int e = lane; e < E; e += 64) wcnt[wave][e] = 0;
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
    if (valid && __popcll(m & lt) == 0) wcnt[wave][e] += __popcll(m);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kThreads) {
    int run = sh.off[e] + (prefix ? prefix[e] : 0);
    for (int w = 0; w < 4; w++) {
      const int t = wcnt[w][e];
      wcnt[w][e] = run;
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
    const int base = valid ? wcnt[wave][e] : 0;
    if (valid && rank == 0) wcnt[wave][e] = base + __popcll(m);
    if (valid) {
      const int row = base + rank;
      if (lds_r2s) lds_r2s[row] = s;
      if (to_global) {
        p.r2s[row] = s;
        p.s2r[s] = row;
        if (p.xsg) {  // the token's activation scales, one dword per K stage, to the row's column
          // (8 loads issued before their 8 stores: the two buffers may alias as far as the
          // compiler knows, so a load after a store would wait for the store's round trip)
          const uint32_t* src = reinterpret_cast<const uint32_t*>(p.x_sf) + (size_t)(s / p.k) * (size_t)(p.H >> 7);
          const int nst = p.H >> 7;
          for (int st0 = 0; st0 < nst; st0 += 8) {
            uint32_t v[8];
#pragma unroll
            for (int j = 0; j < 8; j++) v[j] = st0 + j < nst ? src[st0 + j] : 0u;
#pragma unroll
            for (int j = 0; j < 8; j++)
              if (st0 + j < nst) p.xsg[(size_t)(st0 + j) * p.sg_rows + row] = v[j];
          }
        }
        if (p.out_r2s) p.out_r2s[row] = s;
        if (p.out_s2r) p.out_s2r[s] = row;
      }
    } else if (inr && to_global) {
      p.s2r[s] = -1;
      if (p.out_s2r) p.out_s2r[s] = -1;
    }
  }
  __syncthreads();
}

// Small call: every workgroup routes the whole call in LDS; workgroup 0
// publishes the tables (read by the combine after later barriers).
__device__ void phase_route_local(const KParams& p, Shared& sh, WaveCounters& wcnt, int* lr2s, int S, int bm) {
  const int tid = threadIdx.x;
  for (int e = tid; e < p.E; e += kThreads) sh.cnt[e] = 0;
  __syncthreads();
  int bad = 0;
  for (int s = tid; s < S; s += kThreads) {
    const int e = p.idx[s];
    if ((unsigned)e < (unsigned)p.E) atomicAdd(&sh.cnt[e], 1);
    else if (e != -1) bad = 1;
  }
  __syncthreads();
  if (bad && blockIdx.x == 0) raise_status(p, ST_BAD_EXPERT_INDEX, false);
  build_tables(p, sh, wcnt, bm);
  if (blockIdx.x == 0) publish_tables(p, sh);
  scatter_range(p, sh, wcnt, 0, S, nullptr, lr2s, blockIdx.x == 0);
}

// Large call, R2: every workgroup reads the whole per-chunk histogram (C <= 256
// rows of E counts, coalesced across the threads, eight rows in flight): the
// expert totals give the tables, the counts of the chunks before its own the
// first row of each expert inside its chunk (C <= gridDim.x: one chunk per
// workgroup at most); then the stable scatter of its chunk.
__device__ void phase_scatter_global(const KParams& p, Shared& sh, WaveCounters& wcnt, int S, int C, int cs, int bm) {
  const int tid = threadIdx.x;
  const int own = blockIdx.x;
  for (int e = tid; e < p.E; e += kThreads) {
    int total = 0, before = 0, c = 0;
    for (; c + 8 <= C; c += 8) {
      int v[8];
#pragma unroll
      for (int j = 0; j < 8; j++) v[j] = p.hist[(size_t)(c + j) * p.E + e];
#pragma unroll
      for (int j = 0; j < 8; j++) {
        total += v[j];
        before += c + j < own ? v[j] : 0;
      }
    }
    for (; c < C; c++) {
      const int v = p.hist[(size_t)c * p.E + e];
      total += v;
      before += c < own ? v : 0;
    }
    sh.cnt[e] = total;
    sh.pfx[e] = before;
  }
  __syncthreads();
  build_tables(p, sh, wcnt, bm);
  if (blockIdx.x == 0) publish_tables(p, sh);
  if (own < C) scatter_range(p, sh, wcnt, own * cs, min(S, (own + 1) * cs), sh.pfx, nullptr, true);
}

// ---------------------------------------------------------------------------
// GEMM tiles
// ---------------------------------------------------------------------------
template <bool NT>
__device__ __forceinline__ v4i load16(const uint8_t* ptr) {
  if constexpr (NT) return ldg16_nt(ptr);
  else return ldg16(ptr);
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

// One tile: expert e, token block mb (BM routed rows), feature block nb.
// L1: 4 waves x (32 gate + 32 up rows) = 128 intermediate features;
// L2: 4 waves x 64 rows = 256 hidden outputs.
// TILED (e2m1 weights in the TILED layout): a wave's weight rows of a K stage
// are one contiguous 1 KB piece per 16-row block, already in operand order,
// and a lane's stage scales one dword of its row's group of four stages.
template <int RECIPE, int BM, bool TILED>
__device__ void gemm_tile(const KParams& p, Shared& sh, SharedB<BM>& sb, const int* lr2s, bool local, bool l1, int e, int mb,
                          int nb) {
  using C = Cfg<RECIPE, BM>;
  static_assert(!TILED || RECIPE == 2, "the TILED layout holds e2m1 weights");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, r16 = lane & 15;
  const int H = p.H, I = p.I;
  const int row0 = sh.off[e] + mb * BM;
  const int nrows = min(BM, sh.cnt[e] - mb * BM);
  const int K = l1 ? H : I;
  const int nk = K / C::KS;
  const size_t wrow_bytes = C::kW4 ? (size_t)K / 2 : (C::kBF16 ? (size_t)K * 2 : (size_t)K);
  const size_t wsf_row = (size_t)K / 32;

  // B rows of the tile: gathered x rows (L1) or consecutive h rows (L2)
  const uint8_t* bbase = l1 ? p.x : p.h;
  const uint8_t* bsfbase = l1 ? p.x_sf : p.h_sf;
  if (tid < BM) {
    const int m = tid;
    if (l1) {
      const uint32_t tok = (uint32_t)(route_slot(p, lr2s, local, row0 + (m < nrows ? m : 0)) / p.k);
      sb.boff[m] = tok * (uint32_t)H * (C::kBF16 ? 2u : 1u);
      sb.bsfoff[m] = tok * (uint32_t)(H / 32);
    } else {
      const uint32_t r = (uint32_t)(row0 + m);  // rows past the expert stay inside the padded h buffer
      sb.boff[m] = r * (uint32_t)I * (C::kBF16 ? 2u : 1u);
      sb.bsfoff[m] = r * (uint32_t)(I / 32);
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
    // (1, 128, 128): fp32 scales [E][2I/128][H/128]; else one e8m0 byte per row and 32-block
    Wsf = C::kBF16 ? nullptr
                   : p.w1_sf + (C::kB128 ? (size_t)e * (2 * I / 128) * (K / 128) * 4 : (size_t)e * 2 * I * wsf_row);
  } else {
    const int n0 = nb * 256 + wave * 64;
    active = n0 < H;
    arow[0] = n0; arow[1] = n0 + 16; arow[2] = n0 + 32; arow[3] = n0 + 48;
    W = p.w2 + (size_t)e * H * wrow_bytes;
    Wsf = C::kBF16 ? nullptr
                   : p.w2_sf + (C::kB128 ? (size_t)e * (H / 128) * (K / 128) * 4 : (size_t)e * H * wsf_row);
  }
  const uint8_t* aptr[4];
  const uint8_t* sptr[4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    if constexpr (C::kB128) {
      // e4m3 rows as for FP8 x FP8; the stage scales of the row's 128-row block: K/128 fp32 values
      const size_t r = (size_t)(active ? arow[j] + r16 : r16);
      aptr[j] = W + r * wrow_bytes + (size_t)g * 16;
      sptr[j] = Wsf + (size_t)((active ? arow[j] : 0) / 128) * (size_t)(K / 128) * 4;
    } else if constexpr (TILED) {
      // 16-row block of this row block (inactive waves stream block 0): weights at (blk * nk + s) KB,
      // scales of stage s at (blk * nk + 4 * (s / 4)) * 64 + r16 * 4 * n(s) + (s % 4) * 4
      const size_t blk = (size_t)(active ? arow[j] >> 4 : 0);
      aptr[j] = W + blk * (size_t)nk * 1024 + (size_t)lane * 16;
      sptr[j] = Wsf + blk * (size_t)nk * 64;
    } else {
      const size_t r = (size_t)(active ? arow[j] + r16 : r16);  // inactive waves stream a valid dummy row
      size_t lane_off;
      if constexpr (C::kW4) lane_off = (size_t)g * 16;          // e2m1: elements g*32..g*32+31
      else if constexpr (C::kBF16) lane_off = (size_t)g * 32;   // bf16: elements g*16..g*16+15
      else lane_off = (size_t)g * 16;                           // e4m3: bytes g*16 and 64+g*16
      aptr[j] = W + r * wrow_bytes + lane_off;
      sptr[j] = C::kBF16 ? nullptr : Wsf + r * wsf_row;
    }
  }
  __syncthreads();  // boff / bsfoff visible

  v4f acc[4][C::NTB];
#pragma unroll
  for (int j = 0; j < 4; j++)
#pragma unroll
    for (int t = 0; t < C::NTB; t++) acc[j][t] = v4f{0.f, 0.f, 0.f, 0.f};

  v4i ar[C::P][4][C::ADW / 4];
  uint32_t sar[C::P][4];
  v4i br[C::PB][C::BPT];
  uint32_t bsr[C::PB];

  // Loads are issued without branches (inactive waves read a valid dummy row,
  // spare threads duplicate a B piece) so the waitcnt pass can keep the ring
  // in flight: a load inside a conditional block makes it drain all counters.
  auto load_a = [&](int slot, int ks) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const size_t kb = (size_t)ks * 128;  // 128 bytes of a bf16 row per stage, 64 of e2m1, 128 of e4m3
      if constexpr (TILED) {
        ar[slot][j][0] = load16<C::kStream>(aptr[j] + (size_t)ks * 1024);
        const int g4 = ks & ~3, n = min(4, nk - g4);
        sar[slot][j] = ldg4(sptr[j] + (size_t)g4 * 64 + (size_t)(r16 * 4 * n + (ks & 3) * 4));
      } else if constexpr (C::kW4) {
        ar[slot][j][0] = load16<C::kStream>(aptr[j] + (size_t)ks * 64);
      } else if constexpr (C::kBF16) {
        ar[slot][j][0] = load16<C::kStream>(aptr[j] + kb);
        ar[slot][j][1] = load16<C::kStream>(aptr[j] + kb + 16);
      } else {
        ar[slot][j][0] = load16<C::kStream>(aptr[j] + kb);
        ar[slot][j][1] = load16<C::kStream>(aptr[j] + kb + 64);
      }
      if constexpr (!C::kBF16 && !TILED) sar[slot][j] = ldg4(sptr[j] + (size_t)ks * 4);
    }
  };
  auto load_b = [&](int slot, int ks) {
#pragma unroll
    for (int u = 0; u < C::BPT; u++) {
      const int unit = (tid + u * kThreads) % C::BUNITS;
      br[slot][u] = ldg16(bbase + sb.boff[unit >> 3] + (size_t)ks * 128 + (unit & 7) * 16);
    }
    if constexpr (!C::kBF16) bsr[slot] = ldg4(bsfbase + sb.bsfoff[tid % BM] + (size_t)ks * 4);
  };
  auto store_b = [&](int slot, int buf) {
#pragma unroll
    for (int u = 0; u < C::BPT; u++) {
      const int unit = (tid + u * kThreads) % C::BUNITS;   // duplicates write identical bytes
      const int m = unit >> 3, q = unit & 7;
      const int half = C::kBF16 ? (q & 1) : (q >> 2);
      const int gg = C::kBF16 ? (q >> 1) : (q & 3);
      const int dst = (((m >> 4) * 2 + half) * 64 + gg * 16 + (m & 15)) * 16;
      *(v4i*)(&sb.b[buf][dst]) = br[slot][u];
    }
    if constexpr (!C::kBF16) sb.bsf[buf][tid % BM] = bsr[slot];
  };
  auto compute = [&](int slot, int buf) {
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
      } else if constexpr (C::kB128) {
        // unit block scales in the MFMA (byte 127 = 2^0); the stage's fp32 factors, weight block times
        // token, are folded into the running sum with one FMA per element
        const v8i bb = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        const float fb = __uint_as_float(sb.bsf[buf][t * 16 + r16]);
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const v8i aa = {ar[slot][j][0][0], ar[slot][j][0][1], ar[slot][j][0][2], ar[slot][j][0][3],
                          ar[slot][j][1][0], ar[slot][j][1][1], ar[slot][j][1][2], ar[slot][j][1][3]};
          const v4f part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aa, bb, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0,
                                                                            127, 0, 127);
          const float f = __uint_as_float(sar[slot][j]) * fb;
#pragma unroll
          for (int c = 0; c < 4; c++) acc[j][t][c] = __builtin_fmaf(part[c], f, acc[j][t][c]);
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

  // Pipeline: the A ring runs P stages ahead in registers; B runs PB stages
  // ahead in registers plus one in LDS (double buffer).  Steady-state groups
  // of P stages carry no branches; the last groups drain with guards.
#pragma unroll
  for (int s = 0; s < C::P; s++) load_a(s, s < nk ? s : nk - 1);
#pragma unroll
  for (int s = 0; s < C::PB; s++) load_b(s, s < nk ? s : nk - 1);
  store_b(0, 0);
  int ks0 = 0;
  for (; ks0 + 2 * C::P <= nk; ks0 += C::P) {
#pragma unroll
    for (int s = 0; s < C::P; s++) {
      const int ks = ks0 + s;
      load_b(s % C::PB, ks + C::PB);
      __syncthreads();
      compute(s, s & 1);
      load_a(s, ks + C::P);
      store_b((s + 1) % C::PB, (s + 1) & 1);
    }
  }
  for (; ks0 < nk; ks0 += C::P) {
#pragma unroll
    for (int s = 0; s < C::P; s++) {
      const int ks = ks0 + s;
      if (ks < nk) {
        if (ks + C::PB < nk) load_b(s % C::PB, ks + C::PB);
        __syncthreads();
        compute(s, s & 1);
        if (ks + C::P < nk) load_a(s, ks + C::P);
        if (ks + 1 < nk) store_b((s + 1) % C::PB, (s + 1) & 1);
      }
    }
  }
  __syncthreads();  // every wave is done with the B stages before the next tile refills them

  if constexpr (C::kB128) {
    if (l1) {
      // re-quantisation per 1x128 block of h: the tile's 128 features of a token are spread over the 4
      // waves (32 each; every wave is active, I being a multiple of 128), so the block amax goes through
      // LDS (the first B buffer, free now): s = max(fp32(amax / 448), smallest normal fp32), code = e4m3 of
      // the IEEE fp32 quotient h / s
      float* amx = reinterpret_cast<float*>(&sb.b[0][0]);
#pragma unroll
      for (int t = 0; t < C::NTB; t++) {
        float a = 0.f;
#pragma unroll
        for (int hh = 0; hh < 2; hh++)
#pragma unroll
          for (int j = 0; j < 4; j++)
            a = fmax_nn(a, __builtin_fabsf(swiglu(acc[hh][t][j], acc[2 + hh][t][j], clamp_bound(p.clamp_on, p.clamp))));
        a = max_over_rows(a);
        if (g == 0) amx[wave * 64 + t * 16 + r16] = a;
      }
      __syncthreads();
      const int i0 = nb * 128 + wave * 32;
#pragma unroll
      for (int t = 0; t < C::NTB; t++) {
        const int m = t * 16 + r16;
        const float a = __builtin_fmaxf(__builtin_fmaxf(amx[m], amx[64 + m]), __builtin_fmaxf(amx[128 + m], amx[192 + m]));
        const float sc = __builtin_fmaxf(a / 448.0f, 0x1p-126f);
        if (m < nrows) {
          const size_t row = (size_t)(row0 + m);
#pragma unroll
          for (int hh = 0; hh < 2; hh++) {
            float q[4];
#pragma unroll
            for (int j = 0; j < 4; j++) q[j] = swiglu(acc[hh][t][j], acc[2 + hh][t][j], clamp_bound(p.clamp_on, p.clamp)) / sc;
            stg4(p.h + row * I + (size_t)(i0 + hh * 16 + 4 * g), e4m3x4(q[0], q[1], q[2], q[3]));
          }
          if (wave == 0 && g == 0) stg4(p.h_sf + row * (size_t)(I / 32) + (size_t)nb * 4, __float_as_uint(sc));
        }
      }
      return;
    }
  }
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
        for (int j = 0; j < 4; j++) hv[hh * 4 + j] = swiglu(acc[hh][t][j], acc[2 + hh][t][j], clamp_bound(p.clamp_on, p.clamp));
      const size_t row = (size_t)(row0 + m);
      if constexpr (C::kBF16) {
        if (m < nrows) {
#pragma unroll
          for (int hh = 0; hh < 2; hh++) {
            const uint32_t lo = f32_to_bf16(hv[hh * 4 + 0]) | (f32_to_bf16(hv[hh * 4 + 1]) << 16);
            const uint32_t hi = f32_to_bf16(hv[hh * 4 + 2]) | (f32_to_bf16(hv[hh * 4 + 3]) << 16);
            stg8(p.h + (row * I + (size_t)(i0 + hh * 16 + 4 * g)) * 2, lo, hi);
          }
        }
      } else {
        float amax = 0.f;
#pragma unroll
        for (int j = 0; j < 8; j++) amax = fmax_nn(amax, __builtin_fabsf(hv[j]));
        amax = max_over_rows(amax);
        const int E = block_scale_exp(amax);
        if (m < nrows) {
#pragma unroll
          for (int hh = 0; hh < 2; hh++) {
            const uint32_t word = e4m3x4(__builtin_amdgcn_ldexpf(hv[hh * 4 + 0], -E), __builtin_amdgcn_ldexpf(hv[hh * 4 + 1], -E),
                                          __builtin_amdgcn_ldexpf(hv[hh * 4 + 2], -E), __builtin_amdgcn_ldexpf(hv[hh * 4 + 3], -E));
            stg4(p.h + row * I + (size_t)(i0 + hh * 16 + 4 * g), word);
          }
          if (g == 0) stg1(p.h_sf + row * (size_t)(I / 32) + (size_t)(i0 / 32), (uint8_t)(E + 127));
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
        for (int j = 0; j < 4; j++) store_o4<RECIPE>(p, row * H + (size_t)(arow[j] + 4 * g), acc[j][t]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Wave tiles (token blocks of 16 or 32 rows: the weight-streaming regime).
// Each wave claims its own tile -- 32 intermediate features (gate + up rows)
// of L1 or 64 hidden rows of L2, times the token block -- and streams A
// (weights) and B (token rows) for the same stage into one register ring, so
// stages complete in issue order and no LDS or barrier sits in the K loop.
// ---------------------------------------------------------------------------
template <int RECIPE, int BM>
struct WCfg {
  static constexpr bool kBF16 = RECIPE == 0;
  static constexpr bool kW4 = RECIPE == 2;
  static constexpr int ADW = kW4 ? 4 : 8;          // A dwords per lane per 16-row block per stage
  static constexpr int NTB = BM / 16;
  static constexpr int P = kW4 ? (BM == 16 ? 4 : 3) : 2;  // stages in flight per wave
};

template <int RECIPE, int BM>
__device__ void wave_tile(const KParams& p, const Shared& sh, const int* lr2s, bool local, bool l1, int e, int mb, int blk) {
  using C = WCfg<RECIPE, BM>;
  const int lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
  const int H = p.H, I = p.I;
  const int row0 = sh.off[e] + mb * BM;
  const int nrows = min(BM, sh.cnt[e] - mb * BM);
  const int K = l1 ? H : I;
  const int nk = K / (C::kBF16 ? 64 : 128);
  const size_t wrow_bytes = C::kW4 ? (size_t)K / 2 : (C::kBF16 ? (size_t)K * 2 : (size_t)K);
  const size_t wsf_row = (size_t)K / 32;

  int arow[4];
  const uint8_t* W;
  const uint8_t* Wsf;
  if (l1) {
    const int i0 = blk * 32;
    arow[0] = i0; arow[1] = i0 + 16; arow[2] = I + i0; arow[3] = I + i0 + 16;
    W = p.w1 + (size_t)e * 2 * I * wrow_bytes;
    Wsf = C::kBF16 ? nullptr : p.w1_sf + (size_t)e * 2 * I * wsf_row;
  } else {
    const int n0 = blk * 64;
    arow[0] = n0; arow[1] = n0 + 16; arow[2] = n0 + 32; arow[3] = n0 + 48;
    W = p.w2 + (size_t)e * H * wrow_bytes;
    Wsf = C::kBF16 ? nullptr : p.w2_sf + (size_t)e * H * wsf_row;
  }
  const uint8_t* aptr[4];
  const uint8_t* sptr[4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const size_t r = (size_t)(arow[j] + r16);
    aptr[j] = W + r * wrow_bytes + (size_t)g * (C::kBF16 ? 32 : 16);
    sptr[j] = C::kBF16 ? nullptr : Wsf + r * wsf_row;
  }
  // B rows of this lane (token m = t*16 + r16 of the block)
  const uint8_t* bbase = l1 ? p.x : p.h;
  const uint8_t* bsfbase = l1 ? p.x_sf : p.h_sf;
  uint32_t boff[C::NTB], bsfoff[C::NTB];
#pragma unroll
  for (int t = 0; t < C::NTB; t++) {
    const int m = t * 16 + r16;
    if (l1) {
      const uint32_t tok = (uint32_t)(route_slot(p, lr2s, local, row0 + (m < nrows ? m : 0)) / p.k);
      boff[t] = tok * (uint32_t)H * (C::kBF16 ? 2u : 1u);
      bsfoff[t] = tok * (uint32_t)(H / 32);
    } else {
      const uint32_t r = (uint32_t)(row0 + m);  // rows past the expert stay inside the padded h buffer
      boff[t] = r * (uint32_t)I * (C::kBF16 ? 2u : 1u);
      bsfoff[t] = r * (uint32_t)(I / 32);
    }
  }
  // lane's two 16-byte pieces inside the 128-byte stage chunk of a B row
  const uint32_t bl0 = C::kBF16 ? (uint32_t)g * 32 : (uint32_t)g * 16;
  const uint32_t bl1 = C::kBF16 ? (uint32_t)g * 32 + 16 : 64u + (uint32_t)g * 16;

  v4f acc[4][C::NTB];
#pragma unroll
  for (int j = 0; j < 4; j++)
#pragma unroll
    for (int t = 0; t < C::NTB; t++) acc[j][t] = v4f{0.f, 0.f, 0.f, 0.f};
  v4i ar[C::P][4][C::ADW / 4];
  uint32_t sar[C::P][4];
  v4i brr[C::P][C::NTB][2];
  uint32_t sbr[C::P][C::NTB];

  auto load = [&](int slot, int ks) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const size_t kb = (size_t)ks * 128;
      if constexpr (C::kW4) {
        ar[slot][j][0] = ldg16(aptr[j] + (size_t)ks * 64);
      } else if constexpr (C::kBF16) {
        ar[slot][j][0] = ldg16(aptr[j] + kb);
        ar[slot][j][1] = ldg16(aptr[j] + kb + 16);
      } else {
        ar[slot][j][0] = ldg16(aptr[j] + kb);
        ar[slot][j][1] = ldg16(aptr[j] + kb + 64);
      }
      if constexpr (!C::kBF16) sar[slot][j] = ldg4(sptr[j] + (size_t)ks * 4);
    }
#pragma unroll
    for (int t = 0; t < C::NTB; t++) {
      const uint8_t* rb = bbase + boff[t] + (size_t)ks * 128;
      brr[slot][t][0] = ldg16(rb + bl0);
      brr[slot][t][1] = ldg16(rb + bl1);
      if constexpr (!C::kBF16) sbr[slot][t] = ldg4(bsfbase + bsfoff[t] + (size_t)ks * 4);
    }
  };
  auto compute = [&](int slot) {
#pragma unroll
    for (int t = 0; t < C::NTB; t++) {
      const v4i b0 = brr[slot][t][0], b1 = brr[slot][t][1];
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
        const int sbv = (int)(sbr[slot][t] >> (8 * g));
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

#pragma unroll
  for (int s = 0; s < C::P; s++) load(s, s < nk ? s : nk - 1);
  int ks0 = 0;
  for (; ks0 + 2 * C::P <= nk; ks0 += C::P) {
#pragma unroll
    for (int s = 0; s < C::P; s++) {
      compute(s);
      load(s, ks0 + s + C::P);
    }
  }
  for (; ks0 < nk; ks0 += C::P) {
#pragma unroll
    for (int s = 0; s < C::P; s++) {
      const int ks = ks0 + s;
      if (ks < nk) {
        compute(s);
        if (ks + C::P < nk) load(s, ks + C::P);
      }
    }
  }

  if (l1) {
    const int i0 = blk * 32;
#pragma unroll
    for (int t = 0; t < C::NTB; t++) {
      const int m = t * 16 + r16;
      float hv[8];
#pragma unroll
      for (int hh = 0; hh < 2; hh++)
#pragma unroll
        for (int j = 0; j < 4; j++) hv[hh * 4 + j] = swiglu(acc[hh][t][j], acc[2 + hh][t][j], clamp_bound(p.clamp_on, p.clamp));
      const size_t row = (size_t)(row0 + m);
      if constexpr (C::kBF16) {
        if (m < nrows) {
#pragma unroll
          for (int hh = 0; hh < 2; hh++) {
            const uint32_t lo = f32_to_bf16(hv[hh * 4 + 0]) | (f32_to_bf16(hv[hh * 4 + 1]) << 16);
            const uint32_t hi = f32_to_bf16(hv[hh * 4 + 2]) | (f32_to_bf16(hv[hh * 4 + 3]) << 16);
            stg8(p.h + (row * I + (size_t)(i0 + hh * 16 + 4 * g)) * 2, lo, hi);
          }
        }
      } else {
        float amax = 0.f;
#pragma unroll
        for (int j = 0; j < 8; j++) amax = fmax_nn(amax, __builtin_fabsf(hv[j]));
        amax = max_over_rows(amax);
        const int E = block_scale_exp(amax);
        if (m < nrows) {
#pragma unroll
          for (int hh = 0; hh < 2; hh++) {
            const uint32_t word = e4m3x4(__builtin_amdgcn_ldexpf(hv[hh * 4 + 0], -E), __builtin_amdgcn_ldexpf(hv[hh * 4 + 1], -E),
                                          __builtin_amdgcn_ldexpf(hv[hh * 4 + 2], -E), __builtin_amdgcn_ldexpf(hv[hh * 4 + 3], -E));
            stg4(p.h + row * I + (size_t)(i0 + hh * 16 + 4 * g), word);
          }
          if (g == 0) stg1(p.h_sf + row * (size_t)(I / 32) + (size_t)(i0 / 32), (uint8_t)(E + 127));
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
        for (int j = 0; j < 4; j++) store_o4<RECIPE>(p, row * H + (size_t)(arow[j] + 4 * g), acc[j][t]);
      }
    }
  }
}

// DPP rotate by 8 lanes inside each 16-lane row.
__device__ __forceinline__ int dpp_ror8(int v) { return __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, false); }

// lanes 0-7 of each 16-lane row take x0 (par 0) / rotated x0 (par 1); lanes 8-15 rotated x1 / x1
__device__ __forceinline__ v4i line_shuffle(const v4i& x0, const v4i& x1, int par, bool lo) {
  v4i r;
#pragma unroll
  for (int d = 0; d < 4; d++) {
    const int rot = dpp_ror8(par == 0 ? x1[d] : x0[d]);  // every lane executes the DPP move
    r[d] = par == 0 ? (lo ? x0[d] : rot) : (lo ? rot : x1[d]);
  }
  return r;
}

// ---------------------------------------------------------------------------
// 128-row workgroup tiles for e4m3 rows x e2m1 weights (the MFMA-bound
// regime).  4 waves x 64 weight rows x 128 routed rows, acc[j][t] for weight
// row block j and routed-row block t.  Each wave streams its own weight rows
// into a register ring kBigP stages deep.  The routed rows and the 1x32
// scales of both operands go through a kBigNB-deep LDS ring filled by buffer
// loads that write LDS directly, kBigD stages ahead; one workgroup barrier per
// 128-element K stage publishes a stage to every wave.  Waits on the ring are
// explicit: with the issue order pinned (scheduling barriers), the fill of
// stage s is complete once at most kBigWait younger vector-memory operations
// are outstanding.  Each ring buffer is its own LDS object, so the compiler's
// own wait for a DMA'd buffer only covers the fills of that buffer.
// ---------------------------------------------------------------------------
constexpr int kBigBM = 128, kBigNB = 3, kBigD = 2, kBigP = 3;
constexpr int kBigBsf = kBigBM * 128;               // routed-row scale dwords (+ a second copy)
constexpr int kBigAsf = kBigBsf + 2 * kBigBM * 4;   // weight-row scale dwords
constexpr int kBigBuf = kBigAsf + 256 * 4;          // 18432 bytes per stage
static_assert(kBigP == kBigNB && kBigD == kBigNB - 1, "ring indices assume P = NB = D + 1");
// Younger VMEM operations allowed when stage s is consumed: the weight loads
// of iteration s-D (4) and all of iteration s-1 (row pieces, 2 scale fills,
// 4 weight loads).  A tile of NT 16-row blocks fills NT/2 (at least 1) row
// pieces per wave and stage.
template <int NT>
constexpr int big_row_pieces() { return NT >= 2 ? NT / 2 : 1; }
template <int NT>
constexpr int big_wait() { return 4 + (big_row_pieces<NT>() + 6) * (kBigD - 1); }

struct BigRing {
  uint8_t* b0;
  uint8_t* b1;
  uint8_t* b2;
};

template <int NT>
__device__ __forceinline__ void big_kloop(uint8_t* __restrict__ B0, uint8_t* __restrict__ B1, uint8_t* __restrict__ B2,
                                          v4f (&acc)[4][NT], rsrc_t rW, uint32_t a_off, const uint32_t (&a_soff)[4],
                                          rsrc_t rWs, uint32_t as_full, uint32_t as_last, uint32_t sa_base,
                                          rsrc_t rX, const uint32_t (&xoff)[4],
                                          uint32_t brd0, uint32_t brd1, rsrc_t rXs, uint32_t xs_off, uint32_t xs_stride,
                                          int nk, int wave,
                                          int lane) {
  constexpr int RP = big_row_pieces<NT>();
  const int g = lane >> 4, r16 = lane & 15;
  auto BUF = [&](int u) -> uint8_t* { return u == 0 ? B0 : u == 1 ? B1 : B2; };
#pragma unroll
  for (int j = 0; j < 4; j++)
#pragma unroll
    for (int t = 0; t < NT; t++) acc[j][t] = v4f{0.f, 0.f, 0.f, 0.f};
  v4i ar[kBigP][4];

  // A stage past the end (the ring runs kBigP stages ahead) is fetched from
  // an offset past the buffer's end: the load returns zeros without a memory
  // access and still counts as one vector-memory operation for the waits.
  auto load_a = [&](int slot, int s) {
    const uint32_t voff = s < nk ? a_off : kBufDead;
#pragma unroll
    for (int j = 0; j < 4; j++) ar[slot][j] = buf_load16(rW, voff, a_soff[j] + (uint32_t)s * 1024);
  };
  // Stage s into ring buffer `buf`: 2*NT x 1 KB of routed-row bytes, whole
  // 128-byte lines: instruction q holds rows 8q..8q+7, its lane l row
  // 8q + l/8 and 16-byte chunk (l%8) ^ f, f = 4*(q&1) + l/16 (half the row's
  // index in its 16-row block), so every quad of lanes reads one 64-byte
  // segment and the operand reads below are free of LDS bank conflicts
  // (wave w issues q = RP*w .. RP*w + RP-1; brd0/brd1 address a lane's MFMA
  // operand bytes 0-15 / 16-31 of routed-row block 0), the routed-row scale dwords (waves
  // beyond the first copy load zeros from past the end of the buffer into
  // further copies, so every wave issues the same count) and the scales of
  // the wave's own 64 weight rows from the TILED layout: lane l fetches the
  // stage's dword (4 blocks) of row l%16 of its row block l/16 (the 16 rows'
  // dwords of a full group 16 bytes apart), stored as [wave][block j][row][4 bytes].
  auto dma = [&](int s, int buf) {
    uint8_t* bp = BUF(buf);
    const bool live = s < nk;
#pragma unroll
    for (int i = 0; i < RP; i++)
      buf_load_lds16(rX, bp + (wave * RP + i) * 1024, live ? xoff[i] : kBufDead, (uint32_t)s * 128);
    const int scopy = NT == 8 ? ((wave >> 1) * kBigBM + (wave & 1) * 64) : wave * 64;
    buf_load_lds4(rXs, bp + kBigBsf + scopy * 4, live ? xs_off : kBufDead, (uint32_t)s * xs_stride);
    // stage s = 4G + u: group G at (blk * nk + 4G) * 64, row stride 4 * (stages in G), dword u
    const uint32_t as_off = (s >> 2) < (nk >> 2) ? as_full : as_last;
    buf_load_lds4(rWs, bp + kBigAsf + wave * 256, live ? as_off : kBufDead, (uint32_t)((s >> 2) * 256 + (s & 3) * 4));
  };
  auto compute = [&](int slot, int buf, auto&& mid) {
    const uint8_t* bp = BUF(buf);
    int sa[4];
    // scales: one byte per lane (the dword of row r16 of block j, routed row t*16 + r16, holds the
    // stage's 4 blocks; lane group g takes byte g), read as bytes: a dword read and a shift per
    // value measured slower (the shifts sit between the LDS reads and the MFMAs)
#pragma unroll
    for (int j = 0; j < 4; j++) sa[j] = bp[sa_base + j * 64 + g];
    int sbt = bp[kBigBsf + r16 * 4 + g];
    v4i n0 = *(const v4i*)(bp + brd0);
    v4i n1 = *(const v4i*)(bp + brd1);
    __builtin_amdgcn_sched_group_barrier(0x100, 7, 0);
    __builtin_amdgcn_sched_barrier(0);
    mid();  // issued while the first reads are in flight
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < NT; t++) {
      const v8i bb = {n0[0], n0[1], n0[2], n0[3], n1[0], n1[1], n1[2], n1[3]};
      const int sbc = sbt;
      if (t < NT - 1) {  // the next block's operand and scale, read under this block's MFMAs
        sbt = bp[kBigBsf + ((t + 1) * 16 + r16) * 4 + g];
        n0 = *(const v4i*)(bp + brd0 + (t + 1) * 2048);
        n1 = *(const v4i*)(bp + brd1 + (t + 1) * 2048);
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
      }
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const v8i aa = {ar[slot][j][0], ar[slot][j][1], ar[slot][j][2], ar[slot][j][3], 0, 0, 0, 0};
        acc[j][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aa, bb, acc[j][t], 4, 0, 0, sa[j], 0, sbc);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
  };

  // No drain here: vector-memory operations issued before the ring (the
  // previous tile's stores, the tile claim in flight) only make the count
  // waits below stricter, since the ring's own operations complete in issue
  // order, and they can complete under the prologue's loads.
  // Prologue, in the steady issue order: virtual iterations -P..-1 each issue
  // the fill of stage it + D, then the weight loads of stage it + P.
  load_a(0, 0);
  __builtin_amdgcn_sched_barrier(0);
  dma(0, 0);
  __builtin_amdgcn_sched_barrier(0);
  load_a(1, 1);
  __builtin_amdgcn_sched_barrier(0);
  dma(1, 1);
  __builtin_amdgcn_sched_barrier(0);
  load_a(2, 2);
  __builtin_amdgcn_sched_barrier(0);
  int s0 = 0;
  for (; s0 + kBigP <= nk; s0 += kBigP) {
#pragma unroll
    for (int u = 0; u < kBigP; u++) {
      const int s = s0 + u;
      MOEFFN_WAIT_VMCNT(big_wait<NT>());  // this wave's fill of stage s has landed
      __builtin_amdgcn_s_barrier();       // ... and every other wave's
      // the stage's first LDS reads, then the fill of stage s + D, then the MFMAs
      compute(u, u, [&] { dma(s + kBigD, (u + kBigD) % kBigNB); });
      load_a(u, s + kBigP);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // nk % P trailing stages: already in flight in buffer / slot u
#pragma unroll
  for (int u = 0; u < kBigP - 1; u++) {
    if (s0 + u < nk) {
      MOEFFN_WAIT_VMCNT(0);
      __builtin_amdgcn_s_barrier();
      compute(u, u, [] {});
    }
  }
  // every wave is done with the ring before the next tile refills it or the
  // L2 epilogue writes into it (a full workgroup barrier: its fences keep the
  // compiler from moving LDS accesses across it)
  MOEFFN_WAIT_VMCNT(0);
  __syncthreads();
}

// One 128-row tile: expert e, token block mb, feature block nb (L1: 128
// intermediate features = 4 waves x (32 gate + 32 up rows); L2: 256 hidden
// outputs = 4 waves x 64 rows).
// NT: 16-row blocks computed (the tile's rows rounded up to 16, as 2, 4 or
// 8): a partly filled last token block of an expert skips the MFMAs and the
// routed-row fills of its empty blocks.
template <int RECIPE, int NT>
__device__ __forceinline__ void big_tile(const KParams& p, const Shared& sh, const BigRing& R, bool l1, int e, int mb, int nb) {
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6) & 3;
  const int H = p.H, I = p.I;
  const int row0 = __builtin_amdgcn_readfirstlane(sh.off[e] + mb * kBigBM);
  const int nrows = __builtin_amdgcn_readfirstlane(min(kBigBM, sh.cnt[e] - mb * kBigBM));
  const int K = l1 ? H : I;
  const int nk = K / 128;
  const uint32_t arow = (uint32_t)K / 2, srow = (uint32_t)K / 32;
  const uint32_t wrows = l1 ? 2u * (uint32_t)I : (uint32_t)H;
  // the TILED layout: 16-row block b, K stage s at (b * nk + s) KB in MFMA lane order; its scales in
  // groups of four stages per block
  const uint8_t* W = l1 ? p.w1 + (size_t)e * wrows * arow : p.w2 + (size_t)e * wrows * arow;
  const uint8_t* Ws = l1 ? p.w1_sf + (size_t)e * wrows * srow : p.w2_sf + (size_t)e * wrows * srow;
  int rb[4];  // first weight row of each 16-row block of this wave
  if (l1) {
    const int i0 = nb * 128 + wave * 32;
    rb[0] = i0; rb[1] = i0 + 16; rb[2] = I + i0; rb[3] = I + i0 + 16;
  } else {
    const int n0 = nb * 256 + wave * 64;  // rows past H (last block of an odd H/128) read as zero
    rb[0] = n0; rb[1] = n0 + 16; rb[2] = n0 + 32; rb[3] = n0 + 48;
  }
  const bool active = l1 || rb[0] < H;
  uint32_t a_soff[4];
#pragma unroll
  for (int j = 0; j < 4; j++) a_soff[j] = (uint32_t)(rb[j] >> 4) * (uint32_t)nk * 1024u;
  const rsrc_t rW = make_rsrc(W, wrows * arow);
  const rsrc_t rWs = make_rsrc(Ws, wrows * srow);
  // one 1 KB contiguous load per 16-row block and stage: every quad of lanes
  // reads one 64-byte segment (the texture unit's rate is set by the number
  // of distinct segments a quad touches; row-strided operand loads touch 4)
  const uint32_t a_off = (uint32_t)lane * 16u;
  // TILED weight scales: lane l fetches row l%16 of the wave's row block l/16 (block rb[l/16] / 16):
  // in a full group of four stages at r16 * 16, in the last group of nk % 4 stages at r16 * 4 * (nk % 4)
  const int jl = lane >> 4;
  const uint32_t blk_l = (uint32_t)(l1 ? (nb * 128 + wave * 32) / 16 + (jl & 1) + (jl >> 1) * (I / 16)
                                       : (nb * 256 + wave * 64) / 16 + jl);
  const uint32_t as_full = blk_l * (uint32_t)nk * 64u + (uint32_t)r16 * 16u;
  const uint32_t as_last = blk_l * (uint32_t)nk * 64u + (uint32_t)r16 * 4u * (uint32_t)(nk & 3);
  // ... and reads its row's dword of block j at sa_base + 64 j
  const uint32_t sa_base = (uint32_t)(kBigAsf + wave * 256 + r16 * 4);

  // routed rows of the tile (rows past the expert repeat its first row / read
  // padding): fill instruction i of this wave covers rows 8*(RP*wave + i) + l/8
  constexpr int RP = big_row_pieces<NT>();
  const int r8 = lane >> 3;
  const int ms = NT == 8 ? (wave & 1) * 64 + lane : lane;
  rsrc_t rX, rXs;
  uint32_t xoff[4] = {0u, 0u, 0u, 0u}, xs_off;
  if (l1) {
    rX = make_rsrc(p.x, (uint32_t)p.T * (uint32_t)H);
    rXs = make_rsrc(p.xsg, (uint32_t)(H / 128) * (uint32_t)p.sg_rows * 4u);
#pragma unroll
    for (int i = 0; i < RP; i++) {
      const int q = wave * RP + i, m = 8 * q + r8;
      const uint32_t tok = (uint32_t)(route_slot(p, nullptr, false, row0 + (m < nrows ? m : 0)) / p.k);
      xoff[i] = tok * (uint32_t)H + (uint32_t)(((lane & 7) ^ (4 * (q & 1) + (lane >> 4))) * 16);
    }
    xs_off = (uint32_t)(row0 + ms) * 4u;
  } else {
    const uint32_t rows_end = (uint32_t)(row0 + kBigBM);  // h is padded by kMaxBM rows
    rX = make_rsrc(p.h, rows_end * (uint32_t)I);
    rXs = make_rsrc(p.hsg, (uint32_t)(I / 128) * (uint32_t)p.sg_rows * 4u);
#pragma unroll
    for (int i = 0; i < RP; i++) {
      const int q = wave * RP + i;
      xoff[i] = (uint32_t)(row0 + 8 * q + r8) * (uint32_t)I + (uint32_t)(((lane & 7) ^ (4 * (q & 1) + (lane >> 4))) * 16);
    }
    xs_off = (uint32_t)(row0 + ms) * 4u;
  }
  const uint32_t brd0 = (uint32_t)(((r16 >> 3) * 64 + (r16 & 7) * 8 + (g ^ (r16 >> 1))) * 16);
  const uint32_t brd1 = (uint32_t)(((r16 >> 3) * 64 + (r16 & 7) * 8 + ((4 + g) ^ (r16 >> 1))) * 16);
  // A wave whose scale dwords would repeat rows another wave already loads
  // reads past the end of the buffer instead: that load returns zeros without
  // a memory access (each dword it would fetch is a cache line of its own),
  // and every wave still issues the same count.
  if (NT == 8 ? wave >= 2 : wave >= 1) xs_off = kBufDead;

  v4f acc[4][NT];
  big_kloop<NT>(R.b0, R.b1, R.b2, acc, rW, a_off, a_soff, rWs, as_full, as_last, sa_base, rX, xoff, brd0, brd1,
                rXs, xs_off, (uint32_t)p.sg_rows * 4u, nk, wave, lane);

  // The epilogues' lane indices, taken anew after the K loop: derived from
  // the thread index, their per-lane addresses would be hoisted out of the
  // tile loop and held in registers through the K loop.
  int ep_tid = tid;
  asm volatile("" : "+v"(ep_tid));
  const int ep_lane = ep_tid & 63, ep_g = ep_lane >> 4, ep_r16 = ep_lane & 15;

  if (l1) {
    // h through LDS (the ring buffers are free: the K loop ends on a
    // barrier): the tile's 128 rows x 128 code bytes go to buffer 0 (row
    // stride 144 bytes: the 4-byte writes of a wave hit 64 distinct banks),
    // the four 1x32 scale bytes of each row to buffer 1 as one dword (byte
    // `wave` = block 4 nb + wave); then the tile leaves as whole 128-byte rows
    // of h and one dword per row of h_sf and of the stage-major copy hsg.
    constexpr int kHStride = 144;
    uint8_t* hb = R.b0;
    uint8_t* sfb = R.b1;
    const float cb = clamp_bound(p.clamp_on, p.clamp);
#pragma unroll
    for (int t = 0; t < NT; t++) {
      const int m = t * 16 + ep_r16;
      float hv[8];
#pragma unroll
      for (int hh = 0; hh < 2; hh++)
#pragma unroll
        for (int j = 0; j < 4; j++) hv[hh * 4 + j] = swiglu(acc[hh][t][j], acc[2 + hh][t][j], cb);
      float amax = 0.f;
#pragma unroll
      for (int j = 0; j < 8; j++) amax = fmax_nn(amax, __builtin_fabsf(hv[j]));
      amax = max_over_rows(amax);
      const int E = block_scale_exp(amax);
#pragma unroll
      for (int hh = 0; hh < 2; hh++)
        *(uint32_t*)(hb + m * kHStride + wave * 32 + hh * 16 + 4 * ep_g) =
            e4m3x4(__builtin_amdgcn_ldexpf(hv[hh * 4 + 0], -E), __builtin_amdgcn_ldexpf(hv[hh * 4 + 1], -E),
                   __builtin_amdgcn_ldexpf(hv[hh * 4 + 2], -E), __builtin_amdgcn_ldexpf(hv[hh * 4 + 3], -E));
      if (ep_g == 0) sfb[m * 4 + wave] = (uint8_t)(E + 127);
    }
    __syncthreads();
#pragma unroll 1
    for (int k = 0; k < 4; k++) {  // 1024 pieces of 16 bytes: row piece / 8, chunk piece % 8
      const int piece = k * kThreads + ep_tid, r = piece >> 3, c = piece & 7;
      if (r < nrows)
        stg16(p.h + (size_t)(row0 + r) * I + (size_t)(nb * 128 + c * 16), *(const v4i*)(hb + r * kHStride + c * 16));
    }
    if (ep_tid < nrows) {
      const uint32_t sw = *(const uint32_t*)(sfb + ep_tid * 4);
      stg4(p.h_sf + (size_t)(row0 + ep_tid) * (size_t)(I / 32) + (size_t)nb * 4, sw);
      stg4(p.hsg + (size_t)nb * p.sg_rows + (size_t)(row0 + ep_tid), sw);
    }
  } else {
    // o through LDS, two 16-row blocks at a time (the ring buffers are free:
    // the K loop ends on a barrier): the waves' values of blocks 2q and 2q+1,
    // rounded to bf16, go to buffer q % 3 as [32 rows][256 outputs] (row
    // stride 512 + 16 bytes), then every store instruction writes two whole
    // 512-byte rows of the tile's outputs (lanes 0-31 and 32-63, 16 bytes
    // each).  A buffer is written again three pairs later, after two more
    // barriers that every wave reaches only once done reading it.  Waves
    // whose rows lie past H (the last block of an odd H/128) write nothing
    // but store the other waves' outputs.
    constexpr int kOStride = 528;
    static_assert(32 * kOStride <= kBigBuf, "a pair of 16-row blocks of o fits a ring buffer");
    const int col = (ep_lane & 31) * 8;  // this lane's 8 outputs of the tile's 256
#pragma unroll
    for (int tp = 0; tp < NT / 2; tp++) {
      uint8_t* bp = tp % 3 == 0 ? R.b0 : tp % 3 == 1 ? R.b1 : R.b2;
      if (active) {
#pragma unroll
        for (int hb = 0; hb < 2; hb++)
#pragma unroll
          for (int j = 0; j < 4; j++) {
            const v4f& a = acc[j][2 * tp + hb];
            *(uint2*)(bp + (hb * 16 + ep_r16) * kOStride + (wave * 64 + 16 * j + 4 * ep_g) * 2) =
                uint2{bf16x2(a[0], a[1]), bf16x2(a[2], a[3])};
          }
      }
      __syncthreads();
#pragma unroll
      for (int rr = 0; rr < 4; rr++) {
        const int lr = wave * 8 + rr * 2 + (ep_lane >> 5);  // row of the pair
        const int m = tp * 32 + lr;
        const v4i v = *(const v4i*)(bp + lr * kOStride + col * 2);
        if (m < nrows && nb * 256 + col < H) stg16((uint16_t*)p.o + (size_t)(row0 + m) * H + (size_t)(nb * 256 + col), v);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Wave tiles of the e2m1 x e4m3 recipe with whole-cache-line loads.  A load
// instruction that covers 16 rows x 64 bytes (half of each 128-byte line)
// moves about half as many bytes per cycle through the vector L1 as one that
// covers 8 rows x 128 bytes, so every load here takes whole lines: a weight
// load brings two K stages of 8 weight rows, a routed-row load one K stage of
// 8 rows.  In load half i (rows 8i..8i+7 of a 16-row block) lane l holds row
// 8i + (l%16)%8, 16-byte chunk 4*((l%16)/8) + l/16 of the 128 bytes; a DPP
// rotate by 8 lanes inside each 16-lane row plus a select rebuilds the MFMA
// operand layout (for the weights: stage 2m from chunks 0-3, stage 2m+1 from
// chunks 4-7; for the e4m3 rows: operand bytes 0-15 from chunks 0-3, bytes
// 16-31 from chunks 4-7).
// ---------------------------------------------------------------------------
#ifndef MOEFFN_W4_PP
#define MOEFFN_W4_PP 2
#endif
// TILED: the weights are in the TILED layout (one contiguous 1 KB load per
// 16-row block and K stage, already in operand order) instead of row-major
// (two whole-line loads per block and stage pair, rebuilt by the DPP
// shuffle); a lane's scale load of four stages is 16 contiguous bytes in both
// layouts (its row's dwords of a stage group).
template <int BM, bool TILED>
__device__ void wave_tile_w4(const KParams& p, const Shared& sh, const int* lr2s, bool local, bool l1, int e, int mb,
                             int blk) {
  constexpr int NTB = BM / 16;
  constexpr int PP = MOEFFN_W4_PP;  // weight pairs (2 K stages each) in flight
  const int lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
  const bool lo = r16 < 8;
  const int H = p.H, I = p.I;
  const int row0 = sh.off[e] + mb * BM;
  const int nrows = min(BM, sh.cnt[e] - mb * BM);
  const int K = l1 ? H : I;
  const int nk = K / 128;
  const int npairs = (nk + 1) / 2;
  const uint32_t arow = (uint32_t)K / 2, srow = (uint32_t)K / 32;
  const uint32_t wrows = l1 ? 2u * (uint32_t)I : (uint32_t)H;
  const uint8_t* W = (l1 ? p.w1 : p.w2) + (size_t)e * wrows * arow;
  const uint8_t* Ws = l1 ? p.w1_sf + (size_t)e * wrows * srow : p.w2_sf + (size_t)e * wrows * srow;
  int rb[4];
  if (l1) {
    const int i0 = blk * 32;
    rb[0] = i0; rb[1] = i0 + 16; rb[2] = I + i0; rb[3] = I + i0 + 16;
  } else {
    const int n0 = blk * 64;
    rb[0] = n0; rb[1] = n0 + 16; rb[2] = n0 + 32; rb[3] = n0 + 48;
  }
  const rsrc_t rW = make_rsrc(W, wrows * arow);
  const rsrc_t rWs = make_rsrc(Ws, wrows * srow);
  const uint32_t a_voff = TILED ? (uint32_t)lane * 16u : (uint32_t)(r16 & 7) * arow + (uint32_t)(4 * (r16 >> 3) + g) * 16;
  const uint32_t as_voff = (uint32_t)r16 * srow;

  // routed rows: load half i of token block t covers tile rows t*16 + 8i .. +7
  rsrc_t rB, rBs;
  uint32_t b_voff[NTB][2], bs_voff[NTB];
  const uint32_t bq = (uint32_t)(4 * (r16 >> 3) + g) * 16;
  if (l1) {
    rB = make_rsrc(p.x, (uint32_t)p.T * (uint32_t)H);
    rBs = make_rsrc(p.x_sf, (uint32_t)p.T * (uint32_t)(H / 32));
#pragma unroll
    for (int t = 0; t < NTB; t++) {
#pragma unroll
      for (int i = 0; i < 2; i++) {
        const int m = t * 16 + 8 * i + (r16 & 7);
        const uint32_t tok = (uint32_t)(route_slot(p, lr2s, local, row0 + (m < nrows ? m : 0)) / p.k);
        b_voff[t][i] = tok * (uint32_t)H + bq;
      }
      const int m = t * 16 + r16;
      const uint32_t tok = (uint32_t)(route_slot(p, lr2s, local, row0 + (m < nrows ? m : 0)) / p.k);
      bs_voff[t] = tok * (uint32_t)(H / 32);
    }
  } else {
    const uint32_t rows_end = (uint32_t)(row0 + BM);  // h is padded by kMaxBM rows
    rB = make_rsrc(p.h, rows_end * (uint32_t)I);
    rBs = make_rsrc(p.h_sf, rows_end * (uint32_t)(I / 32));
#pragma unroll
    for (int t = 0; t < NTB; t++) {
#pragma unroll
      for (int i = 0; i < 2; i++) b_voff[t][i] = (uint32_t)(row0 + t * 16 + 8 * i + (r16 & 7)) * (uint32_t)I + bq;
      bs_voff[t] = (uint32_t)(row0 + t * 16 + r16) * (uint32_t)(I / 32);
    }
  }

  v4f acc[4][NTB];
#pragma unroll
  for (int j = 0; j < 4; j++)
#pragma unroll
    for (int t = 0; t < NTB; t++) acc[j][t] = v4f{0.f, 0.f, 0.f, 0.f};
  // Scales are fetched 16 bytes per row, for a group of two pairs (four K
  // stages), with the refill of slot 0; slot 1 takes its pair's half of the
  // group from a copy made before that refill.  Each scale load touches one
  // cache line per row for only 8-16 useful bytes, so halving their number
  // matters for the vector L1 (scale loads cost ~15% of the call at T=128).
  static_assert(PP == 2, "scale groups pair slot 0 with slot 1");
  v4i ar[PP][4][2];          // weight pair: row block j, load half i
  v4i br[PP][NTB][2][2];     // routed rows: block t, stage (0/1 of the pair), load half i
  uint4 sga[4];              // weight scale dwords of the group: pair 0 stage 0/1, pair 1 stage 0/1
  uint4 sgb[NTB];            // routed-row scale dwords of the group
  uint2 nxa[4], nxb[NTB];    // the group's second pair, kept across the refill of slot 0

  auto load = [&](int slot, int m) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
#pragma unroll
      for (int i = 0; i < 2; i++) {
        if constexpr (TILED)  // stage 2m + i of 16-row block rb[j] / 16
          ar[slot][j][i] = buf_load16(rW, a_voff, ((uint32_t)(rb[j] >> 4) * (uint32_t)nk + 2u * (uint32_t)m + i) * 1024u);
        else
          ar[slot][j][i] = buf_load16(rW, a_voff, (uint32_t)(rb[j] + 8 * i) * arow + (uint32_t)m * 128);
      }
      if (slot == 0) {
        if constexpr (TILED)  // group of stages 2m .. 2m+3 (n of them) of 16-row block rb[j] / 16: row r16 at r16 * 4n
          sga[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                       rWs, (uint32_t)r16 * 4u * (uint32_t)min(4, nk - 2 * m),
                       ((uint32_t)(rb[j] >> 4) * (uint32_t)nk + 2u * (uint32_t)m) * 64u, 0));
        else
          sga[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rWs, as_voff, (uint32_t)rb[j] * srow + (uint32_t)m * 8, 0));
      }
    }
#pragma unroll
    for (int t = 0; t < NTB; t++) {
#pragma unroll
      for (int st = 0; st < 2; st++)
#pragma unroll
        for (int i = 0; i < 2; i++) br[slot][t][st][i] = buf_load16(rB, b_voff[t][i], (uint32_t)(2 * m + st) * 128);
      if (slot == 0)
        sgb[t] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rBs, bs_voff[t], (uint32_t)m * 8, 0));
    }
  };
  // scale dwords of the pair in `slot`: slot 0 reads the group directly, slot 1 the saved copy
  auto compute = [&](int slot, int par) {
    v4i a[4];
    int sa[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      if constexpr (TILED) a[j] = par == 0 ? ar[slot][j][0] : ar[slot][j][1];
      else a[j] = line_shuffle(ar[slot][j][0], ar[slot][j][1], par, lo);
      const uint32_t sw = slot == 0 ? (par == 0 ? sga[j].x : sga[j].y) : (par == 0 ? nxa[j].x : nxa[j].y);
      sa[j] = (int)(sw >> (8 * g));
    }
#pragma unroll
    for (int t = 0; t < NTB; t++) {
      const v4i b0 = line_shuffle(br[slot][t][par][0], br[slot][t][par][1], 0, lo);
      const v4i b1 = line_shuffle(br[slot][t][par][0], br[slot][t][par][1], 1, lo);
      const v8i bb = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
      const uint32_t sw = slot == 0 ? (par == 0 ? sgb[t].x : sgb[t].y) : (par == 0 ? nxb[t].x : nxb[t].y);
      const int sb = (int)(sw >> (8 * g));
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const v8i aa = {a[j][0], a[j][1], a[j][2], a[j][3], 0, 0, 0, 0};
        acc[j][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aa, bb, acc[j][t], 4, 0, 0, sa[j], 0, sb);
      }
    }
  };
  auto save_group = [&]() {
#pragma unroll
    for (int j = 0; j < 4; j++) nxa[j] = uint2{sga[j].z, sga[j].w};
#pragma unroll
    for (int t = 0; t < NTB; t++) nxb[t] = uint2{sgb[t].z, sgb[t].w};
  };

  // Steady groups hold only full pairs and carry no branches; the waitcnt
  // pass keeps the ring in flight across them (a guarded compute inside the
  // loop made it drain every load before each pair).  The trailing pairs
  // (at most PP, the last possibly a single stage) are already in flight.
  const int last = npairs - 1;
  const int full = nk / 2;  // pairs with both stages inside K
#pragma unroll
  for (int s = 0; s < PP; s++) load(s, s < npairs ? s : last);
  int m0 = 0;
  for (; m0 + PP <= full && m0 + PP < npairs; m0 += PP) {
    compute(0, 0);
    compute(0, 1);
    save_group();
    // refill a slot only after its last use: interleaving the refill with the
    // MFMAs lets register reuse force near-complete vmcnt drains
    __builtin_amdgcn_sched_barrier(0);
    load(0, m0 + PP);  // m0 + PP < npairs inside this loop
    __builtin_amdgcn_sched_barrier(0);
    compute(1, 0);
    compute(1, 1);
    __builtin_amdgcn_sched_barrier(0);
    load(1, m0 + 1 + PP < npairs ? m0 + 1 + PP : last);
    __builtin_amdgcn_sched_barrier(0);
  }
  save_group();
  if (m0 < npairs) {
    compute(0, 0);
    if (2 * m0 + 1 < nk) compute(0, 1);
  }
  if (m0 + 1 < npairs) {
    compute(1, 0);
    if (2 * (m0 + 1) + 1 < nk) compute(1, 1);
  }

  if (l1) {
    const int i0 = blk * 32;
#pragma unroll
    for (int t = 0; t < NTB; t++) {
      const int m = t * 16 + r16;
      float hv[8];
#pragma unroll
      for (int hh = 0; hh < 2; hh++)
#pragma unroll
        for (int j = 0; j < 4; j++) hv[hh * 4 + j] = swiglu(acc[hh][t][j], acc[2 + hh][t][j], clamp_bound(p.clamp_on, p.clamp));
      float amax = 0.f;
#pragma unroll
      for (int j = 0; j < 8; j++) amax = fmax_nn(amax, __builtin_fabsf(hv[j]));
      amax = max_over_rows(amax);
      const int E = block_scale_exp(amax);
      if (m < nrows) {
        const size_t row = (size_t)(row0 + m);
#pragma unroll
        for (int hh = 0; hh < 2; hh++) {
          const uint32_t word = e4m3x4(__builtin_amdgcn_ldexpf(hv[hh * 4 + 0], -E), __builtin_amdgcn_ldexpf(hv[hh * 4 + 1], -E),
                                        __builtin_amdgcn_ldexpf(hv[hh * 4 + 2], -E), __builtin_amdgcn_ldexpf(hv[hh * 4 + 3], -E));
          stg4(p.h + row * I + (size_t)(i0 + hh * 16 + 4 * g), word);
        }
        if (g == 0) stg1(p.h_sf + row * (size_t)(I / 32) + (size_t)(i0 / 32), (uint8_t)(E + 127));
      }
    }
  } else {
#pragma unroll
    for (int t = 0; t < NTB; t++) {
      const int m = t * 16 + r16;
      if (m < nrows) {
        const size_t row = (size_t)(row0 + m);
#pragma unroll
        for (int j = 0; j < 4; j++) store_o4<2>(p, row * H + (size_t)(rb[j] + 4 * g), acc[j][t]);
      }
    }
  }
}


// Tile queues.  Tile ids run over (expert, feature block, token block), token
// block fastest, so tiles claimed together share a weight slice.
__device__ __forceinline__ void decode_tile(const Shared& sh, int E, int NB, int t, int& e, int& mb, int& blk) {
  e = find_expert(sh.mbo, E, NB, t);
  const int nmb_e = sh.mbo[e + 1] - sh.mbo[e];
  const int loc = t - sh.mbo[e] * NB;
  blk = loc / nmb_e;
  mb = loc % nmb_e;
}

// Wave-tile phase: every streaming wave claims and processes its own tiles.
// The claim for the next tile is issued before the current tile starts, so
// its round trip overlaps the tile's loads.  Three of a workgroup's four
// waves stream the L1 tiles and two the L2 tiles; the others go straight to
// the next grid barrier.  These tiles stream weights, and with all four
// waves loading, the texture unit and L2 contention cost more than the extra
// bytes in flight gain (DeepSeek shape, T=128, waves streaming L1 / L2:
// 4/4 1,299 us, 3/3 1,246-1,262, 2/2 1,255-1,260, 1/1 1,868, 3/4 1,258,
// 4/3 1,272, 3/2 1,239).
constexpr int kWaveTileWavesL1 = 3, kWaveTileWavesL2 = 2;

template <int RECIPE, int BM, bool TILED>
__device__ void phase_wave_tiles(const KParams& p, Shared& sh, const int* lr2s, bool local, bool l1) {
  const int lane = threadIdx.x & 63;
  if ((threadIdx.x >> 6) >= (l1 ? kWaveTileWavesL1 : kWaveTileWavesL2)) return;
  const int E = p.E;
  const int NB = l1 ? p.I / 32 : p.H / 64;
  const uint32_t n = (uint32_t)(sh.mbo[E] * NB);
  uint32_t* q = l1 ? &p.ctrl->tile_next : &p.ctrl->tile_next2;
  uint32_t next = 0;
  if (lane == 0) next = __hip_atomic_fetch_add(q, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (;;) {
    const uint32_t t = __builtin_amdgcn_readfirstlane(next);
    if (t >= n) break;
    if (lane == 0) next = __hip_atomic_fetch_add(q, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int e, mb, blk;
    decode_tile(sh, E, NB, (int)t, e, mb, blk);
    if constexpr (RECIPE == 2) {
      wave_tile_w4<BM, TILED>(p, sh, lr2s, local, l1, __builtin_amdgcn_readfirstlane(e),
                              __builtin_amdgcn_readfirstlane(mb), __builtin_amdgcn_readfirstlane(blk));
    } else {
      wave_tile<RECIPE, BM>(p, sh, lr2s, local, l1, e, mb, blk);
    }
  }
}

// Workgroup-tile phase (token blocks of 64/128).
template <int RECIPE, int BM, bool TILED>
__device__ void phase_wg_tiles(const KParams& p, Shared& sh, SharedB<BM>& sb, const int* lr2s, bool local, bool l1) {
  const int tid = threadIdx.x;
  const int E = p.E;
  const int NB = l1 ? (p.I + 127) / 128 : (p.H + 255) / 256;
  const uint32_t n = (uint32_t)(sh.mbo[E] * NB);
  uint32_t* q = l1 ? &p.ctrl->tile_next : &p.ctrl->tile_next2;
  uint32_t next = 0;
  if (tid == 0) next = __hip_atomic_fetch_add(q, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (;;) {
    if (tid == 0) sh.tile = next;
    __syncthreads();
    const uint32_t t = sh.tile;
    __syncthreads();
    if (t >= n) break;
    if (tid == 0) next = __hip_atomic_fetch_add(q, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int e, mb, nb;
    decode_tile(sh, E, NB, (int)t, e, mb, nb);
    gemm_tile<RECIPE, BM, TILED>(p, sh, sb, lr2s, local, l1, e, mb, nb);
  }
}

// 128-row tile phase.  The 8 XCDs of MI355X have separate L2 caches, so the
// tile list is cut into 8 contiguous ranges, one per XCD, each with its own
// claim counter: a workgroup drains the range of the XCD it runs on, then
// takes tiles from the other ranges.  Inside an expert the tiles are ordered
// in chunks of kBigGM token blocks x all feature blocks, token block fastest,
// so the 32 workgroups of one XCD share about 32 / kBigGM weight slices and
// kBigGM token blocks at a time and fetch each from outside the XCD once.
constexpr int kBigGM = 2;

__device__ __forceinline__ int xcc_id() {
  uint32_t v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return (int)(v & 7u);
}

// Tile t of the list -> expert e, token block mb, feature block nb.
__device__ __forceinline__ void decode_big_tile(const Shared& sh, int E, int NB, int t, int& e, int& mb, int& nb) {
  e = find_expert(sh.mbo, E, NB, t);
  const int nmb_e = sh.mbo[e + 1] - sh.mbo[e];
  const int loc = t - sh.mbo[e] * NB;
  const int c = loc / (kBigGM * NB);
  const int j = loc - c * kBigGM * NB;
  const int gm = min(kBigGM, nmb_e - c * kBigGM);
  nb = j / gm;
  mb = c * kBigGM + (j - nb * gm);
}

__device__ __forceinline__ uint32_t big_range_begin(uint32_t n, int r) {
  return (uint32_t)(((uint64_t)n * (uint32_t)r) >> 3);
}

// Turn a claim into a tile (thread 0).  `c` is the value a fetch-and-add on
// range `cur`'s counter returned; once that range is drained the other ranges
// are tried in turn, synchronously (only at the end of a phase), and `cur`
// moves to the range that yields a tile.  Returns n when every range is
// exhausted.
__device__ __forceinline__ uint32_t resolve_big_claim(uint32_t* ctr, uint32_t n, int& cur, uint32_t c) {
  const uint32_t beg = big_range_begin(n, cur), end = big_range_begin(n, cur + 1);
  if (c < end - beg) return beg + c;
  for (int q = 1; q < 8; q++) {
    const int r = (cur + q) & 7;
    const uint32_t b = big_range_begin(n, r), e = big_range_begin(n, r + 1);
    if (e == b) continue;
    if (ld_relaxed(&ctr[r]) >= e - b) continue;  // already drained: skip the atomic
    const uint32_t v = __hip_atomic_fetch_add(&ctr[r], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (v < e - b) {
      cur = r;
      return b + v;
    }
  }
  cur = (cur + 7) & 7;  // every range is drained; later claims resolve to n as well
  return n;
}

template <int RECIPE>
__device__ __forceinline__ void phase_big_tiles(const KParams& p, Shared& sh, const BigRing& R, bool l1) {
  const int tid = threadIdx.x;
  const int E = p.E;
  const int NB = l1 ? p.I / 128 : (p.H + 255) / 256;
  const uint32_t n = (uint32_t)(sh.mbo[E] * NB);
  uint32_t* ctr = p.ctrl->xq[l1 ? 0 : 1];
  // Thread 0 keeps one claim in flight while a tile runs: a fetch-and-add on
  // the counter of range `cur` (first the XCD's own), issued before the tile
  // and resolved after it, so its round trip to the memory-side atomics
  // overlaps the tile instead of standing between two tiles.  Within the last
  // `near` tiles of a range the next claim waits for the tile's end: a tile
  // claimed ahead there could start only after the list has drained and
  // would stretch the phase's tail by a whole tile.
  const uint32_t near = gridDim.x >> 2;  // ~2 tiles per workgroup of an XCD
  int cur = xcc_id();
  uint32_t pend = 0;
  bool held = false;
  for (;;) {
    if (tid == 0) {
      if (!held) pend = __hip_atomic_fetch_add(&ctr[cur], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t tc = resolve_big_claim(ctr, n, cur, pend);
      sh.tile = tc;
      held = tc < n && tc + near < big_range_begin(n, cur + 1);
      if (held) pend = __hip_atomic_fetch_add(&ctr[cur], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    const uint32_t t = __builtin_amdgcn_readfirstlane(sh.tile);
    __syncthreads();
    if (t >= n) break;
    int e, mb, nb;
    decode_big_tile(sh, E, NB, (int)t, e, mb, nb);
    e = __builtin_amdgcn_readfirstlane(e);
    mb = __builtin_amdgcn_readfirstlane(mb);
    nb = __builtin_amdgcn_readfirstlane(nb);
    const int nrows = __builtin_amdgcn_readfirstlane(min(kBigBM, sh.cnt[e] - mb * kBigBM));
    if (nrows > 64) big_tile<RECIPE, 8>(p, sh, R, l1, e, mb, nb);
    else if (nrows > 32) big_tile<RECIPE, 4>(p, sh, R, l1, e, mb, nb);
    else big_tile<RECIPE, 2>(p, sh, R, l1, e, mb, nb);
  }
}

// ---------------------------------------------------------------------------
// C: combine.  A unit of work is one token x 1024 columns (units spread
// evenly over the waves even when T is not a multiple of the wave count): the
// wave holds the token's k row indices and weights in lanes 0..k-1 (those of
// its first unit loaded before the barrier that ends the L2 phase: routing is
// final long before), then streams the k rows of o and sums in slot order
// j = 0..k-1 with fused multiply-adds in fp32.  bf16 rows (e4m3 recipes): a
// lane takes 8 columns of each 512-column half, so one unit is two 16-byte
// loads per slot, all of them for 8 slots in flight at once.  fp32 rows (BF16
// recipe): 256-column slices of 64 lanes x 4 floats; WIDE (the kernels with
// registers to spare): with k <= 8 all 4 slices of all slots in flight at
// once; else two slices of 8 slots.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void combine_first_meta(const KParams& p, int& myrow, float& myw) {
  const int lane = threadIdx.x & 63;
  const int nc = (p.H + 1023) >> 10;
  const int u = blockIdx.x * 4 + (threadIdx.x >> 6);
  const bool has = u < p.T * nc && lane < p.k;
  myrow = has ? p.s2r[(size_t)(u / nc) * p.k + lane] : -1;
  myw = has ? p.tw[(size_t)(u / nc) * p.k + lane] : 0.f;
}

__device__ __forceinline__ void combine_store(const KParams& p, int t, int c, const v4f& a) {
  if (p.y_fp32) {
    stg16f((float*)p.y + (size_t)t * p.H + c, a);
  } else {
    stg8((uint16_t*)p.y + (size_t)t * p.H + c, f32_to_bf16(a[0]) | (f32_to_bf16(a[1]) << 16),
         f32_to_bf16(a[2]) | (f32_to_bf16(a[3]) << 16));
  }
}

// Eight consecutive outputs y[t, c .. c+7] from fp32 sums.
__device__ __forceinline__ void combine_store8(const KParams& p, int t, int c, const float* a) {
  if (p.y_fp32) {
    stg16f((float*)p.y + (size_t)t * p.H + c, v4f{a[0], a[1], a[2], a[3]});
    stg16f((float*)p.y + (size_t)t * p.H + c + 4, v4f{a[4], a[5], a[6], a[7]});
  } else {
    v4i w;
#pragma unroll
    for (int i = 0; i < 4; i++) w[i] = (int)(f32_to_bf16(a[2 * i]) | (f32_to_bf16(a[2 * i + 1]) << 16));
    stg16((uint16_t*)p.y + (size_t)t * p.H + c, w);
  }
}

// bf16 rows of o (e4m3 recipes).  A wave takes U units at a time (its units
// u, u + nw, .., u + (U-1) nw), all their loads in flight together, and
// fetches the slots of its next U units while they stream in.  H is a
// multiple of 32, so no 8-column piece straddles the end of a row.
template <int U>
__device__ void phase_combine_b16(const KParams& p, int row0, float w0) {
  const int lane = threadIdx.x & 63;
  const int H = p.H, k = p.k;
  const int nw = gridDim.x * 4;
  const int nc = (H + 1023) >> 10;  // 1024-column units per token
  const int units = p.T * nc;
  const int u0 = blockIdx.x * 4 + (threadIdx.x >> 6);
  const uint16_t* o = (const uint16_t*)p.o;
  // lane j < k: slot j's row and weight, for each of the wave's next U units
  // (a unit past the end repeats the last one: loads stay in bounds, nothing is stored)
  int mrow[U];
  float mw[U];
  mrow[0] = row0;
  mw[0] = w0;
#pragma unroll
  for (int q = 1; q < U; q++) {
    const int tq = min(u0 + q * nw, units - 1) / nc;
    mrow[q] = lane < k ? p.s2r[(size_t)tq * k + lane] : -1;
    mw[q] = lane < k ? p.tw[(size_t)tq * k + lane] : 0.f;
  }
  for (int u = u0; u < units; u += U * nw) {
    int crow[U], tt[U], ca[U], la[U], lb[U];
    float cw[U];
    bool live[U], va[U], vb[U];
#pragma unroll
    for (int q = 0; q < U; q++) {
      const int uq = u + q * nw;
      live[q] = uq < units;
      const int uc = live[q] ? uq : u;
      tt[q] = uc / nc;
      const int cu = uc - tt[q] * nc;
      const int cend = min(H, (cu + 1) << 10);
      ca[q] = (cu << 10) + lane * 8;
      va[q] = ca[q] < cend;
      vb[q] = ca[q] + 512 < cend;
      // lanes past the row's end read column 0 and drop it: every load is
      // issued unconditionally, so all of them are in flight together
      la[q] = va[q] ? ca[q] : 0;
      lb[q] = vb[q] ? ca[q] + 512 : 0;
      crow[q] = mrow[q];
      cw[q] = mw[q];
    }
    float acc[U][16];
#pragma unroll
    for (int q = 0; q < U; q++)
#pragma unroll
      for (int i = 0; i < 16; i++) acc[q][i] = 0.f;
    for (int j0 = 0; j0 < k; j0 += 8) {
      v4i oa[U][8], ob[U][8];
      int rows[U][8];
      float ws[U][8];
#pragma unroll
      for (int q = 0; q < U; q++) {
#pragma unroll
        for (int j = 0; j < 8; j++) {
          const int jj = j0 + j;
          // slot jj's row and weight, wave-uniform (a masked slot, or one past k, has row -1 and reads row 0)
          rows[q][j] = jj < k ? __builtin_amdgcn_readlane(crow[q], jj) : -1;
          ws[q][j] = jj < k ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cw[q]), jj)) : 0.f;
          const size_t base = (size_t)(rows[q][j] < 0 ? 0 : rows[q][j]) * H;
          oa[q][j] = ldg16(o + base + la[q]);
          ob[q][j] = ldg16(o + base + lb[q]);
        }
      }
      if (j0 == 0) {
#pragma unroll
        for (int q = 0; q < U; q++) {
          const int tn = min(u + (U + q) * nw, units - 1) / nc;
          mrow[q] = lane < k ? p.s2r[(size_t)tn * k + lane] : -1;
          mw[q] = lane < k ? p.tw[(size_t)tn * k + lane] : 0.f;
        }
      }
#pragma unroll
      for (int q = 0; q < U; q++) {
#pragma unroll
        for (int j = 0; j < 8; j++) {
          if (rows[q][j] >= 0) {
#pragma unroll
            for (int c = 0; c < 4; c++) {
              const uint32_t a = (uint32_t)oa[q][j][c], b = (uint32_t)ob[q][j][c];
              acc[q][2 * c] = __builtin_fmaf(ws[q][j], __uint_as_float(a << 16), acc[q][2 * c]);
              acc[q][2 * c + 1] = __builtin_fmaf(ws[q][j], __uint_as_float(a & 0xFFFF0000u), acc[q][2 * c + 1]);
              acc[q][8 + 2 * c] = __builtin_fmaf(ws[q][j], __uint_as_float(b << 16), acc[q][8 + 2 * c]);
              acc[q][8 + 2 * c + 1] = __builtin_fmaf(ws[q][j], __uint_as_float(b & 0xFFFF0000u), acc[q][8 + 2 * c + 1]);
            }
          }
        }
      }
    }
#pragma unroll
    for (int q = 0; q < U; q++) {
      if (live[q]) {
        if (va[q]) combine_store8(p, tt[q], ca[q], acc[q]);
        if (vb[q]) combine_store8(p, tt[q], ca[q] + 512, acc[q] + 8);
      }
    }
  }
}

template <int RECIPE, bool WIDE>
__device__ void phase_combine(const KParams& p, int myrow, float myw) {
  if constexpr (RECIPE != 0) {
    phase_combine_b16<2>(p, myrow, myw);
    return;
  }
  const float* o = (const float*)p.o;
  const int lane = threadIdx.x & 63;
  const int H = p.H, k = p.k;
  const int nw = gridDim.x * 4;
  const int nc = (H + 1023) >> 10;  // 1024-column units per token
  const int units = p.T * nc;
  const int u0 = blockIdx.x * 4 + (threadIdx.x >> 6);
  for (int u = u0; u < units; u += nw) {
    const int t = u / nc, cu = u - t * nc;
    if (u != u0) {  // lane j < k holds slot j's row and weight
      myrow = lane < k ? p.s2r[(size_t)t * k + lane] : -1;
      myw = lane < k ? p.tw[(size_t)t * k + lane] : 0.f;
    }
    const int cend = min(H, (cu + 1) << 10);
    if constexpr (WIDE) {
      if (k <= 8) {
        int rows[8];
        float ws[8];
        v4f ov[8][4];
#pragma unroll
        for (int j = 0; j < 8; j++) {
          rows[j] = j < k ? __shfl(myrow, j, 64) : -1;
          ws[j] = j < k ? __shfl(myw, j, 64) : 0.f;
          const size_t base = (size_t)(rows[j] < 0 ? 0 : rows[j]) * H;
#pragma unroll
          for (int q = 0; q < 4; q++) {
            const int c = (cu << 10) + q * 256 + lane * 4;
            ov[j][q] = (rows[j] >= 0 && c < cend) ? ldg16f(o + base + c) : v4f{0.f, 0.f, 0.f, 0.f};
          }
        }
#pragma unroll
        for (int q = 0; q < 4; q++) {
          v4f a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int j = 0; j < 8; j++) {
            if (rows[j] >= 0) {
#pragma unroll
              for (int c = 0; c < 4; c++) a[c] = __builtin_fmaf(ws[j], ov[j][q][c], a[c]);
            }
          }
          const int c = (cu << 10) + q * 256 + lane * 4;
          if (c < cend) combine_store(p, t, c, a);
        }
        continue;
      }
    }
    for (int c0 = cu << 10; c0 < cend; c0 += 512) {
      const int ca = c0 + lane * 4;
      const int cb = c0 + 256 + lane * 4;
      const bool va = ca < cend, vb = cb < cend;
      v4f acca = {0.f, 0.f, 0.f, 0.f}, accb = {0.f, 0.f, 0.f, 0.f};
      for (int j0 = 0; j0 < k; j0 += 8) {
        v4f oa[8], ob[8];
        int rows[8];
        float ws[8];
#pragma unroll
        for (int j = 0; j < 8; j++) {
          const int jj = j0 + j;
          rows[j] = jj < k ? __shfl(myrow, jj, 64) : -1;
          ws[j] = jj < k ? __shfl(myw, jj, 64) : 0.f;
          const size_t base = (size_t)(rows[j] < 0 ? 0 : rows[j]) * H;
          oa[j] = (rows[j] >= 0 && va) ? ldg16f(o + base + ca) : v4f{0.f, 0.f, 0.f, 0.f};
          ob[j] = (rows[j] >= 0 && vb) ? ldg16f(o + base + cb) : v4f{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int j = 0; j < 8; j++) {
          if (rows[j] >= 0) {
#pragma unroll
            for (int c = 0; c < 4; c++) {
              acca[c] = __builtin_fmaf(ws[j], oa[j][c], acca[c]);
              accb[c] = __builtin_fmaf(ws[j], ob[j][c], accb[c]);
            }
          }
        }
      }
      if (va) combine_store(p, t, ca, acca);
      if (vb) combine_store(p, t, cb, accb);
    }
  }
}

// ---------------------------------------------------------------------------
// The persistent kernel.  __launch_bounds__(256, 2): registers and LDS sized
// so that two workgroups fit on one CU, which keeps the grid co-resident when
// another stream holds a few CUs of an XCD.
// ---------------------------------------------------------------------------
template <int RECIPE, int BM, bool TILED>
__device__ __forceinline__ void run_call(const KParams& p, Shared& sh, WaveCounters& wcnt, int* lr2s,
                                         SharedB<(BM > 32 && BM < 128 ? BM : 16)>* sb, const BigRing* big) {
  constexpr bool kBig = RECIPE == 2 && BM == kBigBM;
  static_assert(!kBig || TILED, "the 128-row tiles read the TILED layout");
  const int tid = threadIdx.x;
  const int S = p.T * p.k;
  const bool local = !kBig && S <= kLocalRouteSlots;

  const int dirty = entry_verdict(p, sh) != kVerdictClean;

  if (!dirty) {
    if (local) {
      phase_route_local(p, sh, wcnt, lr2s, S, BM);
    } else {
      // chunks of a multiple of 64 slots, at most one per workgroup and kMaxChunks in all
      const int cmax = min((int)gridDim.x, kMaxChunks);
      const int cs = max(64, ((S + cmax - 1) / cmax + 63) / 64 * 64);
      const int C = (S + cs - 1) / cs;
      phase_histogram(p, sh, S, C, cs);
      if (!grid_barrier(p, BAR_HIST, 0, sh)) goto done;
      phase_scatter_global(p, sh, wcnt, S, C, cs, BM);
      if (!grid_barrier(p, BAR_SCATTER, 1, sh)) goto done;
    }
    if constexpr (kBig) phase_big_tiles<RECIPE>(p, sh, *big, true);
    else if constexpr (BM <= 32) phase_wave_tiles<RECIPE, BM, TILED>(p, sh, lr2s, local, true);
    else phase_wg_tiles<RECIPE, BM, TILED>(p, sh, *sb, lr2s, local, true);
    if (!grid_barrier(p, BAR_L1, local ? 0 : 2, sh)) goto done;
    if constexpr (kBig) phase_big_tiles<RECIPE>(p, sh, *big, false);
    else if constexpr (BM <= 32) phase_wave_tiles<RECIPE, BM, TILED>(p, sh, lr2s, local, false);
    else phase_wg_tiles<RECIPE, BM, TILED>(p, sh, *sb, lr2s, local, false);
    {
      int crow;
      float cw;
      combine_first_meta(p, crow, cw);
      if (!grid_barrier(p, BAR_L2, local ? 1 : 3, sh)) goto done;
      phase_combine<RECIPE, !kBig>(p, crow, cw);
    }
  }
done:
  fence_release();
  __syncthreads();
  // A dirty call leaves the control block as it found it (plus the abort
  // flag and verdict set by workgroup 0): no exit count, no reset.
  if (tid == 0 && !dirty) {
    const uint32_t old = add_acq_rel(&p.ctrl->exit_count, 1u);
    // the verdict is re-read: only a call that workgroup 0 found clean resets
    if (old == gridDim.x - 1 && ld_relaxed(&p.ctrl->verdict) == kVerdictClean) {
      // last workgroup out: every other workgroup is past its last access
      const int st = __hip_atomic_load(&p.ctrl->status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (p.out_status) *p.out_status = st;
      for (int i = 0; i < kNumBarriers; i++) st_relaxed(&p.ctrl->bar[i], 0u);
      for (int g = 0; g < kBarGroups; g++) st_relaxed(p.bars + g * kBarLineWords, 0u);
      st_relaxed(&p.ctrl->tile_next, 0u);
      st_relaxed(&p.ctrl->tile_next2, 0u);
      for (int l = 0; l < 2; l++)
        for (int r = 0; r < 8; r++) st_relaxed(&p.ctrl->xq[l][r], 0u);
      st_relaxed(&p.ctrl->abort, 0u);
      __hip_atomic_store(&p.ctrl->status, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      st_relaxed(&p.ctrl->verdict, 0u);
      st_release(&p.ctrl->exit_count, 0u);
    }
  }
}

template <int RECIPE, int BM, bool TILED>
__global__ __launch_bounds__(kThreads, 2) void moe_ffn_kernel(KParams p) {
  __shared__ Shared sh;
  if constexpr (RECIPE == 2 && BM == kBigBM) {
    // three ring buffers, each its own LDS object; the scatter counters of
    // the routing phase live in the first one (routing ends before any tile)
    __shared__ __attribute__((aligned(16))) uint8_t ring0[kBigBuf];
    __shared__ __attribute__((aligned(16))) uint8_t ring1[kBigBuf];
    __shared__ __attribute__((aligned(16))) uint8_t ring2[kBigBuf];
    static_assert(sizeof(WaveCounters) <= kBigBuf, "scatter counters must fit a ring buffer");
    const BigRing R{ring0, ring1, ring2};
    run_call<RECIPE, BM, TILED>(p, sh, *reinterpret_cast<WaveCounters*>(ring0), nullptr, nullptr, &R);
  } else {
    __shared__ WaveCounters wcnt;
    __shared__ int lr2s[kLocalRouteSlots];
    __shared__ SharedB<(BM > 32 && BM < 128 ? BM : 16)> sb;
    run_call<RECIPE, BM, TILED>(p, sh, wcnt, lr2s, &sb, nullptr);
  }
}

int max_block_m(int recipe) { return recipe == 2 ? 128 : 64; }
int min_block_m(int recipe) { return recipe == 3 ? 64 : 16; }

// ---------------------------------------------------------------------------
// Weight-scale transform to the TILED layout: one thread per (expert, row,
// K stage) moves the stage's dword (its four 32-block scales): row r = 16b + i,
// stage s = 4G + u goes to (b * nk + 4G) * 64 + i * 4n + u * 4 of the expert's
// scales, n = min(4, nk - 4G).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void transform_scales_kernel(const uint32_t* __restrict__ src,
                                                                uint32_t* __restrict__ dst, int64_t E, int64_t rows,
                                                                int64_t nk) {
  const int64_t n = E * rows * nk;
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < n; c += (int64_t)gridDim.x * 256) {
    const int64_t er = c / nk, s = c - er * nk;   // er = e * rows + r
    const int64_t e = er / rows, r = er - e * rows;
    const int64_t b = r >> 4, i = r & 15, g4 = s & ~(int64_t)3;
    const int64_t ns = nk - g4 < 4 ? nk - g4 : 4;
    dst[e * rows * nk + (b * nk + g4) * 16 + i * ns + (s & 3)] = src[c];
  }
}

hipError_t launch_transform_scales(const uint8_t* src, uint8_t* dst, int64_t E, int64_t rows, int64_t kb,
                                   hipStream_t stream) {
  const int64_t n = E * rows * (kb / 4);
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(transform_scales_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<const uint32_t*>(src), reinterpret_cast<uint32_t*>(dst), E, rows, kb / 4);
  return hipGetLastError();
}

// Tiled e2m1 weight copy (one thread per 16-byte chunk of a row).
__global__ __launch_bounds__(256) void transform_weights_kernel(const uint8_t* __restrict__ src,
                                                                uint8_t* __restrict__ dst, int64_t E, int64_t rows,
                                                                int64_t kbytes) {
  const int64_t cpr = kbytes >> 4;  // 16-byte chunks per row
  const int64_t n = E * rows * cpr;
  const int64_t nst = kbytes >> 6;  // 64-byte K stages per row
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < n; c += (int64_t)gridDim.x * 256) {
    const int64_t row = c / cpr, ch = c - row * cpr;  // row over all experts (rows % 16 == 0)
    const int64_t b = row >> 4, r = row & 15, s = ch >> 2, g = ch & 3;
    *(v4i*)(dst + ((b * nst + s) << 10) + ((g * 16 + r) << 4)) = ldg16(src + (c << 4));
  }
}

hipError_t launch_transform_weights(const uint8_t* src, uint8_t* dst, int64_t E, int64_t rows, int64_t kbytes,
                                    hipStream_t stream) {
  const int64_t n = E * rows * (kbytes >> 4);
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(transform_weights_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, src, dst, E, rows, kbytes);
  return hipGetLastError();
}

template <int RECIPE, int BM, bool TILED>
static hipError_t launch_one(int grid, const KParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((moe_ffn_kernel<RECIPE, BM, TILED>), dim3(grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int RECIPE, bool TILED>
static hipError_t launch_recipe(int bm, int grid, const KParams& p, hipStream_t stream) {
  if constexpr (RECIPE == 3) {   // the (1, 128, 128) recipe runs on the 64-row workgroup tiles only
    return bm == 64 ? launch_one<RECIPE, 64, TILED>(grid, p, stream) : hipErrorInvalidValue;
  } else {
    switch (bm) {
      case 16: return launch_one<RECIPE, 16, TILED>(grid, p, stream);
      case 32: return launch_one<RECIPE, 32, TILED>(grid, p, stream);
      case 64: return launch_one<RECIPE, 64, TILED>(grid, p, stream);
      case 128:
        if constexpr (RECIPE == 2 && TILED) return launch_one<RECIPE, 128, TILED>(grid, p, stream);
        return hipErrorInvalidValue;
      default: return hipErrorInvalidValue;
    }
  }
}

hipError_t launch_forward(int recipe, int bm, bool tiled, int grid, const KParams& p, hipStream_t stream) {
  switch (recipe) {
    case 0: return tiled ? hipErrorInvalidValue : launch_recipe<0, false>(bm, grid, p, stream);
    case 1: return tiled ? hipErrorInvalidValue : launch_recipe<1, false>(bm, grid, p, stream);
    case 2: return tiled ? launch_recipe<2, true>(bm, grid, p, stream) : launch_recipe<2, false>(bm, grid, p, stream);
    case 3: return tiled ? hipErrorInvalidValue : launch_recipe<3, false>(bm, grid, p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moeffn
