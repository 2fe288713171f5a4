// Workspace layout of the fused MoE forward (host and device).
//
// The layout is a function of the problem only (max_tokens, H, I, E, k,
// recipe): never of the CU count or the reserve, so a caller may cache one
// workspace per problem shape and change the reserve freely.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace moeffn {

constexpr int kThreads = 256;          // one workgroup = 4 waves of 64
constexpr int kMaxExperts = 512;
constexpr int kMaxTopK = 64;
constexpr int kMaxChunks = 256;        // routing chunks of a large call (rows of the per-chunk histogram)
constexpr int kMinBM = 16;             // smallest token block of any tile config
constexpr int kMaxBM = 128;            // largest token block (h rows are padded by this)
constexpr int kNumBarriers = 6;
constexpr int kLocalRouteSlots = 4096;  // up to this many slots every workgroup routes on its own (in LDS)

// Control block at workspace offset 0.  Every field is zero between calls.
struct Ctrl {
  uint32_t bar[kNumBarriers];  // grid barrier arrival counters
  uint32_t exit_count;         // workgroups that reached the end of the call
  uint32_t tile_next;          // next L1 tile to claim
  uint32_t tile_next2;         // next L2 tile to claim
  uint32_t abort;              // set on a fatal condition: every wait gives up
  int32_t status;              // first MOE_FFN_STATUS_* of the call
  uint32_t xq[2][8];           // 128-row tiles: per-XCD range claim counters (L1, L2)
  uint32_t verdict;            // workgroup 0's entry check of this block: 0 none yet, 1 clean, 2 dirty
  uint32_t pad[36];
};
static_assert(sizeof(Ctrl) == 256, "control block must stay 256 bytes");
static_assert(offsetof(Ctrl, bar) == 0, "barrier counters lead the control block");
static_assert(offsetof(Ctrl, exit_count) == 24, "layout change must be deliberate");
static_assert(offsetof(Ctrl, status) == 40, "layout change must be deliberate");
static_assert(offsetof(Ctrl, xq) == 44, "layout change must be deliberate");
static_assert(offsetof(Ctrl, verdict) == 108, "layout change must be deliberate");
constexpr int kCtrlWords = (int)(sizeof(Ctrl) / 4);

// Grid-barrier group counters, right after the control block: 8 groups of
// workgroups (blockIdx % 8), one 128-byte line each, counting the arrivals of
// the group's workgroups over all barriers of a call.  Zero between calls.
constexpr int kBarGroups = 8;
constexpr int kBarLineWords = 32;
constexpr int kBarRegionBytes = kBarGroups * kBarLineWords * 4;
// Bytes at the start of the workspace that must be zero when a call starts.
constexpr int kCtrlRegionBytes = (int)sizeof(Ctrl) + kBarRegionBytes;

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct Layout {
  size_t ctrl, bars, counts, offsets, hist, r2s, s2r, h, h_sf, o, xsg, hsg, total;
  int64_t max_slots;     // max_tokens * k
  int64_t h_rows;        // rows of h (max_slots + kMaxBM padding)
  int64_t h_row_bytes, h_sf_row_bytes, o_row_bytes;
};

// recipe: 0 bf16, 1 fp8xfp8, 2 fp8xfp4 (h is bf16 for recipe 0, e4m3 otherwise)
inline Layout make_layout(int64_t max_tokens, int64_t H, int64_t I, int64_t E, int64_t k, int recipe) {
  Layout L{};
  const size_t A = 256;
  L.max_slots = max_tokens * k;
  L.h_rows = L.max_slots + kMaxBM;
  L.h_row_bytes = recipe == 0 ? I * 2 : I;
  L.h_sf_row_bytes = recipe == 0 ? 0 : I / 32;
  L.o_row_bytes = recipe == 0 ? H * 4 : H * 2;  // the L2 result per routed row: fp32 / bf16
  size_t off = 0;
  L.ctrl = off;    off = align_up(off + sizeof(Ctrl), A);
  L.bars = off;    off = align_up(off + kBarRegionBytes, A);
  L.counts = off;  off = align_up(off + sizeof(int32_t) * (size_t)E, A);
  L.offsets = off; off = align_up(off + sizeof(int32_t) * (size_t)(E + 1), A);
  L.hist = off;    off = align_up(off + sizeof(int32_t) * (size_t)kMaxChunks * (size_t)E, A);
  L.r2s = off;     off = align_up(off + sizeof(int32_t) * (size_t)(L.max_slots + 1), A);
  L.s2r = off;     off = align_up(off + sizeof(int32_t) * (size_t)(L.max_slots + 1), A);
  L.h = off;       off = align_up(off + (size_t)L.h_rows * (size_t)L.h_row_bytes, A);
  L.h_sf = off;    off = align_up(off + (size_t)L.h_rows * (size_t)L.h_sf_row_bytes, A);
  L.o = off;       off = align_up(off + (size_t)(L.max_slots > 0 ? L.max_slots : 1) * (size_t)L.o_row_bytes, A);
  // e4m3 x e2m1 with H and I multiples of 128: stage-major copies of the
  // activation scales of the routed rows, xsg[H/128][h_rows] and
  // hsg[I/128][h_rows] (one dword = the 4 e8m0 bytes of a 128-element K
  // stage), so that a stage's scales of consecutive routed rows are contiguous
  const bool sg = recipe == 2 && H % 128 == 0 && I % 128 == 0;
  L.xsg = off;     off = align_up(off + (sg ? (size_t)(H / 128) * (size_t)L.h_rows * 4 : 0), A);
  L.hsg = off;     off = align_up(off + (sg ? (size_t)(I / 128) * (size_t)L.h_rows * 4 : 0), A);
  L.total = off;
  return L;
}

}  // namespace moeffn
