// Host side of the C ABI declared in include/moe_ffn.h: argument checks,
// workspace layout, launch sizing (CU reserve) and the kernel launch.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>

#include "../../include/moe_ffn.h"
#include "moe_ffn_kernel.h"
#include "moe_ffn_layout.h"

using moeffn::KParams;
using moeffn::Layout;

namespace {

constexpr int kMaxDevices = 64;
// Physical CU count per device: an immutable device property, queried once.
std::atomic<int> g_cus[kMaxDevices];

int physical_cus(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return -1;
  int v = g_cus[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return -1;
  g_cus[dev].store(n, std::memory_order_relaxed);
  return n;
}

long env_long(const char* name, long dflt) {
  const char* s = std::getenv(name);
  if (!s || !*s) return dflt;
  char* end = nullptr;
  long v = std::strtol(s, &end, 10);
  return (end && *end == '\0') ? v : dflt;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_problem(const moe_ffn_problem* p) {
  if (!p) return MOE_FFN_ERR_INVALID_ARG;
  if (p->max_tokens < 0 || p->hidden <= 0 || p->intermediate <= 0 || p->num_experts <= 0 || p->top_k <= 0)
    return MOE_FFN_ERR_INVALID_ARG;
  if (p->recipe < MOE_FFN_RECIPE_BF16 || p->recipe > MOE_FFN_RECIPE_FP8_BLOCK128) return MOE_FFN_ERR_INVALID_ARG;
  if (p->weight_layout != MOE_FFN_WEIGHTS_ROW_MAJOR && p->weight_layout != MOE_FFN_WEIGHTS_TILED)
    return MOE_FFN_ERR_INVALID_ARG;
  if (p->weight_layout == MOE_FFN_WEIGHTS_TILED && p->recipe != MOE_FFN_RECIPE_FP8_FP4) return MOE_FFN_ERR_UNSUPPORTED;
  const int64_t kmul = p->recipe == MOE_FFN_RECIPE_BF16 ? 64 : 128;
  if (p->hidden % kmul || p->intermediate % kmul) return MOE_FFN_ERR_UNSUPPORTED;
  if (p->num_experts > moeffn::kMaxExperts || p->top_k > moeffn::kMaxTopK) return MOE_FFN_ERR_UNSUPPORTED;
  if (p->hidden > (1 << 20) || p->intermediate > (1 << 20)) return MOE_FFN_ERR_UNSUPPORTED;
  // slot indices are 32-bit
  const int64_t lim = int64_t(1) << 31;
  if (p->max_tokens * p->top_k + moeffn::kMaxBM >= lim) return MOE_FFN_ERR_UNSUPPORTED;
  // Every tile kind addresses x rows, h rows (padded by kMaxBM rows) and one
  // expert's weight matrix with 32-bit byte offsets (buffer ranges and
  // per-lane offsets): each of these byte ranges must stay below 2^31.
  const int64_t act = p->recipe == MOE_FFN_RECIPE_BF16 ? 2 : 1;  // bytes per x / h element
  const int64_t w1_bytes = p->recipe == MOE_FFN_RECIPE_BF16   ? 4 * p->intermediate * p->hidden
                           : p->recipe == MOE_FFN_RECIPE_FP8_FP4 ? p->intermediate * p->hidden
                                                                 : 2 * p->intermediate * p->hidden;
  if (p->max_tokens * p->hidden * act >= lim) return MOE_FFN_ERR_UNSUPPORTED;
  if ((p->max_tokens * p->top_k + moeffn::kMaxBM) * p->intermediate * act >= lim) return MOE_FFN_ERR_UNSUPPORTED;
  if (w1_bytes >= lim) return MOE_FFN_ERR_UNSUPPORTED;
  return MOE_FFN_OK;
}

// Token block of the GEMM tiles for this call: the average expert group
// decides between weight streaming (16 tokens, every weight byte read once)
// and larger blocks that reuse each weight tile across more tokens.
int choose_block_m(int recipe, int64_t T, int64_t k, int64_t E) {
  const double avg = E > 0 ? double(T) * double(k) / double(E) : 0.0;
  int bm = avg <= 16.0 ? 16 : avg <= 40.0 ? 32 : avg <= 96.0 ? 64 : 128;
  const int cap = moeffn::max_block_m(recipe), low = moeffn::min_block_m(recipe);
  return bm > cap ? cap : bm < low ? low : bm;
}

// Workgroups a call can keep busy at most, from its sizes alone (the routing is
// not known on the host): token blocks are at most S/bm + min(E, S) (every
// expert with rows adds at most one partial block), each with I/32 (L1) and
// H/64 (L2) wave tiles taken by 3 and 2 waves of a workgroup, or I/128 and
// H/256 workgroup tiles; the combine has T * ceil(H/1024) units over 4 waves
// per workgroup; large calls route with E columns.  A grid larger than this
// only adds workgroups to every grid barrier (measured: ~0.24 us of barrier
// time per workgroup on a 64-token call).
int64_t useful_workgroups(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k, int bm) {
  const int64_t S = T * k;
  const int64_t blocks = S / bm + (E < S ? E : S);
  const bool wave = bm <= 32;
  const int64_t l1 = wave ? (blocks * (I / 32) + 2) / 3 : blocks * ((I + 127) / 128);
  const int64_t l2 = wave ? (blocks * (H / 64) + 1) / 2 : blocks * ((H + 255) / 256);
  const int64_t comb = (T * ((H + 1023) / 1024) + 3) / 4;
  int64_t n = l1 > l2 ? l1 : l2;
  if (comb > n) n = comb;
  if (S > moeffn::kLocalRouteSlots && E > n) n = E;
  return n;
}

}  // namespace

extern "C" {

int moe_ffn_launch_size(int physical, int reserved, int max_cus) {
  if (physical <= 0) return 2;
  const int res = reserved > 0 ? reserved : 0;
  int limit = physical - res;
  if (limit < 2) limit = 2;
  int target = (max_cus > 0 && max_cus < limit) ? max_cus : limit;
  target -= target % 2;
  return target < 2 ? 2 : target;
}

int moe_ffn_get_workspace_size(const moe_ffn_problem* p, size_t* bytes) {
  if (!bytes) return MOE_FFN_ERR_INVALID_ARG;
  const int rc = check_problem(p);
  if (rc) return rc;
  *bytes = moeffn::make_layout(p->max_tokens, p->hidden, p->intermediate, p->num_experts, p->top_k, p->recipe).total;
  return MOE_FFN_OK;
}

int moe_ffn_get_token_alignment(int32_t recipe, int64_t* alignment) {
  if (!alignment || recipe < MOE_FFN_RECIPE_BF16 || recipe > MOE_FFN_RECIPE_FP8_BLOCK128) return MOE_FFN_ERR_INVALID_ARG;
  *alignment = 1;
  return MOE_FFN_OK;
}

int moe_ffn_get_workspace_view(const moe_ffn_problem* p, moe_ffn_workspace_view* v) {
  if (!v) return MOE_FFN_ERR_INVALID_ARG;
  const int rc = check_problem(p);
  if (rc) return rc;
  const Layout L = moeffn::make_layout(p->max_tokens, p->hidden, p->intermediate, p->num_experts, p->top_k, p->recipe);
  v->h = L.h;
  v->h_sf = L.h_sf;
  v->o = L.o;
  v->h_row_bytes = L.h_row_bytes;
  v->h_sf_row_bytes = L.h_sf_row_bytes;
  v->o_row_bytes = L.o_row_bytes;
  return MOE_FFN_OK;
}

int moe_ffn_transform_weight_scales(const uint8_t* src, uint8_t* dst, int64_t num_experts, int64_t rows,
                                    int64_t k_blocks, void* stream) {
  if (!src || !dst || num_experts <= 0 || rows <= 0 || k_blocks <= 0 || rows % 16 != 0 || k_blocks % 4 != 0)
    return MOE_FFN_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(src) & 3u) != 0 || (reinterpret_cast<uintptr_t>(dst) & 3u) != 0)
    return MOE_FFN_ERR_INVALID_ARG;
  const hipError_t e = moeffn::launch_transform_scales(src, dst, num_experts, rows, k_blocks,
                                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_FFN_OK : MOE_FFN_ERR_HIP;
}

int moe_ffn_quantize_activations(const void* x_bf16, int64_t num_tokens, int64_t hidden, void* x_e4m3,
                                 uint8_t* x_sf, void* stream) {
  if (num_tokens < 0 || hidden <= 0) return MOE_FFN_ERR_INVALID_ARG;
  if (hidden % 32 != 0) return MOE_FFN_ERR_UNSUPPORTED;
  if (num_tokens == 0) return MOE_FFN_OK;
  if (!x_bf16 || !x_e4m3 || !x_sf) return MOE_FFN_ERR_INVALID_ARG;
  if (!aligned16(x_bf16) || (reinterpret_cast<uintptr_t>(x_e4m3) & 7u) != 0) return MOE_FFN_ERR_INVALID_ARG;
  if (num_tokens > (int64_t(1) << 40) / hidden) return MOE_FFN_ERR_UNSUPPORTED;
  const hipError_t e = moeffn::launch_quantize_act(static_cast<const uint16_t*>(x_bf16), static_cast<uint8_t*>(x_e4m3),
                                                   x_sf, num_tokens * hidden, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_FFN_OK : MOE_FFN_ERR_HIP;
}

int moe_ffn_route_topk(const void* x_bf16, const void* w_gate_bf16, int64_t num_tokens, int64_t hidden,
                       int64_t num_experts, int64_t top_k, float* logits, int32_t* topk_idx, float* topk_weights,
                       void* stream) {
  if (num_tokens < 0 || hidden <= 0 || num_experts <= 0) return MOE_FFN_ERR_INVALID_ARG;
  if (hidden % 64 != 0 || num_experts > 512 || hidden > (1 << 20)) return MOE_FFN_ERR_UNSUPPORTED;
  if (top_k < 1 || top_k > 64 || top_k > num_experts) return MOE_FFN_ERR_INVALID_ARG;
  if (num_tokens == 0) return MOE_FFN_OK;
  // 32-bit buffer offsets into x and the gate weights
  if (num_tokens * hidden * 2 >= (int64_t(1) << 31) || num_experts * hidden * 2 >= (int64_t(1) << 31))
    return MOE_FFN_ERR_UNSUPPORTED;
  if (!x_bf16 || !w_gate_bf16 || !logits || !topk_idx || !topk_weights) return MOE_FFN_ERR_INVALID_ARG;
  if (!aligned16(x_bf16) || !aligned16(w_gate_bf16) || !aligned16(logits)) return MOE_FFN_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(topk_idx) & 3u) != 0 || (reinterpret_cast<uintptr_t>(topk_weights) & 3u) != 0)
    return MOE_FFN_ERR_INVALID_ARG;
  const hipError_t e = moeffn::launch_router(static_cast<const uint16_t*>(x_bf16), static_cast<const uint16_t*>(w_gate_bf16),
                                             logits, topk_idx, topk_weights, (int)num_tokens, (int)hidden,
                                             (int)num_experts, (int)top_k, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_FFN_OK : MOE_FFN_ERR_HIP;
}

int moe_ffn_transform_weights(const void* src, void* dst, int64_t num_experts, int64_t rows, int64_t k_bytes,
                              void* stream) {
  if (!src || !dst || num_experts <= 0 || rows <= 0 || k_bytes <= 0 || rows % 16 != 0 || k_bytes % 64 != 0)
    return MOE_FFN_ERR_INVALID_ARG;
  if (!aligned16(src) || !aligned16(dst)) return MOE_FFN_ERR_INVALID_ARG;
  const hipError_t e = moeffn::launch_transform_weights(static_cast<const uint8_t*>(src), static_cast<uint8_t*>(dst),
                                                        num_experts, rows, k_bytes, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_FFN_OK : MOE_FFN_ERR_HIP;
}

const char* moe_ffn_strerror(int code) {
  switch (code) {
    case MOE_FFN_OK: return "ok";
    case MOE_FFN_ERR_INVALID_ARG: return "invalid argument";
    case MOE_FFN_ERR_UNSUPPORTED: return "unsupported shape";
    case MOE_FFN_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MOE_FFN_ERR_HIP: return "HIP runtime error";
    case MOE_FFN_STATUS_BAD_EXPERT_INDEX: return "status: expert index outside [-1, E) was masked";
    case MOE_FFN_STATUS_TIMEOUT: return "status: grid barrier or readiness wait timed out";
    case MOE_FFN_STATUS_DIRTY_WORKSPACE: return "status: workspace counters were not zero at entry";
    default: return "unknown code";
  }
}

int moe_ffn_forward(const moe_ffn_problem* p, const moe_ffn_args* a, void* workspace, size_t workspace_bytes,
                    void* stream) {
  return moeffn::forward_enqueue(p, a, workspace, workspace_bytes, static_cast<hipStream_t>(stream), nullptr);
}

}  // extern "C"

namespace moeffn {

int forward_enqueue(const moe_ffn_problem* p, const moe_ffn_args* a, void* workspace, size_t workspace_bytes,
                    hipStream_t stream, hipError_t (*before_launch)(void* workspace, hipStream_t stream)) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (!a || !workspace) return MOE_FFN_ERR_INVALID_ARG;
  const int recipe = p->recipe;
  const bool bf16 = recipe == MOE_FFN_RECIPE_BF16;
  const int64_t T = a->num_tokens;
  if (T < 0 || T > p->max_tokens) return MOE_FFN_ERR_INVALID_ARG;
  if (a->y_dtype != MOE_FFN_Y_BF16 && a->y_dtype != MOE_FFN_Y_FP32) return MOE_FFN_ERR_INVALID_ARG;
  if (!a->w1 || !a->w2 || !aligned16(a->w1) || !aligned16(a->w2)) return MOE_FFN_ERR_INVALID_ARG;
  if (!bf16 && (!a->w1_sf || !a->w2_sf || !aligned16(a->w1_sf) || !aligned16(a->w2_sf))) return MOE_FFN_ERR_INVALID_ARG;
  const bool tiled = p->weight_layout == MOE_FFN_WEIGHTS_TILED;
  if (T > 0) {
    if (!a->x || !a->topk_idx || !a->topk_weights || !a->y) return MOE_FFN_ERR_INVALID_ARG;
    if (!aligned16(a->x) || !aligned16(a->y) || !aligned16(a->topk_idx) || !aligned16(a->topk_weights))
      return MOE_FFN_ERR_INVALID_ARG;
    if (!bf16 && (!a->x_sf || !aligned16(a->x_sf))) return MOE_FFN_ERR_INVALID_ARG;
  }
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return MOE_FFN_ERR_INVALID_ARG;
  const Layout L = moeffn::make_layout(p->max_tokens, p->hidden, p->intermediate, p->num_experts, p->top_k, recipe);
  if (workspace_bytes < L.total) return MOE_FFN_ERR_WORKSPACE_TOO_SMALL;

  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_FFN_ERR_HIP;
  const int cus = physical_cus(dev);
  if (cus <= 0) return MOE_FFN_ERR_HIP;
  const int reserve = a->reserved_cus >= 0 ? a->reserved_cus : (int)env_long("MOE_FFN_RESERVED_CUS", 2);
  int grid = moe_ffn_launch_size(cus, reserve, a->max_cus);
  const long timeout_ms = env_long("MOE_FFN_BARRIER_TIMEOUT_MS", 2000);

  uint8_t* ws = static_cast<uint8_t*>(workspace);
  KParams k{};
  k.T = (int32_t)T;
  k.H = (int32_t)p->hidden;
  k.I = (int32_t)p->intermediate;
  k.E = (int32_t)p->num_experts;
  k.k = (int32_t)p->top_k;
  k.y_fp32 = a->y_dtype == MOE_FFN_Y_FP32;
  k.clamp_on = std::isfinite(a->activation_clamp) && a->activation_clamp > 0.0f;
  k.clamp = k.clamp_on ? a->activation_clamp : 0.0f;
  k.timeout_ticks = (uint64_t)(timeout_ms > 0 ? timeout_ms : 1) * 100000ull;
  k.x = static_cast<const uint8_t*>(a->x);
  k.x_sf = static_cast<const uint8_t*>(a->x_sf);
  k.idx = a->topk_idx;
  k.tw = a->topk_weights;
  k.w1 = static_cast<const uint8_t*>(a->w1);
  k.w1_sf = static_cast<const uint8_t*>(a->w1_sf);
  k.w2 = static_cast<const uint8_t*>(a->w2);
  k.w2_sf = static_cast<const uint8_t*>(a->w2_sf);
  k.tiled = tiled ? 1 : 0;
  k.y = a->y;
  k.out_counts = a->expert_counts;
  k.out_offsets = a->expert_offsets;
  k.out_r2s = a->row_to_slot;
  k.out_s2r = a->slot_to_row;
  k.out_status = a->status;
  k.ctrl = reinterpret_cast<moeffn::Ctrl*>(ws + L.ctrl);
  k.bars = reinterpret_cast<uint32_t*>(ws + L.bars);
  k.counts = reinterpret_cast<int32_t*>(ws + L.counts);
  k.offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
  k.hist = reinterpret_cast<int32_t*>(ws + L.hist);
  k.r2s = reinterpret_cast<int32_t*>(ws + L.r2s);
  k.s2r = reinterpret_cast<int32_t*>(ws + L.s2r);
  k.h = ws + L.h;
  k.h_sf = ws + L.h_sf;
  k.o = ws + L.o;

  int bm = choose_block_m(recipe, T, p->top_k, p->num_experts);
  const long bm_env = env_long("MOE_FFN_BLOCK_M", 0);  // tuning override: 16, 32, 64 or 128
  if ((bm_env == 16 || bm_env == 32 || bm_env == 64 || bm_env == 128) && bm_env <= moeffn::max_block_m(recipe) &&
      bm_env >= moeffn::min_block_m(recipe))
    bm = (int)bm_env;
  // the 128-row tiles read the TILED weight layout (and the stage-major scale copies of the workspace)
  if (bm == 128 && (!tiled || L.hsg == L.xsg)) bm = 64;
  // a small call runs on fewer workgroups than the CU budget allows (never more)
  const int64_t work = useful_workgroups(T, p->hidden, p->intermediate, p->num_experts, p->top_k, bm);
  if (work < grid) grid = work < 2 ? 2 : (int)(work + (work & 1));
  if (env_long("MOE_FFN_LOG", 0) > 0)
    std::fprintf(stderr, "moe_ffn: T=%lld recipe=%d grid=%d (CUs %d, reserve %d, cap %d) block_m=%d\n",
                 (long long)T, recipe, grid, cus, reserve, a->max_cus, bm);
  if (bm == 128) {
    k.xsg = reinterpret_cast<uint32_t*>(ws + L.xsg);
    k.hsg = reinterpret_cast<uint32_t*>(ws + L.hsg);
    k.sg_rows = (int32_t)L.h_rows;
  }
  if (before_launch && before_launch(workspace, stream) != hipSuccess) return MOE_FFN_ERR_HIP;
  const hipError_t err = moeffn::launch_forward(recipe, bm, tiled, grid, k, stream);
  return err == hipSuccess ? MOE_FFN_OK : MOE_FFN_ERR_HIP;
}

}  // namespace moeffn
