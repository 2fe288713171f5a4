// Kernel parameter block and launcher of the fused MoE forward.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_ffn.h"
#include "moe_ffn_layout.h"

namespace moeffn {

// The forward of both entry points: checks the problem and the arguments,
// sizes the grid and launches the persistent kernel on `workspace`.
// `before_launch` (optional) is enqueued on the stream right before the
// kernel, after every check passed.  Returns a MOE_FFN_* code.
int forward_enqueue(const moe_ffn_problem* p, const moe_ffn_args* a, void* workspace, size_t workspace_bytes,
                    hipStream_t stream, hipError_t (*before_launch)(void* workspace, hipStream_t stream));

struct KParams {
  // problem of this call
  int32_t T, H, I, E, k;
  int32_t y_fp32;
  int32_t clamp_on;
  float clamp;
  int32_t tiled;           // weights (and their scales) in the TILED layout (e2m1 recipe)
  uint64_t timeout_ticks;  // bound on every wait, in 100 MHz realtime ticks
  // inputs
  const uint8_t* x;
  const uint8_t* x_sf;
  const int32_t* idx;
  const float* tw;
  const uint8_t* w1;
  const uint8_t* w1_sf;
  const uint8_t* w2;
  const uint8_t* w2_sf;
  void* y;
  // optional outputs
  int32_t* out_counts;
  int32_t* out_offsets;
  int32_t* out_r2s;
  int32_t* out_s2r;
  int32_t* out_status;
  // workspace views
  Ctrl* ctrl;
  uint32_t* bars;          // barrier group counters (kBarGroups lines of kBarLineWords)
  int32_t* counts;
  int32_t* offsets;
  int32_t* hist;
  int32_t* r2s;
  int32_t* s2r;
  uint8_t* h;
  uint8_t* h_sf;
  void* o;                 // per routed row: H fp32 values (BF16 recipe) or H bf16 values (e4m3 recipes)
  // 128-row tiles only (else null): stage-major scale copies, sg_rows rows each
  uint32_t* xsg;
  uint32_t* hsg;
  int32_t sg_rows;
};

// Launches the persistent kernel for `recipe` with token block `bm` on `grid`
// workgroups, reading the weights in the TILED layout when `tiled` (e2m1
// recipe).  Returns the hipError_t of the launch.
hipError_t launch_forward(int recipe, int bm, bool tiled, int grid, const KParams& p, hipStream_t stream);

// e2m1 weights [E][rows][kbytes] -> tiled: per 16-row block and 64-byte K stage one 1 KB piece in
// MFMA lane order (lane g*16 + r holds row r, bytes 16g .. 16g+15 of the stage).
hipError_t launch_transform_weights(const uint8_t* src, uint8_t* dst, int64_t E, int64_t rows, int64_t kbytes,
                                    hipStream_t stream);

// Row-major e8m0 weight scales [E][rows][kb] -> the TILED layout: per 16-row block, groups of four
// 128-element K stages, each group [16 rows][stages in the group][4 blocks].
hipError_t launch_transform_scales(const uint8_t* src, uint8_t* dst, int64_t E, int64_t rows, int64_t kb,
                                   hipStream_t stream);

// Largest token block the recipe supports (register budget of the A ring), and the smallest (the
// (1, 128, 128) recipe re-quantises whole 128-feature blocks, which only the 64-row tiles hold).
int max_block_m(int recipe);
int min_block_m(int recipe);

// bf16 -> e4m3 + e8m0 per 1x32 block over n_elems elements (a multiple of 32).
hipError_t launch_quantize_act(const uint16_t* x, uint8_t* q, uint8_t* sf, int64_t n_elems, hipStream_t stream);

// Softmax router: logits GEMM (bf16 MFMA) then the per-token top-k and renormalised weights.
hipError_t launch_router(const uint16_t* x, const uint16_t* wg, float* logits, int32_t* idx, float* wts, int T, int H,
                         int E, int k, hipStream_t stream);

}  // namespace moeffn
