/*
 * moe_ffn.h -- C ABI of the MI355X (gfx950) fused MoE expert-FFN forward.
 *
 * One call computes, for a batch of tokens already routed to their top-k
 * experts, the "MegaMoE" forward described by the DeepGEMM / sglang pages:
 *   1. routing: per-expert token histogram, exclusive prefix sum and a
 *      stable (ascending slot) index scatter ("SM90 MegaMoE dev log",
 *      Phase-2 entry: expert count, source token / top-k index write);
 *   2. L1 grouped GEMM, hidden -> 2 x intermediate (gate rows, then up rows);
 *   3. SwiGLU with activation clamp, re-quantised per 1x32 block
 *      ("[Blackwell] Reserve SMs for DeepGEMM MegaMoE grid barriers" digest,
 *      key-code section: activation="swiglu", activation_clamp, recipe
 *      (1, 1, 32); dev log Phase-1 entry: l2_acts / l2_acts_sf views);
 *   4. L2 grouped GEMM, intermediate -> hidden;
 *   5. top-k weighted combine into y, deterministic (fixed slot order).
 * The whole call is one persistent kernel whose grid is the CU count minus a
 * tunable reserve, kept even ("[Blackwell] Reserve SMs ..." page, Summary /
 * Fix / root cause; digest, implementation breakdown items 2-3), and which
 * resets its own workspace counters on every call so that graph replay with
 * changed inputs never consumes stale state ("[Bugfix] Reset MegaMoE combine
 * readiness for CUDA graph replay", description).
 *
 * Conventions
 *   - All tensor pointers are DEVICE pointers owned by the caller; the
 *     library never allocates, frees, memsets or synchronises.
 *   - Row-major, last dimension contiguous, 16-byte aligned base pointers.
 *   - e4m3 = OCP FP8 E4M3FN; e2m1 = OCP FP4 (two per byte, element 2j in the
 *     low nibble, 2j+1 in the high nibble); e8m0 = power-of-two scale byte
 *     2^(b-127) applying to one 1x32 block along the contraction dimension.
 *   - Errors: functions return 0 (MOE_FFN_OK) or a negative MOE_FFN_ERR_*
 *     code and never throw.  Device-side conditions are written to the
 *     optional device int *status (MOE_FFN_STATUS_*).
 */
#ifndef MOE_FFN_H
#define MOE_FFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element recipe (the pages' recipe argument): */
#define MOE_FFN_RECIPE_BF16 0     /* x, W1, W2 bf16; no scales; h re-rounded to bf16       */
#define MOE_FFN_RECIPE_FP8_FP8 1  /* x, W e4m3 + e8m0 per 1x32 along K; h e4m3 + e8m0     */
#define MOE_FFN_RECIPE_FP8_FP4 2  /* x e4m3, W e2m1 (packed), e8m0 per 1x32 along K       */
/* Recipe (1, 128, 128) with float scale factors ("SM90 MegaMoE dev log",
   Phase-1 entry: the wrapper's recipe (1, 128, 128) with the float SF path):
   x, W e4m3; one fp32 scale per 1 x 128 block of an activation row and per
   128 x 128 block of a weight matrix; h re-quantised per 1 x 128 block with
   s = max(fp32(amax / 448), 2^-126) and code = e4m3 (nearest even,
   saturating) of the IEEE fp32 quotient h / s.  H and I multiples of 128;
   runs on 64-row token blocks; row-major weights only. */
#define MOE_FFN_RECIPE_FP8_BLOCK128 3

/* Storage layout of the weights (moe_ffn_problem.weight_layout):
   ROW_MAJOR: w1 [E, 2I, H] and w2 [E, H, I] row-major (K contiguous; e2m1 packs
     element 2j in the low nibble of byte j), scales [E, rows, K/32] row-major.
     Every recipe.  Large e2m1 calls run on 64-row token blocks.
   TILED (e2m1 recipe only; the production layout of the e2m1 weights, prepared
     once per set of weights by moe_ffn_transform_weights and
     moe_ffn_transform_weight_scales): per expert, the weight matrix [rows, K]
     stored as 1 KB tiles of 16 rows x one 128-element K stage in MFMA operand
     order, and its scales as groups of four K stages per 16-row block (exact
     offsets at the two transforms).  Same sizes as ROW_MAJOR; the caller holds
     this one copy.  Every token-block size, including the 128-row tiles of
     large calls, reads it with whole-tile loads. */
#define MOE_FFN_WEIGHTS_ROW_MAJOR 0
#define MOE_FFN_WEIGHTS_TILED 1

/* Output element type of y. */
#define MOE_FFN_Y_BF16 0
#define MOE_FFN_Y_FP32 1

/* Synchronous return codes. */
#define MOE_FFN_OK 0
#define MOE_FFN_ERR_INVALID_ARG (-1)        /* null pointer, negative size, misaligned pointer  */
#define MOE_FFN_ERR_UNSUPPORTED (-2)        /* shape outside what the kernels handle            */
#define MOE_FFN_ERR_WORKSPACE_TOO_SMALL (-3)
#define MOE_FFN_ERR_HIP (-4)                /* a HIP runtime call failed (launch, device query) */

/* Device status codes written to args.status (0 = success). */
#define MOE_FFN_STATUS_OK 0
#define MOE_FFN_STATUS_BAD_EXPERT_INDEX 1   /* an index outside [-1, E) was masked (y still valid) */
#define MOE_FFN_STATUS_TIMEOUT 2            /* a grid barrier / readiness wait exceeded its bound; */
                                            /* y is undefined; the workspace is left clean         */
#define MOE_FFN_STATUS_DIRTY_WORKSPACE 3    /* the control block was not zero at entry: the call   */
                                            /* did nothing and left it so; zero the workspace      */

/* Problem: fixes the workspace size and layout.  It does not depend on the
   CU count or the reserve (digest: buffer cache key excludes the SM count).
   The tiles address x rows, h rows and one expert's weight matrix with 32-bit
   byte offsets: a problem with max_tokens*H*a, (max_tokens*k + 128)*I*a
   (a = 2 for BF16, else 1) or one expert's W1 bytes (2I*H times 2, 1 or 1/2)
   at or above 2^31 is MOE_FFN_ERR_UNSUPPORTED (DeepSeek shape, k = 8:
   max_tokens <= 131055). */
typedef struct {
    int64_t max_tokens;   /* capacity of x / y / topk rows (>= num_tokens of any call)         */
    int64_t hidden;       /* H: multiple of 128 (64 for BF16)                                  */
    int64_t intermediate; /* I: multiple of 128 (64 for BF16)                                  */
    int64_t num_experts;  /* E: 1..512                                                         */
    int64_t top_k;        /* k: 1..64                                                          */
    int32_t recipe;       /* MOE_FFN_RECIPE_*                                                  */
    int32_t weight_layout; /* MOE_FFN_WEIGHTS_* (TILED only with MOE_FFN_RECIPE_FP8_FP4)        */
} moe_ffn_problem;

/* Per-call arguments.  Shapes use T = num_tokens. */
typedef struct {
    int64_t num_tokens;          /* 0 <= T <= max_tokens; T = 0 writes no row of y                 */
    const void* x;               /* [T, H] e4m3 bytes, or bf16 for the BF16 recipe                  */
    const void* x_sf;            /* [T, H/32] e8m0 (FP8_BLOCK128: [T, H/128] fp32); NULL for BF16   */
    const int32_t* topk_idx;     /* [T, k] expert ids; -1 masks a slot                              */
    const float* topk_weights;   /* [T, k] combine weights                                          */
    const void* w1;              /* [E, 2I, H] (e2m1: [E, 2I, H/2] bytes); rows [0,I) gate, [I,2I) up; */
                                 /* in the problem's weight_layout                                   */
    const void* w1_sf;           /* [E, 2I, H/32] e8m0 (or its TILED order; FP8_BLOCK128:            */
                                 /* [E, 2I/128, H/128] fp32); NULL for BF16                          */
    const void* w2;              /* [E, H, I] (e2m1: [E, H, I/2] bytes), in the weight_layout       */
    const void* w2_sf;           /* [E, H, I/32] e8m0 (or TILED; FP8_BLOCK128: [E, H/128, I/128]    */
                                 /* fp32); NULL for BF16                                              */
    void* y;                     /* [T, H] of y_dtype; rows >= T untouched                          */
    int32_t y_dtype;             /* MOE_FFN_Y_*                                                      */
    float activation_clamp;      /* finite and > 0: clamp gate and up to [-c, c]; else no clamp      */
    int32_t reserved_cus;        /* CUs left free for other streams; < 0: env MOE_FFN_RESERVED_CUS   */
                                 /* or 2; the grid is even(min(cap, max(2, CUs - reserve)))          */
    int32_t max_cus;             /* cap on the grid (0 = none)                                       */
    int32_t* expert_counts;      /* optional [E] device out: rows per expert                         */
    int32_t* expert_offsets;     /* optional [E+1] device out: exclusive prefix of counts            */
    int32_t* row_to_slot;        /* optional [T*k] device out: first R = offsets[E] entries written  */
    int32_t* slot_to_row;        /* optional [T*k] device out: row of each slot, -1 when masked      */
    int32_t* status;             /* optional device int: MOE_FFN_STATUS_* of this call               */
} moe_ffn_args;

/* Bytes of device workspace one in-flight call needs (buffer-size query of the
   dev log's Phase-1 host API).  The workspace must be zero-filled once after
   allocation; afterwards every call leaves its counters zeroed.  One
   workspace serves one call at a time: calls that overlap on it race. */
int moe_ffn_get_workspace_size(const moe_ffn_problem* problem, size_t* bytes);

/* Multiple that max_tokens must be a multiple of (token-alignment query of the
   dev log's Phase-1 host API).  The kernels handle ragged expert groups, so
   this is 1 for every recipe. */
int moe_ffn_get_token_alignment(int32_t recipe, int64_t* alignment);

/* Enqueue the forward on `stream` (a hipStream_t; NULL = default stream).
   Asynchronous: returns after the launch; never synchronises, allocates or
   memsets, so it can be captured into a HIP graph.  Thread-safe (no mutable
   global state). */
int moe_ffn_forward(const moe_ffn_problem* problem, const moe_ffn_args* args,
                    void* workspace, size_t workspace_bytes, void* stream);

/* The forward without any allocation, for callers that cannot allocate (code
   under HIP graph capture, tight serving loops, harnesses that forbid
   allocation): the same computation and arguments as moe_ffn_forward, on a
   workspace the library keeps in a static device array of
   MOE_FFN_NOALLOC_MAX_WORKSPACE bytes per GPU (held until the process ends).
   Problems whose moe_ffn_get_workspace_size exceeds that return
   MOE_FFN_ERR_WORKSPACE_TOO_SMALL (e.g. the DeepSeek shape up to 496 tokens
   fits: 67.0 MB at 496, 67.5 MB at 500).  Each call clears the array's control block with a kernel on
   `stream` before the forward; calls that overlap on one GPU share the array
   and race.  Calls no hipMalloc / hipFree; other errors as moe_ffn_forward. */
#define MOE_FFN_NOALLOC_MAX_WORKSPACE (64u << 20)
int moe_ffn_forward_noalloc(const moe_ffn_problem* problem, const moe_ffn_args* args, void* stream);

/* Weight-scale transform to the TILED layout (the weight transform step of
   the pages' host API, done once per set of weights).  src: the row-major e8m0
   scales [num_experts, rows, k_blocks] of one weight matrix (W1: rows = 2I,
   k_blocks = H/32; W2: rows = H, k_blocks = I/32); with nk = k_blocks/4 K
   stages of 128 elements, row r = 16b + i, stage s = 4G + u, 32-block c < 4:
     dst[e*rows*k_blocks + (b*nk + 4G)*64 + i*4*n + u*4 + c] = src[e][r][4s + c],
     n = min(4, nk - 4G) (the stages in group G),
   i.e. per 16-row block, groups of four K stages, each group [16 rows][n
   stages][4 blocks]: one 16-byte load brings a row's scales for four stages;
   a stage's scales of the 16 rows lie 4n bytes apart.  src and dst: device buffers
   of num_experts*rows*k_blocks bytes, 4-byte aligned, not overlapping.
   Enqueued on `stream` (a hipStream_t; NULL = default stream); asynchronous,
   allocates nothing.  Returns MOE_FFN_ERR_INVALID_ARG for null or misaligned
   pointers, non-positive sizes, rows not a multiple of 16 or k_blocks not a
   multiple of 4, MOE_FFN_ERR_HIP when the launch fails. */
int moe_ffn_transform_weight_scales(const uint8_t* src, uint8_t* dst, int64_t num_experts, int64_t rows,
                                    int64_t k_blocks, void* stream);

/* Pre-dispatch activation quantisation, the step right before the forward
   ("[Blackwell] Reserve SMs for DeepGEMM MegaMoE grid barriers", Fix section:
   pre-dispatch runs before the kernel call; its digest, key-code section: the
   buffer fetch and pre-dispatch quantisation precede the call).  The pages do
   not state its arithmetic; it applies the forward's own 1x32 re-quantisation
   rule to bf16 activations:
     for every 32-element block b of a row (blocks along H):
       E = smallest integer with amax(|x|) <= 448 * 2^E, clamped to
           [-127, 127]; E = 0 for an all-zero block;
       x_sf[b] = E + 127;
       x_e4m3[i] = E4M3FN code of x[i] * 2^-E, rounded to nearest even,
                   saturating (never NaN).
   x_bf16: [num_tokens, hidden] bf16 bit patterns (device, 16-byte aligned),
   finite values (a block holding inf or NaN gets unspecified codes);
   x_e4m3: [num_tokens, hidden] bytes (device, 8-byte aligned);
   x_sf: [num_tokens, hidden/32] e8m0 bytes (device).  The outputs are exactly
   the x / x_sf inputs of moe_ffn_forward for the e4m3 recipes.  hidden must
   be a positive multiple of 32 (else MOE_FFN_ERR_UNSUPPORTED); num_tokens = 0
   is a no-op.  Enqueued on `stream` (a hipStream_t; NULL = default stream);
   asynchronous, allocates nothing, capturable.  Returns
   MOE_FFN_ERR_INVALID_ARG for negative sizes, null or misaligned pointers
   with num_tokens > 0, MOE_FFN_ERR_HIP when the launch fails. */
int moe_ffn_quantize_activations(const void* x_bf16, int64_t num_tokens, int64_t hidden, void* x_e4m3,
                                 uint8_t* x_sf, void* stream);

/* Gate and top-k: the router that produces topk_idx / topk_weights for
   moe_ffn_forward ("[Blackwell] Reserve SMs for DeepGEMM MegaMoE grid
   barriers", Fix section: gate computation and top-k selection run before
   the MegaMoE call).  The pages give no formula; it is a softmax router:
     logits[t, e] = sum_h x[t, h] * w_gate[e, h]   (bf16 inputs, fp32 sum)
     topk_idx[t, :] = the top_k experts of largest logit, in descending
                      order; equal logits: the lower expert id first
     topk_weights[t, j] = exp(logits[t, idx_j] - max) / sum over the chosen
                      experts (softmax of the top-k, renormalised to 1), fp32.
   x_bf16: [num_tokens, hidden] bf16 bit patterns; w_gate_bf16: [num_experts,
   hidden] bf16; logits: [num_tokens, num_experts] fp32, written (also the
   scratch the top-k reads); topk_idx: [num_tokens, top_k] int32;
   topk_weights: [num_tokens, top_k] fp32.  All device pointers; x, w_gate
   and logits 16-byte aligned, topk_idx / topk_weights 4-byte aligned.
   hidden must be a positive multiple of 64, num_experts at most 512 and
   num_tokens * hidden * 2 below 2^31, else MOE_FFN_ERR_UNSUPPORTED;
   1 <= top_k <= min(64,
   num_experts), else MOE_FFN_ERR_INVALID_ARG; num_tokens = 0 is a no-op.
   Inputs must be finite.  Two kernels enqueued on `stream` (a hipStream_t;
   NULL = default stream); asynchronous, allocates nothing, capturable.
   MOE_FFN_ERR_INVALID_ARG also for negative sizes and null or misaligned
   pointers with num_tokens > 0; MOE_FFN_ERR_HIP when a launch fails. */
int moe_ffn_route_topk(const void* x_bf16, const void* w_gate_bf16, int64_t num_tokens, int64_t hidden,
                       int64_t num_experts, int64_t top_k, float* logits, int32_t* topk_idx, float* topk_weights,
                       void* stream);

/* Weight transform to the TILED layout for the e2m1 recipe (the weight
   transform step of the pages' host API, done once per set of weights):
   re-orders each expert's packed e2m1 weight matrix [rows, k_bytes] into tiles
   of 16 rows x 64 bytes (one 128-element K stage), each tile 1 KB in MFMA
   operand order:
     dst[((e*(rows/16) + b) * (k_bytes/64) + s) * 1024 + (g*16 + r) * 16 + c]
       = src[(e*rows + 16b + r) * k_bytes + 64s + 16g + c]
   for r < 16, g < 4, c < 16.  The GEMM tiles then load one contiguous 1 KB
   piece per 16 weight rows and K stage.  For W1 rows = 2I, k_bytes = H/2; for
   W2 rows = H, k_bytes = I/2.  src and dst: device buffers of
   num_experts*rows*k_bytes bytes, 16-byte aligned, not overlapping.  Enqueued
   on `stream` (a hipStream_t; NULL = default stream); asynchronous,
   allocates nothing.  Returns MOE_FFN_ERR_INVALID_ARG for null or misaligned
   pointers, non-positive sizes, rows not a multiple of 16 or k_bytes not a
   multiple of 64, MOE_FFN_ERR_HIP when the launch fails. */
int moe_ffn_transform_weights(const void* src, void* dst, int64_t num_experts, int64_t rows, int64_t k_bytes,
                              void* stream);

/* Text of a return or status code (static string). */
const char* moe_ffn_strerror(int code);

/* Host-only launch-size rule used by moe_ffn_forward: physical CUs minus the
   reserve (negative reserve = 0), at least 2, capped by max_cus when > 0,
   rounded down to even, at least 2 ("[Blackwell] Reserve SMs ..." digest,
   implementation breakdown items 2-3). */
int moe_ffn_launch_size(int physical_cus, int reserved_cus, int max_cus);

/* Byte offsets of the intermediates inside the workspace, for inspection:
   h ([max_tokens*k + pad, I] e4m3, or bf16), h_sf ([.., I/32] e8m0) and
   o ([max_tokens*k, H] per routed row: the L2 result in bf16 for the e4m3
   recipes, in fp32 for the BF16 recipe; o_row_bytes gives which). */
typedef struct {
    size_t h, h_sf, o;
    int64_t h_row_bytes, h_sf_row_bytes, o_row_bytes;
} moe_ffn_workspace_view;
int moe_ffn_get_workspace_view(const moe_ffn_problem* problem, moe_ffn_workspace_view* view);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FFN_H */
