/*
 * moelora.h -- C ABI of the fused MoE expert-FFN layer with multi-LoRA for
 * AMD Instinct MI355X (gfx950).
 *
 * What the layer computes follows the AWS Machine Learning blog post
 * "Efficiently serve dozens of fine-tuned models with vLLM on Amazon
 * SageMaker AI and Amazon Bedrock" ([AWS] below), section "Implementing
 * multi-LoRA inference for MoE models in vLLM" and its Figure 1: a router
 * sends each token to its top-k experts; each expert applies a gate_up
 * projection and a down projection; a LoRA adapter on a projection with base
 * weight W adds x A B (shrink z = x A to rank r, expand z B back), and every
 * token carries its own adapter id, or none.  For each routed (token, expert)
 * pair with adapter a (a = -1: none):
 *
 *     g   = x W_gu[e]^T + [a >= 0] (x A_gu[a][e]^T) B_gu[a][e]^T   (width 2I)
 *     h   = SiLU(g[0:I]) * g[I:2I],   SiLU(v) = v / (1 + exp(-v))
 *     y   = h W_d[e]^T  + [a >= 0] (h A_d[a][e]^T) B_d[a][e]^T     (width H)
 *     out[t] = sum_j w[t][j] * y(t, ids[t][j])
 *
 * The router, when used, keeps the k largest logits (ties to the lower
 * expert index, listed largest first) and sets w = softmax over the kept
 * logits (softmax over all E followed by renormalisation over the kept k).
 * Logits are expected to be finite: a NaN's place in the order is
 * unspecified (the picks are still k distinct experts in range).
 * The post fixes neither the router formula, the activation nor the gate/up
 * split; these are the readings used here.
 *
 * Storage: row-major, contraction dimension contiguous, elements of the
 * layer dtype (float32, or bf16 as 16-bit patterns):
 *     x        [T][H]          out      [T][H]
 *     W_gu     [E][2I][H]      rows 0..I-1 gate, I..2I-1 up
 *     W_d      [E][H][I]
 *     A_gu     [NA][E][r][H]   B_gu     [NA][E][2I][r]
 *     A_d      [NA][E][r][I]   B_d      [NA][E][H][r]
 *     router_logits [T][E] float32;  topk_ids [T][k] int32;
 *     topk_w [T][k] float32;  adapter_ids [T] int32 (-1 = none)
 * Every device pointer must be 16-byte aligned; the workspace 256-byte
 * aligned.
 *
 * Ownership: the caller allocates and owns every device buffer, the
 * workspace and the stream.  The library owns only the plan (a host
 * object).  moelora_forward only enqueues kernels on the given stream: it
 * never synchronises or allocates, so it can be captured in a HIP graph, and
 * nothing is specialised on the token count.  Kernels are compiled ahead of
 * time; the HIP runtime loads their code on first use, so the first forward
 * of a plan on a device (the current device) looks up every kernel that
 * plan can launch at any token count up to max_tokens, and no later forward
 * loads code ([AWS] "Execution optimizations": loading code for each new
 * context length cost a tenfold time-to-first-token regression).
 *
 * Errors: every entry point returns a status; nothing throws or aborts
 * across the ABI.  Device-resident ids are preconditions: expert ids in
 * [0, E), adapter ids in [-1, NA).  A row with an out-of-range expert id is
 * dropped (adds nothing to its token's output) and an out-of-range adapter
 * id counts as -1; either sets a bit in the device error word that
 * moelora_read_device_error returns.  No kernel reads or writes out of
 * bounds on bad ids.
 */
#ifndef MOELORA_H
#define MOELORA_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define MOELORA_API __attribute__((visibility("default")))
#else
#define MOELORA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moelora_status {
    MOELORA_OK = 0,
    MOELORA_ERR_INVALID_ARG = -1,  /* null / misaligned pointer, bad size  */
    MOELORA_ERR_UNSUPPORTED = -2,  /* shape or dtype outside the limits    */
    MOELORA_ERR_WORKSPACE = -3,    /* workspace too small                  */
    MOELORA_ERR_HIP = -4,          /* a HIP runtime call or launch failed  */
    MOELORA_ERR_DEVICE = -5,       /* the device error word is non-zero    */
    MOELORA_ERR_TOO_LARGE = -6     /* beyond moelora_forward_noalloc's
                                      static scratch buffer                */
} moelora_status;

/* Element types.  MOELORA_BF16_FP8W: x, out and the LoRA weights bf16; the
 * base weights W_gu and W_d one byte per element, an OCP 8-bit floating-point
 * E4M3 code, with one float32 scale per weight row: the weight is
 * scale[row] times the code's value (the aib.vote news item on SageMaker
 * fused-MoE kernel optimizations, second item, routes FP8 MoE layers to a
 * fused path; it gives no quantisation scheme, and one scale per output row
 * is the reading taken here).  Each of w_gate_up / w_down then points at the
 * codes, [E][2I] rows of H codes / [E][H] rows of I codes, each row padded
 * with zero bytes to a multiple of 128 bytes (row pitch P = round_up(H, 128)
 * / round_up(I, 128), so every row starts on a 128-byte line), followed at
 * the next 256-byte boundary (byte offset round_up(E*2I*P, 256) /
 * round_up(E*H*P, 256)) by the scales, float32 [E][2I] / [E][H].  Requires H
 * and I multiples of 64 and r a multiple of 8. */
typedef enum moelora_dtype {
    MOELORA_F32 = 0,
    MOELORA_BF16 = 1,
    MOELORA_BF16_FP8W = 2
} moelora_dtype;

/* Bits of the device error word. */
#define MOELORA_DEVERR_EXPERT_ID 1   /* an expert id outside [0, E)        */
#define MOELORA_DEVERR_ADAPTER_ID 2  /* an adapter id outside [-1, NA)     */

/* Shape of one layer.  Limits (else MOELORA_ERR_UNSUPPORTED):
 * 1 <= E <= 1024, E * (NA + 1) <= 8448, 1 <= k <= min(E, 32),
 * 0 <= NA, 0 <= r <= 256 (r >= 1 when NA >= 1), 1 <= H, I <= 65536,
 * 0 <= max_tokens, max_tokens * k <= 2^24; flags: a combination of the
 * MOELORA_FLAG_* bits below (any other bit: MOELORA_ERR_UNSUPPORTED). */
typedef struct moelora_desc {
    int32_t max_tokens;
    int32_t hidden;      /* H */
    int32_t inter;       /* I (gate_up produces 2I) */
    int32_t n_experts;   /* E */
    int32_t top_k;       /* k */
    int32_t n_adapters;  /* NA */
    int32_t rank;        /* r */
    int32_t dtype;       /* moelora_dtype */
    uint32_t flags;      /* MOELORA_FLAG_* bits */
} moelora_desc;

/* Flags.  Both behaviours are always on in this library, so the bits are
 * accepted and change nothing; they exist so a caller can state that it
 * relies on them.
 *   DETERMINISTIC    results are bitwise repeatable for a given plan, input
 *                    and token count: split contractions (the split-K shrink
 *                    of [AWS] "Kernel optimizations", the split down GEMM)
 *                    write separate fp32 partials that their consumer adds
 *                    in a fixed order; no kernel uses floating-point atomics.
 *   DEBUG_CHECK_IDS  device-resident ids are range-checked: an expert id
 *                    outside [0, E) drops its row, an adapter id outside
 *                    [-1, NA) counts as -1, and either sets a bit of the
 *                    device error word (moelora_read_device_error). */
#define MOELORA_FLAG_DETERMINISTIC 1u
#define MOELORA_FLAG_DEBUG_CHECK_IDS 2u

typedef struct moelora_plan_s *moelora_plan_t;
typedef struct ihipStream_t *moelora_stream_t; /* the same type as hipStream_t */

/* Validate the shape and choose kernels, block size and split-K for every
 * token count up to max_tokens.  Host only: no device memory is touched and
 * no code is compiled or loaded; every kernel is compiled ahead of time and
 * takes the token count as a run-time argument, and the choices are made
 * here, once, for all token counts, because [AWS] "Execution optimizations"
 * traces a tenfold time-to-first-token regression to kernels recompiled for
 * each new context length.  Tuning switches in the environment (MOELORA_*)
 * are read here and never by a forward.  *workspace_bytes receives the
 * largest workspace any forward of 0..max_tokens tokens needs (every token
 * count is checked).  On success *plan must later be released with
 * moelora_plan_destroy.  Errors: MOELORA_ERR_INVALID_ARG for null
 * pointers, MOELORA_ERR_UNSUPPORTED for a shape, dtype or flag outside the
 * limits above. */
MOELORA_API moelora_status moelora_plan(const moelora_desc *desc, moelora_plan_t *plan,
                            size_t *workspace_bytes);

MOELORA_API void moelora_plan_destroy(moelora_plan_t plan);

/* Enqueue one layer call on `stream` (NULL = the null stream).
 *   n_tokens       0 <= n_tokens <= max_tokens; 0 is a no-op
 *   x              [T][H] layer dtype
 *   router_logits  [T][E] float32; NULL exactly when topk_ids and topk_w
 *                  are given
 *   topk_ids       [T][k] int32, or NULL to route from the logits
 *   topk_w         [T][k] float32, or NULL (with topk_ids NULL)
 *   adapter_ids    [T] int32, or NULL: no adapter for any token
 *   w_gate_up, w_down   base expert weights (required)
 *   lora_a_gu, lora_b_gu, lora_a_d, lora_b_d   adapter weights; all four
 *                  NULL (or NA == 0, or adapter_ids NULL) skips every LoRA
 *                  kernel ([AWS] "Execution optimizations": layers without
 *                  adapters exit early); otherwise all four are required
 *   out            [T][H] layer dtype, written (not accumulated)
 *   workspace      >= the size moelora_plan returned, 256-byte aligned; its
 *                  contents need no initialisation.  Concurrent forwards
 *                  need distinct workspaces.
 * The call returns after enqueueing; results are ready when the stream
 * reaches that point. */
MOELORA_API moelora_status moelora_forward(moelora_plan_t plan, int32_t n_tokens,
                               const void *x, const float *router_logits,
                               const int32_t *topk_ids, const float *topk_w,
                               const int32_t *adapter_ids,
                               const void *w_gate_up, const void *w_down,
                               const void *lora_a_gu, const void *lora_b_gu,
                               const void *lora_a_d, const void *lora_b_d,
                               void *out, void *workspace,
                               size_t workspace_bytes,
                               moelora_stream_t stream);

/* moelora_forward for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Same arguments and results as moelora_forward, without the
 * workspace: the call uses a static device array of the library,
 * MOELORA_STATIC_SCRATCH_BYTES (64 MiB) per GPU, allocated with the
 * library's code on each GPU it runs on and held until the process ends.
 * The call allocates nothing; its first call on a GPU looks up that GPU's
 * copy of the array.  `stream` must belong to the current device
 * (else MOELORA_ERR_INVALID_ARG).  A call whose workspace (the size
 * moelora_plan_info reports for n_tokens) exceeds the array returns
 * MOELORA_ERR_TOO_LARGE before touching the device.  Every call on a GPU
 * shares that GPU's array: calls that overlap on one GPU (two streams, two
 * threads) race and must be serialised by the caller, e.g. on one stream.
 * The array's contents need no initialisation; moelora_read_device_error
 * does not apply (its error word lives in the array). */
#define MOELORA_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
MOELORA_API moelora_status moelora_forward_noalloc(moelora_plan_t plan, int32_t n_tokens,
                               const void *x, const float *router_logits,
                               const int32_t *topk_ids, const float *topk_w,
                               const int32_t *adapter_ids,
                               const void *w_gate_up, const void *w_down,
                               const void *lora_a_gu, const void *lora_b_gu,
                               const void *lora_a_d, const void *lora_b_d,
                               void *out, moelora_stream_t stream);

MOELORA_API const char *moelora_status_string(moelora_status status);

/* ---------------------------------------------------------------------
 * Inspection hooks (tests and benchmarks).
 *
 * Alignment: the rows p = t*k + j are grouped per expert, each group padded
 * to a multiple of the block size BM (one BM shared by the four LoRA ops and
 * the base GEMMs, [AWS] "Tuning kernel configurations for Amazon SageMaker
 * AI and Amazon Bedrock"), and inside a group ordered by adapter (base-only
 * rows last), then by p ([AWS] "Implementing multi-LoRA inference for MoE
 * models in vLLM": expert routing compounded with adapter selection).  After
 * a forward of n_tokens tokens the workspace holds, at the offsets below
 * (bytes from the workspace start, int32 arrays):
 *   topk_ids [R], topk_w [R] (float32)  the router's output (only when the
 *                  forward routed from logits)
 *   sorted_rows [cap]       rows per expert; sentinel R in padding and after
 *                           num_padded
 *   block_expert [nblk]     expert of each block, -1 past num_padded
 *   seg_start [E+1]         padded start of each expert's rows
 *   lora_seg [max_seg][4]   (expert, adapter, start, len) for every run of
 *                           rows sharing an expert and an adapter >= 0, in
 *                           (expert, adapter) order; unused (-1, -1, 0, 0)
 *   tiles [max_tiles][4]    (block, adapter, lo, n): each run cut at block
 *                           boundaries, lo and n relative to the block;
 *                           unused (-1, -1, 0, 0)
 *   block_tile_start [nblk+1]  index of the first tile of block >= b
 *   counts [4]              num_padded, n_lora_seg, n_tiles, 0
 * with R = n_tokens * k, cap = BM * ceil((R + min(E, R) * (BM - 1)) / BM),
 * nblk = cap / BM, max_seg = min(R, E * NA), max_tiles = nblk + max_seg.
 * --------------------------------------------------------------------- */
typedef struct moelora_layout {
    int32_t block_m, cap, nblk, max_seg, max_tiles, reserved;
    size_t off_topk_ids, off_topk_w, off_sorted_rows, off_block_expert,
        off_seg_start, off_lora_seg, off_tiles, off_block_tile_start,
        off_counts, off_error;
} moelora_layout;

/* The layout a forward of n_tokens tokens uses (host only). */
MOELORA_API moelora_status moelora_workspace_layout(moelora_plan_t plan, int32_t n_tokens,
                                        moelora_layout *layout);

/* Synchronise `stream`, then copy the device error word of the last forward
 * that used `workspace` into *error_bits (MOELORA_DEVERR_* bits). */
MOELORA_API moelora_status moelora_read_device_error(moelora_plan_t plan,
                                         const void *workspace,
                                         int32_t *error_bits,
                                         moelora_stream_t stream);

/* A one-line description of the kernels and tiles a forward of n_tokens
 * tokens uses (for logs); NUL-terminated, truncated to buf_len. */
MOELORA_API moelora_status moelora_plan_info(moelora_plan_t plan, int32_t n_tokens,
                                 char *buf, size_t buf_len);

/* Stage timing.  Between moelora_timing_begin and moelora_timing_end the
 * plan records HIP events around each stage of every forward (at most
 * max_calls forwards), on the forward's stream.  moelora_timing_end
 * synchronises, writes the summed milliseconds of each stage into
 * stage_ms[0..n_stages) (stages: 0 routing + alignment, 1 gate_up shrink,
 * 2 gate_up GEMM + expand + SiLU*up, 3 down shrink, 4 down GEMM + expand,
 * 5 top-k combine) and the number of timed forwards into *n_calls.  Events
 * are created in begin and destroyed in end, so timed forwards still
 * allocate nothing.  A plan in timing mode must not be used from two
 * threads at once. */
#define MOELORA_N_STAGES 6
MOELORA_API moelora_status moelora_timing_begin(moelora_plan_t plan, int32_t max_calls);
MOELORA_API moelora_status moelora_timing_end(moelora_plan_t plan, double *stage_ms,
                                  int32_t n_stages, int32_t *n_calls);

#ifdef __cplusplus
}
#endif

#endif /* MOELORA_H */
