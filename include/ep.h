/*
 * ep.h — MoE dispatch / combine on one MI355X (gfx950): the C ABI.
 *
 * The operations follow the DeepEP README (community translation),
 * section "Interfaces and examples":
 *   - dispatch (README "Example use in model training or inference
 *     prefilling", dispatch_forward): route each token's hidden row to the
 *     experts of its top-k choice, into expert-contiguous receive rows whose
 *     per-expert counts are padded to expert_alignment for the grouped GEMM;
 *     x may be BF16 or FP8 with per-token scale factors;
 *   - combine (combine_forward): reduce each token's k expert outputs back
 *     into one BF16 row;
 *   - dispatch_backward is a combine (also returning the combined weight
 *     gradients); combine_backward is a dispatch that reuses the handle;
 *   - handle caching for decode (README "Example use in inference decoding"):
 *     a handle is reused across calls and skips the layout and the CPU sync.
 * This library computes one GPU's share of that work: every receive row
 * lives in this GPU's memory; there is no transport.
 *
 * Conventions for every entry point:
 *   - Pointers marked "device" are HIP device pointers (or host pointers the
 *     device can access); "host" pointers are ordinary host memory.
 *   - The caller owns every buffer: inputs, outputs and the workspace. The
 *     library allocates no device memory, keeps no pointer after returning
 *     and holds no global state except a thread-local error message, each
 *     device's CU count (queried once) and the fixed 1 MiB device array of
 *     ep_dispatch_forward_static_scratch (one per GPU, for the process's
 *     lifetime).
 *   - `stream` is a hipStream_t (NULL = the null stream). All work is
 *     enqueued on it and runs asynchronously; only ep_handle_read_counts and
 *     ep_handle_check wait for the stream.
 *   - Argument errors (NULL or misaligned pointer, sizes out of range,
 *     workspace too small) return EP_ERR_INVALID_ARG / EP_ERR_WORKSPACE /
 *     EP_ERR_UNSUPPORTED immediately and enqueue nothing;
 *     ep_last_error_message() says what was wrong. A failed launch returns
 *     EP_ERR_HIP.
 *   - Data errors found on the device (an expert id outside [0, E) that is
 *     not -1; a fixed-capacity overflow) do not fail the call: the pair is
 *     skipped (its slot is -1, it is copied nowhere and contributes nothing
 *     to combine) and a sticky bit is set in the handle's error word, read
 *     with ep_handle_check.
 *   - Alignment: x, recv, y, out and their FP8 counterparts must be 16-byte
 *     aligned; hidden must be a multiple of 8 (BF16) or 128 (FP8).
 *   - Numbers: bf16 = bfloat16 bit patterns (uint16); FP8 = OCP E4M3FN bytes;
 *     scales and weights are IEEE binary32.
 *   - Environment (read at each launch):
 *       EP_BUFFER_DEBUG=1  print, to stderr, the launch geometry each call
 *                          picks (kernel, grid, block, rows per zero-fill
 *                          piece, row pieces per token): the library's form
 *                          of the README's EP_BUFFER_DEBUG (section
 *                          "Environment variables": print buffer set-up and
 *                          SM-count choices).
 *       EP_LAUNCH_CUS=n    size grids as if the device had n compute units
 *                          (1 <= n <= 4096). Results never depend on launch
 *                          geometry; this knob exists so tests can show it.
 */
#ifndef EP_H
#define EP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    EP_OK = 0,
    EP_ERR_INVALID_ARG = 1,
    EP_ERR_UNSUPPORTED = 2,
    EP_ERR_HIP = 3,
    EP_ERR_WORKSPACE = 4
} ep_status;

/* Receive layout.
 * EP_MODE_COMPACT: expert-major rows, expert e owns
 *   [expert_off[e], expert_off[e] + pad[e]) with pad[e] = ceil(cnt[e]/A)*A;
 *   its first cnt[e] rows hold the pairs routed to e, the rest are padding.
 * EP_MODE_FIXED: expert e owns [e*C, e*C + C) (a [E, C, hidden] buffer, the
 *   decode layout); its first min(cnt[e], C) rows are written, the others
 *   are left untouched. */
typedef enum { EP_MODE_COMPACT = 0, EP_MODE_FIXED = 1 } ep_mode;

/* Payload type of a dispatch.
 * EP_BF16: x is bf16 [T, hidden]; recv is bf16 [rows, hidden].
 * EP_FP8_QUANTIZE: x is bf16 [T, hidden]; each 1x128 block of a token is
 *   quantised once (amax = max |x|, scale = amax / 448, code =
 *   E4M3FN(x / scale) rounded to nearest even and saturated to +-448; an
 *   all-zero block has scale 0 and zero codes); recv is E4M3FN
 *   [rows, hidden], recv_scales is binary32 [rows, hidden/128] row-major.
 * EP_FP8_PREQUANT: x is already E4M3FN [T, hidden] with x_scales binary32
 *   [T, hidden/128] (the README's (data, scale_factors) tuple); codes and
 *   scales are copied bitwise.
 * Entry points take the payload type as an int32_t holding one of these
 * values (any other value is EP_ERR_INVALID_ARG), so that a caller's
 * out-of-range value is an error rather than an invalid enum. */
typedef enum { EP_BF16 = 0, EP_FP8_QUANTIZE = 1, EP_FP8_PREQUANT = 2 } ep_dtype;

/* ep_config.flags */
#define EP_FLAG_NO_ZERO_PAD 1u /* COMPACT: leave padding rows unwritten */

/* Bits of the device error word (ep_handle_check). */
#define EP_ERRFLAG_BAD_ID 1u   /* an id outside [0, E) other than -1 */
#define EP_ERRFLAG_OVERFLOW 2u /* FIXED: more than C pairs for an expert */

/* Static sizes of one layout; the README's buffer arguments
 * (num_max_tokens_per_rank, hidden, num_topk, expert_alignment).
 * Limits: 1 <= num_experts <= 1024, 1 <= num_topk <= 32,
 * num_experts % num_dests == 0, max_tokens * num_topk < 2^31,
 * 8 <= hidden <= 2^24 and hidden % 8 == 0 (hidden % 128 == 0 for FP8),
 * expert_alignment >= 1 (must be 1 in FIXED mode), capacity >= 1 in FIXED
 * mode, idx_bits 64 (int64 topk_idx, torch.topk's type) or 32. */
typedef struct {
    int32_t max_tokens;       /* T_max: tokens a layout may hold */
    int32_t hidden;           /* H */
    int32_t num_experts;      /* E */
    int32_t num_topk;         /* k */
    int32_t num_dests;        /* D: experts grouped in D contiguous ranges */
    int32_t expert_alignment; /* A */
    int32_t capacity;         /* C: rows per expert in FIXED mode */
    int32_t mode;             /* ep_mode */
    int32_t idx_bits;         /* 64 or 32 */
    uint32_t flags;           /* EP_FLAG_* */
} ep_config;

/* Routing metadata shared by dispatch, combine and the duals (the README's
 * EPHandle). Plain data: copying it is fine. Every pointer points into the
 * caller's workspace (device memory) and is valid while the workspace
 * lives and no other ep_layout writes into it. Contents after the layout
 * has run on the stream:
 *   cnt[E]         pairs routed to each expert (before any capacity limit)
 *   pad[E]         rows of expert e in the receive buffer (COMPACT: padded
 *                  count; FIXED: min(cnt, C)) — the GEMM row counts
 *   expert_off[E+1] first row of each expert (COMPACT: exclusive scan of pad;
 *                  FIXED: e*C); expert_off[E] is the row total R
 *   dest_off[D+1]  first row of each destination: expert_off[d*E/D]
 *   dest_tokens[D] distinct tokens with a routed pair into destination d
 *   slot[T*k]      receive row of pair (t, j) or -1 when skipped; rows of
 *                  one expert are in ascending (t, j) order
 *   row_src[Rcap]  pair index t*k + j held by each row; -1 on padding rows
 *                  (COMPACT); FIXED rows past pad[e] are not written
 *   row_w[Rcap]    topk_w of the pair held by each row, 0 on padding rows;
 *                  written only when ep_layout got topk_w
 *   err_flags[1]   EP_ERRFLAG_* bits raised by this layout
 *   topk_idx       the caller's topk_idx the layout was built from (not a
 *                  copy: the README's decode example returns
 *                  cached_handle.topk_idx in place of a new recv_topk_idx,
 *                  "Example use in inference decoding"); valid while the
 *                  caller keeps that buffer, NULL for an empty batch */
typedef struct {
    ep_config cfg;
    int32_t num_tokens;
    int32_t num_blocks; /* internal: layout partition of the pairs */
    int32_t* cnt;
    int32_t* pad;
    int32_t* expert_off;
    int32_t* dest_off;
    int32_t* dest_tokens;
    int32_t* slot;
    int32_t* row_src;
    float* row_w;
    uint32_t* err_flags;
    void* internal; /* workspace scratch for the layout kernels */
    const void* topk_idx;
} ep_handle;

/* Bytes of workspace one layout needs (the README's get_buffer_size_hint).
 * Returns 0 when the config is invalid (see ep_last_error_message). */
size_t ep_workspace_bytes(const ep_config* cfg);

/* Rows a receive buffer must have to hold any layout of this config without
 * knowing the counts: max_tokens*k + E*(A-1) (COMPACT) or E*C (FIXED). The
 * README sizes its buffer from num_max_tokens_per_rank and hidden before any
 * routing is known (section "Interfaces and examples", "Buffer
 * initialization": get_buffer_size_hint); this is the same bound for the
 * receive rows, so a caller allocates them once and never waits for counts.
 * Returns -1 when the config is invalid. */
int64_t ep_recv_rows_bound(const ep_config* cfg);

/* Builds the layout of `num_tokens` tokens (README dispatch_forward: the
 * per-expert counts and padded offsets; the stable slot of every pair).
 *   cfg        host; copied into *out.
 *   num_tokens 0 <= num_tokens <= cfg->max_tokens.
 *   topk_idx   device [num_tokens, k], int64 or int32 per cfg->idx_bits;
 *              -1 masks a pair.
 *   topk_w     device [num_tokens, k] binary32, or NULL (row_w not written).
 *   workspace  device, >= ep_workspace_bytes(cfg) bytes, 256-byte aligned;
 *              must not be in use by another in-flight layout.
 *   out        host; receives the handle (valid once the stream reaches it).
 * Enqueues one kernel for small layouts (num_tokens * k <= 4096 and
 * E <= 512), three otherwise. Never synchronises. */
ep_status ep_layout(const ep_config* cfg, int32_t num_tokens, const void* topk_idx,
                    const float* topk_w, void* workspace, size_t workspace_bytes,
                    ep_handle* out, void* stream);

/* Layout and dispatch in one call: the README's dispatch_forward, which
 * builds the handle (per-expert counts, padded offsets, stable slots) and
 * moves the hidden states in the same call. Arguments are those of
 * ep_layout followed by those of ep_dispatch; every argument of both is
 * checked before anything is enqueued. The results (handle contents, recv,
 * recv_scales) are bit-identical to ep_layout followed by ep_dispatch.
 * Small batches (num_tokens * k <= 4096 and E <= 512, the decode sizes of
 * README "Example use in inference decoding", whose zero-fill of padding
 * rows, if any, fits the CUs beside one block per token) take a single
 * kernel launch:
 * every block derives its rows from all the batch's ids (the whole small
 * layout in LDS, or, in FIXED mode and with expert_alignment 1, only the
 * counts that place its own pairs), so no block waits on another. Larger batches enqueue the layout kernels and then the dispatch
 * kernel. Never synchronises. */
ep_status ep_dispatch_forward(const ep_config* cfg, int32_t num_tokens, const void* topk_idx,
                              const float* topk_w, void* workspace, size_t workspace_bytes,
                              int32_t dtype, const void* x, const float* x_scales, void* recv,
                              float* recv_scales, ep_handle* out, void* stream);

/* ep_dispatch_forward for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Same arguments, checks and results (bit-identical handle,
 * recv and recv_scales), except where the multi-block layout keeps its
 * per-block partials (counts [nblk, E], distinct tokens [nblk, D], error
 * bits [nblk]; nblk = ceil(num_tokens * k / 1024), each region rounded up
 * to 256 bytes): in a static device array the library holds (1 MiB per
 * GPU, kept until the process ends) instead of the workspace. The
 * workspace then needs only the handle's arrays; ep_workspace_bytes(cfg)
 * always suffices. Allocates nothing, on the host or the device. The first
 * call on each device looks up the array's address (hipGetSymbolAddress,
 * not a stream operation). A layout whose partials exceed 1 MiB returns
 * EP_ERR_WORKSPACE and enqueues nothing. Every call on one GPU shares the
 * array: calls whose work overlaps on one GPU (concurrent streams) race and
 * must be ordered by the caller; consecutive calls on one stream are safe,
 * since every entry a call reads is written earlier in that call. Small
 * batches (the single launch) use no partials. */
ep_status ep_dispatch_forward_static_scratch(const ep_config* cfg, int32_t num_tokens, const void* topk_idx,
                                             const float* topk_w, void* workspace, size_t workspace_bytes,
                                             int32_t dtype, const void* x, const float* x_scales, void* recv,
                                             float* recv_scales, ep_handle* out, void* stream);

/* Dispatch on an existing handle (README dispatch_forward, or dispatch with a
 * cached handle: no layout work, no synchronisation).
 *   x          device [T, hidden]: bf16 (EP_BF16, EP_FP8_QUANTIZE) or E4M3FN
 *              (EP_FP8_PREQUANT).
 *   x_scales   device [T, hidden/128] binary32 for EP_FP8_PREQUANT, else NULL.
 *   recv       device [ep_recv_rows_bound, hidden] bf16 or E4M3FN. Row
 *              slot[t, j] receives token t's row. COMPACT padding rows are
 *              zero-filled unless EP_FLAG_NO_ZERO_PAD; rows at or past
 *              expert_off[E] are not touched.
 *   recv_scales device [rows bound, hidden/128] binary32 for the FP8 types
 *              (padding rows get 0), else NULL. */
ep_status ep_dispatch(const ep_handle* h, int32_t dtype, const void* x, const float* x_scales,
                      void* recv, float* recv_scales, void* stream);

/* Combine (README combine_forward): for every token t and channel c,
 *   acc = +0; for j = 0..k-1 with slot[t, j] >= 0:
 *       acc = fmaf(topk_w[t, j], float(y[slot[t, j], c]), acc)
 *   (acc = acc + float(y[...]) when topk_w is NULL);
 *   out[t, c] = bf16(acc), round to nearest even.
 *   y          device bf16 [rows bound, hidden] (expert outputs, receive
 *              layout).
 *   topk_w     device [T, k] binary32 or NULL.
 *   out        device bf16 [T, hidden].
 *   row_vals   device [rows bound] binary32 or NULL; with out_vals given,
 *              out_vals[t, j] = row_vals[slot[t, j]] (0 for skipped pairs).
 *   out_vals   device [T, k] binary32 or NULL. */
ep_status ep_combine(const ep_handle* h, const void* y, const float* topk_w, void* out,
                     const float* row_vals, float* out_vals, void* stream);

/* README dispatch_backward: the backward of a dispatch is a combine without
 * weights; grad_row_w (per receive row, e.g. the gradient of row_w) is
 * gathered back to grad_topk_w [T, k] when both are given. */
ep_status ep_dispatch_backward(const ep_handle* h, const void* grad_recv, const float* grad_row_w,
                               void* grad_x, float* grad_topk_w, void* stream);

/* README combine_backward: the backward of a combine is a dispatch of the
 * output gradient on the same handle, which the README lets arrive in BF16
 * or as an FP8 (data, scale_factors) pair. dtype, grad_out, grad_out_scales,
 * grad_y and grad_y_scales are as ep_dispatch's dtype, x, x_scales, recv and
 * recv_scales (grad_out_scales: EP_FP8_PREQUANT only, device [T, hidden/128]
 * binary32; NULL otherwise). With topk_w, the copy for pair (t, j) is the
 * gradient of the weighted combine, bf16(topk_w[t, j] * float(grad_out[t, c]))
 * (one binary32 multiply, round to nearest even); with EP_FP8_QUANTIZE that
 * BF16 copy is then quantised per 1x128 block as ep_dispatch quantises x,
 * each pair with its own scales. EP_FP8_PREQUANT with topk_w returns
 * EP_ERR_UNSUPPORTED (weighting codes would need them re-quantised). */
ep_status ep_combine_backward(const ep_handle* h, int32_t dtype, const void* grad_out,
                              const float* grad_out_scales, const float* topk_w, void* grad_y,
                              float* grad_y_scales, void* stream);

/* Gradient of the weighted combine with respect to its weights (the part of
 * README combine_backward that a weighted combine adds; the gradient with
 * respect to the expert outputs is ep_combine_backward with topk_w):
 *   grad_topk_w[t, j] = sum_c float(grad_out[t, c]) * float(y[slot[t, j], c])
 * in binary32, 0 for skipped pairs.
 *   grad_out     device bf16 [T, hidden] (gradient of combine's out).
 *   y            device bf16 [rows bound, hidden]: the expert outputs the
 *                forward combine read.
 *   grad_topk_w  device binary32 [T, k].
 * The sum is taken in a fixed order (per lane over its channels, then a
 * butterfly over the 64 lanes of a wave, then over the waves in order), so
 * results are deterministic; each product passes through at most
 * 8 * ceil((hidden / 8) / 1024) + 6 + 15 binary32 additions, which bounds
 * the error against the exact sum by that count times 2^-24 times
 * sum_c |grad_out[t, c] * y[slot, c]|. */
ep_status ep_combine_weight_grad(const ep_handle* h, const void* grad_out, const void* y,
                                 float* grad_topk_w, void* stream);

/* FP8 grouped GEMM over the receive layout: the consumer the layout is built
 * for (README: per-expert received-token counts meant for the expert GEMM, rows padded to
 * expert_alignment; "New features": EPv2's new GEMM layout). For every row r
 * of expert e and output channel c < n:
 *   out[r, c] = bf16( sum_kb a_scales[r, kb] * b_scales[e, c/128, kb]
 *                            * sum_{k in block kb} a[r, k] * b[e, c, k] )
 * accumulated in binary32 (MFMA partial sums per 128-wide K block, each
 * promoted with one binary32 product of the two scales and one FMA), rounded
 * to nearest even.
 *   a          device E4M3FN [rows bound, hidden]: the FP8 dispatch's recv.
 *   a_scales   device binary32 [rows bound, hidden/128]: its recv_scales.
 *   b          device E4M3FN [E, n, hidden]: expert e's weights, one row of
 *              hidden codes per output channel.
 *   b_scales   device binary32 [E, n/128, hidden/128]: 128x128 block scales.
 *   out        device bf16 [rows bound, n]. COMPACT: every row below
 *              expert_off[E] is written; padding rows (past expert_off[e] +
 *              cnt[e]) are zero when the receive padding rows are zero (the
 *              default; unspecified under EP_FLAG_NO_ZERO_PAD). FIXED: expert
 *              e's rows [e*C, e*C + ceil(pad[e]/128)*128) are written; those
 *              at or past e*C + pad[e] are unspecified. Other rows are not
 *              touched.
 * a, b and out must be 16-byte aligned, the scale arrays 4-byte aligned
 * (EP_ERR_INVALID_ARG otherwise). Requires hidden % 128 == 0, n % 128 == 0,
 * and expert_alignment % 128 == 0 (COMPACT) or capacity % 128 == 0 (FIXED),
 * so that every 128-row tile belongs to one expert; otherwise
 * EP_ERR_UNSUPPORTED. */
ep_status ep_grouped_gemm_fp8(const ep_handle* h, const void* a, const float* a_scales, const void* b,
                              const float* b_scales, int32_t n, void* out, void* stream);

/* Copies cnt and pad (host arrays of E, either may be NULL) and the row
 * total R (host, may be NULL) to the host. Synchronises the stream: this is
 * the README's CPU synchronisation of a non-cached dispatch. */
ep_status ep_handle_read_counts(const ep_handle* h, int32_t* cnt, int32_t* pad, int64_t* rows,
                                void* stream);

/* Reads the handle's error word (EP_ERRFLAG_* bits) to host *flags.
 * Synchronises the stream. No passage of the pages defines this call: their
 * API has no device-side data errors; it reports the two this library
 * defines (an out-of-range expert id, a fixed-capacity overflow). */
ep_status ep_handle_check(const ep_handle* h, uint32_t* flags, void* stream);

/* Static text for a status code (an ep_status value; any other value
 * gives "EP_ERR_UNKNOWN"). No passage of the pages defines this call: it
 * belongs to this C ABI's error convention. */
const char* ep_status_string(int32_t s);

/* Message of the last failed call on this thread ("" if none). No passage
 * of the pages defines this call: it belongs to this C ABI's error
 * convention (the pages' Python API raises exceptions instead). */
const char* ep_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* EP_H */
