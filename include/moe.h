/*
 * moe.h -- C ABI of the single-GPU sparse Mixture-of-Experts FFN layer
 * forward pass for AMD Instinct MI355X (gfx950).
 *
 * The layer (the computation the MoE pages describe; page titles cited):
 *   1. route:    router GEMM, optional per-expert bias and load-aware penalty,
 *                ranking of the experts with ties to the lower index;
 *   2. dispatch: capacity-capped assignment of each token's top-k choices to
 *                expert queues, re-route of overflow to the next-ranked
 *                candidate or drop, gates, router statistics and the
 *                load-balancing loss, and the permutation of token rows into
 *                per-expert groups;
 *   3. expert_ffn: SwiGLU FFN of every expert over its group of rows;
 *   4. combine:  gate-weighted sum of each token's expert outputs, in token
 *                order;
 *   5. forward:  1-4 on one stream.
 *
 * Conventions shared by every entry point
 *   - Pointers named x, w_*, bias, load, logits, y, h, x_perm, y_perm,
 *     workspace and every member of moe_routing are DEVICE pointers, allocated
 *     and owned by the caller.  The library never allocates or frees memory
 *     and never synchronises: work is enqueued on `stream` (a hipStream_t; NULL
 *     is the legacy default stream) and outputs are valid once the stream has
 *     reached that point.  `p` is a host pointer read during the call only.
 *   - All matrices are row-major.  bf16 means IEEE bfloat16 bit patterns;
 *     conversions from fp32 round to nearest even.  Accumulation is fp32.
 *   - Elements of x, w_router, w1, w3, w2, x_perm and y have the element type
 *     p->dtype.  logits, bias, load, cand_score, gate and y_perm are fp32
 *     (y_perm [R][d] holds the down projection at accumulator precision, so
 *     the staged layer output is rounded to the element type once).
 *   - Intermediate precision of a bf16 layer: the SwiGLU activations h are
 *     fp16 (saturated at +-65504); the down projection multiplies h by W2 in
 *     fp16, W2 being narrowed from bf16 with round-toward-zero (exact for
 *     magnitudes 2^-14 .. 65504; above 65504 a weight clamps to +-65504,
 *     below 2^-14 it keeps fewer bits as an fp16 subnormal, below 2^-24 it
 *     becomes 0).  moe_forward also keeps each kept row's gate-weighted
 *     down projection in fp16 (saturated at +-65504) before the combine.
 *     Layers whose weights or activations reach these limits are outside
 *     the contract of a bf16 layer.  An fp32 layer keeps h and y_perm in
 *     fp32 throughout.
 *   - Every output element listed for an entry point is written on every call.
 *   - NaN or Inf inputs are outside the contract.
 *   - Calls on different streams that share no output buffer may run
 *     concurrently.  The only global mutable state is the static scratch
 *     array of moe_forward_noalloc (one per GPU): calls of that entry point
 *     that overlap on one GPU race; every other entry point works in the
 *     caller's buffers only.  moe_backward runs part of its work on a second
 *     stream of the library's own (made on its first call on a device,
 *     default priority, kept until the process ends), forked from and
 *     joined back to `stream` with events, so its outputs are still valid
 *     once `stream` has reached the call's end; where that stream cannot be
 *     made (e.g. first called inside a graph capture) all its work runs on
 *     `stream`.
 *
 * Return codes: MOE_OK (0) on success, or a negative MOE_ERR_* code; nothing
 * is enqueued when an argument check fails.  moe_strerror() names the code.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_OK 0
#define MOE_ERR_INVALID_ARG (-1) /* null pointer, size out of range, workspace too small */
#define MOE_ERR_UNSUPPORTED (-2) /* dtype, alignment or a dimension the kernels do not take */
#define MOE_ERR_HIP (-3)         /* a kernel launch failed */
#define MOE_ERR_TOO_LARGE (-4)   /* moe_forward_noalloc: the layer's scratch exceeds the static array */

/* Bytes of the static scratch array behind moe_forward_noalloc (32 MiB,
 * one copy per GPU the library runs on, held until the process ends). */
#define MOE_STATIC_SCRATCH_BYTES (32u << 20)

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/*
 * Problem statement: T tokens of hidden size d, E experts, top-k, capacity
 * factor, SwiGLU intermediate size d_ff (the parameters in which the MoE
 * pages state the problem; "MoE架构揭秘" §5.2 names num_experts_per_tok,
 * expert_capacity and the capacity factor).
 *
 * Limits: 0 <= T <= 2^20 (T = 0 is an empty batch); 1 <= E <= 256;
 * 1 <= k <= min(E, 8); d and d_ff positive multiples of 64; d <= 16384 for
 * bf16 and d <= 8192 for fp32; d_ff < 2^22; one expert matrix (d * d_ff
 * elements) below 4 GiB.  Other values return MOE_ERR_INVALID_ARG (sizes) or
 * MOE_ERR_UNSUPPORTED (dtype, multiples, d, d_ff or d * d_ff too large).
 */
typedef struct moe_params {
    int32_t T, d, E, k, d_ff;
    /* capacity C = min(T, ceil(T*k/E * capacity_factor)), evaluated in double
     * in that order ("MoE架构揭秘" §5.2 expert_capacity); capacity_factor <= 0
     * means uncapped (C = T). */
    float capacity_factor;
    /* 1: a token whose chosen expert is full sends its lowest-rank overflowed
     * slot to its rank-k candidate (the third-ranked expert for top-2), else
     * that slot is dropped ("GPT-4稀疏激活真相" §2.3); 0: overflow is dropped. */
    int32_t reroute;
    /* load-aware penalty s = fmaf(-lambda, load[e], raw) ("GPT-4稀疏激活真相"
     * §2.3); ignored when load == NULL. */
    float lambda;
    /* load-balancing loss coefficient; the loss is aux_coef * sum_e
     * (demand[e]/T)^2 ("MoE稀疏激活原理与工程实践" §4.2, coefficient 0.01). */
    float aux_coef;
    int32_t dtype; /* moe_dtype */
    /* gate temperature tau: the gates are the softmax of score / tau over the
     * kept slots ("MoE稀疏激活原理与工程实践" §3.1, third step: a smaller tau
     * sharpens the distribution, a larger one flattens it).  The ranking and
     * every routing decision are independent of tau.  0 means 1 (the plain
     * softmax); a negative, NaN or infinite value is MOE_ERR_INVALID_ARG. */
    float gate_temperature;
    /* top-2 gap threshold delta: where the best two ranking scores differ by
     * less than delta (their fp32 difference), the second choice is replaced
     * by the third-ranked expert (the adg.csdn.net page, §3.1): ranks 1 and 2
     * of cand / cand_score trade places, the displaced expert becoming the
     * fallback candidate.  Applies when k + 1 >= 3 and the third candidate
     * names an expert.  0 turns it off; a negative, NaN or infinite value is
     * MOE_ERR_INVALID_ARG. */
    float top2_gap;
    /* router network: 0 is the linear router (w_router [E][d]); H > 0 is the
     * two-layer router of "MoE稀疏激活原理与工程实践" §3.1, second step, and
     * of its §4.2 code (Linear(d, 2E) -> SiLU -> Linear(2E, E)),
     * raw = silu(x . W1^T + b1) . W2^T + b2 with H hidden units (2E on the
     * page): w_router then holds W1 [H][d] followed by W2 [E][H], and the
     * bias argument of moe_route / moe_forward (when not NULL) holds b1 [H]
     * followed by b2 [E].  1 <= H <= 256 (MOE_ERR_UNSUPPORTED above); a
     * negative value is MOE_ERR_INVALID_ARG. */
    int32_t router_hidden;
    /* 1: the capacity factor grows with the batch, cf = 1 + 0.01 * log2(T)
     * in double ("GPT-4稀疏激活真相" §5.4; 1.05 at 32 tokens), and
     * capacity_factor is ignored; 0: capacity_factor as given.  Any other
     * value is MOE_ERR_INVALID_ARG. */
    int32_t dynamic_capacity;
} moe_params;

/*
 * Routing arrays (all device pointers, caller-allocated, int32 unless noted).
 * K1 = k + 1 candidate columns; R = moe_max_rows(p) = min(T*k, E*C).
 * Arrays with a T dimension may be NULL when T = 0, token_of_row when R = 0;
 * offsets, demand, kept, totals and aux_loss are always required.
 */
typedef struct moe_routing {
    int32_t *cand;       /* [T][K1] experts by (score desc, index asc), NaN scores
                          *         after every number (ranks 1-2 swapped under
                          *         the top-2 gap threshold); -1 past E         */
    float *cand_score;   /* [T][K1] penalised fp32 scores; -inf past E              */
    int32_t *eid;        /* [T][k]  final expert of slot j, -1 when dropped         */
    int32_t *pos;        /* [T][k]  position in that expert's queue, -1 if dropped  */
    int32_t *row;        /* [T][k]  row in the permuted layout, -1 if dropped       */
    uint8_t *flag;       /* [T][k]  0 kept, 1 re-routed, 2 dropped                  */
    float *gate;         /* [T][k]  softmax of the kept slots' scores; 0 if dropped */
    int32_t *offsets;    /* [E+1]   exclusive scan of kept; offsets[E] = rows       */
    int32_t *token_of_row; /* [R]   token of each permuted row; -1 past offsets[E]  */
    int32_t *demand;     /* [E]     rank < k selections before the cap              */
    int32_t *kept;       /* [E]     rows kept per expert (<= C)                     */
    int32_t *totals;     /* [3]     rows, dropped slots, re-routed slots            */
    float *aux_loss;     /* [1]     load-balancing loss                             */
} moe_routing;

/* Host-side, pure: capacity C (see moe_params.capacity_factor); -1 if p is
 * invalid. */
int64_t moe_capacity(const moe_params *p);

/* Host-side, pure: R = min(T*k, E*C), the row bound of the permuted layout;
 * -1 if p is invalid. */
int64_t moe_max_rows(const moe_params *p);

/* Host-side, pure: bytes of scratch moe_expert_ffn needs (the partial
 * products of a down projection split over slices of d_ff); 0 when it needs
 * none, or if p is invalid. */
size_t moe_ffn_workspace_bytes(const moe_params *p);

/* Host-side, pure: bytes of scratch moe_dispatch needs. */
size_t moe_dispatch_workspace_bytes(const moe_params *p);

/* Host-side, pure: bytes of workspace moe_forward needs: the dispatch scratch,
 * h [R][d_ff], the down projection's output rows (bf16: fp16 gated partial
 * products of each d_ff slice, and each row's gate; fp32: y_perm [R][d]),
 * and x_perm [R][d] only when x spans 2 GiB or more (see moe_forward), each
 * 256-byte aligned. */
size_t moe_workspace_bytes(const moe_params *p);

/*
 * Stage 1, route.  raw[t][e] = sum_i x[t][i] * w_router[e][i] + bias[e]
 * ("MoE架构揭秘" §3.1: z = h . W_router; with p->router_hidden > 0 the
 * two-layer router described there), s = fmaf(-lambda, load[e], raw)
 * (or raw when load is NULL), then the K1 best experts by (s desc, e asc)
 * ("MoE架构揭秘" §3.1: softmax then top-k; softmax is monotone, so the ranking
 * is taken on s).
 *   x [T][d], w_router [E][d] (dtype); bias [E] fp32 or NULL ([H + E] for
 *   the two-layer router); load [E] fp32 or NULL.  Writes logits [T][E]
 *   (raw, fp32), r->cand and r->cand_score.
 */
int moe_route(const moe_params *p, const void *x, const void *w_router, const float *bias,
              const float *load, float *logits, moe_routing *r, void *stream);

/*
 * Stage 2, dispatch.  Reads r->cand and r->cand_score; writes every other
 * member of r and x_perm [R][d] (rows past offsets[E] are left untouched).
 * Queue order is rank-major (all rank-0 choices in token order, then rank 1,
 * ..., then one fallback round in token order); a slot is kept while its
 * expert holds fewer than C rows ("GPT-4稀疏激活真相" §2.3; "MoE架构揭秘"
 * §3.3).  Gates are the softmax of the kept slots' scores renormalised over
 * the kept slots.  Deterministic: no atomics.  A candidate outside [0, E)
 * (a caller's own r->cand) names no expert: such a slot is never kept.
 *   workspace: at least moe_dispatch_workspace_bytes(p) bytes, 256-B aligned.
 */
int moe_dispatch(const moe_params *p, const void *x, moe_routing *r, void *x_perm,
                 void *workspace, size_t ws_bytes, void *stream);

/*
 * Stage 3, expert SwiGLU FFN as a grouped GEMM over the permuted rows
 * ("GPT-4稀疏激活真相" §3.1: Linear -> SwiGLU -> Linear per expert):
 *   for rows i in [offsets[e], offsets[e+1]):
 *     h[i]      = silu(x_perm[i] . W1[e]^T) * (x_perm[i] . W3[e]^T)
 *     y_perm[i] = h[i] . W2[e]^T
 *   x_perm [R][d]; w1, w3 [E][d_ff][d]; w2 [E][d][d_ff]; h [R][d_ff] (fp16
 *   for bf16, fp32 for fp32); y_perm [R][d] fp32.  offsets [E+1] is read on
 *   the device and must be as moe_dispatch writes them: non-decreasing,
 *   offsets[0] = 0, offsets[E] <= R and at most C rows per expert (the launch
 *   is sized by these bounds; rows beyond them are not computed).  Rows past
 *   offsets[E] of h and y_perm are left untouched.
 *   workspace: at least moe_ffn_workspace_bytes(p) bytes, 256-B aligned (may
 *   be NULL when that is 0).  Where the down projection is split over slices
 *   of d_ff to fill the chip, the partial products of slices 1.. are kept
 *   there and added to slice 0 in slice order (deterministic, no atomics).
 */
int moe_expert_ffn(const moe_params *p, const void *x_perm, const int32_t *offsets,
                   const void *w1, const void *w3, const void *w2, void *h, void *y_perm,
                   void *workspace, size_t ws_bytes, void *stream);

/*
 * Stage 4, combine ("企业官网建设流程全解析" page §3, step 5: results are put
 * back in token order; "GPT-4稀疏激活真相" §4.3: weighted fusion):
 *   y[t] = sum over slots j with row[t][j] >= 0 of gate[t][j] * y_perm[row[t][j]]
 * accumulated in fp32 (slot order) and rounded once; a token with no kept
 * slot gets zeros.  y_perm [R][d] fp32 (not read when R = 0); row, gate
 * [T][k]; y [T][d].
 */
int moe_combine(const moe_params *p, const void *y_perm, const int32_t *row, const float *gate,
                void *y, void *stream);

/*
 * Stages 1-4 on one stream with no host synchronisation.  workspace holds at
 * least moe_workspace_bytes(p) bytes (256-B aligned) and is carved into the
 * dispatch scratch, h and the down projection's output rows.  When x spans
 * less than 2 GiB the dispatch copy of the token rows is not made: the
 * gate-up GEMM reads its rows from x through token_of_row (same values, one
 * pass over x fewer); otherwise x_perm is materialised in the workspace as
 * moe_dispatch does.  In a bf16 layer the gates are folded into the down
 * projection ("企业官网建设流程全解析" page §5.2: one fused forward;
 * "MoE稀疏激活原理与工程实践" §3.2: the MoE layer's time goes to moving
 * data): each kept row's gate multiplies its fp32 down projection (per d_ff
 * slice) before it is stored in fp16, and the combine adds the k rows of a
 * token (slot order, then slice order) in fp32 and rounds once.  The routing
 * arrays and logits are those of moe_route + moe_dispatch; y agrees with the
 * stage-by-stage result to within the fp16 rounding of the gated rows.
 */
int moe_forward(const moe_params *p, const void *x, const void *w_router, const float *bias,
                const float *load, const void *w1, const void *w3, const void *w2, void *y,
                float *logits, moe_routing *r, void *workspace, size_t ws_bytes, void *stream);

/*
 * moe_forward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * caller passes inputs and outputs only; the workspace is a file-scope
 * device array of MOE_STATIC_SCRATCH_BYTES in the library, one per GPU
 * (its address looked up on the first call on each device).  No allocation
 * of any kind happens in the call.  A layer whose workspace
 * (moe_workspace_bytes(p)) exceeds the array returns MOE_ERR_TOO_LARGE
 * (32 MiB holds, for example, a Mixtral-shape layer of d 4096, E 8, top-2,
 * d_ff 14336, capacity factor 1.25, up to 178 tokens).  Every call on one GPU shares that
 * GPU's array: calls that overlap on one GPU (different streams or host
 * threads) race and must not be issued.  Results are identical to
 * moe_forward's on the same inputs.
 */
int moe_forward_noalloc(const moe_params *p, const void *x, const void *w_router, const float *bias,
                        const float *load, const void *w1, const void *w3, const void *w2, void *y,
                        float *logits, moe_routing *r, void *stream);

/*
 * moe_forward with per-stage timing marks: events is NULL or an array of six
 * hipEvent_t (NULL entries are skipped), recorded on `stream` before the
 * route, the dispatch, the gate-up GEMM, the down GEMM and the combine, and
 * after the combine.  The work enqueued is exactly that of moe_forward.
 */
int moe_forward_events(const moe_params *p, const void *x, const void *w_router, const float *bias,
                       const float *load, const void *w1, const void *w3, const void *w2, void *y,
                       float *logits, moe_routing *r, void *workspace, size_t ws_bytes, void *stream,
                       void *const *events);

/*
 * One-byte expert weights ("企业官网建设流程全解析" page §5.1: the experts'
 * W1/W2/W3 kernels quantised; "GPT-4稀疏激活真相" §2.1 counts FP8 at one byte
 * per parameter).  Each weight matrix is held as OCP FP8 E4M3 codes (no
 * infinities; 0x7F and 0xFF are NaN) with one fp32 scale per output row:
 *   W1[e][j][i] = s1[e][j] * q1[e][j][i], W3 likewise with s3,
 *   W2[e][c][j] = s2[e][c] * q2[e][c][j].
 *   q1, q3 [E][d_ff][d] bytes, s1, s3 [E][d_ff] fp32; q2 [E][d][d_ff] bytes,
 *   s2 [E][d] fp32; q pointers 16-byte aligned, scales 4-byte aligned.
 * The activations are as for the bf16 layer (x_perm bf16, h fp16, y_perm
 * [R][d] fp32); the codes are widened exactly (to bf16 for W1/W3, to fp16
 * for W2) and the scales multiply the fp32 accumulators, so the weights are
 * not narrowed.  dtype MOE_BF16 only (else MOE_ERR_UNSUPPORTED).  Layers
 * whose experts hold at most 32 rows (capacity C = moe_capacity(p) <= 32)
 * run the weight-streaming kernel and need d and d_ff to be multiples of
 * 128; larger groups run the 256 x 256 matrix-core tile (d and d_ff
 * multiples of 64).  Otherwise as moe_expert_ffn, except that the down
 * projection is computed in one K slice here, so no workspace is needed
 * (moe_forward_fp8 splits it like moe_forward).
 */
int moe_expert_ffn_fp8(const moe_params *p, const void *x_perm, const int32_t *offsets,
                       const uint8_t *w1, const float *s1, const uint8_t *w3, const float *s3,
                       const uint8_t *w2, const float *s2, void *h, void *y_perm, void *stream);

/*
 * moe_forward with one-byte expert weights (as moe_expert_ffn_fp8; same
 * workspace size, same limits).  The router weights stay bf16.
 */
int moe_forward_fp8(const moe_params *p, const void *x, const void *w_router, const float *bias,
                    const float *load, const uint8_t *w1, const float *s1, const uint8_t *w3,
                    const float *s3, const uint8_t *w2, const float *s2, void *y, float *logits,
                    moe_routing *r, void *workspace, size_t ws_bytes, void *stream);

/* Host-side, pure: bytes of workspace moe_load_window needs for a window
 * of `window` tokens; 0 if p is invalid or window < 1. */
size_t moe_load_window_workspace_bytes(const moe_params *p, int32_t window);

/*
 * Windowed load statistic ("企业官网建设流程全解析" page §2: an expert's load
 * is its selection frequency over a sliding window of the most recent
 * tokens, 1024 on the page, with a decay factor, 0.99 on the page, so that
 * it follows the current load).  The T tokens of the batch fall, in token
 * order, into consecutive windows of `window` tokens (the last may be
 * shorter); each window updates the statistic once:
 *   load[e] <- decay * load[e] + (1 - decay) * f[e],
 *   f[e] = (selections of e in the window) / (k * tokens in the window),
 * a selection being one of a token's ranks 0..k-1 in cand (the router's
 * top-k choices before the capacity cap; an entry outside [0, E) selects
 * nothing).  Computed in double, windows in order, load rounded to fp32
 * once.  cand [T][k+1] as moe_route writes it; load [E] fp32 (device), read
 * and overwritten, e.g. the `load` of the next batch's penalty.  decay in
 * [0, 1]; window >= 1.  workspace: moe_load_window_workspace_bytes(p,
 * window) bytes, 256-B aligned.  T = 0 leaves load unchanged.
 */
int moe_load_window(const moe_params *p, const int32_t *cand, int32_t window, float decay, float *load,
                    void *workspace, size_t ws_bytes, void *stream);

/* Host-side, pure: bytes of workspace moe_backward needs; 0 if p is invalid. */
size_t moe_backward_workspace_bytes(const moe_params *p);

/*
 * Backward pass (training) of a bf16 layer with the linear router, the
 * routing of the forward pass held fixed.  The router is trained through
 * the experts: its gradient flows back from the experts' outputs through
 * the gates of the kept slots ("MoE架构揭秘" §3.3); the ranking, capacity,
 * re-route and drop decisions are piecewise constant and pass no gradient.
 * The balance loss counts top-k picks without gradient
 * ("MoE稀疏激活原理与工程实践" §4.2) and contributes none; the penalty's
 * load vector is an input without gradient.
 *   Inputs: x [T][d], w_router [E][d], w1, w3 [E][d_ff][d], w2 [E][d][d_ff]
 *   (bf16, as given to the forward pass); r: the routing the forward pass
 *   wrote for this x (eid, row, gate, offsets, token_of_row are read); dy
 *   [T][d] bf16, the gradient of the loss with respect to the layer output.
 *   Outputs (fp32, every element written): dx [T][d]; dlogits [T][E], the
 *   gradient with respect to the router logits (nonzero only at a token's
 *   kept experts; each row sums to 0); dw_router [E][d]; dbias [E] (the
 *   gradient of a per-expert router bias); dw1, dw3 [E][d_ff][d]; dw2
 *   [E][d][d_ff].  An expert without rows gets zero weight gradients.
 *   workspace: at least moe_backward_workspace_bytes(p) bytes, 256-B aligned.
 * The a = x W1^T, b = x W3^T products are recomputed.  The GEMMs run on
 * matrix cores with fp32 accumulation:
 *   - u = dy W2 on bf16 (dy and W2 exact);
 *   - dx, dw1, dw3 and dw2 on fp16.  The fp32 SwiGLU gradients da, db and
 *     g * h are rounded once to fp16 (2^-12 relative), after scaling by a
 *     power of 2 per expert that puts the expert's largest magnitude in
 *     [2^14, 2^15).  dy is scaled likewise by its largest magnitude.  x, W1
 *     and W3 enter as fp16 conversions of their bf16 values: exact for
 *     magnitudes from 2^-14 up to 65504, fp16 subnormal steps of 2^-24
 *     below, and infinite above (the forward pass already takes W2 and h on
 *     the same range).
 * Measured against the oracle, the weight and input gradients stay within
 * 0.8% of their RMS.  Deterministic: the per-expert maxima are atomic
 * maxima, the same in any order, and every sum runs in a fixed order.
 * MOE_ERR_UNSUPPORTED: an
 * fp32 layer, the two-layer router, x of 2 GiB and more, or 2 GiB and more
 * in 256 rows of the kept rows' transposed K axis (1024 (R + 64 E) bytes, R
 * the kept row bound moe_max_rows rounded up to 64: about two million kept
 * rows).
 */
int moe_backward(const moe_params *p, const void *x, const void *w_router, const void *w1, const void *w3,
                 const void *w2, const moe_routing *r, const void *dy, float *dx, float *dlogits,
                 float *dw_router, float *dbias, float *dw1, float *dw3, float *dw2, void *workspace,
                 size_t ws_bytes, void *stream);

/*
 * One-byte expert weights as INT8 codes (two's complement, -128..127) with
 * one fp32 scale per output row: W[e][j][i] = s[e][j] * q[e][j][i]
 * ("MoE稀疏激活原理与工程实践" §3.2 quantises the experts to INT8;
 * "企业官网建设流程全解析" page §5.1 to integer formats).  The codes are
 * widened exactly to bf16 (gate-up) and fp16 (down) in registers and the
 * scales multiply the fp32 accumulators.  Layouts, limits, activations and
 * workspace as for moe_expert_ffn_fp8 / moe_forward_fp8.
 */
int moe_expert_ffn_i8(const moe_params *p, const void *x_perm, const int32_t *offsets,
                      const int8_t *w1, const float *s1, const int8_t *w3, const float *s3,
                      const int8_t *w2, const float *s2, void *h, void *y_perm, void *stream);
int moe_forward_i8(const moe_params *p, const void *x, const void *w_router, const float *bias,
                   const float *load, const int8_t *w1, const float *s1, const int8_t *w3,
                   const float *s3, const int8_t *w2, const float *s2, void *y, float *logits,
                   moe_routing *r, void *workspace, size_t ws_bytes, void *stream);

/*
 * INT4 expert weights: two's complement codes -8..7, two per byte (element 2j
 * of a row in the low nibble of byte j, 2j + 1 in the high nibble), with one
 * fp32 scale per output row: W[e][j][i] = s[e][j] * q[e][j][i]
 * ("企业官网建设流程全解析" page §5.1 quantises some experts to INT4;
 * "MoE稀疏激活原理与工程实践" §5.4 names INT4 expert weights as the remedy
 * for a bandwidth-bound dispatch).  The scale granularity is not on the
 * pages; one scale per output row keeps each dot product a scaled sum, as for
 * the one-byte codes.
 *   q1, q3 [E][d_ff][d/2] bytes, s1, s3 [E][d_ff] fp32; q2 [E][d][d_ff/2]
 *   bytes, s2 [E][d] fp32; q pointers 16-byte aligned, scales 4-byte aligned.
 * The codes are widened exactly to bf16 (W1/W3) or fp16 (W2) in registers
 * and the scales multiply the fp32 accumulators.  Activations and outputs as
 * for moe_expert_ffn_fp8 / moe_forward_fp8 (same workspace size).  Only the
 * weight-streaming kernel takes INT4 codes: dtype MOE_BF16, every expert at
 * most 32 rows (moe_capacity(p) <= 32) and d, d_ff multiples of 128, else
 * MOE_ERR_UNSUPPORTED.
 */
int moe_expert_ffn_i4(const moe_params *p, const void *x_perm, const int32_t *offsets,
                      const uint8_t *w1, const float *s1, const uint8_t *w3, const float *s3,
                      const uint8_t *w2, const float *s2, void *h, void *y_perm, void *stream);
int moe_forward_i4(const moe_params *p, const void *x, const void *w_router, const float *bias,
                   const float *load, const uint8_t *w1, const float *s1, const uint8_t *w3,
                   const float *s3, const uint8_t *w2, const float *s2, void *y, float *logits,
                   moe_routing *r, void *workspace, size_t ws_bytes, void *stream);

/* Static description of a return code. */
const char *moe_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
