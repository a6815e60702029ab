/*
 * libmoe — the Mixture-of-Experts layer's hot path on one AMD Instinct MI355X
 * (gfx950): router with top-k gating, dispatch into expert-contiguous (or
 * per-destination-rank contiguous) buffers, grouped SwiGLU GEMM, combine, and the
 * backward of each step.
 *
 * [EFA] = Perplexity (N. Licker, K. Hu, V. Zaytsev, L. Chen), "Enabling
 * trillion-parameter models on AWS EFA", 2025-11-04. Section names follow its table
 * of contents. The article describes the layer only in prose; the readings this
 * library takes where it is silent are stated at each call.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Memory: every pointer argument is DEVICE memory owned by the caller (allocate
 *   it with hipMalloc or any device allocator). The library allocates nothing;
 *   scratch space comes in through `ws`. Its only process-wide state is one-time
 *   set-up per device (kernel LDS limits, the compute-unit count), done on a device's
 *   first call under std::call_once, so concurrent first calls are safe.
 * - Layout: all matrices are row-major and dense. A "row" of a token tensor is
 *   d contiguous elements. Rows and pointers must be 16-byte aligned
 *   (d * element size % 16 == 0, pointers % 16 == 0); otherwise MOE_ERR_ALIGN.
 * - dtype: MOE_BF16 (bfloat16 storage, float32 arithmetic, round-to-nearest-even
 *   on every store) or MOE_F32. Gate weights, logits and weight gradients are
 *   always float32; indices always int32.
 * - Execution: each call only enqueues work on `stream` (a hipStream_t; NULL is
 *   the default stream) and returns. Results are ready when the stream is. Calls
 *   on one stream run in order, which also orders the reuse of buffers between
 *   dispatch and combine ([EFA] Dispatch and combine: receive buffers are read
 *   before later kernels overwrite them).
 * - Errors: a non-zero moe_status_t means nothing was enqueued. All argument
 *   checks run on the host before any HIP call. Problems only the device can see
 *   (an expert id out of range, a token listing an expert twice, a destination
 *   region over capacity) never cause out-of-bounds accesses: the offending pair is
 *   skipped and a flag is raised in the dispatch workspace; read it with
 *   moe_dispatch_status(). MOE_ERR_HIP reports a failed launch.
 * - Determinism: no floating-point atomics anywhere; every output is bitwise
 *   reproducible for the same inputs and sizes.
 */
#ifndef LIBMOE_MOE_H
#define LIBMOE_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

typedef int32_t moe_status_t;
#define MOE_OK               0
#define MOE_ERR_INVALID_ARG  1  /* null pointer, negative size, bad flag or dtype  */
#define MOE_ERR_SHAPE        2  /* sizes inconsistent (k > E, T % n_src, ...)       */
#define MOE_ERR_ALIGN        3  /* row length or pointer not 16-byte aligned        */
#define MOE_ERR_CAPACITY     4  /* workspace or destination region too small        */
#define MOE_ERR_BAD_INDEX    5  /* (device flag) expert id out of range / repeated  */
#define MOE_ERR_HIP          6  /* a HIP launch or query failed                     */
#define MOE_ERR_UNSUPPORTED  7  /* sizes outside what the kernels implement         */

typedef int32_t moe_dtype_t;
#define MOE_F32   0
#define MOE_BF16  1

/* moe_route flags */
#define MOE_ROUTE_RENORM        0  /* gates = softmax over the k selected logits     */
#define MOE_ROUTE_FULL_SOFTMAX  1  /* gates = full softmax's probabilities of the k  */

/* Where dispatched rows go. n_src = n_dst = 1 with cap_rows_per_dst = T*k is the
 * plain expert-major layout. Otherwise the T tokens are n_src equal consecutive
 * groups (source ranks) and the E experts n_dst equal consecutive groups
 * (destination ranks; expert e lives on rank e / (E / n_dst)); destination r owns
 * rows [r*cap, (r+1)*cap) of the dispatch buffer. */
typedef struct moe_layout {
    int32_t n_src;
    int32_t n_dst;
    int64_t cap_rows_per_dst;
} moe_layout_t;

int32_t     moe_abi_version(void);
const char *moe_status_str(moe_status_t status);

/* Workspace bytes of one call, by operation (the per-call functions below give the
 * same numbers): MOE_OP_DISPATCH for moe_dispatch / moe_dispatch_fp8 (uses T, E, k,
 * layout), MOE_OP_EXPERT_FFN for moe_expert_ffn and MOE_OP_EXPERT_FFN_BWD for
 * moe_expert_ffn_bwd (use E, rows, d, F, dtype). Arguments an operation does not use
 * are ignored. Every other call needs no workspace (0). Invalid sizes give 0.
 * [EFA] NVSHMEM-based pplx-kernels: one interface, whatever moves the bytes; the
 * caller sizes every buffer up front, once. */
typedef int32_t moe_op_t;
#define MOE_OP_DISPATCH        0
#define MOE_OP_EXPERT_FFN      1
#define MOE_OP_EXPERT_FFN_BWD  2
size_t moe_workspace_size(moe_op_t op, int64_t T, int32_t E, int32_t k,
                          const struct moe_layout *layout, int64_t rows, int64_t d, int64_t F,
                          moe_dtype_t dtype);

/* ------------------------------------------------------------------ router
 * [EFA] Introduction: a small linear routing layer decides which experts multiply a
 * token; [EFA] Send and receive buffers: each token goes to R (here k) of E experts.
 *
 *   logit[t,e] = sum_{i<d} x[t,i] * w_router[e,i]        (no bias)
 *   computed in float32 as acc = fmaf(x[t,i], w[e,i], acc) for i = 0..d-1 from +0,
 *   one fixed order, so the integer routing decision is reproducible exactly.
 *   topk_idx[t,:] = the k largest logits, descending; equal logits -> lower id first.
 *   topk_w[t,j]   = exp(l_j - l_0) / sum_{j'<k} exp(l_j' - l_0)   (MOE_ROUTE_RENORM)
 *                 = full softmax probability of expert idx[t,j]    (MOE_ROUTE_FULL_SOFTMAX)
 *   The gating function is not on the pages; softmax over the selection is the
 *   reading that makes the gate-weighted average of combine a true average.
 *
 * x [T,d] dtype, w_router [E,d] dtype; logits [T,E] f32 (NULL: not written);
 * topk_idx [T,k] int32; topk_w [T,k] f32. Limits: 1 <= k <= min(E, 32); E <= 1024
 * for bf16, E <= 512 for f32; for bf16 also d <= 2^26 and E*d*2 < 2^31 bytes (32-bit
 * buffer offsets), else MOE_ERR_UNSUPPORTED before anything is launched. T = 0 is a
 * no-op. */
moe_status_t moe_route(const void *x, const void *w_router, int64_t T, int64_t d, int32_t E,
                       int32_t k, moe_dtype_t dtype, int32_t flags, float *logits,
                       int32_t *topk_idx, float *topk_w, void *stream);

/* ---------------------------------------------------------------- dispatch
 * [EFA] Dispatch and combine: count the tokens of every expert (the article does it
 * with atomics in shared memory of one block), take the cumulative sum of the
 * counts as offsets that pack the tokens into contiguous per-destination send
 * buffers, then copy the tokens in. [EFA] Send and receive buffers: each sender's
 * rows at a destination are one contiguous chunk, so one write per peer suffices,
 * and a destination receives at most N*T*max(R, E/N) rows.
 *
 * Plan (all int32 outputs):
 *   counts     [n_src, E]        pairs of source s routed to expert e
 *   expert_off [E+1]             exclusive cumulative sum of per-expert totals
 *   chunk_off  [n_dst, n_src+1]  start of source s's chunk inside destination r;
 *                                chunk_off[r][n_src] = rows live at r
 *   pair_slot  [T, k]            row of pair (t, j) in x_disp
 *   row_pair   [n_dst * cap]     t*k + j of the pair in each row; -1 where unused
 * Row of pair (t,j) with s = t / (T/n_src), e = topk_idx[t,j], r = e / (E/n_dst):
 *   r*cap + chunk_off[r][s] + sum_{e' in r, e' < e} counts[s][e']
 *         + #{t' < t in source s routed to e}
 * i.e. chunks by sender, experts ascending inside a chunk, tokens ascending inside
 * an expert (a stable order: the article's atomics leave it open). With the
 * expert-major layout this is expert_off[e] + #{t' < t routed to e}.
 * Copy: x_disp[pair_slot[t,j], :] = x[t, :] (bit copy). Rows of x_disp that no pair
 * uses are not written. x and x_disp may both be NULL (plan only).
 *
 * layout NULL = expert-major. Requires T % n_src == 0, E % n_dst == 0 and
 * cap_rows_per_dst >= (T/n_src) * n_src * min(k, E/n_dst) (the tight form of the
 * article's bound: a token sends at most min(k, E/N) rows to one destination).
 * Tokens must list k distinct experts in [0, E); violations raise the device flag.
 * Limits: E <= 1024, k <= 32, T*k < 2^31, n_dst*cap < 2^31. The rank-major layout
 * (n_src or n_dst > 1) also scans its plan in one workgroup's LDS: it needs
 *   B*E + n_src*E + E + 1 + n_dst*(n_src+1) + n_src*n_dst <= 32768 ints,
 * B = n_src * ceil(T/n_src / 256) plan blocks (e.g. 32 sources x 128 tokens at E = 384
 * uses 25,665); larger plans return MOE_ERR_UNSUPPORTED. The expert-major layout has
 * no such limit.
 * T = 0 (an empty batch): topk_idx, pair_slot, x and x_disp are not read; counts,
 * expert_off and chunk_off are written as zeros, every row_pair entry as -1, and the
 * status flag is cleared.
 * ws: at least moe_dispatch_workspace_size() bytes, 256-byte aligned; its first
 * bytes hold the device status flag that moe_dispatch_status() reads. */
size_t moe_dispatch_workspace_size(int64_t T, int32_t E, int32_t k, const moe_layout_t *layout);
moe_status_t moe_dispatch(const void *x, const int32_t *topk_idx, int64_t T, int64_t d,
                          int32_t E, int32_t k, moe_dtype_t dtype, const moe_layout_t *layout,
                          int32_t *counts, int32_t *expert_off, int32_t *chunk_off,
                          int32_t *pair_slot, int32_t *row_pair, void *x_disp, void *ws,
                          size_t ws_bytes, void *stream);
/* moe_dispatch_noalloc: moe_dispatch for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same plan and copy, bit for bit, with the workspace taken from a fixed array of
 * 4 MiB per GPU inside the library (a __device__ array, resident from the library's
 * load until the process ends) instead of `ws`. The call itself allocates nothing.
 * Limit: the plan's workspace (moe_dispatch_workspace_size of the same sizes) must fit
 * 4 MiB, e.g. T <= 209,408 tokens at E = 384 or T <= 104,704 at E = 1024 in the
 * expert-major layout; larger plans return MOE_ERR_CAPACITY before anything runs.
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU (two
 * streams, two host threads) race and must be serialised by the caller. Nothing in
 * the array needs clearing between calls. The device status flag lives in the array
 * and moe_dispatch_status cannot read it; a skipped pair shows as pair_slot = -1 and
 * an over-full destination as chunk_off[r][n_src] > cap_rows_per_dst. */
moe_status_t moe_dispatch_noalloc(const void *x, const int32_t *topk_idx, int64_t T, int64_t d,
                                  int32_t E, int32_t k, moe_dtype_t dtype,
                                  const moe_layout_t *layout, int32_t *counts,
                                  int32_t *expert_off, int32_t *chunk_off, int32_t *pair_slot,
                                  int32_t *row_pair, void *x_disp, void *stream);
/* Waits for `stream`, then returns MOE_OK, MOE_ERR_BAD_INDEX or MOE_ERR_CAPACITY
 * from the flag the last moe_dispatch on `ws` raised. */
moe_status_t moe_dispatch_status(const void *ws, void *stream);

/* moe_dispatch_fp8: the same plan, with the rows sent as block-scaled fp8 ([EFA]
 * evaluation: dispatch in block-scaled fp8, combine in bf16; the format is not on the
 * pages, this is the reading taken). x is bf16 [T,d] with d % 128 == 0. For every
 * row r and 128-element block b of its token, with m = max |x| over the block:
 *   q_scale[r, b]  = m / 448                                         (f32)
 *   q_disp[r, i]   = E4M3(x[t,i] * (448 / m)), round to nearest even, saturating at
 *                    +-448 (OCP FP8 E4M3: bias 7, 3 mantissa bits); 0 codes, scale 0
 *                    for an all-zero block. Every f32 operation rounds once.
 * q_disp [rows, d] uint8 (16-byte aligned), q_scale [rows, d/128] f32 (16-byte
 * aligned), rows = n_dst * cap; unused rows are not written. Other arguments, the
 * plan outputs, limits and errors as for moe_dispatch. */
moe_status_t moe_dispatch_fp8(const void *x, const int32_t *topk_idx, int64_t T, int64_t d,
                              int32_t E, int32_t k, const moe_layout_t *layout, int32_t *counts,
                              int32_t *expert_off, int32_t *chunk_off, int32_t *pair_slot,
                              int32_t *row_pair, uint8_t *q_disp, float *q_scale, void *ws,
                              size_t ws_bytes, void *stream);

/* -------------------------------------------------------------- expert FFN
 * [EFA] MoE all-to-all over EFA: grouped GEMM kernels multiply the received tokens
 * with the expert weights; [EFA] Dispatch and combine: the receiver moves tokens
 * into the tensor handed to the grouped GEMM. Expert form (not on the pages):
 * SwiGLU without biases. For every expert e, rows R_e = [expert_off[e],
 * expert_off[e+1]) of the expert-major x_disp:
 *   h = X W1^T, u = X W3^T, a = silu(h) * u with silu(z) = z / (1 + exp(-z)),
 *   y_disp[R_e] = a W2^T
 * w13 [E, 2F, d] (rows 0..F-1 = W1, F..2F-1 = W3), w2 [E, d, F], x_disp and y_disp
 * [rows, d], rows >= expert_off[E] (the host cannot see expert_off: rows is the
 * allocation). float32 accumulation; bf16 stores round to nearest even (a is
 * stored in bf16 between the two GEMMs). hu_save [rows, 2F] (NULL: not written)
 * keeps h and u for the backward. Requires d % 64 == 0 and F % 64 == 0 for bf16,
 * E <= 1024. ws: moe_expert_ffn_workspace_size() bytes (it holds a), 256-byte
 * aligned. */
size_t moe_expert_ffn_workspace_size(int32_t E, int64_t rows, int64_t d, int64_t F,
                                     moe_dtype_t dtype);
/* The two halves of moe_expert_ffn, one kernel each, for callers that schedule
 * them separately (overlap, timing): gate_up writes act [rows, F] = silu(h) * u
 * (and hu_save if non-NULL); down writes y_disp = act W2^T. No workspace. */
moe_status_t moe_expert_ffn_gate_up(const void *x_disp, const int32_t *expert_off,
                                    const void *w13, int32_t E, int64_t rows, int64_t d,
                                    int64_t F, moe_dtype_t dtype, void *act, void *hu_save,
                                    void *stream);
moe_status_t moe_expert_ffn_down(const void *act, const int32_t *expert_off, const void *w2,
                                 int32_t E, int64_t rows, int64_t d, int64_t F,
                                 moe_dtype_t dtype, void *y_disp, void *stream);
moe_status_t moe_expert_ffn(const void *x_disp, const int32_t *expert_off, const void *w13,
                            const void *w2, int32_t E, int64_t rows, int64_t d, int64_t F,
                            moe_dtype_t dtype, void *y_disp, void *hu_save, void *ws,
                            size_t ws_bytes, void *stream);

/* ----------------------------------------------------------------- combine
 * [EFA] Introduction and Dispatch and combine: the combine kernel returns each
 * token's processed copies and computes their weighted average into the output
 * tensor, accumulating at the receiver ([EFA] Dispatch/combine latency).
 *   y[t,:] = sum_{j<k} topk_w[t,j] * y_disp[pair_slot[t,j], :]
 * float32 accumulation in j order, one rounding to dtype. rows_total bounds
 * pair_slot (entries outside [0, rows_total) contribute nothing; with rows_total = 0
 * y_disp is never read). k <= 64, else MOE_ERR_UNSUPPORTED (also for combine_add). */
moe_status_t moe_combine(const void *y_disp, const int32_t *pair_slot, const float *topk_w,
                         int64_t T, int32_t k, int64_t d, int64_t rows_total, moe_dtype_t dtype,
                         void *y, void *stream);

/* ------------------------------------------- receive side of the rank-major layout
 * [EFA] Dispatch and combine: the receiver moves the tokens it got into the tensor
 * handed to the grouped GEMM; [EFA] Send and receive buffers: destination r's region
 * holds one contiguous chunk per sender. These calls give one destination its
 * expert-major input and return the expert outputs to the region for combine.
 *
 * moe_ep_recv_plan: from the plan of a rank-major moe_dispatch (counts [n_src,E],
 *   chunk_off [n_dst, n_src+1]; E/n_dst = epr local experts), destination r's order:
 *   local expert le = e - r*epr ascending, inside it senders ascending, inside those
 *   the sender's own (ascending token) order.
 *     local_off [epr+1]  exclusive cumulative sum of the local experts' rows
 *     row_src   [cap]    region row (0-based inside r's region) of local row j for
 *                        j < local_off[epr]; -1 for the rest
 *   Limits: epr <= 1024, epr * n_src <= 8192, cap < 2^31. A plan the dispatch
 *   flagged over capacity is cut at cap.
 * moe_ep_recv_gather:  x_local[j]  = x_region[row_src[j]]  (bit copy, rows with -1
 *                      untouched); x_region = x_disp + r*cap rows.
 * moe_ep_recv_scatter: y_region[row_src[j]] = y_local[j]   (bit copy).
 * Between the two, moe_expert_ffn(x_local, local_off, w13 + r*epr experts, w2 + ...,
 * epr, rows = cap, ...) is destination r's grouped GEMM; combine then runs at the
 * sources on the whole rank-major y_disp with the dispatch's pair_slot. */
moe_status_t moe_ep_recv_plan(const int32_t *counts, const int32_t *chunk_off, int32_t n_src,
                              int32_t n_dst, int32_t E, int32_t r, int64_t cap,
                              int32_t *local_off, int32_t *row_src, void *stream);
moe_status_t moe_ep_recv_gather(const void *x_region, const int32_t *row_src, int64_t cap,
                                int64_t d, moe_dtype_t dtype, void *x_local, void *stream);
/* moe_ep_recv_gather_fp8: x_local[j] = bf16(decode(q[row_src[j], i]) * scale[row_src[j], i/128])
 * (the receiver's dequantization of the moe_dispatch_fp8 payload, one f32 product,
 * one rounding); row_src NULL means row j itself (the expert-major layout). q_region
 * [cap, d] uint8 (8-byte aligned), scale_region [cap, d/128] f32, x_local [cap, d]
 * bf16; d % 128 == 0. */
moe_status_t moe_ep_recv_gather_fp8(const uint8_t *q_region, const float *scale_region,
                                    const int32_t *row_src, int64_t cap, int64_t d, void *x_local,
                                    void *stream);
moe_status_t moe_ep_recv_scatter(const void *y_local, const int32_t *row_src, int64_t cap,
                                 int64_t d, moe_dtype_t dtype, void *y_region, void *stream);

/* moe_combine_add: y[t,:] = residual[t,:] + sum_{j<k} topk_w[t,j] * y_disp[pair_slot[t,j], :]
 * (the float32 sum starts from the residual, then the j-ordered fmas, one rounding).
 * [EFA] Dispatch and combine: while the sender half of dispatch waits on the network
 * the GPU computes other work such as the shared expert; this call adds that shared
 * expert's output (residual [T,d] dtype, e.g. moe_expert_ffn with E = 1 on x) into the
 * combine. y may alias neither y_disp nor residual. */
moe_status_t moe_combine_add(const void *y_disp, const int32_t *pair_slot, const float *topk_w,
                             int64_t T, int32_t k, int64_t d, int64_t rows_total,
                             moe_dtype_t dtype, const void *residual, void *y, void *stream);

/* ------------------------------------------------ partial combine (rank-major)
 * [EFA] Dispatch/combine latency: the article accumulates only at the receiver of the
 * combine. The variant here lets each destination of the rank-major layout first sum,
 * per token, the gate-weighted outputs of that token's experts it holds, so one row per
 * (token, destination) travels back instead of one per (token, expert); the source
 * then adds its partial rows. The partial is rounded to dtype before the return (the
 * payload precision), so the result carries one more rounding than moe_combine.
 *   moe_combine_partial:  partial[r*T + t] = sum_{j: pair_slot[t,j] in [r*cap,(r+1)*cap)}
 *                         topk_w[t,j] * y_disp[pair_slot[t,j]]      (float32 fma in j
 *                         order, one rounding); rows of absent (t, r) are not written
 *   moe_combine_partials: y[t] = sum over the destinations r holding rows of t, r
 *                         ascending, of partial[r*T + t]   (float32, one rounding)
 * partial [n_dst*T, d] dtype; other arguments as for moe_combine with rows_total =
 * n_dst*cap; n_dst <= 64 and k <= 64, else MOE_ERR_UNSUPPORTED. */
moe_status_t moe_combine_partial(const void *y_disp, const int32_t *pair_slot,
                                 const float *topk_w, int64_t T, int32_t k, int64_t d,
                                 int32_t n_dst, int64_t cap, moe_dtype_t dtype, void *partial,
                                 void *stream);
moe_status_t moe_combine_partials(const void *partial, const int32_t *pair_slot, int64_t T,
                                  int32_t k, int64_t d, int32_t n_dst, int64_t cap,
                                  moe_dtype_t dtype, void *y, void *stream);

/* ---------------------------------------------------------------- backward
 * The transposes of the steps above (the layer's gradient; the article covers
 * only the forward data movement).
 *
 * moe_combine_bwd:  dy_disp[pair_slot[t,j]] = topk_w[t,j] * dy[t]      (dtype)
 *                   dtopk_w[t,j] = <dy[t], y_disp[pair_slot[t,j]]>    (f32)
 * moe_expert_ffn_bwd (bf16 only), per expert e with X, dO = dy_disp rows of e, h, u
 * from hu_save (written by moe_expert_ffn):
 *                   dA = dO W2;  dh = dA * u * s * (1 + h (1 - s)), s = sigmoid(h);
 *                   du = dA * silu(h);  dX = dh W1 + du W3      -> dx_disp (dtype)
 *                   dW2 = dO^T a;  dW1 = dh^T X;  dW3 = du^T X  -> dw2, dw13 (f32)
 *                   a = silu(h) * u is recomputed from hu_save. ws: at least
 *                   moe_expert_ffn_bwd_workspace_size() bytes, 256-byte aligned (it
 *                   holds [dh du] and a in bf16; contents undefined afterwards).
 *                   d and F multiples of 64, 2F * d * 2 bytes < 2^31, E <= 1024;
 *                   otherwise MOE_ERR_UNSUPPORTED. Every dw13/dw2 entry is written,
 *                   zeros for experts without rows.
 * moe_route_bwd:   (T = 0: only dw_router is written, as zeros; nothing else is read)
 *                   dlogits_sel[t,j] = g_j (dg_j - sum_i g_i dg_i)   (f32, RENORM gating)
 *                   dw_router[e,:] = sum over the rows of expert e in the expert-major
 *                                    plan (expert_off, row_pair from moe_dispatch),
 *                                    i.e. over its tokens, of
 *                                    dlogits_sel[t,j] * x[t,:]      (f32, summed in
 *                                    one fixed order: bitwise reproducible)
 * moe_dispatch_bwd: dx[t] = sum_j dx_disp[pair_slot[t,j]]
 *                           + sum_j dlogits_sel[t,j] * w_router[topk_idx[t,j]]
 *                   (second term skipped if dlogits_sel is NULL), float32 sum in
 *                   j order, one rounding to dtype; k <= 64.
 * Shapes as in the forward calls; dw13 [E,2F,d], dw2 [E,d,F], dw_router [E,d]. */
moe_status_t moe_combine_bwd(const void *dy, const void *y_disp, const int32_t *pair_slot,
                             const float *topk_w, int64_t T, int32_t k, int64_t d,
                             int64_t rows_total, moe_dtype_t dtype, void *dy_disp,
                             float *dtopk_w, void *stream);
size_t moe_expert_ffn_bwd_workspace_size(int32_t E, int64_t rows, int64_t d, int64_t F,
                                         moe_dtype_t dtype);
moe_status_t moe_expert_ffn_bwd(const void *x_disp, const void *dy_disp, const void *hu_save,
                                const int32_t *expert_off, const void *w13, const void *w2,
                                int32_t E, int64_t rows, int64_t d, int64_t F,
                                moe_dtype_t dtype, void *dx_disp, float *dw13, float *dw2,
                                void *ws, size_t ws_bytes, void *stream);
moe_status_t moe_route_bwd(const void *x, const int32_t *topk_idx, const float *topk_w,
                           const float *dtopk_w, const int32_t *expert_off,
                           const int32_t *row_pair, int64_t T, int64_t d, int32_t E, int32_t k,
                           moe_dtype_t dtype, float *dlogits_sel, float *dw_router, void *stream);
moe_status_t moe_dispatch_bwd(const void *dx_disp, const int32_t *pair_slot,
                              const int32_t *topk_idx, const float *dlogits_sel,
                              const void *w_router, int64_t T, int32_t k, int64_t d, int32_t E,
                              int64_t rows_total, moe_dtype_t dtype, void *dx, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* LIBMOE_MOE_H */
