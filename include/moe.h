/*
 * moe.h -- C-ABI of the MI355X (gfx950) MoE expert-layer library (libmoe_mi355x.so).
 *
 * The library computes one mixture-of-experts expert layer on the experts resident on
 * one GPU: router scores, top-k gating, a stable rowwise permutation that writes routed
 * tokens straight into per-expert input buffers, grouped SwiGLU expert GEMMs, and the
 * weighted combine, forward and backward.  The structure follows the pages' statement
 * of the problem: E experts with k chosen per token (unite.ai, "Ai2 κυκλοφορεί το
 * Olmo-Core 3…", opening section; ettayeb.fr, "Olmo-core 3 ouvre l'entraînement des
 * MoE…", section "Le problème que les MoE n'ont jamais tout à fait résolu"); routed data
 * placed directly into expert input buffers, routing metadata kept on the GPU so the
 * host never waits for a copy-back, and a grouped GEMM over the many small expert
 * computations (unite.ai, section "Παραλληλισμός, Ακρίβεια και Τεχνικές Μνήμης";
 * ettayeb.fr, section "Trois parallélismes, trois optimisations de routage").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor argument is a DEVICE pointer owned by the caller.  The library never
 *    allocates, frees, synchronises, or reads device memory from the host.  All work is
 *    enqueued on `stream` (a hipStream_t; NULL = the default stream).  No call copies
 *    anything back to the host, so expert counts and offsets never leave the GPU.
 *  - Notation: T tokens, d model width, f expert hidden width, E experts, k experts per
 *    token, R = T*k routed rows.  All matrices are row-major.  Weights are stored
 *    [out, in] per expert: Wr [E, d], W1 and W3 [E, f, d], W2 [E, d, f].
 *  - `act` dtype (moe_shape.act) is the element type of x, weights, y, every [R, *]
 *    activation buffer and every gradient except those documented as float.
 *    MOE_F32 -> float, MOE_BF16 -> bf16 (bit pattern in uint16).  Scores, gates and
 *    their gradients are always float.
 *  - Return value: MOE_OK, or a negative moe_status for an error detected on the host
 *    before anything was enqueued (bad shape, null pointer, misalignment, workspace too
 *    small).  MOE_ELAUNCH means a kernel launch failed (the stream state is then
 *    unspecified).  Data errors that only the device can see (an invalid pre-routed
 *    expert id) are reported by OR-ing bits into a caller-provided device word.
 *  - Determinism: every output is bitwise reproducible run to run (no float atomics,
 *    fixed reduction orders).
 *  - Re-entrancy: calls on different streams, or from different host threads, with disjoint
 *    buffers may run concurrently; calls that share a workspace must be ordered.  The only
 *    state the library keeps is host-side and filled once: each device's compute-unit count,
 *    the occupancy of each kernel at each dynamic-LDS size (it sizes the persistent GEMM
 *    grids), and the tuning overrides below; all three are read and filled under a lock or
 *    atomically.  moe_route_noalloc adds one fixed device array per GPU (see there).
 *  - Tuning overrides: MOE_TILE_<GEMM> / MOE_TILE, MOE_GEMM_BK, MOE_GEMM_STAGES,
 *    MOE_GEMM_LOADERS and MOE_MX_TILE select other GEMM tile shapes, k-depths, stage counts
 *    and loader waves than the measured defaults.  Each is read from the environment once,
 *    at the first launch that consults it, and kept until moe_tuning_reload.  They
 *    change only how the work is tiled and scheduled: every output element is still one fp32
 *    reduction over the same values in ascending order of the reduction index.
 *  - Limits: 1 <= k <= E <= 1024, T*k < 2^31, d and f multiples of 64; with MOE_MXFP8
 *    GEMMs d and f must be multiples of 128.  bf16 buffers need 16-byte alignment.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,        /* shape or argument out of the supported range */
  MOE_ENULL = -2,         /* a required pointer is NULL */
  MOE_EALIGN = -3,        /* a pointer is not aligned as required */
  MOE_EWORKSPACE = -4,    /* workspace smaller than moe_workspace_size() */
  MOE_EUNSUPPORTED = -5,  /* dtype combination not implemented */
  MOE_ELAUNCH = -6,       /* a kernel launch failed */
  MOE_ESCRATCH = -7       /* shape too large for moe_route_noalloc's fixed scratch */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_MXFP8 = 2 } moe_dtype;

/* The six expert GEMMs, as bits of moe_shape.mx_scope. */
#define MOE_MX_GEMM1 1   /* a, b = X W1^T, X W3^T (+ SwiGLU) */
#define MOE_MX_GEMM2 2   /* y_perm = h W2^T */
#define MOE_MX_DGRAD2 4  /* dh = dy_perm W2 (+ SwiGLU gradient) */
#define MOE_MX_WGRAD2 8  /* dW2 = dy_perm^T h */
#define MOE_MX_DGRAD1 16 /* dx_perm = [da | db] [W1; W3] */
#define MOE_MX_WGRAD1 32 /* [dW1; dW3] = [da | db]^T X */
#define MOE_MX_ALL 63
/* The default MXFP8 scope: the two GEMMs that reduce over the hidden width and produce the
 * d-wide rows returned to the tokens (y_perm and dx_perm).  Each output and gradient of the
 * layer then passes through at most one E4M3-quantised GEMM, which keeps the layer within
 * 6e-2 (normwise) of the unquantised result; with all six, two or three quantised GEMMs in
 * series put it 6-14% away.  The pages enable MXFP8 on selected operations, where it helped
 * most (bigchange.ai, "Olmo-core 3 открывает стек обучения MoE от Ai2…", section "Главное
 * изменение"; ettayeb.fr, "Olmo-core 3 ouvre l'entraînement des MoE…", section "Trois
 * parallélismes, trois optimisations de routage"). */
#define MOE_MX_DEFAULT (MOE_MX_GEMM2 | MOE_MX_DGRAD1)

/* All sizes are known on the host; nothing about the routing is. */
typedef struct {
  int32_t T, d, f, E, k;
  int32_t act;       /* MOE_F32 or MOE_BF16 */
  int32_t gemm;      /* grouped-GEMM arithmetic: MOE_F32 (act F32), MOE_BF16 or MOE_MXFP8 (act BF16) */
  int32_t mx_scope;  /* with gemm = MOE_MXFP8: the MOE_MX_* bits of the expert GEMMs that take E4M3
                        operands (0 means MOE_MX_DEFAULT); the other expert GEMMs run bf16.  Must be
                        0 for other gemm values. */
} moe_shape;

/* Bits OR-ed into *dev_err by moe_route_given. */
#define MOE_DEVERR_EXPERT_RANGE 1  /* an expert id outside [0, E) (clamped before use) */
#define MOE_DEVERR_DUPLICATE 2     /* one token lists the same expert twice */

const char* moe_status_str(int status);

/* Bytes of device workspace any call below may need for this shape (pure host
 * function; no HIP call).  Calls taking (ws, ws_bytes) use it as scratch only: its
 * contents on entry are ignored and on exit are unspecified. */
size_t moe_workspace_size(const moe_shape* s);

/* ---------------------------------------------------------------- forward */

/* Router scores: logits[t, e] = sum_i x[t, i] * Wr[e, i] (+ bias[e]).
 * x [T, d] act, Wr [E, d] act, bias [E] float or NULL, logits [T, E] float (written).
 * Router of the learned-routing rows (bigchange.ai, "Olmo-core 3 открывает стек
 * обучения MoE от Ai2…", section "Что инженер может попробовать на практике"). */
moe_status moe_router_fwd(const moe_shape* s, const void* x, const void* Wr, const float* bias,
                          float* logits, void* stream);

/* Top-k gating and dispatch metadata, all on the device: each token picks k of the E
 * experts (top-four routing in the production rows: bigchange.ai, "Olmo-core 3 открывает
 * стек обучения MoE от Ai2…", section "Что инженер может попробовать на практике"), and the
 * counts and offsets stay in device memory so the host never waits for them (unite.ai,
 * "Ai2 κυκλοφορεί το Olmo-Core 3…", section "Παραλληλισμός, Ακρίβεια και Τεχνικές
 * Μνήμης").  The gate function is not on the pages; the softmax over the chosen k scores
 * is the reading taken.
 * In:  logits [T, E] float (finite).
 * Out: topk_idx [T, k] int32, the k largest scores per token in value-descending order,
 *      equal scores broken toward the lower expert index;
 *      gates [T, k] float, softmax over the k selected scores;
 *      counts [E] int32 rows routed to each expert;
 *      offsets [E + 1] int32 exclusive prefix sum of counts (offsets[E] = T*k);
 *      slot_row [T, k] int32, packed row of routed slot (t, j): rows of one expert keep
 *      ascending slot order t*k + j (a stable counting sort).
 * ws: scratch of at least moe_workspace_size(s) bytes. */
moe_status moe_route(const moe_shape* s, const float* logits, int32_t* topk_idx, float* gates,
                     int32_t* counts, int32_t* offsets, int32_t* slot_row, void* ws, size_t ws_bytes,
                     void* stream);

/* moe_route for callers that cannot allocate device memory: code under HIP graph capture
 * that must not call hipMalloc, tight serving loops, harnesses that forbid allocation.  Same
 * arguments, kernels and results (bit for bit) as moe_route, without the workspace: the
 * per-chunk histograms and ranks live in a fixed array of 2^20 int32 (4 MiB) in the
 * library's own device memory, one per GPU, held until the process ends.  The first call on
 * a device takes that array's address on the current device (hipGetSymbolAddress, no
 * allocation); no call allocates or frees anything.  Shapes needing more than 4 MiB
 * (ceil(T/32)*E + T*k int32 values; e.g. T up to 131072 at E = 128, k = 4) return
 * MOE_ESCRATCH before anything is enqueued.  Every call on one GPU shares that GPU's array,
 * so calls that may overlap on one GPU (other streams, other host threads) race and must be
 * ordered by the caller.  No clearing is needed: every histogram entry and rank a launch reads
 * is written earlier in the same call. */
moe_status moe_route_noalloc(const moe_shape* s, const float* logits, int32_t* topk_idx, float* gates,
                             int32_t* counts, int32_t* offsets, int32_t* slot_row, void* stream);

/* Dispatch metadata for tokens that arrive already routed (random routing of the large
 * benchmark rows: bigchange.ai, section "Три числа, три знаменателя"; unite.ai, section
 * "Δοκιμές τρισεκατομμυρίων παραμέτρων").  topk_idx [T, k] int32 is the input; counts,
 * offsets and slot_row are written as in moe_route.  Invalid ids set bits in *dev_err
 * (a device int32 the caller zeroes and reads at its own sync point) and are clamped
 * into [0, E) so every later kernel stays in bounds. */
moe_status moe_route_given(const moe_shape* s, const int32_t* topk_idx, int32_t* counts,
                           int32_t* offsets, int32_t* slot_row, int32_t* dev_err, void* ws,
                           size_t ws_bytes, void* stream);

/* Rowwise dispatch into per-expert input buffers: x_perm[slot_row[t, j]] = x[t] and
 * row_src[slot_row[t, j]] = t.  Routed rows are written straight into the experts' input
 * buffers (unite.ai, section "Παραλληλισμός, Ακρίβεια και Τεχνικές Μνήμης"; ettayeb.fr,
 * "Olmo-core 3 ouvre l'entraînement des MoE…", section "Trois parallélismes, trois
 * optimisations de routage").  x [T, d] act, slot_row [T, k], row_src [R] int32 (written,
 * may be NULL), x_perm [R, d] act (written). */
moe_status moe_permute(const moe_shape* s, const void* x, const int32_t* slot_row, int32_t* row_src,
                       void* x_perm, void* stream);

/* Grouped SwiGLU expert FFN over the packed buffers (one group per expert, rows
 * [offsets[e], offsets[e+1])):  a = X_e W1_e^T, b = X_e W3_e^T, h = silu(a) * b,
 * y_e = h W2_e^T.  Equivalent to moe_ffn_gemm1_fwd followed by moe_ffn_gemm2_fwd.
 * x_perm [R, d] act; ab [R, 2f] act written (a in columns [0, f), b in [f, 2f), kept for
 * the backward); h [R, f] act written; y_perm [R, d] act written.  Accumulation is
 * float; with MOE_MXFP8 the GEMMs in moe_shape.mx_scope take E4M3 operands with one E8M0
 * scale per 32 elements along K (MXFP8 for the expert FFN: unite.ai, section
 * "Παραλληλισμός, Ακρίβεια και Τεχνικές Μνήμης"). */
moe_status moe_grouped_ffn_fwd(const moe_shape* s, const void* x_perm, const void* W1, const void* W3,
                               const void* W2, const int32_t* offsets, void* ab, void* h, void* y_perm,
                               void* ws, size_t ws_bytes, void* stream);

/* The two forward GEMMs as separate calls (moe_grouped_ffn_fwd runs both): GEMM1 with the
 * SwiGLU epilogue writes ab and h, GEMM2 writes y_perm.  Arguments as above; ws is used by
 * MOE_MXFP8 shapes (operand quantisation) and may be NULL otherwise. */
moe_status moe_ffn_gemm1_fwd(const moe_shape* s, const void* x_perm, const void* W1, const void* W3,
                             const int32_t* offsets, void* ab, void* h, void* ws, size_t ws_bytes,
                             void* stream);
moe_status moe_ffn_gemm2_fwd(const moe_shape* s, const void* h, const void* W2, const int32_t* offsets,
                             void* y_perm, void* ws, size_t ws_bytes, void* stream);

/* Weighted combine: y[t] = y_add[t] + sum_j gates[t, j] * y_perm[slot_row[t, j]] (float
 * accumulation, y_add first, then j in order).  y_perm [R, d] act, gates [T, k] float,
 * y_add [T, d] act or NULL (the always-on shared expert's output, when the layer has one:
 * bigchange.ai, "Olmo-core 3 открывает стек обучения MoE…", section "Что инженер может
 * попробовать на практике", top-four routing plus one shared expert), y [T, d] act
 * (written). */
moe_status moe_combine(const moe_shape* s, const void* y_perm, const float* gates, const int32_t* slot_row,
                       const void* y_add, void* y, void* stream);

/* ---------------------------------------------------------------- backward */

/* Backward of moe_combine: dy_perm[slot_row[t, j]] = gates[t, j] * dy[t] and
 * dgates[t, j] = <dy[t], y_perm[slot_row[t, j]]>.  The pages train the layer (forward and
 * backward) and route every token through its experts, whose outputs it gets back
 * (bigchange.ai, section "Главное изменение", where moving tokens to the experts is named
 * as a cost of its own); the gate-weighted sum differentiated here is the reading taken for
 * the combine.
 * dy [T, d] act, y_perm [R, d] act, gates [T, k] float; dy_perm [R, d] act and
 * dgates [T, k] float written. */
moe_status moe_combine_bwd(const moe_shape* s, const void* dy, const void* y_perm, const float* gates,
                           const int32_t* slot_row, void* dy_perm, float* dgates, void* stream);

/* Backward of the grouped FFN (equivalent to moe_ffn_dgrad2, moe_ffn_wgrad2,
 * moe_ffn_dgrad1, moe_ffn_wgrad1 in that order): the grouped expert GEMMs of the training
 * step (unite.ai, section "Παραλληλισμός, Ακρίβεια και Τεχνικές Μνήμης"), differentiated for
 * the SwiGLU reading of the expert FFN.
 *   dh = dy_e W2_e;  da = dh * b * s * (1 + a (1 - s)), db = dh * silu(a), s = sigmoid(a)
 *   dW2_e = dy_e^T h_e;  dx_e = da W1_e + db W3_e;  dW1_e = da^T X_e;  dW3_e = db^T X_e
 * dy_perm [R, d], x_perm [R, d], ab [R, 2f], h [R, f]: act inputs.  dab [R, 2f] act written
 * (da | db), dx_perm [R, d] act written, dW1 dW3 [E, f, d] and dW2 [E, d, f] act written;
 * an expert with no rows gets exactly zero weight gradients. */
moe_status moe_grouped_ffn_bwd(const moe_shape* s, const void* dy_perm, const void* x_perm, const void* ab,
                               const void* h, const void* W1, const void* W3, const void* W2,
                               const int32_t* offsets, void* dab, void* dx_perm, void* dW1, void* dW3,
                               void* dW2, void* ws, size_t ws_bytes, void* stream);

/* The four backward GEMMs as separate calls, in the order moe_grouped_ffn_bwd runs them:
 * dgrad2 (with the SwiGLU gradient, writes dab), wgrad2 (dW2), dgrad1 (dx_perm), wgrad1
 * (dW1, dW3).  ws: MOE_MXFP8 shapes quantise their operands into it; with one expert
 * (E = 1, as for a shared expert) the bf16 weight gradients split their reduction over the
 * rows and keep fp32 partial sums in it, added in a fixed order (MOE_EWORKSPACE if ws_bytes
 * is below moe_workspace_size). */
moe_status moe_ffn_dgrad2(const moe_shape* s, const void* dy_perm, const void* W2, const void* ab,
                          const int32_t* offsets, void* dab, void* ws, size_t ws_bytes, void* stream);
moe_status moe_ffn_wgrad2(const moe_shape* s, const void* h, const void* dy_perm, const int32_t* offsets,
                          void* dW2, void* ws, size_t ws_bytes, void* stream);
moe_status moe_ffn_dgrad1(const moe_shape* s, const void* dab, const void* W1, const void* W3,
                          const int32_t* offsets, void* dx_perm, void* ws, size_t ws_bytes, void* stream);
moe_status moe_ffn_wgrad1(const moe_shape* s, const void* x_perm, const void* dab, const int32_t* offsets,
                          void* dW1, void* dW3, void* ws, size_t ws_bytes, void* stream);

/* Gradient of the gates w.r.t. the scores: dlogits[t, e] = g_e (dg_e - sum_i g_i dg_i) for
 * the k chosen experts, 0 for the others (the derivative of the softmax gate of moe_route).
 * The router is trained in the learned-routing rows (bigchange.ai, section "Что инженер
 * может попробовать на практике").  dgates, gates [T, k] float, topk_idx [T, k],
 * dlogits [T, E] float (written in full). */
moe_status moe_route_bwd(const moe_shape* s, const float* dgates, const float* gates,
                         const int32_t* topk_idx, float* dlogits, void* stream);

/* Router backward: dx_r = dlogits Wr ([T, d] act, written), dWr = dlogits^T x ([E, d]
 * float, written), the gradients of the learned router's scores (bigchange.ai, section
 * "Что инженер может попробовать на практике").  The reduction over T is split into partial sums held in ws and added
 * in a fixed order (deterministic).  dx_r may be NULL: then only dWr is computed (the caller
 * folds dx_r into moe_permute_bwd_router). */
moe_status moe_router_bwd(const moe_shape* s, const void* x, const void* Wr, const float* dlogits,
                          void* dx_r, float* dWr, void* ws, size_t ws_bytes, void* stream);

/* Un-permute and sum, the backward of the rowwise dispatch (unite.ai, section
 * "Παραλληλισμός, Ακρίβεια και Τεχνικές Μνήμης"): each token gathers the input gradients of
 * its k routed rows.  dx[t] = dx_r[t] + dx_add[t] + sum_j dx_perm[slot_row[t, j]] (float
 * accumulation in that order; dx_r, the router's input gradient, and dx_add, the shared
 * expert's, may each be NULL).  dx_perm [R, d], dx_r / dx_add [T, d], dx [T, d] act. */
moe_status moe_permute_bwd(const moe_shape* s, const void* dx_perm, const int32_t* slot_row,
                           const void* dx_r, const void* dx_add, void* dx, void* stream);

/* Un-permute with the router's input gradient folded in (the same dispatch backward as
 * moe_permute_bwd, plus the gradient through the learned router's scores: bigchange.ai,
 * section "Что инженер может попробовать на практике").  The gates are a softmax over each
 * token's k chosen scores, so dlogits is zero outside them and dx_r[t] = sum_e dlogits[t, e]
 * Wr[e] has k terms: dx[t] = dx_add[t] + sum_j (dx_perm[slot_row[t, j]] + dlogits[t, e_j]
 * Wr[e_j]), e_j = topk_idx[t, j] (float accumulation in that order, one rounding to act;
 * dx_add may be NULL).  dlogits [T, E] float as written by moe_route_bwd, topk_idx [T, k]
 * from moe_route (ids outside [0, E) are clamped, never read out of range), Wr [E, d] act,
 * dx_perm [R, d], dx [T, d] act.  Replaces moe_router_bwd's dx_r and its read here. */
moe_status moe_permute_bwd_router(const moe_shape* s, const void* dx_perm, const int32_t* slot_row,
                                  const int32_t* topk_idx, const float* dlogits, const void* Wr,
                                  const void* dx_add, void* dx, void* stream);

/* ---------------------------------------------------------------- MXFP8 */

/* Block quantisation bf16 -> E4M3 codes + E8M0 scales, 32 elements per block.
 * src [rows, cols] bf16.  The scale of a block is the smallest power of two 2^s with
 * amax * 2^-s <= 448 (s clamped to [-127, 127]; an all-zero block gets s = -127); each
 * element is rounded to nearest-even on the E4M3 grid.
 * axis 0: blocks run along each row (32 consecutive columns); q [rows, cols] u8 and
 *         scales [rows, cols/32] u8; cols must be a multiple of 32.
 * axis 1: blocks run down the columns, restarting at every segment start
 *         seg_offsets[e] (e < nseg; seg_offsets has nseg + 1 entries, seg_offsets[nseg] =
 *         rows); the output is TRANSPOSED into the padded layout the weight-gradient GEMM
 *         reads: segment e occupies columns [P_e, P_e + roundup(n_e, 128)) of
 *         q [cols, rows_pad] with P_e = sum_{e'<e} roundup(n_e', 128), rows_pad = rows +
 *         128 * nseg, and scales [cols, rows_pad / 32]; padding is written as zero codes
 *         and zero-block scales.
 * MXFP8 for the expert FFN: unite.ai, section "Παραλληλισμός, Ακρίβεια και Τεχνικές
 * Μνήμης"; ettayeb.fr, section "Trois parallélismes, trois optimisations de routage". */
moe_status moe_mx_quantize(int32_t rows, int32_t cols, int32_t axis, const int32_t* seg_offsets,
                           int32_t nseg, const void* src, uint8_t* q, uint8_t* scales, void* stream);

/* ---------------------------------------------------------------------------------------
 * MXFP8 dispatch (shapes with gemm = MOE_MXFP8).  The routed rows leave the dispatch
 * already block-quantised, so no bf16 copy of x_perm or dy_perm is written and the expert
 * GEMMs quantise no activation that the dispatch has produced: MXFP8 serves the data moved
 * to the experts as well as the expert FFN compute (unite.ai, "Ai2 κυκλοφορεί το
 * Olmo-Core 3…", section "Παραλληλισμός, Ακρίβεια και Τεχνικές Μνήμης"; ettayeb.fr,
 * "Olmo-core 3 ouvre l'entraînement des MoE…", section "Trois parallélismes, trois
 * optimisations de routage").
 *
 * Each dispatch writes an [R, d] row set v in two layouts, with exactly the bytes
 * moe_mx_quantize would write for v:
 *   row layout     q_rows [R, d] u8, s_rows [R, d/32] u8     (axis 0)
 *   column layout  q_cols [d, L] u8, s_cols [d, L/32] u8     (axis 1 with seg_offsets =
 *                  offsets: blocks down each column restarting at every expert, expert e
 *                  at columns [P_e, P_e + roundup(n_e, 128)), padding zero)
 * with L = moe_mx_cols_ld(s) = R + 128 E.  Columns of the column layout past the last
 * expert's padded end are not written.  Every buffer is caller-owned device memory,
 * 16-byte aligned; the row and column layouts are what the *_mx GEMM calls below read.
 * --------------------------------------------------------------------------------------- */

/* L = T*k + 128*E, the row count of a column layout (pure host function; 0 for a bad shape). */
size_t moe_mx_cols_ld(const moe_shape* s);

/* Forward dispatch: v[r] = x[row_src[r]], with row_src[slot_row[t, j]] = t written first
 * (as moe_permute).  x [T, d] bf16, slot_row [T, k], offsets [E + 1] (from moe_route /
 * moe_route_given), row_src [R] int32 written.  Returns MOE_EUNSUPPORTED unless gemm =
 * MOE_MXFP8. */
moe_status moe_permute_mx(const moe_shape* s, const void* x, const int32_t* slot_row, const int32_t* offsets,
                          int32_t* row_src, uint8_t* q_rows, uint8_t* s_rows, uint8_t* q_cols,
                          uint8_t* s_cols, void* stream);

/* Combine backward with the routed gradient quantised in the dispatch:
 * dgates[t, j] = <dy[t], y_perm[slot_row[t, j]]> (float, bit-identical with
 * moe_combine_bwd), and v[slot_row[t, j]] = bf16(gates[t, j] * dy[t]) (the values
 * moe_combine_bwd would store in dy_perm) written only in the two MXFP8 layouts.
 * row_src is the one moe_permute_mx wrote. */
moe_status moe_combine_bwd_mx(const moe_shape* s, const void* dy, const void* y_perm, const float* gates,
                              const int32_t* slot_row, const int32_t* row_src, const int32_t* offsets,
                              float* dgates, uint8_t* q_rows, uint8_t* s_rows, uint8_t* q_cols,
                              uint8_t* s_cols, void* stream);

/* The expert GEMMs of moe_ffn_gemm1_fwd, moe_ffn_dgrad2, moe_ffn_wgrad2 and moe_ffn_wgrad1
 * with the dispatched operand given in its MXFP8 layout instead of bf16 (bit-identical
 * results, since the bytes are those the GEMM would have produced itself):
 *   gemm1_fwd_mx: x rows (q_rows, s_rows of moe_permute_mx)
 *   dgrad2_mx:    dy rows (q_rows, s_rows of moe_combine_bwd_mx)
 *   wgrad2_mx:    dy columns (q_cols, s_cols of moe_combine_bwd_mx)
 *   wgrad1_mx:    x columns (q_cols, s_cols of moe_permute_mx)
 * Each needs its GEMM in moe_shape.mx_scope (MOE_EUNSUPPORTED otherwise, before anything is
 * enqueued).  Other arguments, workspace and errors as the bf16-operand calls. */
moe_status moe_ffn_gemm1_fwd_mx(const moe_shape* s, const uint8_t* xq_rows, const uint8_t* xs_rows,
                                const void* W1, const void* W3, const int32_t* offsets, void* ab, void* h,
                                void* ws, size_t ws_bytes, void* stream);
moe_status moe_ffn_dgrad2_mx(const moe_shape* s, const uint8_t* dyq_rows, const uint8_t* dys_rows,
                             const void* W2, const void* ab, const int32_t* offsets, void* dab, void* ws,
                             size_t ws_bytes, void* stream);
moe_status moe_ffn_wgrad2_mx(const moe_shape* s, const void* h, const uint8_t* dyq_cols,
                             const uint8_t* dys_cols, const int32_t* offsets, void* dW2, void* ws,
                             size_t ws_bytes, void* stream);
moe_status moe_ffn_wgrad1_mx(const moe_shape* s, const uint8_t* xq_cols, const uint8_t* xs_cols,
                             const void* dab, const int32_t* offsets, void* dW1, void* dW3, void* ws,
                             size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * MXFP8 operands written by the producing GEMM's epilogue (the default scope: GEMM1 and
 * dgrad2 in bf16, GEMM2 and dgrad1 in MXFP8).  GEMM1 writes h and dgrad2 writes [da | db]
 * also as MXFP8 row blocks (blocks of 32 along the row, the layout of moe_mx_quantize with
 * axis 0), bit for bit the bytes the row quantiser writes for the stored bf16 values, so the
 * MXFP8 GEMM that reads them quantises nothing itself and its results are unchanged.  This
 * keeps the quantisation inside the expert FFN compute that MXFP8 serves (unite.ai,
 * section "Παραλληλισμός, Ακρίβεια και Τεχνικές Μνήμης").
 *
 * moe_ffn_gemm1_fwd_q: moe_ffn_gemm1_fwd (bf16), plus hq_rows [R, f] u8 codes and
 *   hs_rows [R, f/32] u8 scales of h.  Needs GEMM2 in the MXFP8 scope and GEMM1 outside it.
 * moe_ffn_gemm2_fwd_mx: moe_ffn_gemm2_fwd with h given as those rows.  Needs GEMM2 in scope.
 * moe_ffn_dgrad2_q: moe_ffn_dgrad2 (bf16), plus dabq_rows [R, 2f] codes and dabs_rows
 *   [R, 2f/32] scales of [da | db].  Needs dgrad1 in the MXFP8 scope and dgrad2 outside it.
 * moe_ffn_dgrad1_mx: moe_ffn_dgrad1 with [da | db] given as those rows.  Needs dgrad1 in scope.
 * A call whose scope condition fails returns MOE_EUNSUPPORTED before anything is enqueued;
 * buffers are caller-owned device memory, 16-byte aligned; other arguments and errors as the
 * plain calls.
 * --------------------------------------------------------------------------------------- */
moe_status moe_ffn_gemm1_fwd_q(const moe_shape* s, const void* x_perm, const void* W1, const void* W3,
                               const int32_t* offsets, void* ab, void* h, uint8_t* hq_rows, uint8_t* hs_rows,
                               void* stream);
moe_status moe_ffn_gemm2_fwd_mx(const moe_shape* s, const uint8_t* hq_rows, const uint8_t* hs_rows, const void* W2,
                                const int32_t* offsets, void* y_perm, void* ws, size_t ws_bytes, void* stream);
moe_status moe_ffn_dgrad2_q(const moe_shape* s, const void* dy_perm, const void* W2, const void* ab,
                            const int32_t* offsets, void* dab, uint8_t* dabq_rows, uint8_t* dabs_rows,
                            void* stream);
moe_status moe_ffn_dgrad1_mx(const moe_shape* s, const uint8_t* dabq_rows, const uint8_t* dabs_rows, const void* W1,
                             const void* W3, const int32_t* offsets, void* dx_perm, void* ws, size_t ws_bytes,
                             void* stream);

/* ---------------------------------------------------------------------------------------
 * moe_tuning_reload: forget the tuning overrides read so far (see the file header), so each
 * is read from the environment again at its next use.  For tuning sweeps and tests that
 * change them within one process; it must not run while another host thread launches
 * through the library.
 * --------------------------------------------------------------------------------------- */
void moe_tuning_reload(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
