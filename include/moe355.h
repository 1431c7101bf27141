/*
 * libmoe355 -- one GPU's hot path of an expert-parallel MoE layer, forward and
 * backward, hand-written HIP for gfx950 (MI355X).
 *
 * The path follows the numbered forward-pass steps of the textbook section
 * "Expert parallelism" (zerotofrontier.app/moe/expert-parallel): route (step 1),
 * permute and count by destination (step 2), expert compute as one grouped
 * matrix product (step 5), unpermute and weight (step 7).  The cross-GPU
 * exchanges (steps 3, 4, 6) are not here; moe_send_counts gives the matrix of
 * rows each simulated rank would send to each other rank.
 *
 * Conventions for every call:
 *  - Every pointer is a DEVICE pointer (hipMalloc'd or equivalent) unless
 *    stated; every call is asynchronous on `stream` (NULL = the null stream)
 *    and performs no device-to-host synchronisation.
 *  - The caller owns every buffer, including scratch.  The library never
 *    allocates device memory.  Between calls it keeps only per-device caches
 *    of launch-shape queries (compute-unit count, kernel occupancy), held in
 *    atomics, so calls are reentrant and may run concurrently on different
 *    host threads and streams when their buffers do not overlap.
 *  - Outputs are fully overwritten.  Inputs are not modified.  Inputs and
 *    outputs must not alias.
 *  - Results are deterministic: the same inputs give the same output bits.
 *  - Host-side validation happens before any launch; on error nothing is
 *    launched.  T == 0 (or M == 0) returns MOE_OK and launches nothing,
 *    except where a call states otherwise.
 *  - Row-major layouts; all row strides are dense.  Device pointers to
 *    activations and weights must be 16-byte aligned.
 *  - No C++ exception crosses this interface.
 */
#ifndef MOE355_H
#define MOE355_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1,   /* null pointer, bad size, misalignment, workspace too small */
    MOE_ERR_UNSUPPORTED = -2,   /* a shape or option outside what the kernels implement */
    MOE_ERR_HIP = -3            /* the HIP runtime reported an error at launch */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;
typedef enum { MOE_SOFTMAX = 0, MOE_SIGMOID = 1 } moe_gating;

/* Human-readable name of a status code (static string, never NULL). */
const char *moe_status_string(moe_status s);

/*
 * Route: top-k experts and gates per token (step 1 of the forward pass;
 * "05 - Expert Parallelism (MoE)", section "The all-to-all pattern"; the
 * group limit is DeepSeek-V3's node-limited routing, "What DeepSeek-V3 did
 * about it").
 *
 *   logits    [T, E] fp32, the router output for each token.
 *   k         experts per token, 1 <= k <= min(E, 16).
 *   gating    MOE_SOFTMAX or MOE_SIGMOID.
 *   renormalize  1: gates normalised over the k chosen experts
 *                   (softmax: exp(l_j - l_0) / sum_i exp(l_i - l_0);
 *                    sigmoid: s(l_j) / sum_i s(l_i));
 *                0: softmax over all E experts, or the bare sigmoid.
 *   n_groups, topk_groups  group limit: the E experts form n_groups
 *                contiguous groups; each group scores the fp32 sum of its two
 *                largest sigmoid affinities; only experts of the topk_groups
 *                best groups may be chosen.  1, 1 = no limit.
 *   topk_ids  [T, k] int32 out: slot 0 is the best expert.
 *   topk_w    [T, k] fp32 out: the gates.
 *
 * Selection ranks experts by their fp32 logit (-0 counts as +0), ties to the
 * lower expert id; group ties go to the lower group id.  The sigmoid used for
 * group scores is the pinned fp32 function of moe_sigmoid_pinned, so group
 * choices are reproducible bit for bit.  NaN logits are outside the contract.
 * Errors: INVALID_ARG for null pointers, T < 0, k outside [1, E], E % n_groups,
 * topk_groups outside [1, n_groups], a group of fewer than 2 experts, or
 * topk_groups * (E / n_groups) < k; UNSUPPORTED for E > 1024, k > 16,
 * n_groups > 64.
 */
moe_status moe_route_topk(const float *logits, int T, int E, int k, moe_gating gating,
                          int renormalize, int n_groups, int topk_groups, int32_t *topk_ids,
                          float *topk_w, hipStream_t stream);

/*
 * moe_route_topk with auxiliary-loss-free balancing ("05 - Expert
 * Parallelism (MoE)", section "Load balancing", family (b)): the choice is
 * TopK(logits + bias).  Every selection -- the group scores of the group
 * limit included -- ranks the fp32 keys fl32(logit + bias[e]) (-0 counts as
 * +0), while the gates are the formulas of moe_route_topk evaluated on the
 * unbiased logits of the chosen experts.
 *
 *   bias  [E] fp32 device array, one entry per expert.
 * Every other argument, and every error, as in moe_route_topk; a null bias
 * is INVALID_ARG (for T > 0).  A zero bias gives moe_route_topk's results bit
 * for bit.
 */
moe_status moe_route_topk_biased(const float *logits, const float *bias, int T, int E, int k,
                                 moe_gating gating, int renormalize, int n_groups,
                                 int topk_groups, int32_t *topk_ids, float *topk_w,
                                 hipStream_t stream);

/*
 * Router product (step 1 of the forward pass computes the router before the
 * top-k choice): logits[t][e] = sum_i x[t][i] w_router[e][i], accumulated in
 * fp32 (MFMA), written in fp32.
 *
 *   x         [T, d] token rows, dtype dt.
 *   w_router  [E, d] one row of d inputs per expert (K-contiguous, like the
 *             expert matrices), dtype dt.
 *   logits    [T, E] fp32 out.
 * Errors: INVALID_ARG for null pointers, T < 0, d < 1, E < 1, misaligned x or
 * w_router; UNSUPPORTED for d elem not a multiple of 128 bytes, or x or
 * w_router of 64 GiB or more.
 */
moe_status moe_router_logits(const void *x, moe_dtype dt, int T, int d, const void *w_router,
                             int E, float *logits, hipStream_t stream);

/*
 * Bias update of auxiliary-loss-free balancing ("05 - Expert Parallelism
 * (MoE)", section "Load balancing", family (b)): after a step,
 *     bias[e] += lr * (avg - counts[e]),   avg = fl(M) / fl(E),
 * M the sum of the counts (moe_permute's per-expert histogram), one fp32
 * rounding per operation, so an under-loaded expert's bias rises and an
 * over-loaded one's falls.
 *
 *   counts  [E] int32 device array; bias [E] fp32 device array, updated in
 *   place.  lr is a host value.
 * Errors: INVALID_ARG for null pointers or E < 1; UNSUPPORTED for E > 1024.
 */
moe_status moe_router_bias_update(const int32_t *counts, int E, float lr, float *bias,
                                  hipStream_t stream);

/*
 * The pinned fp32 sigmoid applied elementwise: y[i] = s(x[i]), n elements.
 * s(x) = 1/(1+t) for x >= 0 and t/(1+t) otherwise, t = exp(-|x|), where exp
 * is Cody & Waite reduction (ln2 split into a 12-significant-bit head and a
 * tail) and a degree-7 Taylor polynomial in fp32 fmaf, scaled by 2^n; inputs
 * below -87 give 0.  Exposed so the group scores of moe_route_topk can be
 * checked bit for bit.  Errors: INVALID_ARG for null pointers or n < 0.
 */
moe_status moe_sigmoid_pinned(const float *x, float *y, int64_t n, hipStream_t stream);

/*
 * Send-count matrix (step 2; "A dispatch you can check by hand"): entry
 * (s, q) = number of assignments of source rank s's tokens whose expert lives
 * on rank q.  Token t belongs to rank floor(t / (T / n_ep)); expert e lives on
 * rank floor(e * n_ep / E).  Each row sums to k T / n_ep.
 *
 *   topk_ids     [T, k] int32, values in [0, E).
 *   send_counts  [n_ep, n_ep] int32 out, row = source rank.
 * T = 0 writes an all-zero matrix.
 * Errors: INVALID_ARG for null pointers, n_ep < 1, T % n_ep or E % n_ep != 0;
 * UNSUPPORTED for n_ep > 1024.
 */
moe_status moe_send_counts(const int32_t *topk_ids, int T, int k, int E, int n_ep,
                           int32_t *send_counts, hipStream_t stream);

/*
 * Bytes of device scratch moe_permute needs for M = T k assignments over E
 * experts (per-chunk histograms).  Host function, no device work.
 */
size_t moe_permute_workspace_bytes(int T, int k, int E);

/*
 * Permute (step 2 and step 5's sort by local expert; "Token permutation and
 * grouped GEMMs"): order is the stable argsort of the expert ids of the M = T k
 * assignments (assignment a = t k + j), counts the per-expert histogram,
 * offsets its exclusive prefix sum, inv the inverse permutation
 * (inv[order[p]] = p), and x_perm = X[order]: packed row p is a bit copy of
 * token order[p] / k.  Rows of one expert are contiguous in x_perm, in token
 * order.
 *
 *   x          [T, d] activations, dtype dt.
 *   topk_ids   [T, k] int32, values in [0, E).  An id outside [0, E) breaks
 *              the permutation; the kernels never write out of bounds for it
 *              but leave the affected outputs undefined.
 *   counts     [E] int32 out;  offsets [E+1] int32 out (offsets[E] = M).
 *   order, inv [M] int32 out.
 *   x_perm     [M, d] out, dtype dt.
 *   workspace  at least moe_permute_workspace_bytes(T, k, E) bytes of device
 *              scratch owned by the caller; its contents on entry do not matter.
 * Index-only mode: x and x_perm both NULL computes counts, offsets, order and
 * inv and copies no rows (for moe_grouped_gate_up_gather, which reads the rows
 * of x through order itself).
 * Errors: INVALID_ARG for null pointers (exactly one of x, x_perm NULL
 * included), T < 0, k < 1, E < 1, workspace too small, misaligned x / x_perm;
 * UNSUPPORTED for E > 1024, d % 8 != 0, or T k >= 2^31.
 */
moe_status moe_permute(const void *x, moe_dtype dt, int T, int d, const int32_t *topk_ids,
                       int k, int E, int32_t *counts, int32_t *offsets, int32_t *order,
                       int32_t *inv, void *x_perm, void *workspace, size_t workspace_bytes,
                       hipStream_t stream);

/*
 * moe_permute for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * call without the workspace argument.  Its per-chunk histograms go to a
 * library-owned device array of 1 MiB (moe_permute_workspace_bytes(T, k, E)
 * must not exceed 1048576: every call with E <= 256 fits, E = 1024 up to
 * T k = 2^19), one copy per GPU, held until the process ends.  The
 * call allocates nothing; its first call on a device looks up that device's
 * copy.  Same arguments, outputs, layouts and errors as moe_permute, plus
 * UNSUPPORTED when the workspace would exceed the array and MOE_ERR_HIP when
 * the array cannot be looked up.  Calls that overlap on one GPU (several
 * streams or host threads at once) share the array and race; serialise them.
 */
moe_status moe_permute_noalloc(const void *x, moe_dtype dt, int T, int d, const int32_t *topk_ids,
                               int k, int E, int32_t *counts, int32_t *offsets, int32_t *order,
                               int32_t *inv, void *x_perm, hipStream_t stream);

/*
 * Grouped SwiGLU expert MLP (step 5; "Token permutation and grouped GEMMs":
 * one launch computes the products of all experts' row segments, scheduling
 * output tiles from all of them, with no padding beyond the tile and nothing
 * dropped).  For each expert g and each packed row p in
 * [offsets[g], offsets[g+1]):
 *     h[p] = SiLU(a[p] W_gate,g^T) * (a[p] W_up,g^T),   y[p] = h[p] W_down,g^T,
 * SiLU(z) = z / (1 + exp(-z)); 6 d ffn FLOPs per row ("A worked example at
 * DeepSeek-V3's shape").
 *
 *   a        [M, d] packed rows, dtype dt.
 *   offsets  [G+1] int32 device array, non-decreasing, offsets[0] = 0,
 *            offsets[G] = M.  Row segments may be empty.
 *   w13      [G, 2, ffn, d]: per expert the gate matrix then the up matrix,
 *            each row an output feature with d contiguous inputs.
 *   w2       [G, d, ffn]: the down matrix, ffn contiguous inputs per row.
 *   h        [M, ffn] caller scratch, dtype dt; holds the SwiGLU activations
 *            on return.
 *   y        [M, d] out, dtype dt.
 * Accumulation is fp32; bf16 outputs are rounded to nearest even.  A single
 * always-active shared expert is the same call with G = 1 and offsets {0, M}
 * ("Fine-grained vs coarse experts").
 * Errors: INVALID_ARG for null pointers, M < 0, G < 1, misalignment;
 * UNSUPPORTED for d or ffn not a multiple of 128, G > 4096, M >= 2^31, or
 * one expert's gate and up matrices of 4 GiB or more (2 ffn d elem >= 2^32).
 * An offsets array that breaks its precondition is clamped to [0, M] and
 * never causes an out-of-bounds access.
 */
moe_status moe_grouped_swiglu(const void *a, moe_dtype dt, int M, int d, int ffn,
                              const int32_t *offsets, int G, const void *w13, const void *w2,
                              void *h, void *y, hipStream_t stream);

/*
 * The two halves of moe_grouped_swiglu as separate launches, so a caller can
 * time, overlap or fuse around each product on its own.  Same arguments,
 * layouts, precision and errors as moe_grouped_swiglu; the pair
 * moe_grouped_gate_up then moe_grouped_down gives bit-identical h and y.
 *
 * moe_grouped_gate_up: h[p] = SiLU(a[p] W_gate,g^T) * (a[p] W_up,g^T) for
 *   each packed row p of expert g's segment (4 d ffn FLOPs per row).
 *   a [M, d] in, w13 [G, 2, ffn, d] in, h [M, ffn] out.
 * moe_grouped_down: y[p] = h[p] W_down,g^T (2 d ffn FLOPs per row).
 *   h [M, ffn] in, w2 [G, d, ffn] in, y [M, d] out.  Argument order follows
 *   the product: M, then K = ffn, then N = d.
 */
moe_status moe_grouped_gate_up(const void *a, moe_dtype dt, int M, int d, int ffn,
                               const int32_t *offsets, int G, const void *w13, void *h,
                               hipStream_t stream);
moe_status moe_grouped_down(const void *h, moe_dtype dt, int M, int ffn, int d,
                            const int32_t *offsets, int G, const void *w2, void *y,
                            hipStream_t stream);

/*
 * One expert's SwiGLU MLP on few rows: the always-active shared expert of a
 * decode step ("05 -- Expert Parallelism (MoE)", section "Fine-grained vs
 * coarse experts": DeepSeek-V3 has one shared expert beside its routed ones;
 * same page, "The serving asymmetry": decode time is weight reads).
 *   h = SiLU(x W_gate^T) * (x W_up^T),  y = h W_down^T
 * which is moe_grouped_swiglu with G = 1, computed with each product's
 * reduction split into K ranges over many workgroups; fp32 partial sums go
 * to the workspace and are added in a fixed order (split 0 first), so the
 * result does not depend on scheduling.  It may differ from
 * moe_grouped_swiglu's in the last bits (another summation order).
 *   x [M, d], w13 [2, ffn, d] (gate rows, then up rows), w2 [d, ffn] in;
 *   h [M, ffn] and y [M, d] out; gu [M, 2 ffn] out (optional, NULL skips
 *   it): the pre-activations (gate, then up) in bf16, for a backward.
 *   workspace: device memory of at least
 *   moe_dense_swiglu_workspace_bytes(M, d, ffn) bytes, owned by the caller
 *   and overwritten.  Calls sharing a workspace must not overlap.
 * bf16 only.  Errors: INVALID_ARG for M < 0, d or ffn < 1, an unknown dtype
 * code, a null pointer (other than gu), pointers not 16-byte aligned, or a
 * workspace too small;
 * UNSUPPORTED for fp32, M > 256, or d or ffn not a multiple of 64.  M = 0
 * launches nothing.
 */
size_t moe_dense_swiglu_workspace_bytes(int M, int d, int ffn);
moe_status moe_dense_swiglu(const void *x, moe_dtype dt, int M, int d, int ffn, const void *w13,
                            const void *w2, void *h, void *gu, void *y, void *workspace,
                            size_t workspace_bytes, hipStream_t stream);

/*
 * moe_grouped_gate_up with the permute's row copy folded into the product's
 * loads ("Token permutation and grouped GEMMs": X[order] is only ever read by
 * the first expert product, so the rows can be gathered where they are
 * consumed).  Packed row p (p < M) is token order[p] / k of x; with M = T k
 * and moe_permute's order the result is bit-identical to moe_permute's x_perm
 * followed by moe_grouped_gate_up.  M may exceed T k: entries order[p] = t k
 * past T k add token t again, e.g. as the rows of an always-active shared
 * expert placed as one more group after the routed ones.
 *
 *   x        [T, d] activations in token order, dtype dt.
 *   k        assignments per token (the divisor applied to order).
 *   M        packed rows of the product; offsets[G] = M.
 *   order    [M] int32, every entry in [0, T k).
 *   offsets, w13, h, G, d, ffn as in moe_grouped_gate_up.
 * Errors: those of moe_grouped_gate_up, and INVALID_ARG for k < 1 or a null
 * order; UNSUPPORTED also for x of 4 GiB or more (T d elem >= 2^32).  An
 * order entry outside [0, T k) is outside the contract: the read it steers is
 * bounded by x's extent, the row it produces is undefined.
 */
moe_status moe_grouped_gate_up_gather(const void *x, moe_dtype dt, int T, int k, int M, int d,
                                      int ffn, const int32_t *order, const int32_t *offsets,
                                      int G, const void *w13, void *h, hipStream_t stream);

/*
 * Unpermute and weight (step 7; "Token permutation and grouped GEMMs":
 * Y_sorted[inv] restores the token order): for each token t,
 *     y[t] = sum_{j<k} topk_w[t, j] * y_perm[inv[t k + j]]  (+ y_shared[t]),
 * summed in fp32 in slot order, the shared row last with weight 1.
 *
 *   y_perm    [T k, d] expert outputs in packed (expert) order, dtype dt.
 *   inv       [T k] int32 from moe_permute.  Entries outside [0, T k) are
 *             skipped (contribute nothing).
 *   topk_w    [T, k] fp32 gates, or NULL: every gate 1 (the sum of a
 *             token's k rows, which is the permute's backward).
 *   y_shared  [T, d] dtype dt, or NULL for none.
 *   y         [T, d] out, dtype dt.
 * Errors: INVALID_ARG for null required pointers, T < 0, k < 1, misalignment;
 * UNSUPPORTED for d % 8 != 0, k > 64, T k >= 2^31.
 */
moe_status moe_unpermute_combine(const void *y_perm, moe_dtype dt, int T, int k, int d,
                                 const int32_t *inv, const float *topk_w, const void *y_shared,
                                 void *y, hipStream_t stream);

/*
 * moe_unpermute_combine over expert outputs of any row count: y_perm has
 * `rows` rows (for the capacity form below, E cap), and inv entries outside
 * [0, rows) -- a dropped assignment's -1 -- contribute nothing.
 * moe_unpermute_combine is this call with rows = T k.  Same layouts,
 * precision and errors, plus INVALID_ARG for rows < 0; y_perm may be NULL
 * only when rows = 0.
 */
moe_status moe_unpermute_combine_rows(const void *y_perm, int64_t rows, moe_dtype dt, int T,
                                      int k, int d, const int32_t *inv, const float *topk_w,
                                      const void *y_shared, void *y, hipStream_t stream);

/* ========================================================================
 * The two other ways to run the E expert products ("Expert parallelism",
 * section "Token permutation and grouped GEMMs", which weighs three: a loop
 * of products, padding every expert to a fixed capacity and batching, and
 * the grouped product above).  Both are here for comparison with the grouped
 * path, which is dropless and pads only inside a tile.
 * ======================================================================== */

/*
 * The capacity: cap = ceil(cf M / E), cf times an expert's fair share of the
 * M = T k assignments ("Load imbalance becomes idle time": a capacity factor
 * caps every expert at CF times its fair share), evaluated in double
 * precision.  Host function.  Returns -1 for E < 1, M < 0 or cf <= 0.
 */
int64_t moe_expert_capacity(int64_t M, int E, double cf);

/* Bytes of device scratch moe_permute_capacity needs.  Host function. */
size_t moe_permute_capacity_workspace_bytes(int T, int k, int E);

/*
 * Pad to capacity ("Token permutation and grouped GEMMs": every expert's
 * block is exactly cap rows, so one batched product of E blocks runs all
 * experts; overflowing rows are dropped).  Expert e keeps its first cap
 * assignments in increasing a = t k + j -- the order moe_permute's stable
 * sort gives -- at slots e cap + 0, 1, ...; its later assignments are
 * dropped.  Blocks with fewer assignments are padded.
 *
 *   x, dt, T, d, topk_ids, k, E   as moe_permute.
 *   cap        rows per expert block, >= 0 (moe_expert_capacity).
 *   counts     [E] int32 out: assignments per expert BEFORE the cap (so the
 *              dropped count is sum max(0, counts[e] - cap)).
 *   offsets    [E+1] int32 out: offsets[e] = e cap, the segment list that
 *              makes moe_grouped_swiglu (or its halves) one batched product.
 *   order      [E cap] int32 out: the assignment in each slot, -1 for a
 *              padding slot.  moe_grouped_gate_up_gather accepts it as is
 *              (a padding slot then computes a row of x[T-1], never read).
 *   inv        [T k] int32 out: each assignment's slot, -1 when dropped;
 *              moe_unpermute_combine_rows(rows = E cap) skips those.
 *   x_cap      [E cap, d] out, dtype dt: slot s holds token order[s] / k bit
 *              for bit, a padding slot zeros.  x and x_cap both NULL:
 *              index-only mode.
 *   workspace  moe_permute_capacity_workspace_bytes(T, k, E) bytes of device
 *              scratch owned by the caller.
 * Errors: INVALID_ARG for null required pointers, T < 0, k < 1, E < 1,
 * cap < 0, a small workspace, misaligned x / x_cap; UNSUPPORTED for E > 1024,
 * d % 8 != 0, T k >= 2^31 or E cap >= 2^31.
 */
moe_status moe_permute_capacity(const void *x, moe_dtype dt, int T, int d, const int32_t *topk_ids,
                                int k, int E, int cap, int32_t *counts, int32_t *offsets,
                                int32_t *order, int32_t *inv, void *x_cap, void *workspace,
                                size_t workspace_bytes, hipStream_t stream);

/*
 * A loop of products ("Token permutation and grouped GEMMs": one kernel
 * launch per expert): moe_grouped_swiglu's result, computed as two launches
 * per expert with rows, each sized and tiled for that expert's rows alone.
 * The launch count and grid sizes come from offsets_host, a HOST copy of the
 * device array offsets (the loop form needs the segment sizes on the host;
 * getting them costs the caller a device-to-host copy).  Same layouts,
 * precision and errors as moe_grouped_swiglu, plus INVALID_ARG when
 * offsets_host is NULL or not non-decreasing within [0, M].  The results
 * equal moe_grouped_swiglu's bit for bit when each expert's row count picks
 * the same tile family as the grouped call's mean rows per expert.
 */
moe_status moe_expert_loop_swiglu(const void *a, moe_dtype dt, int M, int d, int ffn,
                                  const int32_t *offsets, const int32_t *offsets_host, int G,
                                  const void *w13, const void *w2, void *h, void *y,
                                  hipStream_t stream);

/* ========================================================================
 * Training: the forward product that keeps what the backward needs, and the
 * backward pass.  The backward runs the forward's steps in reverse: the
 * combine's gradient goes out to the expert rows as the dispatch did, and
 * the dispatch's gradient is combined back into the tokens ("Expert
 * parallelism", section "How many bytes move"); its products cost twice the
 * forward's, 12 d ffn FLOPs per assignment (section "A worked example at
 * DeepSeek-V3's shape").  All values are the chain rule applied to the
 * forward's definitions.
 *
 * Precision (bf16).  The backward reads what the forward kept in bf16: the
 * pre-activations gu, h, and the dispatched gradient dy_perm (rounded once
 * each, to nearest even), and accumulates in fp32.  The SwiGLU backward's
 * dgate = dh u SiLU'(g) then carries an error that scales with |dh u|, not
 * with dgate itself, and a weight-gradient row sums only the rows of its
 * expert: for an expert with one or two rows, a single row of dW13 can be
 * off by as much as its own magnitude.  Over a whole matrix the error stays
 * within about 1e-2 of the matrix's largest magnitude (the GPU tests' bar is
 * 2e-2 per matrix).  fp32 layers keep fp32 pre-activations and agree with
 * the exact gradients to about 1e-6 per row.
 * ====================================================================== */

/*
 * moe_grouped_gate_up / moe_grouped_gate_up_gather that also stores the
 * pre-activations: gu [M, 2 ffn] row p = (W_gate,e x_p, W_up,e x_p) in the
 * dtype of x (gate columns 0 .. ffn-1, then up columns), besides h.
 * order == NULL: x is the packed rows [M, d] (T and k unused); otherwise row
 * p is x[order[p] / k] as in moe_grouped_gate_up_gather.  Errors as the
 * calls it extends, plus a NULL or misaligned gu.
 */
moe_status moe_grouped_gate_up_save(const void *x, moe_dtype dt, int T, int k, int M, int d,
                                    int ffn, const int32_t *order, const int32_t *offsets, int G,
                                    const void *w13, void *h, void *gu, hipStream_t stream);

/*
 * Backward of moe_unpermute_combine: for each token t and slot j, with
 * p = inv[t k + j],
 *     dy_perm[p]  = topk_w[t,j] dy[t]                (dtype of dy, [T k, d])
 *     dgate[t,j]  = sum_m dy[t,m] y_perm[p,m]         (fp32, [T, k])
 *     dy_shared[t] = dy[t]                            (optional copy, [T, d])
 * dgate and y_perm are both given or both NULL (no gate gradient).  The dot
 * products sum in a fixed order, so results are deterministic.  Errors:
 * INVALID_ARG for a NULL dy / inv / topk_w / dy_perm, one of dgate and
 * y_perm without the other, misaligned rows, T < 0, k < 1, d < 1;
 * UNSUPPORTED for d not a multiple of 8, k > 64 or T k >= 2^31.
 */
moe_status moe_combine_backward(const void *dy, moe_dtype dt, int T, int k, int d,
                                const int32_t *inv, const float *topk_w, const void *y_perm,
                                void *dy_perm, float *dgate, void *dy_shared, hipStream_t stream);

/*
 * Backward of the gates of moe_route_topk (the gate formulas of O1; the
 * choice is piecewise constant and a balancing bias is outside the
 * gradient, "05 - Expert Parallelism (MoE)", section "Load balancing"):
 * dlogits [T, E] fp32 from dgate [T, k], the route's topk_ids and topk_w and
 * the logits.  With dot = sum_j w_j dgate_j:
 *   softmax, renormalised:  dl[c_j] = w_j (dgate_j - dot)
 *   softmax, not renorm.:   dl[e] = P_e ([e = c_j] dgate_j - dot), P = softmax(l)
 *   sigmoid, renormalised:  dl[c_j] = s_j (1 - s_j) (dgate_j - dot) / sum_i s_i
 *   sigmoid, not renorm.:   dl[c_j] = s_j (1 - s_j) dgate_j,  s_j = 1/(1+e^-l_j)
 * every other entry 0.  Errors: INVALID_ARG for NULL pointers, T < 0,
 * k < 1, k > E, an unknown gating; UNSUPPORTED for k > 64 or E > 4096.
 */
moe_status moe_gate_backward(const float *logits, const int32_t *topk_ids, const float *topk_w,
                             const float *dgate, int T, int E, int k, moe_gating gating,
                             int renormalize, float *dlogits, hipStream_t stream);

/*
 * Backward of the second expert product and of SwiGLU, per expert segment
 * (offsets as in moe_grouped_swiglu): dh = dy_perm W_down,e ([M, d] x
 * [d, ffn], W_down,e = w2[e] row-major), then with (g, u) = gu[p] the
 * forward's pre-activations (moe_grouped_gate_up_save),
 *     dgu[p] = (dh u SiLU'(g), dh SiLU(g)),   SiLU'(g) = s (1 + g (1 - s)),
 * s = 1/(1+e^-g); dgu [M, 2 ffn], gate columns then up columns.
 * bf16 or fp32 (fp32 accumulation; bf16 outputs rounded to nearest even).
 * Errors: INVALID_ARG for NULL or misaligned pointers, M < 0, G < 1, an
 * unknown dtype; UNSUPPORTED for d or ffn not a multiple of 128, G > 1024,
 * or operands of 4 GiB or more.
 */
moe_status moe_grouped_down_backward(const void *dy_perm, moe_dtype dt, int M, int d, int ffn,
                                     const int32_t *offsets, int G, const void *w2,
                                     const void *gu, void *dgu, hipStream_t stream);

/*
 * Backward of the first expert product to its rows: dx_perm [M, d] =
 * dgu [M, 2 ffn] W13,e per segment, with W13,e = w13[e] read as [2 ffn, d]
 * (gate rows then up rows).  The token gradient is then
 * moe_unpermute_combine(dx_perm, inv, NULL gates) (+ the shared expert's).
 * bf16 or fp32; errors as moe_grouped_down_backward.
 */
moe_status moe_grouped_gate_up_backward(const void *dgu, moe_dtype dt, int M, int d, int ffn,
                                        const int32_t *offsets, int G, const void *w13,
                                        void *dx_perm, hipStream_t stream);

/*
 * Weight gradients: for each expert segment e = [offsets[e], offsets[e+1]),
 *     c[e] = a[seg]^T b[rows of seg]        c [G, m_dim, n_dim], a [M, m_dim]
 * where row p of b is b[b_order[p] / b_k] (b has b_rows rows), or b[p] when
 * b_order is NULL (then b has M rows).  An empty segment gives zeros.  Uses:
 * dW_down = weight_grad(dy_perm, h), dW13 = weight_grad(dgu, x, order, k)
 * (the second is [G, 2 ffn, d] = w13's layout).  bf16 or fp32.  Errors:
 * INVALID_ARG for NULL or misaligned pointers, M < 0, G < 1, b_k < 1, an
 * unknown dtype; UNSUPPORTED for m_dim or n_dim not a multiple of 128,
 * G > 1024, or operands of 4 GiB or more.
 */
moe_status moe_grouped_weight_grad(const void *a, const void *b, moe_dtype dt, int M, int m_dim,
                                   int n_dim, const int32_t *offsets, int G,
                                   const int32_t *b_order, int b_k, int b_rows, void *c,
                                   hipStream_t stream);

/*
 * Backward of the router product (logits = x w_router^T, moe_router_logits):
 *     dx        += dlogits w_router          [T, E] x [E, d]   (dx: [T, d], added to)
 *     dw_router  = dlogits^T x               [E, T] x [T, d]   (overwritten)
 * dlogits [T, E] fp32 (moe_gate_backward) is rounded once to bf16, the
 * products' operand type, into the workspace (moe_router_backward_workspace_bytes
 * bytes, which also holds the products' one-segment offsets); fp32
 * accumulation, bf16 results.  Either output may be NULL (not computed).
 * Errors: INVALID_ARG for NULL or misaligned pointers, a small workspace,
 * T < 0, d < 1, E < 1; UNSUPPORTED for fp32, E or d not a multiple of 256,
 * 0 < T < 96, or operands of 4 GiB or more.
 */
size_t moe_router_backward_workspace_bytes(int T, int E);
moe_status moe_router_backward(const float *dlogits, const void *x, moe_dtype dt, int T, int d,
                               const void *w_router, int E, void *dx, void *dw_router,
                               void *workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE355_H */
