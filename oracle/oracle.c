/*
 * CPU oracle for one GPU's share of an expert-parallel MoE layer: forward
 * pass and its backward.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is what the HIP path is checked
 * against; it is never part of the product.  Only the tests, the smoke
 * check and the CPU-baseline leg of the benchmark load it.  It shares no
 * source with the HIP library and includes nothing from it.
 *
 * Plain loops, written for a reader to check against the pages by eye:
 *   - "Expert parallelism" (zerotofrontier.app/moe/expert-parallel), the
 *     textbook section: the numbered forward-pass steps in section "Expert
 *     parallelism", the send matrix in "A dispatch you can check by hand",
 *     the byte count in "How many bytes move", node-limited routing in "What
 *     DeepSeek-V3 did about it", and order / counts / inverse in "Token
 *     permutation and grouped GEMMs".
 *   - "05 - Expert Parallelism (MoE)" (project-fortress), section "The
 *     all-to-all pattern": top-k routing and the router-probability-weighted
 *     sum; section "Fine-grained vs coarse experts": the always-active shared
 *     expert.
 *
 * Precision: routing keys and the group scores are fp32 (the logits are fp32
 * inputs and the selection must be bit-exact); every other floating-point
 * result is accumulated and returned in fp64.  bf16 values are widened
 * exactly.  Build with -ffp-contract=off and without fast-math.
 *
 * Parity: every function here is pinned by the CPU tests (hand-worked
 * example, invariants, brute force, closed forms); none is unpinned.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_F64 2

#define ORC_SOFTMAX 0
#define ORC_SIGMOID 1

static double widen(const void *base, int dtype, int64_t i)
{
    if (dtype == ORC_F32) return (double)((const float *)base)[i];
    if (dtype == ORC_F64) return ((const double *)base)[i];
    uint32_t u = (uint32_t)((const uint16_t *)base)[i] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ------------------------------------------------------------------------
 * Pinned fp32 sigmoid.
 *
 * In DeepSeek-V3's node-limited routing ("What DeepSeek-V3 did about it") a
 * group's score for a token adds up the token's two largest affinities among
 * the group's experts, and an affinity is the sigmoid of a logit.  Which groups survive is an
 * integer decision taken on fp32 sums, so both sides must produce the same
 * fp32 sigmoid bits.  This is that function, written from the mathematics:
 *
 *   exp(y), y <= 0: Cody & Waite range reduction y = n ln2 + r, |r| <= ln2/2,
 *   with ln2 split as C_HI + C_LO (C_HI has 12 significant bits, so n*C_HI is
 *   exact), then the degree-7 Taylor polynomial of exp(r) in Horner form with
 *   coefficients fl(1/i!), then scaling by 2^n.  Every operation is one IEEE
 *   fp32 operation (fmaf where written), rounded to nearest even.
 *   Results that would leave the normal range (y < -87) return 0.
 *
 *   sigmoid(x) = 1/(1+t) for x >= 0 and t/(1+t) for x < 0, with t = exp(-|x|).
 * ---------------------------------------------------------------------- */
static float pinned_exp_nonpos(float y)
{
    const float log2e = (float)1.4426950408889634074;       /* fl(log2 e) */
    const float c_hi = 2839.0f / 4096.0f;                    /* ln2 to 12 significant bits */
    const float c_lo = (float)(0.69314718055994530942 - 2839.0 / 4096.0);
    static const float inv_fact[8] = {
        1.0f, 1.0f, (float)(1.0 / 2), (float)(1.0 / 6), (float)(1.0 / 24),
        (float)(1.0 / 120), (float)(1.0 / 720), (float)(1.0 / 5040)};
    if (y < -87.0f) return 0.0f;
    float n = rintf(y * log2e);
    float r = fmaf(-n, c_hi, y);
    r = fmaf(-n, c_lo, r);
    float p = inv_fact[7];
    for (int i = 6; i >= 0; --i) p = fmaf(p, r, inv_fact[i]);
    return ldexpf(p, (int)n);
}

float orc_sigmoid_pinned(float x)
{
    float t = pinned_exp_nonpos(-fabsf(x));
    float den = 1.0f + t;
    return x >= 0.0f ? 1.0f / den : t / den;
}

void orc_sigmoid_pinned_array(const float *x, float *y, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) y[i] = orc_sigmoid_pinned(x[i]);
}

/* ------------------------------------------------------------------------
 * O1  Route: top-k per token, optionally node (group) limited, plus gates.
 *
 * Step 1 of the forward pass ("Expert parallelism", section "Expert
 * parallelism"): every GPU picks k experts for each of its own tokens.  The key of expert e is the fp32
 * logit with -0 read as +0; both gating maps are increasing, so ranking by
 * the logit ranks by the gate.  Among equal keys the lower expert id wins,
 * and slot j holds the j-th pick.
 *
 * Group limit ("What DeepSeek-V3 did about it"): score each of n_groups
 * contiguous groups by the fp32 sum of its two highest pinned-sigmoid
 * affinities, keep the best topk_groups groups (lower group id on ties), and
 * pick the k experts only among them.
 *
 * Gates, in fp64, rounded once to fp32:
 *   softmax, renormalised: exp(l_j - l_0) / sum_{i<k} exp(l_i - l_0)
 *   softmax, not renorm.:  exp(l_j - m) / sum_e exp(l_e - m), m = max_e l_e
 *   sigmoid, renormalised: s(l_j) / sum_{i<k} s(l_i)
 *   sigmoid, not renorm.:  s(l_j)
 *
 * Auxiliary-loss-free balancing ("05 - Expert Parallelism (MoE)", section
 * "Load balancing", family (b)): with a per-expert bias b (NULL = none) the
 * choice is TopK(logits + bias) -- the key becomes fl32(l_e + b_e), and the
 * group scores, being part of the choice, are taken on those keys -- while
 * the gates above stay functions of the unbiased logits l.  Without a bias
 * the key is l_e and nothing changes.
 * Returns 0, or -1 on arguments outside the contract.
 * ---------------------------------------------------------------------- */
int orc_route(const float *logits, const float *bias, int T, int E, int k, int gating, int renorm,
              int n_groups, int topk_groups, int32_t *ids, float *w)
{
    if (T < 0 || E < 1 || k < 1 || k > E || k > 64 || n_groups < 1 || E % n_groups != 0 ||
        topk_groups < 1 || topk_groups > n_groups)
        return -1;
    const int gs = E / n_groups;
    if (n_groups > 1 && (gs < 2 || topk_groups * gs < k)) return -1;

#pragma omp parallel
    {
        float *key = malloc(sizeof(float) * (size_t)E);
        char *allowed = malloc((size_t)E);
        char *taken = malloc((size_t)E);
        float *gscore = malloc(sizeof(float) * (size_t)n_groups);
        char *gkept = malloc((size_t)n_groups);
#pragma omp for schedule(static)
        for (int t = 0; t < T; ++t) {
            const float *l = logits + (int64_t)t * E;
            for (int e = 0; e < E; ++e) {
                key[e] = (bias ? l[e] + bias[e] : l[e]) + 0.0f;   /* -0 + +0 = +0 */
                allowed[e] = 1;
                taken[e] = 0;
            }
            if (n_groups > 1) {
                for (int g = 0; g < n_groups; ++g) {
                    float a1 = -INFINITY, a2 = -INFINITY;
                    for (int e = g * gs; e < (g + 1) * gs; ++e) {
                        float a = orc_sigmoid_pinned(key[e]);
                        if (a > a1) { a2 = a1; a1 = a; }
                        else if (a > a2) { a2 = a; }
                    }
                    gscore[g] = a1 + a2;
                    gkept[g] = 0;
                }
                for (int r = 0; r < topk_groups; ++r) {
                    int best = -1;
                    for (int g = 0; g < n_groups; ++g)
                        if (!gkept[g] && (best < 0 || gscore[g] > gscore[best])) best = g;
                    gkept[best] = 1;
                }
                for (int e = 0; e < E; ++e) allowed[e] = gkept[e / gs];
            }
            int32_t *id = ids + (int64_t)t * k;
            for (int j = 0; j < k; ++j) {
                int best = -1;
                for (int e = 0; e < E; ++e)
                    if (allowed[e] && !taken[e] && (best < 0 || key[e] > key[best])) best = e;
                taken[best] = 1;
                id[j] = best;
            }
            float *wt = w + (int64_t)t * k;
            double v[64], sum = 0.0;     /* k <= 64 is checked above */
            if (gating == ORC_SOFTMAX) {
                if (renorm) {
                    double l0 = (double)l[id[0]];
                    for (int j = 0; j < k; ++j) { v[j] = exp((double)l[id[j]] - l0); sum += v[j]; }
                } else {
                    double m = (double)l[0];
                    for (int e = 1; e < E; ++e) if ((double)l[e] > m) m = (double)l[e];
                    for (int e = 0; e < E; ++e) sum += exp((double)l[e] - m);
                    for (int j = 0; j < k; ++j) v[j] = exp((double)l[id[j]] - m);
                }
            } else {
                for (int j = 0; j < k; ++j) { v[j] = 1.0 / (1.0 + exp(-(double)l[id[j]])); sum += v[j]; }
                if (!renorm) sum = 1.0;
            }
            for (int j = 0; j < k; ++j) wt[j] = (float)(v[j] / sum);
        }
        free(key); free(allowed); free(taken); free(gscore); free(gkept);
    }
    return 0;
}

/* ------------------------------------------------------------------------
 * O2  Send-count matrix ("A dispatch you can check by hand").
 * Entry (s, q) counts the rows GPU s sends to GPU q.  Token t belongs to
 * source rank s = floor(t / T_loc) (each GPU holds its own T_loc tokens,
 * section "Expert parallelism"), and expert i lives on GPU floor(i n_ep / E)
 * (step 2 of the forward pass).
 * ---------------------------------------------------------------------- */
int orc_send_counts(const int32_t *ids, int T, int k, int E, int n_ep, int32_t *S)
{
    if (n_ep < 1 || T % n_ep != 0 || E % n_ep != 0) return -1;
    const int T_loc = T / n_ep;
    memset(S, 0, sizeof(int32_t) * (size_t)n_ep * (size_t)n_ep);
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            int e = ids[(int64_t)t * k + j];
            if (e < 0 || e >= E) return -1;
            int s = t / T_loc;
            int q = (int)(((int64_t)e * n_ep) / E);
            S[(int64_t)s * n_ep + q] += 1;
        }
    return 0;
}

/* ------------------------------------------------------------------------
 * O3  Permutation ("Token permutation and grouped GEMMs").
 * order is the stable argsort of the expert ids of the M = T k assignments
 * (assignment a = t k + j), counts the per-expert histogram, offsets its
 * exclusive prefix sum (offsets[E] = M), and inv the inverse permutation,
 * inv[order[p]] = p.  Written as a textbook stable counting sort.
 * ---------------------------------------------------------------------- */
int orc_permute_index(const int32_t *ids, int64_t M, int E, int32_t *counts,
                      int32_t *offsets, int32_t *order, int32_t *inv)
{
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t a = 0; a < M; ++a) {
        if (ids[a] < 0 || ids[a] >= E) return -1;
        counts[ids[a]] += 1;
    }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t *cursor = malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
    for (int e = 0; e < E; ++e) cursor[e] = offsets[e];
    for (int64_t a = 0; a < M; ++a) {
        int32_t p = cursor[ids[a]]++;
        order[p] = (int32_t)a;
        inv[a] = p;
    }
    free(cursor);
    return 0;
}

/* ------------------------------------------------------------------------
 * N2  Pad to capacity and batch ("Expert parallelism", "Token permutation
 * and grouped GEMMs", the second of its three ways to run the E expert
 * products).  Every expert's block holds exactly cap rows, so one batched
 * product of E blocks covers all of them; assignments beyond an expert's cap
 * are dropped and blocks with fewer rows are padded.  cap is CF times an
 * expert's fair share T k / E ("Load imbalance becomes idle time"), rounded
 * up to a whole row, evaluated in double precision.
 * ---------------------------------------------------------------------- */
int64_t orc_expert_capacity(int64_t M, int E, double cf)
{
    if (E < 1 || M < 0 || !(cf > 0.0)) return -1;
    return (int64_t)ceil(cf * (double)M / (double)E);
}

/* Which assignments an expert keeps: its assignments a = t k + j in
 * increasing a (the order a stable sort leaves them in), the first cap of
 * them.  Kept assignment number r of expert e goes to slot e cap + r.
 *   counts[e]     all assignments to e, before the cap;
 *   slot_of[a]    its slot, or -1 when the assignment is dropped;
 *   assign_of[s]  the assignment in slot s, or -1 when the slot is padding.
 * Written as a direct walk over the assignments with a fill count per
 * expert. */
int orc_permute_capacity(const int32_t *ids, int64_t M, int E, int64_t cap, int32_t *counts,
                         int32_t *slot_of, int32_t *assign_of)
{
    if (cap < 0) return -1;
    for (int64_t s = 0; s < (int64_t)E * cap; ++s) assign_of[s] = -1;
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t a = 0; a < M; ++a) {
        int e = ids[a];
        if (e < 0 || e >= E) return -1;
        int64_t r = counts[e]++;
        if (r < cap) {
            slot_of[a] = (int32_t)(e * cap + r);
            assign_of[e * cap + r] = (int32_t)a;
        } else {
            slot_of[a] = -1;
        }
    }
    return 0;
}

/* X[order]: packed row p is a copy of token order[p] / k, bit for bit. */
void orc_gather_rows(const void *x, int64_t row_bytes, const int32_t *order, int64_t M,
                     int k, void *x_perm)
{
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < M; ++p)
        memcpy((char *)x_perm + p * row_bytes, (const char *)x + (int64_t)(order[p] / k) * row_bytes,
               (size_t)row_bytes);
}

/* ------------------------------------------------------------------------
 * O4  Expert MLP on a list of rows (step 5 of the forward pass).
 * A SwiGLU expert has three d x ffn matrices and costs 6 d ffn forward FLOPs
 * per row ("A worked example at DeepSeek-V3's shape", "DeepSeek-V3's layout,
 * counted"):
 *   g = W_gate x,  u = W_up x,  h = SiLU(g) * u,  y = W_down h,
 *   SiLU(z) = z / (1 + exp(-z)).
 * w13 is [G][2][ffn][d] (gate rows, then up rows), w2 is [G][d][ffn].  Row r
 * uses expert expert_of_row[r].  All sums run in fp64 in index order.
 * ---------------------------------------------------------------------- */
void orc_expert_swiglu_rows(const void *xrows, int dtype, int64_t R, int d, int ffn,
                            const int32_t *expert_of_row, const void *w13, const void *w2,
                            double *y)
{
#pragma omp parallel
    {
        double *xv = malloc(sizeof(double) * (size_t)d);
        double *h = malloc(sizeof(double) * (size_t)ffn);
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < R; ++r) {
            int64_t e = expert_of_row[r];
            for (int i = 0; i < d; ++i) xv[i] = widen(xrows, dtype, r * d + i);
            int64_t gate0 = e * 2 * (int64_t)ffn * d;
            int64_t up0 = gate0 + (int64_t)ffn * d;
            for (int n = 0; n < ffn; ++n) {
                double g = 0.0, u = 0.0;
                for (int i = 0; i < d; ++i) {
                    g += widen(w13, dtype, gate0 + (int64_t)n * d + i) * xv[i];
                    u += widen(w13, dtype, up0 + (int64_t)n * d + i) * xv[i];
                }
                h[n] = g / (1.0 + exp(-g)) * u;
            }
            int64_t down0 = e * (int64_t)d * ffn;
            for (int m = 0; m < d; ++m) {
                double acc = 0.0;
                for (int n = 0; n < ffn; ++n) acc += widen(w2, dtype, down0 + (int64_t)m * ffn + n) * h[n];
                y[r * d + m] = acc;
            }
        }
        free(xv);
        free(h);
    }
}

/* ------------------------------------------------------------------------
 * O5  Unpermute and weight (step 7 of the forward pass; "Token permutation
 * and grouped GEMMs": Y_sorted[inv] restores token order).  Each token's k
 * expert outputs are added with their gates, slot order j = 0..k-1, then the
 * shared expert's output (weight 1) if given:
 *   y[t] = sum_j w[t,j] y_perm[inv[t k + j]]  (+ y_shared[t]).
 * An assignment that a capacity limit dropped (inv = -1; "Token permutation
 * and grouped GEMMs": overflowing rows are dropped) has no expert output and
 * adds nothing.
 * ---------------------------------------------------------------------- */
void orc_combine(const void *y_perm, int dtype, int64_t T, int k, int d, const int32_t *inv,
                 const float *w, const void *y_shared, int sh_dtype, double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int m = 0; m < d; ++m) {
            double acc = 0.0;
            for (int j = 0; j < k; ++j) {
                int64_t p = inv[t * k + j];
                if (p < 0) continue;
                acc += (double)w[t * k + j] * widen(y_perm, dtype, p * d + m);
            }
            if (y_shared) acc += widen(y_shared, sh_dtype, t * d + m);
            y[t * d + m] = acc;
        }
    }
}

/* ------------------------------------------------------------------------
 * Bytes one GPU sends in the dispatch plus the combine all-to-all ("How many
 * bytes move"): each of the T_loc k assignments carries d numbers, of which
 * a fraction (n_ep - 1)/n_ep leaves the GPU; dispatch at s_disp bytes per
 * number, combine at s_comb.  A training step does both twice.
 * ---------------------------------------------------------------------- */
double orc_alltoall_bytes(int64_t T_loc, int k, int64_t d, int n_ep, double s_disp,
                          double s_comb, int training)
{
    double per = (double)T_loc * k * (double)d * (double)(n_ep - 1) / (double)n_ep;
    double b = per * s_disp + per * s_comb;
    return training ? 2.0 * b : b;
}

/* ------------------------------------------------------------------------
 * O0  Router logits (step 1 of the forward pass: "compute the router").
 * logits[t][e] = sum_i x[t][i] wg[e][i]: one row of wg per expert, d inputs
 * per row (the same K-contiguous layout as the expert matrices).  The sum
 * runs in fp64 in index order and is rounded once to fp32, the precision
 * routing takes its decisions in.
 * ---------------------------------------------------------------------- */
void orc_router_logits(const void *x, int dtype, int64_t T, int d, const void *wg, int E,
                       float *logits)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int i = 0; i < d; ++i)
                acc += widen(x, dtype, t * d + i) * widen(wg, dtype, (int64_t)e * d + i);
            logits[t * E + e] = (float)acc;
        }
    }
}

/* ------------------------------------------------------------------------
 * Bias update of auxiliary-loss-free balancing ("05 - Expert Parallelism
 * (MoE)", section "Load balancing", family (b)): after a step, with load[i]
 * the tokens expert i received, bias[i] += lr * (avg_load - load[i]), so an
 * under-loaded expert's bias rises and an over-loaded one's falls.  In fp32,
 * one rounding per operation: avg = fl(M) / fl(E) with M = sum of the loads,
 * then fl(avg - fl(load[i])), times lr, added to bias[i].
 * Returns 0, or -1 on arguments outside the contract.
 * ---------------------------------------------------------------------- */
int orc_bias_update(const int32_t *counts, int E, float lr, float *bias)
{
    if (E < 1) return -1;
    int64_t M = 0;
    for (int e = 0; e < E; ++e) M += counts[e];
    const float avg = (float)M / (float)E;
    for (int e = 0; e < E; ++e) {
        const float dev = avg - (float)counts[e];
        const float step = lr * dev;
        bias[e] = bias[e] + step;
    }
    return 0;
}

/* ========================================================================
 * Backward pass.
 *
 * The pages give the backward's shape, not its formulas: it runs the
 * forward's steps in reverse, the gradient of the combine going out the way
 * the dispatch did and the gradient of the dispatch coming back the way the
 * combine did ("Expert parallelism", section "How many bytes move"), and it
 * costs twice the forward's products, 12 d d_e per assignment (section "A
 * worked example at DeepSeek-V3's shape").  What it computes is fixed by the
 * forward definition and the chain rule; each function below is that
 * derivative written out, in fp64.  dy is the gradient of the loss at the
 * layer output y.
 * ====================================================================== */

/* ------------------------------------------------------------------------
 * B5  Backward of O5 (unpermute and weight).  From
 *   y[t] = sum_j w[t,j] y_perm[inv[t k + j]]  (+ y_sh[t]):
 *   dy_perm[inv[t k + j]] = w[t,j] dy[t]          (the combine's gradient,
 *                                                   dispatched to the rows)
 *   dw[t,j]               = sum_m dy[t,m] y_perm[inv[t k + j], m]
 *   (dy_sh[t] = dy[t], not written here.)
 * dy_perm is [T k, d] indexed by packed position; dw is [T, k].
 * ---------------------------------------------------------------------- */
void orc_combine_backward(const void *dy, int dy_dt, int64_t T, int k, int d, const int32_t *inv,
                          const float *w, const void *y_perm, int yp_dt, double *dy_perm,
                          double *dw)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int j = 0; j < k; ++j) {
            const int64_t p = inv[t * k + j];
            const double g = (double)w[t * k + j];
            double acc = 0.0;
            for (int m = 0; m < d; ++m) {
                const double v = widen(dy, dy_dt, t * d + m);
                dy_perm[p * d + m] = g * v;
                acc += v * widen(y_perm, yp_dt, p * d + m);
            }
            dw[t * k + j] = acc;
        }
    }
}

/* ------------------------------------------------------------------------
 * B4  Backward of O4 (one expert's SwiGLU MLP) for a set of rows.  Forward,
 * per row x of expert e:  g = W_gate x,  u = W_up x,  h = SiLU(g) u,
 * y = W_down h.  With dy the gradient at y:
 *   dh      = W_down^T dy
 *   dg      = dh u SiLU'(g),   SiLU'(z) = s(z) (1 + z (1 - s(z))),  s = 1/(1+e^-z)
 *   du      = dh SiLU(g)
 *   dx      = W_gate^T dg + W_up^T du
 *   dW_down += dy h^T,   dW_gate += dg x^T,   dW_up += du x^T
 * The forward is recomputed from x in fp64.  First pass, row by row: g, u,
 * h, dh, dg, du and dx.  Second pass, one weight-gradient row at a time:
 * the sums over each expert's rows, in increasing row order.  Outputs, each
 * may be NULL: dx [R, d]; gu [R, 2 ffn] = (g, u) and dgu [R, 2 ffn] =
 * (dg, du) per row; dw13 [G, 2, ffn, d] and dw2 [G, d, ffn], overwritten.
 * ---------------------------------------------------------------------- */
void orc_expert_swiglu_backward_rows(const void *xrows, int dtype, int64_t R, int d, int ffn,
                                     const int32_t *expert_of_row, int G, const void *w13,
                                     const void *w2, const double *dyrows, double *dx,
                                     double *gu, double *dgu, double *dw13, double *dw2)
{
    double *h = malloc(sizeof(double) * (size_t)(R > 0 ? R : 1) * ffn);
    double *dg = malloc(sizeof(double) * (size_t)(R > 0 ? R : 1) * ffn);
    double *du = malloc(sizeof(double) * (size_t)(R > 0 ? R : 1) * ffn);
#pragma omp parallel
    {
        double *xv = malloc(sizeof(double) * (size_t)d);
        double *g = malloc(sizeof(double) * (size_t)ffn);
        double *u = malloc(sizeof(double) * (size_t)ffn);
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < R; ++r) {
            const int64_t e = expert_of_row[r];
            const int64_t gate0 = e * 2 * ffn * d, up0 = gate0 + (int64_t)ffn * d;
            const int64_t down0 = e * d * ffn;
            const double *dyv = dyrows + r * d;
            for (int i = 0; i < d; ++i) xv[i] = widen(xrows, dtype, r * d + i);
            for (int n = 0; n < ffn; ++n) {
                double a = 0.0, b = 0.0;
                for (int i = 0; i < d; ++i) {
                    a += widen(w13, dtype, gate0 + (int64_t)n * d + i) * xv[i];
                    b += widen(w13, dtype, up0 + (int64_t)n * d + i) * xv[i];
                }
                g[n] = a;
                u[n] = b;
            }
            for (int n = 0; n < ffn; ++n) {
                double dh = 0.0;
                for (int m = 0; m < d; ++m)
                    dh += widen(w2, dtype, down0 + (int64_t)m * ffn + n) * dyv[m];
                const double s = 1.0 / (1.0 + exp(-g[n]));
                const double silu = g[n] * s;
                const double dsilu = s * (1.0 + g[n] * (1.0 - s));
                h[r * ffn + n] = silu * u[n];
                dg[r * ffn + n] = dh * u[n] * dsilu;
                du[r * ffn + n] = dh * silu;
            }
            if (gu)
                for (int n = 0; n < ffn; ++n) {
                    gu[r * 2 * ffn + n] = g[n];
                    gu[r * 2 * ffn + ffn + n] = u[n];
                }
            if (dgu)
                for (int n = 0; n < ffn; ++n) {
                    dgu[r * 2 * ffn + n] = dg[r * ffn + n];
                    dgu[r * 2 * ffn + ffn + n] = du[r * ffn + n];
                }
            if (dx) {
                for (int i = 0; i < d; ++i) {
                    double acc = 0.0;
                    for (int n = 0; n < ffn; ++n)
                        acc += widen(w13, dtype, gate0 + (int64_t)n * d + i) * dg[r * ffn + n] +
                               widen(w13, dtype, up0 + (int64_t)n * d + i) * du[r * ffn + n];
                    dx[r * d + i] = acc;
                }
            }
        }
        free(xv); free(g); free(u);
    }
    if (dw2) {
#pragma omp parallel for schedule(dynamic, 4)
        for (int64_t em = 0; em < (int64_t)G * d; ++em) {      /* row m of dW_down,e */
            const int64_t e = em / d, m = em % d;
            double *row = dw2 + em * ffn;
            for (int n = 0; n < ffn; ++n) row[n] = 0.0;
            for (int64_t r = 0; r < R; ++r) {
                if (expert_of_row[r] != e) continue;
                const double a = dyrows[r * d + m];
                for (int n = 0; n < ffn; ++n) row[n] += a * h[r * ffn + n];
            }
        }
    }
    if (dw13) {
#pragma omp parallel for schedule(dynamic, 4)
        for (int64_t en = 0; en < (int64_t)G * 2 * ffn; ++en) { /* row n of dW_gate,e / dW_up,e */
            const int64_t e = en / (2 * ffn), n = en % (2 * ffn);
            const double *src = n < ffn ? dg : du;
            const int64_t nn = n < ffn ? n : n - ffn;
            double *row = dw13 + en * d;
            for (int i = 0; i < d; ++i) row[i] = 0.0;
            for (int64_t r = 0; r < R; ++r) {
                if (expert_of_row[r] != e) continue;
                const double a = src[r * ffn + nn];
                for (int i = 0; i < d; ++i) row[i] += a * widen(xrows, dtype, r * d + i);
            }
        }
    }
    free(h); free(dg); free(du);
}

/* ------------------------------------------------------------------------
 * B4's steps one at a time, each taking the previous step's result as an
 * input (so a stage of an implementation can be fed the same values):
 *
 * B4a  dgu from the output gradient and given pre-activations:
 *        dh = W_down^T dy;  dg = dh u SiLU'(g);  du = dh SiLU(g)
 *      with (g, u) = gu[r] ([R, 2 ffn], gate then up); dgu [R, 2 ffn].
 * B4b  dx = W_gate^T dg + W_up^T du from given (dg, du) = dgu[r]; dx [R, d].
 * B4c  the weight-gradient sum over each expert's rows,
 *        c[e] = sum_{r in e, increasing} a[r]^T b[src(r)]   ([G, m, n]),
 *      src(r) = b_order[r] / b_k, or r when b_order is NULL: dW_down =
 *      B4c(dy, h), dW13 = B4c(dgu, x rows).
 * ---------------------------------------------------------------------- */
void orc_down_backward_rows(const double *dyrows, int64_t R, int d, int ffn,
                            const int32_t *expert_of_row, const void *w2, int dtype,
                            const double *gu, double *dgu)
{
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t r = 0; r < R; ++r) {
        const int64_t down0 = (int64_t)expert_of_row[r] * d * ffn;
        for (int n = 0; n < ffn; ++n) {
            double dh = 0.0;
            for (int m = 0; m < d; ++m)
                dh += widen(w2, dtype, down0 + (int64_t)m * ffn + n) * dyrows[r * d + m];
            const double g = gu[r * 2 * ffn + n], u = gu[r * 2 * ffn + ffn + n];
            const double s = 1.0 / (1.0 + exp(-g));
            dgu[r * 2 * ffn + n] = dh * u * (s * (1.0 + g * (1.0 - s)));
            dgu[r * 2 * ffn + ffn + n] = dh * (g * s);
        }
    }
}

void orc_gate_up_backward_rows(const double *dgu, int64_t R, int d, int ffn,
                               const int32_t *expert_of_row, const void *w13, int dtype,
                               double *dx)
{
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t r = 0; r < R; ++r) {
        const int64_t gate0 = (int64_t)expert_of_row[r] * 2 * ffn * d, up0 = gate0 + (int64_t)ffn * d;
        for (int i = 0; i < d; ++i) {
            double acc = 0.0;
            for (int n = 0; n < ffn; ++n)
                acc += widen(w13, dtype, gate0 + (int64_t)n * d + i) * dgu[r * 2 * ffn + n] +
                       widen(w13, dtype, up0 + (int64_t)n * d + i) * dgu[r * 2 * ffn + ffn + n];
            dx[r * d + i] = acc;
        }
    }
}

void orc_weight_grad(const double *a, int64_t R, int m, const double *b, int n,
                     const int32_t *offsets, int G, const int32_t *b_order, int b_k, double *c)
{
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t ei = 0; ei < (int64_t)G * m; ++ei) {
        const int64_t e = ei / m, i = ei % m;
        double *row = c + ei * n;
        for (int j = 0; j < n; ++j) row[j] = 0.0;
        int64_t lo = offsets[e], hi = offsets[e + 1];
        if (lo < 0) lo = 0;
        if (hi > R) hi = R;
        for (int64_t r = lo; r < hi; ++r) {
            const int64_t src = b_order ? b_order[r] / b_k : r;
            const double ar = a[r * m + i];
            for (int j = 0; j < n; ++j) row[j] += ar * b[src * n + j];
        }
    }
}

/* ------------------------------------------------------------------------
 * B1  Backward of the gates (O1, the gate formulas).  The choice of experts
 * is piecewise constant in the logits and the bias of auxiliary-loss-free
 * balancing is outside the gradient ("05 - Expert Parallelism (MoE)",
 * section "Load balancing", family (b)), so the gradient reaches the logits
 * through the gate formulas only.  With c_j the chosen experts and dw the
 * gradient at the gates:
 *   softmax, renormalised:  p_j = w_j;  dl[c_j] = p_j (dw_j - sum_i p_i dw_i)
 *   softmax, not renorm.:   P = softmax over all E;
 *                           dl[e] = P_e ([e = c_j] dw_j - sum_i P_{c_i} dw_i)
 *   sigmoid, renormalised:  s_j = s(l_{c_j}), S = sum s_j, w_j = s_j / S;
 *                           dl[c_j] = s_j (1 - s_j) (dw_j - sum_i w_i dw_i) / S
 *   sigmoid, not renorm.:   dl[c_j] = s_j (1 - s_j) dw_j
 * All other entries are 0.  dlogits is [T, E], overwritten.
 * Returns 0, or -1 on arguments outside the contract.
 * ---------------------------------------------------------------------- */
int orc_gate_backward(const float *logits, int T, int E, int k, const int32_t *ids, int gating,
                      int renorm, const double *dw, double *dlogits)
{
    if (T < 0 || E < 1 || k < 1 || k > E || k > 64) return -1;
#pragma omp parallel
    {
        double *P = malloc(sizeof(double) * (size_t)E);
#pragma omp for schedule(static)
        for (int t = 0; t < T; ++t) {
            const float *l = logits + (int64_t)t * E;
            const int32_t *c = ids + (int64_t)t * k;
            const double *g = dw + (int64_t)t * k;
            double *out = dlogits + (int64_t)t * E;
            for (int e = 0; e < E; ++e) out[e] = 0.0;
            double v[64], sum = 0.0, dot = 0.0;
            if (gating == ORC_SOFTMAX && renorm) {
                const double l0 = (double)l[c[0]];
                for (int j = 0; j < k; ++j) { v[j] = exp((double)l[c[j]] - l0); sum += v[j]; }
                for (int j = 0; j < k; ++j) { v[j] /= sum; dot += v[j] * g[j]; }
                for (int j = 0; j < k; ++j) out[c[j]] = v[j] * (g[j] - dot);
            } else if (gating == ORC_SOFTMAX) {
                double m = (double)l[0];
                for (int e = 1; e < E; ++e) if ((double)l[e] > m) m = (double)l[e];
                for (int e = 0; e < E; ++e) { P[e] = exp((double)l[e] - m); sum += P[e]; }
                for (int e = 0; e < E; ++e) P[e] /= sum;
                for (int j = 0; j < k; ++j) dot += P[c[j]] * g[j];
                for (int e = 0; e < E; ++e) out[e] = -P[e] * dot;
                for (int j = 0; j < k; ++j) out[c[j]] += P[c[j]] * g[j];
            } else {
                for (int j = 0; j < k; ++j) { v[j] = 1.0 / (1.0 + exp(-(double)l[c[j]])); sum += v[j]; }
                if (renorm) {
                    for (int j = 0; j < k; ++j) dot += v[j] / sum * g[j];
                    for (int j = 0; j < k; ++j) out[c[j]] = v[j] * (1.0 - v[j]) * (g[j] - dot) / sum;
                } else {
                    for (int j = 0; j < k; ++j) out[c[j]] = v[j] * (1.0 - v[j]) * g[j];
                }
            }
        }
        free(P);
    }
    return 0;
}

/* ------------------------------------------------------------------------
 * B0  Backward of the router product O0, logits = x wg^T:
 *   dx[t][i]  = sum_e dlogits[t][e] wg[e][i]
 *   dwg[e][i] = sum_t dlogits[t][e] x[t][i]
 * Either output may be NULL.
 * ---------------------------------------------------------------------- */
void orc_router_backward(const void *x, int dtype, int64_t T, int d, const void *wg, int E,
                         const double *dlogits, double *dx, double *dwg)
{
    if (dx) {
#pragma omp parallel for schedule(static)
        for (int64_t t = 0; t < T; ++t)
            for (int i = 0; i < d; ++i) {
                double acc = 0.0;
                for (int e = 0; e < E; ++e) acc += dlogits[t * E + e] * widen(wg, dtype, (int64_t)e * d + i);
                dx[t * d + i] = acc;
            }
    }
    if (dwg) {
#pragma omp parallel for schedule(static)
        for (int e = 0; e < E; ++e)
            for (int i = 0; i < d; ++i) {
                double acc = 0.0;
                for (int64_t t = 0; t < T; ++t) acc += dlogits[t * E + e] * widen(x, dtype, t * d + i);
                dwg[(int64_t)e * d + i] = acc;
            }
    }
}

/* Number of OpenMP threads the oracle's parallel loops use. */
#ifdef _OPENMP
#include <omp.h>
int orc_num_threads(void) { return omp_get_max_threads(); }
void orc_set_num_threads(int n) { if (n > 0) omp_set_num_threads(n); }
#else
int orc_num_threads(void) { return 1; }
void orc_set_num_threads(int n) { (void)n; }
#endif
