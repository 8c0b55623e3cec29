/* spec_oracle.c -- plain fp64 CPU oracle of the speculative-decoding verify step.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark, never by the library path.  Slow on purpose:
 * scalar loops in ascending index order, double arithmetic, libm exp, no blocking.
 *
 * Sources (web pages on speculative decoding):
 *   [atlas]   llm-infra-atlas, "Speculative Decoding -- lossless acceleration of
 *             autoregressive decode": section 0 (core idea), section 2 (notation:
 *             bonus token, correction/residual norm(max(0, p - q)), tau counts the bonus).
 *   [ricardo] ricardokevins, "Speculative Decoding: real gains, correction sampling and
 *             production limits": "mechanism" (draft / verify / accept / correct),
 *             "correction sampling" with Eq. a(x) = min(1, p(x)/q(x)) and
 *             Eq. r(x) = max(p(x) - q(x), 0) / sum_y max(p(y) - q(y), 0).
 *   [origins] zdszero, "spec_origins": "Blockwise Parallel Decoding" (verify: accept the
 *             longest prefix that equals the scorer's argmax, always advance >= 1 token),
 *             "Speculative Decoding" -> acceptance rule items 1-3 (accept with prob
 *             min(1, p/q); on rejection resample from norm(max(0, p - q)) and stop; if
 *             all gamma accepted draw a bonus from position gamma+1), "in SGLang"
 *             (target-only tree walk: per level, accumulate sibling target probabilities
 *             prob_acc, accept when coin <= prob_acc / threshold_acc or a single
 *             probability >= threshold_single; rejected children are removed from the
 *             final distribution relu(target - draft_probs)).
 *
 * Readings where the pages are silent (each one is also taken by the HIP library):
 *   - p = softmax(logits / T) with the row maximum subtracted; q arrives as fp32
 *     probabilities at T and is used as given.
 *   - coins lie in (0, 1]; every comparison is "coin <= threshold"; a token with p = 0 is
 *     never accepted.
 *   - the correction / bonus / final draw uses its own coin (chain: coins[G],
 *     tree: coins[D]); the draw is the inverse CDF in ascending token id: the first j
 *     with w_j > 0 and u * S <= C_j, C_j the inclusive prefix sum of w.
 *   - if the residual mass S is not positive the draw falls back to w = p of that row.
 *   - greedy argmax ties go to the lowest token id.
 *   - tree: node 0 is the root, parents[i] < i, siblings are tried in ascending node id,
 *     one coin per level coins[d] and a final coin coins[D]; a leaf draws its bonus
 *     from its own row.
 *   - a request is invalid when something the verify consults is unusable: chains and
 *     trees are walked in order and stop at the first rejection, so rows (and drafts,
 *     q values, per-position coins) beyond the stop are not checked.
 */
#include "spec_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- reading the inputs ------------------------------------------------------- */

typedef struct {
    const void* base;
    int dtype;
    size_t offset; /* element offset of the row start */
    int V;
} Row;

static Row row_of(const void* logits, int dtype, size_t row_index, int V) {
    Row r;
    r.base = logits;
    r.dtype = dtype;
    r.offset = row_index * (size_t)V;
    r.V = V;
    return r;
}

/* One logit, widened exactly to double (a bf16 value is the high half of an fp32). */
static double logit(Row r, int x) {
    size_t i = r.offset + (size_t)x;
    if (r.dtype == ORACLE_F32) return (double)((const float*)r.base)[i];
    uint32_t bits = (uint32_t)((const uint16_t*)r.base)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static double row_max(Row r) {
    double m = -INFINITY;
    for (int x = 0; x < r.V; ++x)
        if (logit(r, x) > m) m = logit(r, x);
    return m;
}

/* Lowest token id attaining the row maximum (greedy reading: ties -> lowest id). */
static int row_argmax(Row r) {
    int best = 0;
    for (int x = 1; x < r.V; ++x)
        if (logit(r, x) > logit(r, best)) best = x;
    return best;
}

/* Normaliser of the temperature softmax, Z = sum_x exp((l_x - m) / T). */
static double row_partition(Row r, double m, double T) {
    double Z = 0.0;
    for (int x = 0; x < r.V; ++x) Z += exp((logit(r, x) - m) / T);
    return Z;
}

/* Target probability p(x) = exp((l_x - m) / T) / Z. */
static double row_prob(Row r, int x, double m, double Z, double T) {
    return exp((logit(r, x) - m) / T) / Z;
}

static void note_margin(double* mm, double margin) {
    if (margin < *mm) *mm = margin;
}

static int coin_ok(float u) { return u > 0.0f && u <= 1.0f; }

static int temperature_ok(float T) { return isfinite(T) && T > 0.0f; }

/* ---- the final draw --------------------------------------------------------------
 * Inverse CDF over w (probability units): t = u * S, the first token with positive weight
 * whose inclusive prefix reaches t.  The distances of t to both ends of the chosen bucket
 * are recorded as margins.  If rounding left t beyond the last bucket the last token with
 * positive weight is returned and a zero margin recorded. */
static int draw_inverse_cdf(const double* w, int V, double u, double* mm) {
    double S = 0.0;
    for (int j = 0; j < V; ++j) S += w[j];
    double t = u * S;
    double C = 0.0;
    int last = -1;
    for (int j = 0; j < V; ++j) {
        if (w[j] > 0.0) {
            double before = C;
            C += w[j];
            last = j;
            if (t <= C) {
                note_margin(mm, t - before);
                note_margin(mm, C - t);
                return j;
            }
        }
    }
    note_margin(mm, 0.0);
    return last;
}

/* ---- greedy chain ------------------------------------------------------------------
 * [origins] Blockwise Parallel Decoding, verify: the scorer checks the k proposals in
 * parallel and keeps the longest prefix that agrees with its own argmax, so every step
 * advances by at least one token and the result equals token-by-token greedy decoding.
 * The token emitted after the prefix is the scorer's argmax at the first mismatch (or
 * at position G+1 when every proposal matched). */
static void greedy_one(const void* logits, int dtype, const int32_t* draft, int G, int V,
                       size_t b, int32_t* accept_len, int32_t* out) {
    int R = G + 1;
    int valid = 1, k = G, a = -1;
    for (int i = 0; i <= G; ++i) { /* positions in order, up to the first mismatch */
        Row r = row_of(logits, dtype, b * (size_t)R + (size_t)i, V);
        if (row_max(r) == -INFINITY) { /* a row the verify consults has no finite logit */
            valid = 0;
            break;
        }
        a = row_argmax(r);
        if (i == G) break;
        if (draft[i] < 0 || draft[i] >= V) {
            valid = 0;
            break;
        }
        if (draft[i] != a) {
            k = i;
            break;
        }
    }
    if (!valid) {
        *accept_len = -1;
        for (int i = 0; i < R; ++i) out[i] = -1;
        return;
    }
    for (int i = 0; i < k; ++i) out[i] = draft[i];
    out[k] = a;
    for (int i = k + 1; i < R; ++i) out[i] = -1;
    *accept_len = k;
}

int oracle_verify_greedy(const void* logits, int dtype, const int32_t* draft_tokens,
                         int B, int G, int V, int32_t* accept_len, int32_t* out_tokens) {
    if (!logits || !draft_tokens || !accept_len || !out_tokens) return -1;
    if (B < 0 || G < 1 || V < 1 || (dtype != ORACLE_F32 && dtype != ORACLE_BF16)) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < B; ++b)
        greedy_one(logits, dtype, draft_tokens + (size_t)b * G, G, V, (size_t)b,
                   accept_len + b, out_tokens + (size_t)b * (G + 1));
    return 0;
}

/* ---- chain rejection sampling --------------------------------------------------------
 * [origins] acceptance rule: (1) accept x ~ q with probability min(1, p(x)/q(x));
 * (2) at the first rejection resample from p' = norm(max(0, p - q)) and stop;
 * (3) when all gamma drafts are accepted, draw a bonus token from position gamma+1.
 * [ricardo] correction sampling: Eq. a(x) and Eq. r(x) state the same two steps.
 * With coin u_i the test "accept with probability min(1, p/q)" reads u_i <= p/q. */
static void chain_one(const void* logits, int dtype, const float* q, const int32_t* draft,
                      const float* coins, float temperature, int G, int V, size_t b,
                      int32_t* accept_len, int32_t* out, double* probs, double* margin,
                      double* amargin, double* beta, double* w) {
    int R = G + 1;
    double T = (double)temperature;
    double m[R > 0 ? R : 1], Z[R > 0 ? R : 1];
    /* Positions are consulted in order up to the first rejection (or the bonus row): only
     * what is consulted must be usable -- its row, draft token, q(token) and coin -- plus
     * the temperature and the final coin. */
    int valid = temperature_ok(temperature) && coin_ok(coins[G]);
    int k = G;
    double pacc[R > 0 ? R : 1];
    *margin = INFINITY;
    if (amargin) *amargin = INFINITY;
    for (int i = 0; i <= G && valid; ++i) {
        Row r = row_of(logits, dtype, b * (size_t)R + (size_t)i, V);
        m[i] = row_max(r);
        if (m[i] == -INFINITY) {
            valid = 0;
            break;
        }
        Z[i] = row_partition(r, m[i], T);
        if (i == G) break;
        int x = draft[i];
        if (x < 0 || x >= V || !coin_ok(coins[i])) {
            valid = 0;
            break;
        }
        float qf = q[(size_t)i * V + (size_t)x];
        if (!(qf >= 0.0f) || !isfinite(qf)) {
            valid = 0;
            break;
        }
        double p = row_prob(r, x, m[i], Z[i], T);
        double qx = (double)qf;
        double u = (double)coins[i];
        int accept;
        if (qx > 0.0) {
            double ratio = p / qx;
            note_margin(margin, fabs(u - ratio));
            accept = p > 0.0 && u <= ratio;
        } else {
            accept = p > 0.0; /* q(x) = 0 < p(x): ratio is +inf */
        }
        if (!accept) {
            k = i;
            break;
        }
        pacc[i] = p;
    }
    if (!valid) {
        *margin = INFINITY;
        if (amargin) *amargin = INFINITY;
        *accept_len = -1;
        for (int i = 0; i < R; ++i) out[i] = -1;
        if (probs)
            for (int i = 0; i < R; ++i) probs[i] = 0.0;
        if (beta)
            for (int i = 0; i < G; ++i) beta[i] = 0.0;
        return;
    }

    if (beta) { /* beta_i = sum_x min(p_i(x), q_i(x)): per-position acceptance rate
                 * (a diagnostic over every position; 0 where a row has no finite logit) */
        for (int i = 0; i < G; ++i) {
            Row r = row_of(logits, dtype, b * (size_t)R + (size_t)i, V);
            double mi = row_max(r);
            double s = 0.0;
            if (mi != -INFINITY) {
                double Zi = row_partition(r, mi, T);
                for (int x = 0; x < V; ++x) {
                    double p = row_prob(r, x, mi, Zi, T);
                    double qq = (double)q[(size_t)i * V + (size_t)x];
                    s += p < qq ? p : qq;
                }
            }
            beta[i] = s;
        }
    }

    /* Weights of the final draw: residual max(0, p_k - q_k) after a rejection, the
     * target row G itself for the bonus. */
    Row rk = row_of(logits, dtype, b * (size_t)R + (size_t)k, V);
    double S = 0.0;
    for (int x = 0; x < V; ++x) {
        double p = row_prob(rk, x, m[k], Z[k], T);
        if (k < G) {
            double d = p - (double)q[(size_t)k * V + (size_t)x];
            w[x] = d > 0.0 ? d : 0.0;
        } else {
            w[x] = p;
        }
        S += w[x];
    }
    if (k < G) note_margin(margin, S);
    if (amargin) *amargin = *margin; /* every margin so far: the tests before the draw */
    if (!(S > 0.0))
        for (int x = 0; x < V; ++x) w[x] = row_prob(rk, x, m[k], Z[k], T);
    int y = draw_inverse_cdf(w, V, (double)coins[G], margin);

    for (int i = 0; i < k; ++i) out[i] = draft[i];
    out[k] = y;
    for (int i = k + 1; i < R; ++i) out[i] = -1;
    *accept_len = k;
    if (probs) {
        for (int i = 0; i < k; ++i) probs[i] = pacc[i];
        probs[k] = row_prob(rk, y, m[k], Z[k], T);
        for (int i = k + 1; i < R; ++i) probs[i] = 0.0;
    }
}

int oracle_verify_chain(const void* logits, int dtype, const float* draft_probs,
                        const int32_t* draft_tokens, const float* coins,
                        const float* temperature, int B, int G, int V,
                        int32_t* accept_len, int32_t* out_tokens, double* probs_out,
                        double* min_margin, double* beta_out, double* accept_margin) {
    if (!logits || !draft_probs || !draft_tokens || !coins || !temperature || !accept_len ||
        !out_tokens || !min_margin)
        return -1;
    if (B < 0 || G < 1 || V < 1 || (dtype != ORACLE_F32 && dtype != ORACLE_BF16)) return -1;
    int R = G + 1;
#pragma omp parallel
    {
        double* w = (double*)malloc(sizeof(double) * (size_t)V);
#pragma omp for schedule(dynamic, 1)
        for (int b = 0; b < B; ++b)
            chain_one(logits, dtype, draft_probs + (size_t)b * G * V, draft_tokens + (size_t)b * G,
                      coins + (size_t)b * R, temperature[b], G, V, (size_t)b, accept_len + b,
                      out_tokens + (size_t)b * R, probs_out ? probs_out + (size_t)b * R : NULL,
                      min_margin + b, accept_margin ? accept_margin + b : NULL,
                      beta_out ? beta_out + (size_t)b * G : NULL, w);
        free(w);
    }
    return 0;
}

/* ---- token tree, target only ----------------------------------------------------------
 * [origins] "in SGLang": walk down the tree; at each level add up the target
 * probabilities of the siblings tried so far (prob_acc) and accept a child when
 * coin <= prob_acc / threshold_acc or its own probability >= threshold_single (both
 * thresholds 1.0 by default, which amounts to drawing one child from the target
 * distribution and checking whether it is on the tree).  A rejected child's target
 * probability is written into draft_probs, and the final token is drawn from
 * relu(target - draft_probs): the children tried and rejected at the last level are
 * removed.  At a leaf nothing was rejected and the draw is from the leaf's own row.
 * [origins] SpecInfer: the tree is flattened, each node sees only its ancestors; here the
 * ancestry is the parent array and row j holds the target distribution after node j.
 * Greedy mode follows the child whose token equals the argmax of the current row. */
static void tree_one(const void* logits, int dtype, const int32_t* tok, const int32_t* par,
                     const float* coins, float temperature, int N, int V, int D, int mode,
                     double th_single, double th_acc, size_t b, int32_t* accept_len,
                     int32_t* out, int32_t* nodes, double* probs, double* margin,
                     double* amargin, double* w, int* depth, int32_t* excl) {
    int sampling = mode == ORACLE_TREE_SAMPLING;
    int valid = par[0] == -1;
    depth[0] = 0;
    for (int i = 1; i < N && valid; ++i) {
        if (par[i] < 0 || par[i] >= i) {
            valid = 0;
            break;
        }
        depth[i] = depth[par[i]] + 1;
        if (depth[i] > D) valid = 0;
        if (tok[i] < 0 || tok[i] >= V) valid = 0;
    }
    if (sampling) {
        if (!temperature_ok(temperature)) valid = 0;
        for (int d = 0; d <= D; ++d)
            if (!coin_ok(coins[d])) valid = 0;
    }
    *margin = INFINITY;
    if (amargin) *amargin = INFINITY;

    double T = (double)temperature;
    int cur = 0, d = 0, nexcl = 0;
    for (; valid;) {
        Row r = row_of(logits, dtype, b * (size_t)N + (size_t)cur, V);
        if (row_max(r) == -INFINITY) { /* a row the walk reaches has no finite logit */
            valid = 0;
            break;
        }
        int any_child = 0;
        for (int c = cur + 1; c < N; ++c)
            if (par[c] == cur) any_child = 1;
        if (!any_child) break; /* leaf: bonus from its own row */
        int chosen = -1;
        double pchosen = 0.0;
        if (!sampling) {
            int a = row_argmax(r);
            for (int c = cur + 1; c < N; ++c)
                if (par[c] == cur && tok[c] == a) {
                    chosen = c;
                    break;
                }
        } else {
            double m = row_max(r), Z = row_partition(r, m, T);
            double u = (double)coins[d];
            double acc = 0.0;
            nexcl = 0;
            for (int c = cur + 1; c < N; ++c) {
                if (par[c] != cur) continue;
                double pc = row_prob(r, tok[c], m, Z, T);
                acc += pc;
                note_margin(margin, fabs(u - acc / th_acc));
                note_margin(margin, fabs(pc - th_single));
                if (u <= acc / th_acc || pc >= th_single) {
                    chosen = c;
                    pchosen = pc;
                    break;
                }
                excl[nexcl++] = tok[c];
            }
        }
        if (chosen < 0) break;
        out[d] = tok[chosen];
        nodes[d] = chosen;
        if (probs) probs[d] = pchosen;
        cur = chosen;
        ++d;
        nexcl = 0;
    }
    if (!valid) {
        *margin = INFINITY;
        *accept_len = -1;
        for (int e = 0; e <= D; ++e) out[e] = -1;
        for (int e = 0; e < D; ++e) nodes[e] = -1;
        if (probs)
            for (int e = 0; e <= D; ++e) probs[e] = 0.0;
        return;
    }

    Row r = row_of(logits, dtype, b * (size_t)N + (size_t)cur, V);
    int y;
    double py = 0.0;
    if (!sampling) {
        y = row_argmax(r);
    } else {
        double m = row_max(r), Z = row_partition(r, m, T);
        double S = 0.0;
        for (int x = 0; x < V; ++x) w[x] = row_prob(r, x, m, Z, T);
        for (int e = 0; e < nexcl; ++e) w[excl[e]] = 0.0;
        for (int x = 0; x < V; ++x) S += w[x];
        if (nexcl > 0) note_margin(margin, S);
        if (amargin) *amargin = *margin; /* every margin so far: the tests before the draw */
        if (!(S > 0.0))
            for (int x = 0; x < V; ++x) w[x] = row_prob(r, x, m, Z, T);
        y = draw_inverse_cdf(w, V, (double)coins[D], margin);
        py = row_prob(r, y, m, Z, T);
    }
    out[d] = y;
    if (probs) probs[d] = py;
    for (int e = d + 1; e <= D; ++e) out[e] = -1;
    for (int e = d; e < D; ++e) nodes[e] = -1;
    if (probs)
        for (int e = d + 1; e <= D; ++e) probs[e] = 0.0;
    *accept_len = d;
}

int oracle_verify_tree(const void* logits, int dtype, const int32_t* node_tokens,
                       const int32_t* parents, const float* coins, const float* temperature,
                       int B, int N, int V, int D, int mode, float threshold_single,
                       float threshold_acc, int32_t* accept_len, int32_t* out_tokens,
                       int32_t* accepted_nodes, double* probs_out, double* min_margin,
                       double* accept_margin) {
    if (!logits || !node_tokens || !parents || !accept_len || !out_tokens || !accepted_nodes ||
        !min_margin)
        return -1;
    if (B < 0 || N < 1 || V < 1 || D < 1 || (dtype != ORACLE_F32 && dtype != ORACLE_BF16)) return -1;
    if (mode != ORACLE_TREE_GREEDY && mode != ORACLE_TREE_SAMPLING) return -1;
    if (mode == ORACLE_TREE_SAMPLING &&
        (!coins || !temperature || !(threshold_single > 0.0f) || !(threshold_acc > 0.0f)))
        return -1;
#pragma omp parallel
    {
        double* w = (double*)malloc(sizeof(double) * (size_t)V);
        int* depth = (int*)malloc(sizeof(int) * (size_t)N);
        int32_t* excl = (int32_t*)malloc(sizeof(int32_t) * (size_t)N);
#pragma omp for schedule(dynamic, 1)
        for (int b = 0; b < B; ++b)
            tree_one(logits, dtype, node_tokens + (size_t)b * N, parents + (size_t)b * N,
                     coins ? coins + (size_t)b * (D + 1) : NULL,
                     temperature ? temperature[b] : 1.0f, N, V, D, mode,
                     (double)threshold_single, (double)threshold_acc, (size_t)b,
                     accept_len + b, out_tokens + (size_t)b * (D + 1),
                     accepted_nodes + (size_t)b * D,
                     probs_out ? probs_out + (size_t)b * (D + 1) : NULL, min_margin + b,
                     accept_margin ? accept_margin + b : NULL, w, depth, excl);
        free(w);
        free(depth);
        free(excl);
    }
    return 0;
}

/* ---- token tree, multi-step speculative sampling with draft distributions ---------
 * [origins] SpecInfer, multi-step speculative sampling (MSS): the children of a node are
 * tested one after another with the rule min(1, p(x)/q(x)); when a child is rejected the
 * target distribution of that node is replaced by the residual norm(max(0, p - q)) and
 * the next sibling is tested against the updated distribution; once every child has been
 * rejected the token is drawn from the last updated distribution.  An accepted child
 * becomes the next node, with its own target row and draft row.
 * Readings: draft_probs row j is the distribution the children of node j were drawn
 * from (shared by all of them; used as given, as in the chain); the siblings are tried in
 * ascending node id; node c is tested with coins[c - 1] and the final draw uses
 * coins[N - 1]; if the updated distribution has no positive mass the remaining siblings
 * are not tested and the final token is drawn from the node's target row; a request is
 * invalid when a row the walk reaches has no finite logit (rows off the walk are never
 * read, so they are not checked).  The output
 * follows the target law when the children of each node are independent draws from
 * that node's draft row. */
static void tree_mss_one(const void* logits, int dtype, const float* q, const int32_t* tok,
                         const int32_t* par, const float* coins, float temperature, int N,
                         int V, int D, size_t b, int32_t* accept_len, int32_t* out,
                         int32_t* nodes, double* probs, double* margin, double* amargin,
                         double* w, int* depth) {
    int valid = par[0] == -1 && temperature_ok(temperature);
    depth[0] = 0;
    for (int i = 1; i < N && valid; ++i) {
        if (par[i] < 0 || par[i] >= i) {
            valid = 0;
            break;
        }
        depth[i] = depth[par[i]] + 1;
        if (depth[i] > D) valid = 0;
        if (tok[i] < 0 || tok[i] >= V) {
            valid = 0;
            break;
        }
        float qx = q[(size_t)par[i] * V + (size_t)tok[i]];
        if (!(qx >= 0.0f) || !isfinite(qx)) valid = 0;
    }
    for (int c = 0; c < N && valid; ++c)
        if (!coin_ok(coins[c])) valid = 0;
    *margin = INFINITY;
    if (amargin) *amargin = INFINITY;

    double T = (double)temperature;
    int cur = 0, d = 0;
    double m = 0.0, Z = 0.0;
    for (; valid;) {
        Row r = row_of(logits, dtype, b * (size_t)N + (size_t)cur, V);
        const float* qc = q + (size_t)cur * V;
        m = row_max(r);
        if (m == -INFINITY) { /* a row the walk reaches has no finite logit */
            valid = 0;
            break;
        }
        Z = row_partition(r, m, T);
        for (int x = 0; x < V; ++x) w[x] = row_prob(r, x, m, Z, T); /* current distribution */
        int chosen = -1;
        for (int c = cur + 1; c < N; ++c) {
            if (par[c] != cur) continue;
            int x = tok[c];
            double qx = (double)qc[x];
            double u = (double)coins[c - 1];
            int accept;
            if (qx > 0.0) {
                double ratio = w[x] / qx;
                note_margin(margin, fabs(u - ratio));
                accept = w[x] > 0.0 && u <= ratio;
            } else {
                accept = w[x] > 0.0;
            }
            if (accept) {
                chosen = c;
                break;
            }
            /* rejected: the distribution becomes norm(max(0, w - q)) */
            double S = 0.0;
            for (int v = 0; v < V; ++v) {
                double dv = w[v] - (double)qc[v];
                w[v] = dv > 0.0 ? dv : 0.0;
                S += w[v];
            }
            note_margin(margin, S);
            if (!(S > 0.0)) { /* no residual mass left: draw from the target row */
                for (int v = 0; v < V; ++v) w[v] = row_prob(r, v, m, Z, T);
                break;
            }
            for (int v = 0; v < V; ++v) w[v] /= S;
        }
        if (chosen < 0) break; /* a leaf, or every child rejected: final draw from w */
        out[d] = tok[chosen];
        nodes[d] = chosen;
        if (probs) probs[d] = row_prob(r, tok[chosen], m, Z, T);
        cur = chosen;
        ++d;
    }
    if (!valid) {
        *accept_len = -1;
        for (int e = 0; e <= D; ++e) out[e] = -1;
        for (int e = 0; e < D; ++e) nodes[e] = -1;
        if (probs)
            for (int e = 0; e <= D; ++e) probs[e] = 0.0;
        return;
    }

    Row r = row_of(logits, dtype, b * (size_t)N + (size_t)cur, V);
    if (amargin) *amargin = *margin; /* every margin so far: the tests before the draw */
    int y = draw_inverse_cdf(w, V, (double)coins[N - 1], margin);
    out[d] = y;
    if (probs) probs[d] = row_prob(r, y, m, Z, T);
    for (int e = d + 1; e <= D; ++e) out[e] = -1;
    for (int e = d; e < D; ++e) nodes[e] = -1;
    if (probs)
        for (int e = d + 1; e <= D; ++e) probs[e] = 0.0;
    *accept_len = d;
}

int oracle_verify_tree_mss(const void* logits, int dtype, const float* draft_probs,
                           const int32_t* node_tokens, const int32_t* parents,
                           const float* coins, const float* temperature, int B, int N, int V,
                           int D, int32_t* accept_len, int32_t* out_tokens,
                           int32_t* accepted_nodes, double* probs_out, double* min_margin,
                           double* accept_margin) {
    if (!logits || !draft_probs || !node_tokens || !parents || !coins || !temperature ||
        !accept_len || !out_tokens || !accepted_nodes || !min_margin)
        return -1;
    if (B < 0 || N < 1 || V < 1 || D < 1 || (dtype != ORACLE_F32 && dtype != ORACLE_BF16)) return -1;
#pragma omp parallel
    {
        double* w = (double*)malloc(sizeof(double) * (size_t)V);
        int* depth = (int*)malloc(sizeof(int) * (size_t)N);
#pragma omp for schedule(dynamic, 1)
        for (int b = 0; b < B; ++b)
            tree_mss_one(logits, dtype, draft_probs + (size_t)b * N * V,
                         node_tokens + (size_t)b * N, parents + (size_t)b * N,
                         coins + (size_t)b * N, temperature[b], N, V, D, (size_t)b,
                         accept_len + b, out_tokens + (size_t)b * (D + 1),
                         accepted_nodes + (size_t)b * D,
                         probs_out ? probs_out + (size_t)b * (D + 1) : NULL, min_margin + b,
                         accept_margin ? accept_margin + b : NULL, w, depth);
        free(w);
        free(depth);
    }
    return 0;
}

/* ---- chain rejection sampling from logits, with top-k / top-p filtering ------------
 * [ricardo] mechanism: serving samples with temperature, top-p, top-k and the like, so
 * "accept if it matches the target's top-1" is not unbiased sampling; correction
 * sampling keeps the law only when the acceptance test and the residual use the
 * distributions the drafter and the target actually sample from.
 * Readings: both rows are filtered the same way before the acceptance rule.
 *   p = softmax(l / T) from the target logits, q = softmax(d / T) from the draft logits;
 *   top-k (0 < k < V): keep the tokens whose logit is at least the k-th largest (ties
 *   kept); top-p (0 < top_p < 1), on the top-k-filtered row: sorted by probability, the
 *   shortest head whose mass reaches top_p of the kept mass ends at probability tau;
 *   keep every token with probability >= tau (ties kept); then renormalise.
 * The acceptance rule, the residual and the bonus then run on the filtered rows exactly
 * as in the unfiltered chain.  The top-p boundary (the kept-mass fraction before and
 * after the threshold group, against top_p) is recorded as a margin. */
static int cmp_desc(const void* a, const void* b) {
    double x = *(const double*)a, y = *(const double*)b;
    return x < y ? 1 : (x > y ? -1 : 0);
}

/* w[x] = exp((l_x - m) / T) for the kept tokens, 0 for the others; returns the kept
 * mass.  tmp has room for V doubles. */
static double filter_row(Row r, double m, double T, int top_k, double top_p, double* w,
                         double* tmp, double* margin) {
    int V = r.V;
    for (int x = 0; x < V; ++x) w[x] = exp((logit(r, x) - m) / T);
    if (top_k > 0 && top_k < V) {
        for (int x = 0; x < V; ++x) tmp[x] = logit(r, x);
        qsort(tmp, (size_t)V, sizeof(double), cmp_desc);
        double th = tmp[top_k - 1];
        for (int x = 0; x < V; ++x)
            if (logit(r, x) < th) w[x] = 0.0;
    }
    double S = 0.0;
    for (int x = 0; x < V; ++x) S += w[x];
    if (top_p < 1.0) {
        for (int x = 0; x < V; ++x) tmp[x] = w[x];
        qsort(tmp, (size_t)V, sizeof(double), cmp_desc);
        double target = top_p * S, cum = 0.0, tau = tmp[0];
        for (int i = 0; i < V; ++i) {
            if (cum + tmp[i] >= target) {
                tau = tmp[i];
                break;
            }
            cum += tmp[i];
        }
        double before = 0.0, through = 0.0;
        for (int i = 0; i < V; ++i) {
            if (tmp[i] > tau) before += tmp[i];
            if (tmp[i] >= tau) through += tmp[i];
        }
        note_margin(margin, (target - before) / S);
        note_margin(margin, (through - target) / S);
        for (int x = 0; x < V; ++x)
            if (w[x] < tau) w[x] = 0.0;
        S = through;
    }
    return S;
}

static void chain_filtered_one(const void* logits, const void* dlogits, int dtype,
                               const int32_t* draft, const float* coins, float temperature,
                               int top_k, float top_p, int G, int V, size_t b,
                               int32_t* accept_len, int32_t* out, double* probs,
                               double* margin, double* amargin, double* wp, double* wq,
                               double* tmp) {
    int R = G + 1;
    double T = (double)temperature;
    double tp = (double)top_p;
    int valid = temperature_ok(temperature) && top_p > 0.0f && !isnan(top_p);
    for (int i = 0; i < G; ++i)
        if (draft[i] < 0 || draft[i] >= V) valid = 0;
    for (int i = 0; i < R; ++i)
        if (!coin_ok(coins[i])) valid = 0;
    double m[R > 0 ? R : 1], mq[R > 0 ? R : 1];
    for (int i = 0; i < R && valid; ++i) {
        m[i] = row_max(row_of(logits, dtype, b * (size_t)R + (size_t)i, V));
        if (m[i] == -INFINITY) valid = 0;
    }
    for (int i = 0; i < G && valid; ++i) {
        mq[i] = row_max(row_of(dlogits, dtype, b * (size_t)G + (size_t)i, V));
        if (mq[i] == -INFINITY) valid = 0;
    }
    *margin = INFINITY;
    if (amargin) *amargin = INFINITY;
    if (!valid) {
        *accept_len = -1;
        for (int i = 0; i < R; ++i) out[i] = -1;
        if (probs)
            for (int i = 0; i < R; ++i) probs[i] = 0.0;
        return;
    }
    int k = G;
    double pacc[R > 0 ? R : 1];
    for (int i = 0; i < G; ++i) {
        Row r = row_of(logits, dtype, b * (size_t)R + (size_t)i, V);
        Row rq = row_of(dlogits, dtype, b * (size_t)G + (size_t)i, V);
        double Zp = filter_row(r, m[i], T, top_k, tp, wp, tmp, margin);
        double Zq = filter_row(rq, mq[i], T, top_k, tp, wq, tmp, margin);
        int x = draft[i];
        double p = wp[x] / Zp, qx = wq[x] / Zq;
        double u = (double)coins[i];
        int accept;
        if (qx > 0.0) {
            double ratio = p / qx;
            note_margin(margin, fabs(u - ratio));
            accept = p > 0.0 && u <= ratio;
        } else {
            accept = p > 0.0;
        }
        if (!accept) {
            k = i;
            break;
        }
        pacc[i] = p;
    }
    Row rk = row_of(logits, dtype, b * (size_t)R + (size_t)k, V);
    double Zp = filter_row(rk, m[k], T, top_k, tp, wp, tmp, margin);
    for (int x = 0; x < V; ++x) wp[x] /= Zp;
    double S = 0.0;
    if (k < G) {
        Row rq = row_of(dlogits, dtype, b * (size_t)G + (size_t)k, V);
        double Zq = filter_row(rq, mq[k], T, top_k, tp, wq, tmp, margin);
        for (int x = 0; x < V; ++x) {
            double d = wp[x] - wq[x] / Zq;
            wq[x] = d > 0.0 ? d : 0.0;
            S += wq[x];
        }
        note_margin(margin, S);
    }
    if (amargin) *amargin = *margin; /* every margin so far: the tests before the draw */
    double* w = (k < G && S > 0.0) ? wq : wp;
    int y = draw_inverse_cdf(w, V, (double)coins[G], margin);
    for (int i = 0; i < k; ++i) out[i] = draft[i];
    out[k] = y;
    for (int i = k + 1; i < R; ++i) out[i] = -1;
    *accept_len = k;
    if (probs) {
        for (int i = 0; i < k; ++i) probs[i] = pacc[i];
        probs[k] = wp[y];
        for (int i = k + 1; i < R; ++i) probs[i] = 0.0;
    }
}

int oracle_verify_chain_filtered(const void* logits, const void* draft_logits, int dtype,
                                 const int32_t* draft_tokens, const float* coins,
                                 const float* temperature, const int32_t* top_k,
                                 const float* top_p, int B, int G, int V, int32_t* accept_len,
                                 int32_t* out_tokens, double* probs_out, double* min_margin,
                                 double* accept_margin) {
    if (!logits || !draft_logits || !draft_tokens || !coins || !temperature || !accept_len ||
        !out_tokens || !min_margin)
        return -1;
    if (B < 0 || G < 1 || V < 1 || (dtype != ORACLE_F32 && dtype != ORACLE_BF16)) return -1;
    int R = G + 1;
#pragma omp parallel
    {
        double* wp = (double*)malloc(sizeof(double) * (size_t)V);
        double* wq = (double*)malloc(sizeof(double) * (size_t)V);
        double* tmp = (double*)malloc(sizeof(double) * (size_t)V);
#pragma omp for schedule(dynamic, 1)
        for (int b = 0; b < B; ++b)
            chain_filtered_one(logits, draft_logits, dtype, draft_tokens + (size_t)b * G,
                               coins + (size_t)b * R, temperature[b], top_k ? top_k[b] : 0,
                               top_p ? top_p[b] : 1.0f, G, V, (size_t)b, accept_len + b,
                               out_tokens + (size_t)b * R,
                               probs_out ? probs_out + (size_t)b * R : NULL, min_margin + b,
                               accept_margin ? accept_margin + b : NULL, wp, wq, tmp);
        free(wp);
        free(wq);
        free(tmp);
    }
    return 0;
}

/* ---- tree attention mask and positions ---------------------------------------------
 * [origins] SpecInfer, tree attention mask: the token tree is flattened into one sequence
 * and every node attends only to its ancestors, so one target forward scores every
 * branch and the branches share one KV.  Readings: a node also attends to itself (the
 * diagonal of causal attention); the root (node 0) is the last committed token, and a
 * node's position is the root's position plus its depth.
 * Row i of the mask is the path from node i up to the root: walk the parent pointers
 * from i and set the bit of every node met, i included. */
static void tree_mask_one(const int32_t* par, int32_t base, int N, int W, uint32_t* mask,
                          int32_t* pos) {
    int valid = par[0] == -1;
    for (int i = 1; i < N; ++i)
        if (par[i] < 0 || par[i] >= i) valid = 0;
    for (size_t e = 0; e < (size_t)N * (size_t)W; ++e) mask[e] = 0u;
    for (int i = 0; i < N; ++i) {
        if (!valid) {
            if (pos) pos[i] = -1;
            continue;
        }
        int steps = 0;
        for (int j = i; j >= 0; j = par[j]) {
            mask[(size_t)i * W + (size_t)(j / 32)] |= 1u << (j % 32);
            ++steps;
        }
        if (pos) pos[i] = base + steps - 1;
    }
}

int oracle_tree_mask(const int32_t* parents, const int32_t* base_pos, int B, int N,
                     uint32_t* mask_bits, int32_t* positions) {
    if (!parents || !mask_bits || B < 0 || N < 1) return -1;
    int W = (N + 31) / 32;
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < B; ++b)
        tree_mask_one(parents + (size_t)b * N, base_pos ? base_pos[b] : 0, N, W,
                      mask_bits + (size_t)b * N * W, positions ? positions + (size_t)b * N : NULL);
    return 0;
}

/* ---- committing the accepted path of a token tree ----------------------------------
 * [atlas] the tree chapter covers how the KV of a token tree is laid out and rolled
 * back after a rejection; the serving section lists rolling back the KV of rejected
 * drafts as a cost that speculation adds.  [origins] SpecInfer: the verify forward
 * computes every node of the flattened tree over one shared KV.
 * Readings: the verify forward left one KV row per tree node, node j in row j of the
 * request's block; committing keeps the root and the accepted nodes in path order, so
 * output row d is the KV row of the d-th node of the path (row 0 the root) and the KV of
 * rejected nodes is dropped.  Output rows past the path are left as they were.
 * slots[d] names the tree node copied into output row d (-1 past the path).  A request
 * with accept_len outside [0, D] or an accepted node outside [0, N) copies nothing and
 * gets slots -1. */
static void commit_one(const int32_t* nodes, int32_t k, int D, int N, const uint8_t* src,
                       uint8_t* dst, size_t row_bytes, int32_t* slots) {
    int valid = k >= 0 && k <= D;
    for (int d = 0; d < k && valid; ++d)
        if (nodes[d] < 0 || nodes[d] >= N) valid = 0;
    for (int d = 0; d <= D; ++d) {
        int node = -1;
        if (valid && d <= k) node = d == 0 ? 0 : nodes[d - 1];
        if (slots) slots[d] = node;
        if (node >= 0) memcpy(dst + (size_t)d * row_bytes, src + (size_t)node * row_bytes, row_bytes);
    }
}

int oracle_tree_commit_kv(const int32_t* accepted_nodes, const int32_t* accept_len, int B,
                          int D, int N, const void* kv_tree, void* kv_out, size_t row_bytes,
                          int32_t* slots) {
    if (!accepted_nodes || !accept_len || !kv_tree || !kv_out || B < 0 || D < 1 || N < 1)
        return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < B; ++b)
        commit_one(accepted_nodes + (size_t)b * D, accept_len[b], D, N,
                   (const uint8_t*)kv_tree + (size_t)b * N * row_bytes,
                   (uint8_t*)kv_out + (size_t)b * (D + 1) * row_bytes, row_bytes,
                   slots ? slots + (size_t)b * (D + 1) : NULL);
    return 0;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
