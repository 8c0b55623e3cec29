/* spec_oracle.h -- plain fp64 CPU oracle of the speculative-decoding verify step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark may load this library.  It shares no source with the HIP
 * library: no header, helper, table or constant.
 *
 * All pointers are host pointers.  Logits are stored row-major [B][R][V] as fp32
 * (dtype 0) or as raw bf16 bit patterns (dtype 1).  Everything is widened to double;
 * sums run sequentially in ascending index order; exp() is libm's double exp.
 *
 * min_margin[b] receives the smallest distance between a coin and the threshold it was
 * compared against along request b's decision trace, or +inf when no coin decided
 * anything (greedy, invalid requests).  The distances are: |u - p/q| for an acceptance
 * test (ratio units, the coin's own scale); |u - prob_acc/threshold_acc| and
 * |p - threshold_single| for a tree sibling; the residual mass S itself where a residual
 * is formed (a mass near 0 decides between the residual and the fallback); the distance
 * of the top-p target to the ends of its boundary group (filtered calls, as a fraction
 * of the row's mass); and for the final inverse-CDF draw, the distances from t = u * S
 * to both ends of the chosen token's step, in WEIGHT units (probability mass), i.e. S
 * times the coin-space distance.  The draw's distance is kept in weight units because
 * that is the scale on which another implementation's rounding acts: a prefix sum of
 * fp32 weights is off by a small absolute amount of mass, whatever S is; and since
 * S <= 1 it is never larger than the coin-space distance, so the band it defines
 * contains every coin-space near-tie.  A request whose margin is below a small band can
 * legitimately come out differently under another rounding order.
 *
 * accept_margin[b] (every verify call; may be NULL) receives the same minimum over the
 * decision trace without the final draw's distances: the margin of everything that
 * decides how many drafts are accepted and which row and weights the last token is drawn
 * from.  min_margin[b] = min(accept_margin[b], the final draw's distance).
 *
 * Invalid requests (a token outside [0,V), a temperature that is not finite and > 0, a
 * coin outside (0,1], a row whose maximum is -inf, a drafted token whose q is negative
 * or not finite, a malformed parent array or a node deeper than D) get accept_len = -1
 * and every output slot of the request set to -1 (tokens, nodes) or 0 (probs).
 *
 * Return value: 0, or -1 if an argument is unusable (NULL pointer, non-positive size).
 */
#ifndef SPEC_ORACLE_H
#define SPEC_ORACLE_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_TREE_GREEDY 0
#define ORACLE_TREE_SAMPLING 1

/* Greedy chain verify: accept the longest draft prefix equal to the target argmax,
 * then emit the target argmax at the first mismatch (or at position G). */
int oracle_verify_greedy(const void* logits, int dtype, const int32_t* draft_tokens,
                         int B, int G, int V, int32_t* accept_len, int32_t* out_tokens);

/* Chain rejection sampling.  probs_out [B][G+1] (may be NULL): target probability of each
 * emitted token under the row it was emitted from, 0 past the last emitted token.
 * beta_out [B][G] (may be NULL): beta_i = sum_x min(p_i(x), q_i(x)) per drafted position. */
int oracle_verify_chain(const void* logits, int dtype, const float* draft_probs,
                        const int32_t* draft_tokens, const float* coins,
                        const float* temperature, int B, int G, int V,
                        int32_t* accept_len, int32_t* out_tokens, double* probs_out,
                        double* min_margin, double* beta_out, double* accept_margin);

/* Token-tree verify, target-only.  mode 0 = greedy, mode 1 = sampling.
 * out_tokens [B][D+1], accepted_nodes [B][D], probs_out [B][D+1] (may be NULL). */
int oracle_verify_tree(const void* logits, int dtype, const int32_t* node_tokens,
                       const int32_t* parents, const float* coins, const float* temperature,
                       int B, int N, int V, int D, int mode, float threshold_single,
                       float threshold_acc, int32_t* accept_len, int32_t* out_tokens,
                       int32_t* accepted_nodes, double* probs_out, double* min_margin,
                       double* accept_margin);

/* Token-tree verify by multi-step speculative sampling with draft distributions:
 * draft_probs [B][N][V] fp32 (row j = the distribution the children of node j were drawn
 * from), coins [B][N] (coins[c-1] tests node c, coins[N-1] drives the final draw).
 * Outputs as oracle_verify_tree. */
int oracle_verify_tree_mss(const void* logits, int dtype, const float* draft_probs,
                           const int32_t* node_tokens, const int32_t* parents,
                           const float* coins, const float* temperature, int B, int N, int V,
                           int D, int32_t* accept_len, int32_t* out_tokens,
                           int32_t* accepted_nodes, double* probs_out, double* min_margin,
                           double* accept_margin);

/* Chain rejection sampling from target logits [B][G+1][V] and draft logits [B][G][V]
 * (same dtype), both at temperature T and both filtered with top_k[b] (NULL or <= 0 or
 * >= V: off; ties at the k-th largest logit kept) and then top_p[b] (NULL or >= 1: off;
 * must be > 0; every token at least as probable as the end of the shortest head
 * reaching top_p of the mass is kept).  Outputs as oracle_verify_chain. */
int oracle_verify_chain_filtered(const void* logits, const void* draft_logits, int dtype,
                                 const int32_t* draft_tokens, const float* coins,
                                 const float* temperature, const int32_t* top_k,
                                 const float* top_p, int B, int G, int V, int32_t* accept_len,
                                 int32_t* out_tokens, double* probs_out, double* min_margin,
                                 double* accept_margin);

/* Tree attention mask: mask_bits [B][N][W], W = ceil(N/32); bit (j % 32) of word j / 32 of
 * row i is set iff node j lies on the path from node i to the root (i included).
 * positions [B][N] (may be NULL) = base_pos[b] (0 when base_pos is NULL) + depth(i).
 * A request whose parent array is malformed gets all-zero rows and positions -1. */
int oracle_tree_mask(const int32_t* parents, const int32_t* base_pos, int B, int N,
                     uint32_t* mask_bits, int32_t* positions);

/* Commit the accepted path of a token tree: kv_tree [B][N][row_bytes] (one KV row per
 * node), kv_out [B][D+1][row_bytes]: row d = kv_tree row of the d-th node of the path
 * (row 0 the root, rows 1..k the accepted nodes); rows past the path untouched.
 * slots [B][D+1] (may be NULL): the node copied into each row, -1 past the path.
 * accept_len outside [0, D] or an accepted node outside [0, N): nothing copied, slots -1. */
int oracle_tree_commit_kv(const int32_t* accepted_nodes, const int32_t* accept_len, int B,
                          int D, int N, const void* kv_tree, void* kv_out, size_t row_bytes,
                          int32_t* slots);

/* Number of OpenMP threads the oracle runs with (1 when built without OpenMP). */
int oracle_num_threads(void);

/* Threads for the calling thread's later oracle calls (n >= 1; no effect without OpenMP). */
void oracle_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
