/* spec_verify.h -- C ABI of the MI355X (gfx950) speculative-decoding verify library.
 *
 * The verify step of speculative decoding: a cheap drafter proposes tokens, the target
 * model scores every proposed position in one forward pass, and the verifier decides
 * which proposals to keep and which single extra token to emit so that the output
 * follows the target distribution exactly.  Sources:
 *   llm-infra-atlas, "Speculative Decoding -- lossless acceleration of autoregressive
 *     decode", section 0 (target logits for gamma+1 positions from one forward;
 *     rejection sampling keeps the output law equal to the target's) and section 2
 *     (notation: bonus token, correction from norm(max(0, p - q)), tau counts the bonus);
 *   ricardokevins, "Speculative Decoding: real gains, correction sampling and production
 *     limits", "mechanism" (draft / verify / accept / correct) and "correction sampling"
 *     (Eq. a(x) = min(1, p(x)/q(x)), Eq. r(x) = norm(max(p - q, 0)));
 *   zdszero, "spec_origins": "Blockwise Parallel Decoding" (greedy verify keeps the
 *     longest prefix equal to the scorer's argmax), "Speculative Decoding" acceptance
 *     rule items 1-3, "SpecInfer" (token tree flattened with an ancestor-only mask) and
 *     "in SGLang" (greedy tree verify; the target-only tree walk with prob_acc, per-level
 *     coin, threshold_single and threshold_acc, rejected children removed from the final
 *     distribution relu(target - draft_probs); chain p/q rejection sampling with topk 1).
 *
 * Conventions shared by every entry point
 *   - All array arguments are DEVICE pointers owned by the caller.  The library never
 *     allocates, frees or synchronises, and keeps no pointer after the call returns.
 *     Work is enqueued on `stream` (a hipStream_t passed as void*; NULL = default stream)
 *     and the call returns immediately.  No host synchronisation and no allocation
 *     happen inside a call, so calls can be captured into a HIP graph.
 *   - Layouts are dense row-major with the last dimension contiguous.  Target logits are
 *     fp32 (SPEC_F32) or bf16 (SPEC_BF16, raw 16-bit patterns) and must be aligned to
 *     their element size; rows need not be 16-byte aligned (a scalar head/tail handles
 *     that), but 16-byte aligned rows (V * element size a multiple of 16 and an aligned
 *     base) take the fast path.  A row holds at most 2^31 - 1 bytes (V * element size;
 *     SPEC_ERR_SHAPE beyond).  Draft probabilities are fp32.  Token ids and parents
 *     are int32.  Coins are fp32 uniforms in (0, 1] supplied by the caller.
 *   - Target distribution: p = softmax(logits / T) per row, T > 0 per request.  Draft
 *     probabilities q are used exactly as given (already at temperature T).
 *   - Return value: SPEC_OK, or a negative status for an argument error found on the
 *     host before anything is enqueued (nothing is written), or SPEC_ERR_HIP if a launch
 *     failed.  Errors in the data are reported in-band per request: accept_len[b] =
 *     SPEC_ROW_INVALID (-1), token / node rows of that request filled with -1 and
 *     probability rows with 0.  accept_len[b] = SPEC_ROW_RETRY (-2) means the request
 *     was not verified (see "Walks" below); its other output rows are then unspecified.
 *     A request is invalid when something the verify consults is unusable: a token id
 *     outside [0, V), a temperature that is not finite and > 0, a coin outside (0, 1], a
 *     row with no finite logit (all -inf), a drafted token's q that is negative or not
 *     finite, or (tree) a malformed parent array or a node deeper than D.  Chains and
 *     trees are walked in order and stop at the first rejection (or mismatch), so
 *     positions, rows and coins after the stop are not consulted and not checked (the
 *     temperature and the final draw's coin always are; spec_verify_chain_filtered
 *     checks every row).  NaN or +inf logits are undefined.
 *   - Workspace: a device buffer of at least spec_workspace_bytes(op, B, R, V) bytes,
 *     256-byte aligned, owned by the caller, ZERO-FILLED ONCE before its first use
 *     (hipMemset).  Its header holds a call counter that tags the words the workgroups
 *     of one request hand to each other, and one exit word per request; each call
 *     advances the counter on the device once every workgroup of the call has finished,
 *     and leaves the exit words at zero, so a call captured into a HIP graph replays
 *     correctly and one workspace serves calls of any shape in turn.  Everything else in
 *     it is written before it is read within a call.  Calls that may run at the same time
 *     (on different streams) need separate workspaces; calls issued in order on one
 *     stream can share one.
 *   - Walks: by default the greedy, chain and tree calls spread each request over a
 *     cluster of workgroups that walk it position by position (node by node) and stop
 *     where the method stops, handing row statistics to each other through the
 *     workspace.  Every wait for another workgroup is bounded (spec_options.spin_limit
 *     polls, 2^18 by default: far longer than a walk takes while its workgroups run).  A
 *     wait that runs out, which only happens when other work keeps a cluster's
 *     workgroups off the device for that long, ends that request with accept_len =
 *     SPEC_ROW_RETRY instead of hanging; the other requests are unaffected, the next
 *     call on the same workspace is unaffected, and calling again verifies the request.
 *   - Determinism: identical inputs give bitwise-identical outputs.
 *   - Coin convention: every comparison is coin <= threshold.  The final draw (the
 *     correction, the bonus, or the tree's last token) is the inverse CDF in ascending
 *     token id with its own coin: the first token j with weight w_j > 0 and
 *     u * sum(w) <= w_0 + ... + w_j.  If the residual mass is not positive the draw
 *     falls back to the target row itself.  Greedy argmax ties go to the lowest id.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* In-band results of a request (accept_len[b]) other than an accepted length. */
#define SPEC_ROW_INVALID (-1) /* something the verify consults is unusable */
#define SPEC_ROW_RETRY (-2)   /* not verified: a wait between the request's workgroups ran out */

enum {
    SPEC_OK = 0,
    SPEC_ERR_NULL = -1,      /* a required pointer is NULL */
    SPEC_ERR_SHAPE = -2,     /* B, G, N, V or D outside the supported range */
    SPEC_ERR_DTYPE = -3,     /* unknown logit dtype */
    SPEC_ERR_PARAM = -4,     /* bad mode / threshold / misaligned pointer */
    SPEC_ERR_WORKSPACE = -5, /* workspace too small or not 256-byte aligned */
    SPEC_ERR_HIP = -6,       /* a HIP launch failed */
    SPEC_ERR_TOO_LARGE = -7  /* spec_verify_chain_noalloc: sizes beyond its static scratch */
};

enum { SPEC_F32 = 0, SPEC_BF16 = 1 };                   /* target-logit dtype */
enum { SPEC_TREE_GREEDY = 0, SPEC_TREE_SAMPLING = 1 };  /* spec_verify_tree mode */
enum { SPEC_OP_GREEDY = 0, SPEC_OP_CHAIN = 1, SPEC_OP_TREE = 2, SPEC_OP_CHAIN_FILTERED = 3,
       SPEC_OP_TREE_MSS = 4 };

#define SPEC_MAX_G 64     /* drafted positions per request (chain) */
#define SPEC_MAX_N 1024   /* tree nodes per request, root included */

enum { SPEC_PATH_WALK = 0, SPEC_PATH_EAGER = 1 };
enum { SPEC_LOADS_DEFAULT = 0, SPEC_LOADS_CACHED = 1, SPEC_LOADS_STREAMING = 2 };

/* Launch options of the *_opt entry points.  Zero-initialise and set what you need: a
 * field left at 0 keeps the library's own choice, which is all the plain entry points use.
 * The same options give the same kernels and launch shapes on the same device, whatever
 * the process environment.  Greedy results never depend on them.  Sampling results agree
 * across options except where a coin lies within rounding of a threshold (the paths add
 * the same fp32 terms in different groupings); timing and the SPEC_ROW_RETRY behaviour
 * depend on them.
 *   path        SPEC_PATH_WALK: walk each request and read only the rows the method
 *               consults (default); SPEC_PATH_EAGER: stream every row once, then decide
 *               in separate kernels (greedy, chain and tree; the multi-step tree always
 *               walks).
 *   cluster     walks: workgroups per request.  0: the largest width at which every
 *               request's workgroups are resident at once.  A request is never spread
 *               over more workgroups than the device holds at once for the batch, nor
 *               over more than 16.
 *   splits      eager row passes: workgroups per row (0: about 64 KB of logits each).
 *   row_loads   chain walk's row loads: SPEC_LOADS_CACHED (the default) or
 *               SPEC_LOADS_STREAMING (non-temporal).
 *   spin_limit  walks: polls before a wait for another workgroup gives up (0: 2^18);
 *               a tiny value forces SPEC_ROW_RETRY, for tests of that path. */
typedef struct spec_options {
    int path;
    int cluster;
    int splits;
    int row_loads;
    int spin_limit;
} spec_options;

/* Bytes of workspace a call of kind `op` needs for B requests, R logit rows per request
 * (G+1 for the chain calls, N for the tree) and vocabulary V.  0 for unusable sizes. */
size_t spec_workspace_bytes(int op, int B, int R, int V);

/* Human-readable name of a status code (static string). */
const char* spec_status_str(int status);

/* Greedy chain verify (spec_origins, "Blockwise Parallel Decoding", verify).
 *   logits       [B][G+1][V] target logits; row i scores the token after draft i-1.
 *   draft_tokens [B][G]      proposed tokens.
 * Per request: a_i = lowest id attaining max_x logits[b][i][x] (raw logits, no
 * temperature); k = the first i < G with draft_tokens[b][i] != a_i, else G.
 *   accept_len [B]    = k;
 *   out_tokens [B][G+1] = draft_tokens[b][0..k-1], then a_k, then -1 padding. */
int spec_verify_greedy(const void* logits, int dtype, const int32_t* draft_tokens,
                       int B, int G, int V, int32_t* accept_len, int32_t* out_tokens,
                       void* workspace, size_t ws_bytes, void* stream);
/* The same with launch options (NULL: the defaults). */
int spec_verify_greedy_opt(const void* logits, int dtype, const int32_t* draft_tokens,
                           int B, int G, int V, int32_t* accept_len, int32_t* out_tokens,
                           void* workspace, size_t ws_bytes, void* stream,
                           const spec_options* opt);

/* Chain rejection sampling (spec_origins, "Speculative Decoding", acceptance rule;
 * ricardokevins, "correction sampling", Eq. a(x) and Eq. r(x)).
 *   logits       [B][G+1][V] target logits;
 *   draft_probs  [B][G][V]   draft distribution q_i at each drafted position (fp32);
 *   draft_tokens [B][G]      x_i ~ q_i;
 *   coins        [B][G+1]    coins[b][i] (i < G) decides position i: x_i is accepted iff
 *                            p_i(x_i) > 0 and coins[b][i] <= p_i(x_i) / q_i(x_i);
 *                            coins[b][G] drives the final draw;
 *   temperature  [B].
 * k = the first rejected position, else G.  The final token is drawn from
 * norm(max(0, p_k - q_k)) if k < G (the correction), else from p_G (the bonus).
 *   accept_len [B] = k; out_tokens [B][G+1] = x_0..x_{k-1}, final token, -1 padding;
 *   probs_out  [B][G+1] (optional, may be NULL) = target probability of each emitted
 *              token under the row it was emitted from, 0 for padding. */
int spec_verify_chain(const void* logits, int dtype, const float* draft_probs,
                      const int32_t* draft_tokens, const float* coins,
                      const float* temperature, int B, int G, int V, int32_t* accept_len,
                      int32_t* out_tokens, float* probs_out, void* workspace,
                      size_t ws_bytes, void* stream);
/* The same with launch options (NULL: the defaults). */
int spec_verify_chain_opt(const void* logits, int dtype, const float* draft_probs,
                          const int32_t* draft_tokens, const float* coins,
                          const float* temperature, int B, int G, int V, int32_t* accept_len,
                          int32_t* out_tokens, float* probs_out, void* workspace,
                          size_t ws_bytes, void* stream, const spec_options* opt);

/* Chain rejection sampling (as spec_verify_chain, same arguments and results) for callers
 * that cannot allocate device memory: code under HIP graph capture, tight serving loops,
 * and harnesses that forbid hipMalloc.  There is no workspace argument: the call uses a
 * static scratch array of 32 MiB inside the library (each GPU the library runs on holds
 * its own copy until the process ends; zero when the library is loaded), and allocates
 * nothing.  Calls whose spec_workspace_bytes(SPEC_OP_CHAIN, B, G+1, V) exceeds 32 MiB
 * return SPEC_ERR_TOO_LARGE before anything is enqueued (B = 256, G = 4 fits up to
 * V ~ 700k; at V = 152064, B up to ~1200).  Every call on one GPU shares that GPU's
 * array: calls on one stream run in turn and may differ in shape, but calls that overlap
 * on one GPU (other streams, other host threads) race and give wrong results.  The
 * array's header (the walks' call counter and exit words) is left ready by every call;
 * everything else in it is written before it is read within a call.  SPEC_ERR_HIP if the
 * array's device address cannot be obtained. */
int spec_verify_chain_noalloc(const void* logits, int dtype, const float* draft_probs,
                              const int32_t* draft_tokens, const float* coins,
                              const float* temperature, int B, int G, int V,
                              int32_t* accept_len, int32_t* out_tokens, float* probs_out,
                              void* stream);

/* Chain rejection sampling from draft logits, with top-k / top-p filtering
 * (ricardokevins, "mechanism": serving samples with temperature, top-p and top-k;
 * "correction sampling", Eq. a(x) and Eq. r(x): acceptance and residual keep the
 * target's law only on the distributions actually sampled from).
 *   logits       [B][G+1][V] target logits;
 *   draft_logits [B][G][V]   draft logits, same dtype (q_i = softmax(draft_logits / T));
 *   draft_tokens, coins, temperature as spec_verify_chain;
 *   top_k [B] (NULL: off)    keep the tokens whose logit is at least the k-th largest
 *                            (ties kept); k <= 0 or k >= V: off;
 *   top_p [B] (NULL: off)    on the top-k-filtered row, keep every token at least as
 *                            probable as the last token of the shortest head (in
 *                            decreasing probability) whose mass reaches top_p of the
 *                            row's mass (ties kept); top_p >= 1: off; top_p <= 0 or NaN
 *                            makes the request invalid.
 * Target and draft rows are filtered alike and renormalised; then the acceptance rule,
 * the residual and the bonus run as in spec_verify_chain on the filtered rows.  The
 * filtered masses are summed in fixed point, so the kept sets are deterministic.
 * Workspace: spec_workspace_bytes(SPEC_OP_CHAIN_FILTERED, B, G+1, V).  Outputs and
 * probs_out as spec_verify_chain (probabilities under the filtered target rows). */
int spec_verify_chain_filtered(const void* logits, const void* draft_logits, int dtype,
                               const int32_t* draft_tokens, const float* coins,
                               const float* temperature, const int32_t* top_k,
                               const float* top_p, int B, int G, int V, int32_t* accept_len,
                               int32_t* out_tokens, float* probs_out, void* workspace,
                               size_t ws_bytes, void* stream);

/* Token-tree verify (spec_origins, "SpecInfer" and "in SGLang").
 *   logits      [B][N][V] row j = target logits of the token after node j (node 0 is the
 *               root, i.e. the last committed token);
 *   node_tokens [B][N]    token carried by each node ([b][0] unused);
 *   parents     [B][N]    parents[b][0] = -1 and 0 <= parents[b][i] < i; siblings should
 *               carry distinct tokens (duplicates are accumulated as given);
 *   coins       [B][D+1]  sampling mode: coins[b][d] decides level d, coins[b][D] drives
 *               the final draw (NULL allowed in greedy mode);
 *   temperature [B]       sampling mode (NULL allowed in greedy mode);
 *   D           maximum depth, 1 <= D <= SPEC_MAX_N: every node must lie at depth <= D.
 * Sampling (target-only): from cur = root, level d: try the children of cur in ascending
 * node id, adding their target probabilities p_cur(token) into acc; the first child with
 * coins[b][d] <= acc / threshold_acc or p_cur(token) >= threshold_single is accepted and
 * the walk moves to it; if none is, the walk stops.  The final token is drawn from p_cur
 * with the tokens of the children tried at the last level removed (a leaf keeps its whole
 * row).  threshold_single = threshold_acc = 1.0 is the lossless setting.
 * Greedy: follow the first child whose token equals the argmax of row cur; emit the argmax
 * of the row where the walk stops.
 *   accept_len [B] = number of accepted nodes d; out_tokens [B][D+1] = their tokens, then
 *   the final token, -1 padding; accepted_nodes [B][D] = accepted node ids, -1 padding;
 *   probs_out [B][D+1] (optional) = target probability of each emitted token under the row
 *   it was emitted from (sampling mode; 0 in greedy mode and for padding). */
int spec_verify_tree(const void* logits, int dtype, const int32_t* node_tokens,
                     const int32_t* parents, const float* coins, const float* temperature,
                     int B, int N, int V, int D, int mode, float threshold_single,
                     float threshold_acc, int32_t* accept_len, int32_t* out_tokens,
                     int32_t* accepted_nodes, float* probs_out, void* workspace,
                     size_t ws_bytes, void* stream);
/* The same with launch options (NULL: the defaults). */
int spec_verify_tree_opt(const void* logits, int dtype, const int32_t* node_tokens,
                         const int32_t* parents, const float* coins, const float* temperature,
                         int B, int N, int V, int D, int mode, float threshold_single,
                         float threshold_acc, int32_t* accept_len, int32_t* out_tokens,
                         int32_t* accepted_nodes, float* probs_out, void* workspace,
                         size_t ws_bytes, void* stream, const spec_options* opt);

/* Token-tree verify by multi-step speculative sampling with draft distributions
 * (spec_origins, "SpecInfer": the children of a node are tested in turn with
 * min(1, p(x)/q(x)); after a rejection the node's distribution becomes the residual
 * norm(max(0, p - q)) and the next sibling is tested against it).
 *   logits      [B][N][V] row j = target logits of the token after node j;
 *   draft_probs [B][N][V] fp32, row j = the draft distribution the children of node j were
 *               drawn from (shared by all of them; used as given).  The result follows the
 *               target law when the children are independent draws from that row
 *               (duplicate tokens are then allowed);
 *   node_tokens, parents [B][N] as spec_verify_tree;
 *   coins       [B][N]    coins[b][c-1] tests node c; coins[b][N-1] drives the final draw;
 *   temperature [B];
 *   D           maximum depth, 1 <= D <= SPEC_MAX_N.
 * From cur = root, children are tried in ascending node id; the first accepted child
 * becomes cur.  When every child of cur is rejected, the final token is drawn from the
 * last residual.  At a leaf, or when a residual has no mass left (remaining siblings
 * untried), the final token is drawn from p_cur.
 * Only the rows the walk reaches are read.  A request is invalid (-1) when such a row
 * has no finite logit, or when parents, tokens, temperature, coins, depth or the
 * q(token) of any child are bad.
 * Workspace: spec_workspace_bytes(SPEC_OP_TREE_MSS, B, N, V).  Outputs and probs_out as
 * spec_verify_tree sampling mode. */
int spec_verify_tree_mss(const void* logits, int dtype, const float* draft_probs,
                         const int32_t* node_tokens, const int32_t* parents,
                         const float* coins, const float* temperature, int B, int N, int V,
                         int D, int32_t* accept_len, int32_t* out_tokens,
                         int32_t* accepted_nodes, float* probs_out, void* workspace,
                         size_t ws_bytes, void* stream);
/* The same with launch options (NULL: the defaults; `path` is ignored). */
int spec_verify_tree_mss_opt(const void* logits, int dtype, const float* draft_probs,
                             const int32_t* node_tokens, const int32_t* parents,
                             const float* coins, const float* temperature, int B, int N,
                             int V, int D, int32_t* accept_len, int32_t* out_tokens,
                             int32_t* accepted_nodes, float* probs_out, void* workspace,
                             size_t ws_bytes, void* stream, const spec_options* opt);

/* Tree attention mask and positions (spec_origins, "SpecInfer": the token tree is
 * flattened into one sequence and each node attends only to its ancestors, so one target
 * forward scores every branch over a shared KV).  This is the step before verify: it
 * builds, from the same parent array spec_verify_tree takes, the mask and the position
 * ids of that forward.  A node also attends to itself (the causal diagonal).
 *   parents   [B][N]  parents[b][0] = -1 and 0 <= parents[b][i] < i (node 0 = root, the
 *             last committed token);
 *   base_pos  [B]     position id of the root, or NULL for 0;
 *   mask      [B][N][W] uint32 out, W = (N + 31) / 32: bit (j % 32) of word j / 32 of row i
 *             is set iff node j lies on the path from node i to the root, i included;
 *   positions [B][N]  out, base_pos[b] + depth of node i; may be NULL.
 * A request whose parent array is malformed gets all-zero mask rows and positions -1.
 * 1 <= N <= SPEC_MAX_N.  No workspace; device pointers; enqueued on `stream`. */
int spec_tree_mask(const int32_t* parents, const int32_t* base_pos, int B, int N,
                   uint32_t* mask, int32_t* positions, void* stream);

/* Commit the accepted path of a token tree (llm-infra-atlas "Speculative Decoding": the
 * tree chapter covers how a tree's KV is laid out and rolled back after a rejection;
 * spec_origins, "SpecInfer": one verify forward computes every node of the flattened
 * tree over a shared KV).  After spec_verify_tree, the KV rows of the root and of the
 * accepted nodes are gathered, in path order, into a contiguous block; the rows of
 * rejected branches are dropped.
 *   accepted_nodes [B][D], accept_len [B]  as written by spec_verify_tree;
 *   kv_tree  [B][N][row_bytes]  the verify forward's KV, one row per tree node;
 *   kv_out   [B][D+1][row_bytes] out: row d = kv_tree row of the d-th node of the path
 *            (row 0 = the root, rows 1..k = the accepted nodes); rows past the path are
 *            left as they were.  Must not overlap kv_tree;
 *   slots    [B][D+1] out (may be NULL): the node copied into each row, -1 past the path.
 * A request with accept_len outside [0, D] or an accepted node outside [0, N) copies
 * nothing and gets slots -1.  Rows whose size and bases are 16-byte multiples take the
 * vector path.  No workspace; device pointers; enqueued on `stream`. */
int spec_tree_commit_kv(const int32_t* accepted_nodes, const int32_t* accept_len, int B, int D,
                        int N, const void* kv_tree, void* kv_out, size_t row_bytes,
                        int32_t* slots, void* stream);

/* Measurement utilities (not part of the verify path).  They calibrate the figures the
 * verify kernels are measured against on the device at hand.
 *
 * spec_calib_read: streams `bytes` bytes of device memory from `data` with 16-byte loads
 * that do not allocate in the caches, the access pattern of the row passes, and reduces
 * them to nothing observable; the caller times the call to get the achievable read
 * bandwidth.  `data` 16-byte aligned, `bytes` a multiple of 16 (SPEC_ERR_PARAM
 * otherwise), 0 is a no-op.  `sink` (one float, device) is written only in the
 * impossible case that the reduction hits a sentinel, which keeps the reads from being
 * optimised away.
 *
 * spec_calib_exp: `blocks` workgroups of 256 lanes each evaluate iters * 8 independent
 * v_exp_f32 (the row passes' exponential), so the caller gets the exponential throughput
 * as blocks * 256 * iters * 8 / time.  1 <= blocks <= 65535, 1 <= iters <= 1 << 20
 * (SPEC_ERR_PARAM otherwise).  `sink` as above.
 *
 * Both enqueue on `stream` and return SPEC_OK, an argument error, or SPEC_ERR_HIP. */
int spec_calib_read(const void* data, size_t bytes, float* sink, void* stream);
int spec_calib_exp(int blocks, int iters, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
