/*
 * ddt.h - one DDTree verification round on AMD Instinct MI355X (gfx950).
 *
 * The method is DDTree (Diffusion Draft Tree), as summarised on the page
 * "策展 · X (Twitter)" at easyvibecoding.app/curated/665 (Liran Ringel's DDTree
 * post).  Sections of that page are cited by heading:
 *   核心創新  core innovation: draft tree from per-position marginals, node budget B,
 *             best-first heap, ancestor-only attention mask
 *   運作流程  procedure: bonus token b, step 1 (marginals q_i), step 2 (tree under
 *             budget B), step 3 (compile the tree, one target forward with tree
 *             attention), step 4 (tree walk)
 *   理論基礎  theory: Proposition 1 (expected acceptance = sum of prefix
 *             probabilities), Proposition 2 (the top-B prefixes form a tree)
 *
 * One round for S sequences is
 *   ddt_topk -> ddt_build_tree -> ddt_tree_mask -> ddt_tree_attention -> ddt_tree_walk
 * and ddt_draft_tree does the first three in two launches, with identical results.
 * (the target model's layers around the attention are the caller's).
 *
 * Conventions shared by every entry point
 *   - Array arguments are device pointers (hipMalloc'd or equivalent, visible to
 *     the current device); scalars are host values.  The caller owns every buffer.
 *     The library allocates no device memory and keeps no per-call state; it
 *     caches the current device's compute-unit count.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue work
 *     and never synchronise; outputs are valid once the stream reaches that point.
 *     Calls are reentrant; two calls that share output or workspace buffers must
 *     be ordered by the caller.
 *   - Errors that the host can see are reported before anything is launched and
 *     leave every output untouched: DDT_ERR_INVALID_ARG (null required pointer,
 *     size out of range), DDT_ERR_UNSUPPORTED (a head size or dtype without a
 *     kernel), DDT_ERR_WORKSPACE (workspace too small).  DDT_ERR_HIP means a launch
 *     failed.  No C++ exception crosses this interface.
 *   - Data preconditions, not checked: logits are finite; token ids are in
 *     [0, vocab); parent/depth arrays come from ddt_build_tree (or obey the same
 *     layout); cu_prefix is non-decreasing with cu_prefix[0] = 0.
 *   - Tree arrays have N = B + 1 entries per sequence.  Node 0 is the root (the
 *     bonus token).  A sequence whose candidate tree holds fewer than B prefixes
 *     gets num_nodes < N; its trailing entries are padding (ids -1, logq -inf,
 *     mask rows zero, attention rows zero) and every call honours num_nodes.
 */
#ifndef DDT_H_
#define DDT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DDT_OK = 0,
  DDT_ERR_INVALID_ARG = -1,
  DDT_ERR_UNSUPPORTED = -2,
  DDT_ERR_WORKSPACE = -3,
  DDT_ERR_HIP = -4
} ddt_status;

typedef enum { DDT_F32 = 0, DDT_BF16 = 1 } ddt_dtype;

enum {
  DDT_MAX_K = 64,    /* top-K width per position */
  DDT_MAX_L = 64,    /* draft positions per round */
  DDT_MAX_B = 1023   /* node budget (non-root nodes) */
};

/* Human-readable name of a status code (static string, never NULL). */
const char* ddt_status_string(int status);

/* ---------------------------------------------------------------- step 1
 * Per-position softmax and top-K (運作流程 step 1: the drafter's marginal q_i for
 * each of the next L positions; 核心創新: nodes at depth i are candidate tokens
 * for position i).
 *
 * logits     [rows, vocab] fp32, row r at logits + r * row_stride (row_stride >=
 *            vocab).  A row is one (sequence, position) pair: rows = S * L.
 *            Finite values, or -inf for masked tokens; at least one finite value
 *            per row, no NaN and no +inf (the softmax is undefined otherwise).
 * k          1 <= k <= min(vocab, DDT_MAX_K).
 * out_tok    [rows, k] int32: the k largest logits of the row, largest first;
 *            equal logits in increasing token id.
 * out_logq   [rows, k] fp32: log q(token) = logit - logsumexp(row), the
 *            full-vocabulary log-softmax at temperature 1 (not renormalised over
 *            the k kept tokens).  Sums of exp are formed in fp32 over at most 32
 *            logits per lane and in fp64 beyond that.
 * ws         device workspace of at least ddt_topk_workspace_size(rows, vocab, k)
 *            bytes (per-chunk lists and statistics; contents ignored).
 * Errors: null pointer; rows < 1; vocab < 1 or > INT32_MAX; row_stride < vocab;
 *         k out of range; ws_bytes too small.
 */
size_t ddt_topk_workspace_size(int64_t rows, int64_t vocab, int k);
int ddt_topk(const float* logits, int64_t rows, int64_t vocab, int64_t row_stride, int k,
             int32_t* out_tok, float* out_logq, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- step 2
 * Draft tree under a node budget (核心創新; 運作流程 step 2; 理論基礎).
 *
 * The candidates are the prefixes (r_1..r_d), 1 <= d <= L, of the K-ary tree whose
 * depth-i children are the K tokens of position i; a prefix's log-probability is
 * sum_i topk_logq[s, i-1, r_i] (the factorised draft).  A best-first heap selects
 * the B most probable prefixes; by Proposition 2 they are prefix-closed, and by
 * Proposition 1 they maximise the expected acceptance length under the draft.
 * Sums are formed in fp64.
 *
 * topk_tok, topk_logq  [S, L, K] from ddt_topk (rows of one sequence consecutive);
 *                      logq non-increasing along K.
 * bonus                [S] int32: the round's bonus token b, the tree root.
 * 1 <= S, 1 <= L <= DDT_MAX_L, 1 <= K <= DDT_MAX_K, 0 <= B <= DDT_MAX_B.
 * Outputs, [S, N] with N = B + 1, in canonical order: node 0 is the root (token
 *   b, parent -1, depth 0); then nodes sorted by (depth, parent index, sibling
 *   rank), so parents precede children and a parent's children are contiguous,
 *   most probable first.  The order depends only on the selected set.
 * tree_tok   token of each node (-1 padding).
 * parent     parent node index (-1 for the root and padding).
 * depth      0 for the root, d for a depth-d prefix (-1 padding).
 * node_logq  nullable; fp32 log-probability of each node's prefix (0 for the
 *            root, -inf padding).
 * num_nodes  [S]: 1 + number of selected prefixes (= N unless the candidate tree
 *            holds fewer than B prefixes).
 */
int ddt_build_tree(const int32_t* topk_tok, const float* topk_logq, const int32_t* bonus,
                   int S, int L, int K, int B,
                   int32_t* tree_tok, int32_t* parent, int32_t* depth, float* node_logq,
                   int32_t* num_nodes, void* stream);

/* ---------------------------------------------------------------- step 3
 * Compile the tree into the ancestor-only attention mask (核心創新; 運作流程 step 3).
 *
 * parent, depth  [S, N] as written by ddt_build_tree; num_nodes [S].
 * cu_prefix      nullable; [S+1] int64 prefix offsets (P_s = cu_prefix[s+1] -
 *                cu_prefix[s]).  When NULL, pos_ids is not written.
 * mask           [S, N, W] uint32, W = ceil(N / 32): bit j of word j / 32 of row n
 *                is set iff node j is node n or one of its ancestors.  The prefix
 *                context is visible to every node and is not part of the mask.
 *                Rows n >= num_nodes[s] are zero.
 * pos_ids        nullable; [S, N] int32 position of each node in the target's
 *                sequence, P_s + depth (-1 padding).
 * Errors: null parent/depth/num_nodes/mask; S < 1; B outside [0, DDT_MAX_B].
 */
int ddt_tree_mask(const int32_t* parent, const int32_t* depth, const int32_t* num_nodes,
                  const int64_t* cu_prefix, int S, int B, uint32_t* mask, int32_t* pos_ids,
                  void* stream);

/* ---------------------------------------------------------------- steps 1-3 fused
 * ddt_topk, ddt_build_tree and ddt_tree_mask in two launches (a top-K pass over the
 * vocabulary chunks, then one workgroup per sequence that merges the chunks, builds
 * the tree and forms its mask).  Every output is bit-identical to the three calls.
 *
 * logits      [S, L, vocab] fp32; row (s, i) at logits + (s * L + i) * row_stride;
 *             values as for ddt_topk.
 * bonus       [S]; cu_prefix nullable [S+1] (needed for pos_ids).
 * Limits as for the three calls: 1 <= L <= DDT_MAX_L, 1 <= K <= min(vocab,
 * DDT_MAX_K), 0 <= B <= DDT_MAX_B.
 * topk_tok, topk_logq [S, L, K]: the top-K step's outputs.
 * When a workgroup cannot give every draft position its own merge wave next to the
 * tree builder's registers (large budgets or long chunk lists), the call runs the
 * merge, the builder and the mask as three kernels instead of one; results are the
 * same either way.
 * tree_tok, parent, depth, node_logq (nullable), num_nodes: as ddt_build_tree.
 * mask [S, N, W] and pos_ids (nullable; written only with cu_prefix): as ddt_tree_mask.
 * ws          at least ddt_draft_tree_workspace_size(S, L, vocab, K) bytes.
 * Errors: null required pointer; a size out of range; ws_bytes too small.
 */
size_t ddt_draft_tree_workspace_size(int S, int L, int64_t vocab, int K);
int ddt_draft_tree(const float* logits, int64_t row_stride, const int32_t* bonus,
                   const int64_t* cu_prefix, int S, int L, int64_t vocab, int K, int B,
                   int32_t* topk_tok, float* topk_logq, int32_t* tree_tok, int32_t* parent,
                   int32_t* depth, float* node_logq, int32_t* num_nodes, uint32_t* mask,
                   int32_t* pos_ids, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- step 4 (attention)
 * Grouped-query tree attention: the whole tree is scored in one target forward
 * under the ancestor-only mask (運作流程 step 3).
 *
 * For sequence s, node n < num_nodes[s] and query head h, with g = h / (Hq / Hkv):
 *   keys   = prefix K[cu_prefix[s] .. cu_prefix[s+1]) of KV head g, followed by
 *            k_tree[s, j, g] for every j visible in mask[s, n]
 *   out[s, n, h] = softmax(scale * q[s, n, h] . keys^T) . values
 *   lse[s, n, h] = natural log of sum exp(scale * q . k) over those keys
 * q          [S, N, Hq, D]                 (dtype)
 * k_cache,   [sum_s P_s, Hkv, D]           (dtype) sequences packed back to back
 * v_cache
 * cu_prefix  [S+1] int64
 * k_tree,    [S, N, Hkv, D]                (dtype) the tree nodes' own K/V
 * v_tree
 * mask       [S, N, W] from ddt_tree_mask; num_nodes [S]
 * dtype      DDT_F32 or DDT_BF16 for q, K, V and out; accumulation is fp32.
 * D          32, 64 or 128; Hq % Hkv == 0; scale finite and > 0.
 * max_prefix host upper bound on every P_s: it sizes the key-split plan and the
 *            workspace.  A larger P_s is still computed correctly, more slowly.
 * out        [S, N, Hq, D] (dtype); rows n >= num_nodes[s] are written as 0.
 * lse        nullable; [S, N, Hq] fp32 (-inf for padding rows).
 * ws         at least ddt_tree_attention_workspace_size(...) bytes, computed for
 *            the device current at the call (its compute-unit count shapes the
 *            plan).  Contents are ignored.
 */
size_t ddt_tree_attention_workspace_size(int S, int B, int Hq, int Hkv, int D, int dtype,
                                         int64_t max_prefix);
int ddt_tree_attention(const void* q, const void* k_cache, const void* v_cache,
                       const int64_t* cu_prefix, const void* k_tree, const void* v_tree,
                       const uint32_t* mask, const int32_t* num_nodes,
                       int S, int B, int Hq, int Hkv, int D, int dtype, float scale,
                       int64_t max_prefix, void* out, float* lse, void* ws, size_t ws_bytes,
                       void* stream);

/* ---------------------------------------------------------------- step 5
 * Greedy tree walk (運作流程 step 4): from the root, take the target's greedy
 * token at the current node; if a child carries it, accept that child and move
 * there; otherwise stop and return the token as the next round's bonus.  A node
 * at depth L has no children, so the walk ends there.
 *
 * tree_tok, parent  [S, N] from ddt_build_tree; num_nodes [S].
 * target_logits     [S, N, vocab] fp32 target logits at every node (rows past
 *                   num_nodes are not read).  Greedy = argmax, equal logits to the
 *                   smaller token id (-0 and +0 are equal).  No NaN.
 * accept_len [S]     accepted draft tokens a (the round emits a + 1 tokens).
 * acc_nodes  [S, L]  accepted node indices in order, -1 padded.
 * acc_tok    [S, L]  their tokens, -1 padded.
 * bonus_out  [S]     the target's token at the last accepted node.
 * ws        at least ddt_tree_walk_workspace_size(S, B, vocab) bytes of device memory,
 *           zero-filled before its first use; every call leaves it zero-filled again
 *           (completion counters and arg-max keys).  Calls that share a workspace
 *           must not overlap.
 * Errors: null pointer; S < 1; L outside [1, DDT_MAX_L]; B outside [0, DDT_MAX_B];
 *         vocab < 1 or > INT32_MAX; ws too small.
 */
size_t ddt_tree_walk_workspace_size(int S, int B, int64_t vocab);
int ddt_tree_walk(const int32_t* tree_tok, const int32_t* parent, const int32_t* num_nodes,
                  const float* target_logits, int S, int B, int L, int64_t vocab,
                  int32_t* accept_len, int32_t* acc_nodes, int32_t* acc_tok, int32_t* bonus_out,
                  void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- benchmark aid
 * Timing of the attention's main kernel (the round's dominant kernel) with HIP
 * events on the stream it runs on.  While profiling is on, every
 * ddt_tree_attention call attaches a start/stop event pair to that kernel's
 * dispatch (hipExtLaunchKernelGGL), so the pair brackets the kernel's execution.
 * Use it on eagerly launched calls: event pairs recorded during a HIP graph
 * capture are not readable afterwards.  ddt_attention_timing waits for the
 * recorded pairs, returns the sum of their elapsed times in milliseconds and their
 * count, and forgets them.  ddt_attention_profiling(0) releases the events.  This
 * is the only state the library keeps; it is process-wide and guarded by a mutex.
 * Returns DDT_OK or DDT_ERR_HIP.
 */
int ddt_attention_profiling(int enable);
int ddt_attention_timing(double* total_ms, int* count);

#ifdef __cplusplus
}
#endif
#endif /* DDT_H_ */
