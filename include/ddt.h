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
 * Across rounds, ddt_commit_kv appends the accepted path's K/V to each sequence's cache
 * and the walk's bonus token becomes the next round's root.
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
 *   - The prefix (context) of sequence s is described by cu_prefix [S+1] int64 and an
 *     optional prefix_len [S] int64.  Without prefix_len, its P_s = cu_prefix[s+1] -
 *     cu_prefix[s] keys are cache rows cu_prefix[s] .. cu_prefix[s+1] (sequences packed
 *     back to back).  With prefix_len, they are rows cu_prefix[s] .. cu_prefix[s] +
 *     prefix_len[s], and the rows up to cu_prefix[s+1] are room for ddt_commit_kv to
 *     append to (0 <= prefix_len[s] <= cu_prefix[s+1] - cu_prefix[s]).
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
  DDT_ERR_HIP = -4,
  DDT_ERR_TOO_LARGE = -5
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
 * cu_prefix      nullable; [S+1] int64 prefix offsets, with prefix_len (nullable) as
 *                described above: they give P_s.  When cu_prefix is NULL, pos_ids is
 *                not written.
 * mask           [S, N, W] uint32, W = ceil(N / 32): bit j of word j / 32 of row n
 *                is set iff node j is node n or one of its ancestors.  The prefix
 *                context is visible to every node and is not part of the mask.
 *                Rows n >= num_nodes[s] are zero.
 * pos_ids        nullable; [S, N] int32 position of each node in the target's
 *                sequence, P_s + depth (-1 padding).
 * Errors: null parent/depth/num_nodes/mask; S < 1; B outside [0, DDT_MAX_B].
 */
int ddt_tree_mask(const int32_t* parent, const int32_t* depth, const int32_t* num_nodes,
                  const int64_t* cu_prefix, const int64_t* prefix_len, int S, int B,
                  uint32_t* mask, int32_t* pos_ids, void* stream);

/* ---------------------------------------------------------------- steps 1-3 fused
 * ddt_topk, ddt_build_tree and ddt_tree_mask in two launches (a top-K pass over the
 * vocabulary chunks, then one workgroup per sequence that merges the chunks, builds
 * the tree and forms its mask).  Every output is bit-identical to the three calls.
 *
 * logits      [S, L, vocab] fp32; row (s, i) at logits + (s * L + i) * row_stride;
 *             values as for ddt_topk.
 * bonus       [S]; cu_prefix nullable [S+1] and prefix_len nullable [S] (needed for
 *             pos_ids; see the conventions above).
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
                   const int64_t* cu_prefix, const int64_t* prefix_len, int S, int L,
                   int64_t vocab, int K, int B,
                   int32_t* topk_tok, float* topk_logq, int32_t* tree_tok, int32_t* parent,
                   int32_t* depth, float* node_logq, int32_t* num_nodes, uint32_t* mask,
                   int32_t* pos_ids, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- adaptive budget (after step 2)
 * Choice of the node budget per sequence (實驗結果與權衡: the speedup peaks at an
 * intermediate budget as verification cost grows; 理論基礎: by Proposition 1 the
 * expected acceptance E(b) of the best tree with b nodes is the sum of its prefix
 * probabilities, and by Proposition 2 that tree is the b most probable prefixes, the
 * heap's first b pops).  For a tree built at budget B:
 *   B*_s = argmax over b = 0 .. num_nodes[s]-1 of (E(b) + 1) / cost[b]
 * (sums and ratios in fp64; equal ratios to the smaller b), and the tree is cut, in
 * place, to its B*_s most probable prefixes: pop order is log-probability
 * descending, equal values by smaller node index (shallower first, then canonical
 * order within a depth).  The survivors keep their canonical order and are
 * renumbered; entries past B*_s + 1 become padding.  Call ddt_tree_mask afterwards
 * for the cut tree's mask; attention and walk honour the new num_nodes.
 *
 * cost        [B+1] fp32 device array: the caller's verify cost at each budget
 *             (for instance measured microseconds per round); finite and > 0.
 * tree_tok, parent, depth, node_logq, num_nodes: as written by ddt_build_tree
 *             (node_logq required), rewritten in place.
 * budget_out  [S] int32: B*_s.
 * expected_out nullable [S] fp32: E(B*_s).
 * Errors: null required pointer; S < 1; B outside [0, DDT_MAX_B].
 */
int ddt_adapt_budget(const float* cost, int S, int B, int32_t* tree_tok, int32_t* parent,
                     int32_t* depth, float* node_logq, int32_t* num_nodes, int32_t* budget_out,
                     float* expected_out, void* stream);

/* ---------------------------------------------------------------- step 4 (attention)
 * Grouped-query tree attention: the whole tree is scored in one target forward
 * under the ancestor-only mask (運作流程 step 3).
 *
 * For sequence s, node n < num_nodes[s] and query head h, with g = h / (Hq / Hkv):
 *   keys   = prefix K[cu_prefix[s] .. cu_prefix[s] + P_s) of KV head g, followed by
 *            k_tree[s, j, g] for every j visible in mask[s, n]
 *   out[s, n, h] = softmax(scale * q[s, n, h] . keys^T) . values
 *   lse[s, n, h] = natural log of sum exp(scale * q . k) over those keys
 * q          [S, N, Hq, D]                 (dtype)
 * k_cache,   [rows, Hkv, D]                (dtype) sequences back to back, cu_prefix[S] rows
 * v_cache
 * cu_prefix  [S+1] int64; prefix_len nullable [S] int64 (conventions above)
 * k_tree,    [S, N, Hkv, D]                (dtype) the tree nodes' own K/V
 * v_tree
 * mask       [S, N, W] from ddt_tree_mask; num_nodes [S]
 * dtype      DDT_F32 or DDT_BF16 for q, K, V and out; accumulation is fp32.
 * D          32, 64 or 128; Hq % Hkv == 0; scale finite and > 0.  For DDT_BF16,
 *            64 key rows (64 * Hkv * D * 2 bytes) must span less than 2 GiB, else
 *            DDT_ERR_UNSUPPORTED.
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
                       const int64_t* cu_prefix, const int64_t* prefix_len,
                       const void* k_tree, const void* v_tree,
                       const uint32_t* mask, const int32_t* num_nodes,
                       int S, int B, int Hq, int Hkv, int D, int dtype, float scale,
                       int64_t max_prefix, void* out, float* lse, void* ws, size_t ws_bytes,
                       void* stream);

/* ---------------------------------------------------------------- between rounds
 * KV commit (運作流程: each round starts from a bonus token that the target produced
 * but has not run forward, and the walk's first mismatch is carried into the next
 * round as its bonus).  After the walk, the root and the accepted nodes n_1..n_a have
 * been run through the target, each attending to exactly the prefix and its
 * ancestors, which is their causal context in the continued sequence: their tree K/V
 * rows, root first, become cache rows cu_prefix[s] + P_s .. cu_prefix[s] + P_s + a,
 * and prefix_len[s] becomes P_s + a + 1.  The next round's root is the walk's
 * bonus_out.
 *
 * k_cache, v_cache   [rows, Hkv, D] (dtype), written in place; 16-byte aligned.
 * cu_prefix          [S+1]: sequence s owns rows cu_prefix[s] .. cu_prefix[s+1].
 * prefix_len         [S] int64, read and advanced in place.
 * k_tree, v_tree     [S, N, Hkv, D] (dtype) as given to ddt_tree_attention; 16-byte aligned.
 * acc_nodes [S, L], accept_len [S]: from ddt_tree_walk.
 * appended           nullable [S] int32: rows appended (a + 1), or -1 when the
 *                    sequence's room cannot take them or its walk outputs are out of
 *                    range; such a sequence's cache and prefix_len are left unchanged.
 * 1 <= S, 0 <= B <= DDT_MAX_B, 1 <= L <= DDT_MAX_L, Hkv >= 1, D in {32, 64, 128}.
 * Errors: null required pointer, unaligned cache or tree pointer, size out of range
 *         (DDT_ERR_INVALID_ARG); D or dtype without a kernel (DDT_ERR_UNSUPPORTED).
 */
int ddt_commit_kv(void* k_cache, void* v_cache, const int64_t* cu_prefix, int64_t* prefix_len,
                  const void* k_tree, const void* v_tree, const int32_t* acc_nodes,
                  const int32_t* accept_len, int S, int B, int L, int Hkv, int D, int dtype,
                  int32_t* appended, void* stream);

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
 *           (completion counters, arg-max keys, the hybrid walk's hand-off state and
 *           subtree rows).  Calls that share a workspace must not overlap.
 * Errors: null pointer; S < 1; L outside [1, DDT_MAX_L]; B outside [0, DDT_MAX_B];
 *         vocab < 1 or > INT32_MAX; ws too small.
 */
size_t ddt_tree_walk_workspace_size(int S, int B, int64_t vocab);
int ddt_tree_walk(const int32_t* tree_tok, const int32_t* parent, const int32_t* num_nodes,
                  const float* target_logits, int S, int B, int L, int64_t vocab,
                  int32_t* accept_len, int32_t* acc_nodes, int32_t* acc_tok, int32_t* bonus_out,
                  void* ws, size_t ws_bytes, void* stream);

/* Strategy of ddt_tree_walk, ddt_tree_walk_sample and ddt_tree_walk_noalloc, for the
 * whole process (all give identical outputs; the walk's result depends only on the
 * rows of the nodes it visits):
 *   DDT_WALK_AUTO   (0)  the library chooses per call (the default);
 *   DDT_WALK_SCAN   (1)  arg-max of every node's row by many workgroups, then the walk;
 *   DDT_WALK_PATH   (2)  one workgroup per sequence follows the walk and scans only the
 *                        rows of the nodes it visits (at most L + 1 rows, one after
 *                        another), leaving the workspace untouched;
 *   DDT_WALK_HYBRID (3)  the path walk for up to 3 accepted tokens; a sequence whose
 *                        walk goes on is handed to the scan, which reads only the rows
 *                        of the reached node's subtree and finishes the walk.
 * AUTO takes PATH where it is expected to beat the full scan with half the block
 * accepted (many long rows: S * (B + 1) rows of a large vocabulary), SCAN where the
 * full scan is short, and HYBRID in between.  Returns the previous strategy, or
 * DDT_ERR_INVALID_ARG for a value outside 0..3 (the strategy is then unchanged).  Not
 * synchronised with calls in flight on other threads.
 */
#define DDT_WALK_AUTO 0
#define DDT_WALK_SCAN 1
#define DDT_WALK_PATH 2
#define DDT_WALK_HYBRID 3
int ddt_tree_walk_strategy(int mode);

/* The strategy (DDT_WALK_SCAN, DDT_WALK_PATH or DDT_WALK_HYBRID) that a walk call of
 * this shape would use now: the forced one if ddt_tree_walk_strategy set one, else the
 * planner's choice.  No device access.  Errors: the shape errors of ddt_tree_walk.
 */
int ddt_tree_walk_mode(int S, int B, int L, int64_t vocab);

/* ---------------------------------------------------------------- step 5 at temperature > 0
 * Tree walk under the target's sampling rule at temperature T > 0 (中文摘要 counts
 * temperature among the evaluated settings; 運作流程 step 4 follows the target's
 * decoding rule): the target's token at node n is a draw from softmax(logits / T),
 * taken by the Gumbel-max rule,
 *   token(n) = argmax_v  fl( fl(target_logits[s, n, v] * inv_temperature)
 *                            + gumbel[s, depth[s, n], v] ),
 * each fp32 multiply and add rounded on its own (no fused multiply-add), equal scores
 * to the smaller token id (-0 and +0 equal).  The walk then proceeds as ddt_tree_walk.
 * The noise row is chosen by the node's depth, so every node of a depth shares it and
 * the walk emits exactly the tokens that plain one-token-at-a-time sampling with the
 * same noise emits (lossless).
 *
 * depth            [S, N] from ddt_build_tree.
 * gumbel           [S, L + 1, vocab] fp32 standard Gumbel draws, the caller's random
 *                  numbers for this round (row d serves depth d); finite.
 * inv_temperature  1 / T as an fp32 value, finite and >= 0 (0 samples uniformly).
 * Other arguments, outputs, workspace (the same size) and errors as ddt_tree_walk.
 */
int ddt_tree_walk_sample(const int32_t* tree_tok, const int32_t* parent, const int32_t* depth,
                         const int32_t* num_nodes, const float* target_logits, const float* gumbel,
                         float inv_temperature, int S, int B, int L, int64_t vocab,
                         int32_t* accept_len, int32_t* acc_nodes, int32_t* acc_tok,
                         int32_t* bonus_out, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- step 5, no allocation
 * ddt_tree_walk without a workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Arguments, outputs and errors are those of ddt_tree_walk; the kernels
 * are the same.  Its workspace is a static device array of the library,
 * ddt_tree_walk_noalloc_max_bytes() = 1 MiB, of which a call needs
 * ddt_tree_walk_workspace_size(S, B, vocab) bytes (each part 256-byte-rounded: 4 and
 * 16 bytes per sequence, 4 + 8 + 4 bytes per node row: S * (B + 1) rows up to about
 * 65000).  A larger problem returns DDT_ERR_TOO_LARGE before any launch.
 * Each GPU the library runs on holds its own copy of the array until the process
 * ends.  The first call on a device looks up the array's address there and enqueues
 * a zero fill of it on `stream` ahead of the walk; every walk leaves the part it used
 * zero-filled again.  All calls on one GPU share that array: calls that may overlap
 * on one GPU (different streams, or concurrently replayed graphs) race and must be
 * ordered by the caller.  The call allocates nothing: no hipMalloc, no hipFree.
 */
size_t ddt_tree_walk_noalloc_max_bytes(void);
int ddt_tree_walk_noalloc(const int32_t* tree_tok, const int32_t* parent, const int32_t* num_nodes,
                          const float* target_logits, int S, int B, int L, int64_t vocab,
                          int32_t* accept_len, int32_t* acc_nodes, int32_t* acc_tok,
                          int32_t* bonus_out, void* stream);

/* ---------------------------------------------------------------- verifier epilogue
 * The target's last layer and greedy choice at every tree node without storing the
 * logits: the tree is scored in one target forward (運作流程 step 3) and the walk
 * needs only each node's greedy token (step 4).  Node n's logits are its final hidden
 * state times the LM-head weight, logit_v = h_n . w_v, and its token is their
 * arg-max, equal values to the smaller id.
 *
 * hidden     [S, N, d] bf16 (N = B + 1), 16-byte aligned: final hidden states.
 * weight     [V, d] bf16 (V = vocab), 16-byte aligned: one row per vocabulary entry.
 * num_nodes  nullable [S]: nodes n >= num_nodes[s] are padding (token -1, max -inf);
 *            every row is still multiplied, so padding rows must hold finite values
 *            or their (unused) products may be anything.
 * node_tok   [S, N] int32 out: arg-max_v of the fp32 logits (bf16 products, fp32 sums).
 * node_max   nullable [S, N] fp32 out: that logit.
 * d          multiple of 64, 64 <= d <= 65536; 1 <= vocab <= 2^31 - 512;
 *            1 <= S, 0 <= B <= DDT_MAX_B.  Logits must not overflow fp32.
 * ws         at least ddt_lm_head_argmax_workspace_size(S, B, vocab, d) bytes: the
 *            partial arg-max of each (node, 256-entry vocabulary tile).  Contents are
 *            ignored.
 * Errors: null required pointer, unaligned hidden or weight, size out of range
 *         (DDT_ERR_INVALID_ARG); d not a multiple of 64 (DDT_ERR_UNSUPPORTED); ws_bytes
 *         too small (DDT_ERR_WORKSPACE).
 */
size_t ddt_lm_head_argmax_workspace_size(int S, int B, int64_t vocab, int d);
int ddt_lm_head_argmax(const void* hidden, const void* weight, const int32_t* num_nodes, int S,
                       int B, int d, int64_t vocab, int32_t* node_tok, float* node_max, void* ws,
                       size_t ws_bytes, void* stream);

/* Tree walk of 運作流程 step 4 driven by given per-node target tokens (from
 * ddt_lm_head_argmax): from the root, while a child of the current node (the smallest
 * index first) carries the current node's token, accept it and move there; the token
 * at the node where the walk stops is the next round's bonus.  Inputs and outputs as
 * ddt_tree_walk, with node_tok [S, N] int32 in place of the logits.
 * Errors: null pointer; S < 1; L outside [1, DDT_MAX_L]; B outside [0, DDT_MAX_B].
 */
int ddt_tree_walk_tokens(const int32_t* tree_tok, const int32_t* parent, const int32_t* num_nodes,
                         const int32_t* node_tok, int S, int B, int L, int32_t* accept_len,
                         int32_t* acc_nodes, int32_t* acc_tok, int32_t* bonus_out, void* stream);

/* ---------------------------------------------------------------- benchmark aid
 * Timing of the attention step (the round's dominant cost) with HIP events on the
 * stream it runs on.  While profiling is on, every ddt_tree_attention call attaches
 * a start/stop event pair to its main kernel's dispatch (hipExtLaunchKernelGGL), so
 * the pair brackets that kernel's execution, and a third event to the stop of the
 * split-merge kernel that completes the step (for fp32 inputs the step is the one
 * kernel).  Use it on eagerly launched calls: events recorded during a HIP graph
 * capture are not readable afterwards.  ddt_attention_timing waits for the recorded
 * calls and returns, summed over them in milliseconds, the main kernel's time and
 * the whole step's (main kernel start to merge end), with their count, and forgets
 * them.  ddt_attention_profiling(0) releases the events.  This is the only state
 * the library keeps; it is process-wide and guarded by a mutex.
 * Returns DDT_OK, DDT_ERR_INVALID_ARG (null pointer) or DDT_ERR_HIP.
 */
int ddt_attention_profiling(int enable);
int ddt_attention_timing(double* main_ms, double* step_ms, int* count);

/* The same for the verifier epilogue's tile kernel (the LM-head product and the
 * per-tile arg-max; the per-node reduce that follows is not included):
 * ddt_lm_head_timing returns the summed milliseconds and the count of the recorded
 * ddt_lm_head_argmax calls since the last read.  Same rules and errors as above.
 */
int ddt_lm_head_profiling(int enable);
int ddt_lm_head_timing(double* tiles_ms, int* count);

#ifdef __cplusplus
}
#endif
#endif /* DDT_H_ */
