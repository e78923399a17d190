"""Plain CPU fp64 oracle of one DDTree verification round.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the bench's CPU-baseline
leg may import this module.  It shares no code with the HIP path; both take their
inputs from the seeded generator in ``ddt_synthetic``.

Source of the method: the DDTree page ("策展 · X (Twitter)",
easyvibecoding.app/curated/665), a summary of Liran Ringel and Yaniv Romano's
DDTree.  Sections are cited by their headings:
  核心創新 (core innovation), 運作流程 (procedure, steps 1-4), 理論基礎 (theory,
  Propositions 1 and 2).
Readings where the page leaves a step open are marked [R#]; the list is kept with
the design notes of this repository.

Every step is the plain definition, in fp64, one sequence at a time:
  topk            log-softmax of the draft logits, K best tokens per position
  build_tree      best-first heap over draft prefixes under a node budget B
  tree_mask       ancestor-only visibility as a per-node bitmask
  tree_attention  softmax(scale * q k^T) v over prefix keys plus visible tree keys
  tree_walk       greedy walk of the target's argmax through the tree
"""
import heapq
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np


# ============================================================================ step 1
def softmax_topk_row(x_row: np.ndarray, k: int) -> Tuple[np.ndarray, np.ndarray, float]:
    """One position's draft marginal q_i (運作流程 step 1) and its K best tokens.

    [R1] q_i is the softmax of the draft logits over the full vocabulary at
    temperature 1; the K kept log-probabilities are not renormalised.
    [R2] Order is by logit descending, equal logits by smaller token id.
    Returns (token ids [k], log q_i(token) [k], log-sum-exp of the row).
    """
    x = np.asarray(x_row, dtype=np.float64)
    m = np.max(x)
    lse = float(m + np.log(np.sum(np.exp(x - m))))
    ids = np.arange(x.size)
    order = np.lexsort((ids, -x))  # last key is primary: -x ascending, then id ascending
    tok = order[:k]
    return tok.astype(np.int64), x[tok] - lse, lse


def topk(logits: np.ndarray, k: int) -> Tuple[np.ndarray, np.ndarray]:
    """Rows of logits [rows, V] -> (tok [rows, k] int32, logq [rows, k] fp64)."""
    logits = np.asarray(logits)
    rows = logits.reshape(-1, logits.shape[-1])
    tok = np.empty((rows.shape[0], k), dtype=np.int32)
    lq = np.empty((rows.shape[0], k), dtype=np.float64)
    for r in range(rows.shape[0]):
        t, l, _ = softmax_topk_row(rows[r], k)
        tok[r], lq[r] = t, l
    return tok.reshape(logits.shape[:-1] + (k,)), lq.reshape(logits.shape[:-1] + (k,))


# ============================================================================ step 2
def best_first_prefixes(logq: np.ndarray, B: int) -> List[Tuple[Tuple[int, ...], float]]:
    """The best-first heap of 核心創新 / 運作流程 step 2, in pop order.

    A candidate is a rank path (r_1..r_d): the r_i-th best token at position i, with
    1 <= d <= L [R4: the candidate tree is the K-ary tree of per-position top-K
    tokens].  Its log-probability under the factorised draft (理論基礎) is
    sum_i log q_i(r_i).  The heap starts from the root's children, pops the most
    probable candidate, and pushes that candidate's K children, until B candidates
    have been taken [R3: B counts non-root nodes].  Ties pop shallower first, then
    the lexicographically smaller rank path.
    Returns [(rank path, log-probability)] in pop order.
    """
    L, K = logq.shape
    heap = [(-float(logq[0, r]), 1, (r,)) for r in range(K)]
    heapq.heapify(heap)
    taken: List[Tuple[Tuple[int, ...], float]] = []
    while len(taken) < B and heap:
        neg, d, path = heapq.heappop(heap)
        taken.append((path, -neg))
        if d < L:
            for r in range(K):
                heapq.heappush(heap, (neg - float(logq[d, r]), d + 1, path + (r,)))
    return taken


def build_tree(tok: np.ndarray, logq: np.ndarray, bonus: int, B: int) -> Dict[str, np.ndarray]:
    """The draft tree of one sequence in canonical order.

    Node 0 is the root, the bonus token b (運作流程, opening paragraph), with
    parent -1 and depth 0.  [R5] The B selected prefixes follow, ordered by
    (depth, parent's index, sibling rank): parents precede children and a parent's
    children are contiguous, most probable first.  The order depends only on the
    selected set.
    Arrays have B+1 entries; entries past num_nodes (a candidate tree smaller than
    B) hold tok/parent/depth/rank = -1 and logq = -inf.
    """
    L, K = tok.shape
    N = B + 1
    taken = best_first_prefixes(logq, B)
    score = {p: lp for p, lp in taken}
    # canonical order, one depth at a time
    order: List[Tuple[int, ...]] = [()]
    index = {(): 0}
    depth = 1
    while True:
        level = [p for p in score if len(p) == depth]
        if not level:
            break
        level.sort(key=lambda p: (index[p[:-1]], p[-1]))
        for p in level:
            index[p] = len(order)
            order.append(p)
        depth += 1
    out = {
        "tree_tok": np.full(N, -1, dtype=np.int32),
        "parent": np.full(N, -1, dtype=np.int32),
        "depth": np.full(N, -1, dtype=np.int32),
        "rank": np.full(N, -1, dtype=np.int32),
        "node_logq": np.full(N, -np.inf, dtype=np.float64),
    }
    for n, p in enumerate(order):
        d = len(p)
        out["depth"][n] = d
        if d == 0:
            out["tree_tok"][n] = bonus
            out["node_logq"][n] = 0.0
        else:
            out["tree_tok"][n] = tok[d - 1, p[-1]]
            out["parent"][n] = index[p[:-1]]
            out["rank"][n] = p[-1]
            out["node_logq"][n] = score[p]
    out["num_nodes"] = np.int32(len(order))
    return out


# ============================================================================ step 3
def ancestors(parent: np.ndarray, n: int) -> List[int]:
    """Node n and every node on its path to the root, root first."""
    chain = []
    while n >= 0:
        chain.append(n)
        n = int(parent[n])
    return chain[::-1]


def tree_mask(parent: np.ndarray, num_nodes: int, N: int) -> np.ndarray:
    """Ancestor-only attention mask (核心創新; 運作流程 step 3) as bits.

    [R6] Node n sees its ancestors and itself (the whole prefix context is visible
    to every node and is not part of the mask).  Bit j of word j // 32 of row n is
    set iff node j is visible to node n.  Rows past num_nodes are zero.
    """
    W = (N + 31) // 32
    mask = np.zeros((N, W), dtype=np.uint32)
    for n in range(num_nodes):
        for j in ancestors(parent, n):
            mask[n, j // 32] |= np.uint32(1 << (j % 32))
    return mask


def position_ids(depth: np.ndarray, num_nodes: int, prefix_len: int) -> np.ndarray:
    """[R7] A node at depth d sits at position P + d; -1 past num_nodes."""
    pos = np.full(depth.shape[0], -1, dtype=np.int32)
    pos[:num_nodes] = prefix_len + depth[:num_nodes]
    return pos


def visible_nodes(mask_row: np.ndarray, N: int) -> List[int]:
    return [j for j in range(N) if (int(mask_row[j // 32]) >> (j % 32)) & 1]


# ============================================================================ step 4
def attend(q: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float) -> Tuple[np.ndarray, float]:
    """softmax(scale * keys @ q) @ values for one query row, fp64.
    Returns (output [D], natural-log log-sum-exp of the scaled scores)."""
    if keys.shape[0] == 0:
        return np.zeros(values.shape[1]), float("-inf")
    s = scale * (keys @ q)
    m = np.max(s)
    e = np.exp(s - m)
    z = np.sum(e)
    return (e @ values) / z, float(m + np.log(z))


def tree_attention(q: np.ndarray, k_prefix: np.ndarray, v_prefix: np.ndarray,
                   k_tree: np.ndarray, v_tree: np.ndarray, mask: np.ndarray, num_nodes: int,
                   scale: float, rows: Optional[Sequence[Tuple[int, int]]] = None):
    """Tree attention of one sequence (運作流程 step 3: the whole tree is scored in
    one target forward under the ancestor-only mask).

    q [N,Hq,D]; k_prefix, v_prefix [P,Hkv,D]; k_tree, v_tree [N,Hkv,D]; mask [N,W].
    [R8] scale is the caller's (1/sqrt(D) in the workloads).  [R9] query head h
    reads KV head h // (Hq // Hkv).  Keys are the prefix followed by the visible
    tree nodes.  Rows past num_nodes get output 0 and lse -inf.
    With ``rows`` = [(n, h), ...] only those rows are computed and returned as
    ([len, D], [len]); otherwise ([N,Hq,D], [N,Hq]).
    """
    q = np.asarray(q, dtype=np.float64)
    N, Hq, D = q.shape
    Hkv = k_prefix.shape[1]
    G = Hq // Hkv
    kp = np.asarray(k_prefix, dtype=np.float64)
    vp = np.asarray(v_prefix, dtype=np.float64)
    kt = np.asarray(k_tree, dtype=np.float64)
    vt = np.asarray(v_tree, dtype=np.float64)

    def one(n: int, h: int):
        if n >= num_nodes:
            return np.zeros(D), float("-inf")
        vis = visible_nodes(mask[n], N)
        g = h // G
        keys = np.concatenate([kp[:, g, :], kt[vis, g, :]], axis=0)
        vals = np.concatenate([vp[:, g, :], vt[vis, g, :]], axis=0)
        return attend(q[n, h], keys, vals, scale)

    if rows is not None:
        o = np.zeros((len(rows), D))
        lse = np.zeros(len(rows))
        for i, (n, h) in enumerate(rows):
            o[i], lse[i] = one(n, h)
        return o, lse
    o = np.zeros((N, Hq, D))
    lse = np.full((N, Hq), -np.inf)
    for n in range(num_nodes):
        for h in range(Hq):
            o[n, h], lse[n, h] = one(n, h)
    return o, lse


# ============================================================================ step 5
def greedy_token(logits_row: np.ndarray) -> int:
    """[R11] The greedy target rule: argmax, equal logits to the smaller id."""
    x = np.asarray(logits_row, dtype=np.float64)
    return int(np.flatnonzero(x == np.max(x))[0])


def tree_walk(tree_tok: np.ndarray, parent: np.ndarray, num_nodes: int,
              target_logits: np.ndarray, L: int) -> Dict[str, np.ndarray]:
    """Tree walk of 運作流程 step 4 under greedy decoding.

    From the root, take the target's token at the current node; if a child carries
    that token, accept the child and continue from it; otherwise stop, and the
    target's token becomes the next round's bonus.  [R12] A node at depth L has no
    children, so the walk ends there.  [R13] accept_len counts accepted draft
    nodes; a round emits accept_len + 1 tokens.  If two children carry the wanted
    token (impossible in a tree built from distinct top-K tokens) the one with the
    smaller index is taken.
    Returns accept_len, acc_nodes [L] and acc_tok [L] (-1 padded), bonus.
    """
    cur = 0
    acc: List[int] = []
    while True:
        want = greedy_token(target_logits[cur])
        nxt = -1
        for c in range(num_nodes):
            if int(parent[c]) == cur and int(tree_tok[c]) == want:
                nxt = c
                break
        if nxt < 0:
            bonus = want
            break
        acc.append(nxt)
        cur = nxt
    acc_nodes = np.full(L, -1, dtype=np.int32)
    acc_tok = np.full(L, -1, dtype=np.int32)
    acc_nodes[:len(acc)] = acc
    acc_tok[:len(acc)] = [int(tree_tok[n]) for n in acc]
    return {"accept_len": np.int32(len(acc)), "acc_nodes": acc_nodes, "acc_tok": acc_tok,
            "bonus": np.int32(bonus)}


# ============================================================================ step 5 at temperature > 0
def sample_token(logits_row: np.ndarray, gumbel_row: np.ndarray, inv_temperature: float) -> int:
    """The target's decoding rule at temperature T > 0 (中文摘要 counts temperature
    among the evaluated settings; 運作流程 step 4 follows the target's decoding rule):
    a draw from softmax(logits / T).  [R24] It is taken by the Gumbel-max rule: with
    g_v independent standard Gumbel draws, argmax_v (x_v / T + g_v) is distributed as
    softmax(x / T).  The scores are formed in fp32 as fl(fl(x_v * t) + g_v) with
    t = 1/T given as an fp32 value (the precision the kernel decides in); equal scores
    go to the smaller id."""
    x = np.asarray(logits_row, dtype=np.float32)
    g = np.asarray(gumbel_row, dtype=np.float32)
    y = (x * np.float32(inv_temperature)).astype(np.float32) + g
    y = y.astype(np.float32)
    return int(np.flatnonzero(y == np.max(y))[0])


def tree_walk_sample(tree_tok: np.ndarray, parent: np.ndarray, depth: np.ndarray, num_nodes: int,
                     target_logits: np.ndarray, gumbel: np.ndarray, inv_temperature: float,
                     L: int) -> Dict[str, np.ndarray]:
    """Tree walk of 運作流程 step 4 at temperature > 0: as tree_walk, but the target's
    token at node n is sample_token(target_logits[n], gumbel[depth[n]], t).  [R24]
    The noise row is chosen by depth, not by node, so the walk emits exactly the
    tokens that plain one-token-at-a-time sampling with the same noise emits."""
    cur = 0
    acc: List[int] = []
    while True:
        want = sample_token(target_logits[cur], gumbel[int(depth[cur])], inv_temperature)
        nxt = -1
        for c in range(num_nodes):
            if int(parent[c]) == cur and int(tree_tok[c]) == want:
                nxt = c
                break
        if nxt < 0:
            bonus = want
            break
        acc.append(nxt)
        cur = nxt
    acc_nodes = np.full(L, -1, dtype=np.int32)
    acc_tok = np.full(L, -1, dtype=np.int32)
    acc_nodes[:len(acc)] = acc
    acc_tok[:len(acc)] = [int(tree_tok[n]) for n in acc]
    return {"accept_len": np.int32(len(acc)), "acc_nodes": acc_nodes, "acc_tok": acc_tok,
            "bonus": np.int32(bonus)}


# ============================================================================ adaptive budget
def score_order(node_logq: np.ndarray, num_nodes: int) -> List[int]:
    """The tree's non-root nodes in the heap's pop order: log-probability descending,
    equal values by canonical index (shallower first, then lexicographic rank path,
    which is the canonical order within a depth [R5])."""
    return sorted(range(1, num_nodes), key=lambda n: (-float(node_logq[n]), n))


def choose_budget(node_logq: np.ndarray, num_nodes: int, cost: np.ndarray) -> Tuple[int, float]:
    """[R25] The budget B* <= num_nodes - 1 that maximises tokens per unit of verify
    cost, (E[accept](b) + 1) / cost[b] (實驗結果與權衡: speedup peaks at an
    intermediate budget; 理論基礎 Prop. 1: E[accept](b) is the sum of the b largest
    prefix probabilities, the first b pops of the heap).  cost[b] > 0 is the caller's
    verify cost at budget b.  Sums and ratios in fp64; equal ratios to the smaller b.
    Returns (B*, E[accept](B*))."""
    order = score_order(node_logq, num_nodes)
    e = 0.0
    best_b, best_j, best_e = 0, (0.0 + 1.0) / float(cost[0]), 0.0
    for b in range(1, num_nodes):
        e += float(np.exp(float(node_logq[order[b - 1]])))
        j = (e + 1.0) / float(cost[b])
        if j > best_j:
            best_b, best_j, best_e = b, j, e
    return best_b, best_e


def prune_tree(tree: Dict[str, np.ndarray], b: int) -> Dict[str, np.ndarray]:
    """The tree cut to its b most probable prefixes (the first b pops): they are
    prefix-closed (Prop. 2), and keeping the survivors in their canonical order keeps
    the order canonical [R5].  Arrays keep their length; the rest is padding."""
    nn = int(tree["num_nodes"])
    keep = [0] + sorted(score_order(tree["node_logq"], nn)[:b])
    new = {old: i for i, old in enumerate(keep)}
    N = tree["tree_tok"].shape[0]
    out = {"tree_tok": np.full(N, -1, dtype=np.int32), "parent": np.full(N, -1, dtype=np.int32),
           "depth": np.full(N, -1, dtype=np.int32), "node_logq": np.full(N, -np.inf, dtype=np.float64)}
    for i, old in enumerate(keep):
        out["tree_tok"][i] = tree["tree_tok"][old]
        out["depth"][i] = tree["depth"][old]
        out["node_logq"][i] = tree["node_logq"][old]
        p = int(tree["parent"][old])
        out["parent"][i] = -1 if p < 0 else new[p]
    out["num_nodes"] = np.int32(len(keep))
    return out


# ============================================================================ helpers for tests
def candidate_logprobs(logq: np.ndarray) -> np.ndarray:
    """Log-probability of every candidate prefix of the K-ary depth-L candidate
    tree (理論基礎: the factorised draft probability of a prefix is the product of
    its positions' marginals).  Only for tiny L and K."""
    L, K = logq.shape
    out = []
    level = [0.0]
    for d in range(L):
        level = [lp + float(logq[d, r]) for lp in level for r in range(K)]
        out.extend(level)
    return np.array(out)


def selection_gap(logq: np.ndarray, B: int) -> float:
    """log-prob of the B-th selected prefix minus that of the best unselected one
    (+inf when B = 0 or the candidate tree holds at most B prefixes)."""
    if B <= 0:
        return float("inf")
    taken = best_first_prefixes(logq, B + 1)
    if len(taken) <= B:
        return float("inf")
    return taken[B - 1][1] - taken[B][1]


def expected_acceptance(node_logq: np.ndarray, num_nodes: int) -> float:
    """Proposition 1 (理論基礎): the surrogate objective of a tree is the sum of its
    non-root nodes' prefix probabilities."""
    return float(np.sum(np.exp(node_logq[1:num_nodes])))
