"""Several verification rounds in a row, with the KV cache carried between them.

TEST INFRASTRUCTURE (see ``oracle/ddtree.py``): imported only by the tests, the
smoke check and the bench's CPU-baseline leg.

Source: the DDTree page ("策展 · X (Twitter)", easyvibecoding.app/curated/665),
section 運作流程: a round starts from a bonus token b that the target produced but has
not yet run forward; step 3 runs the whole tree through the target in one forward;
step 4 walks it and carries the first mismatch into the next round as its bonus.
The page does not spell out what happens to the cache between rounds; the readings
taken here:
  [R22] After a round, the root b and the accepted nodes n_1..n_a have been run
        through the target, each attending to exactly the prefix and its own
        ancestors, which is their causal context in the continued sequence.  Their
        K/V rows, in path order (root first), are appended to the sequence's cache.
        The new bonus token has not been run forward; it is the next round's root.
  [R23] The next round's prefix therefore holds P + a + 1 rows, and its nodes sit at
        positions P + a + 1 + depth.
"""
from typing import Callable, Dict, List, Sequence, Tuple

import numpy as np

from . import ddtree
from .round import widen


def commit_kv(k_prefix: np.ndarray, v_prefix: np.ndarray, k_tree: np.ndarray, v_tree: np.ndarray,
              acc_nodes: np.ndarray, accept_len: int) -> Tuple[np.ndarray, np.ndarray]:
    """[R22] The cache after a round: the prefix rows [P, Hkv, D] followed by the tree
    K/V rows [N, Hkv, D] of the root and the accepted nodes, root first.  A copy:
    the arrays keep their dtype (bfloat16 encodings stay encodings)."""
    rows = [0] + [int(n) for n in np.asarray(acc_nodes)[:int(accept_len)]]
    return (np.concatenate([k_prefix, k_tree[rows]], axis=0),
            np.concatenate([v_prefix, v_tree[rows]], axis=0))


def greedy_decode(target_fn: Callable[[List[int]], np.ndarray], g: Sequence[int], n: int) -> List[int]:
    """Plain decoding, one token at a time: append the target's greedy token n times.
    target_fn(g) gives the target's next-token logits after the generated tokens g."""
    g = list(g)
    out = []
    for _ in range(n):
        t = ddtree.greedy_token(target_fn(g))
        out.append(t)
        g.append(t)
    return out


def run_rounds(draft_fn: Callable[[List[int]], np.ndarray],
               inputs_fn: Callable[[List[int], Dict[str, np.ndarray]], Dict[str, np.ndarray]],
               k_prefix: np.ndarray, v_prefix: np.ndarray, b0: int, K: int, B: int, rounds: int,
               scale: float, attention_rows: Sequence[Tuple[int, int]] = None) -> Tuple[List[int], List[Dict]]:
    """``rounds`` verification rounds of one sequence, each a full round of
    ddtree's steps followed by the cache commit [R22].

    draft_fn(g) -> the round's draft logits [L, V] given the generated tokens g (g
    ends with the round's bonus token).  inputs_fn(g, tree) -> {q [N,Hq,D], k_tree,
    v_tree [N,Hkv,D], target [N,V]}: the verifier's inputs at the tree.  The cache
    starts as k_prefix/v_prefix [P0, Hkv, D].  attention_rows restricts the attention
    to those (node, head) rows.
    Returns the generated tokens (b0 and everything emitted) and one record per round
    (its tree, mask, positions, attention, walk and the cache length after commit).
    """
    g = [int(b0)]
    kc, vc = k_prefix, v_prefix
    records = []
    for _ in range(rounds):
        logits = draft_fn(g)
        L = logits.shape[0]
        tok, lq = ddtree.topk(logits, K)
        tree = ddtree.build_tree(tok, lq, g[-1], B)
        nn = int(tree["num_nodes"])
        x = inputs_fn(g, tree)
        mask = ddtree.tree_mask(tree["parent"], nn, B + 1)
        P = kc.shape[0]
        pos = ddtree.position_ids(tree["depth"], nn, P)
        o, lse = ddtree.tree_attention(widen(x["q"]), widen(kc), widen(vc), widen(x["k_tree"]),
                                       widen(x["v_tree"]), mask, nn, scale, attention_rows)
        walk = ddtree.tree_walk(tree["tree_tok"], tree["parent"], nn, x["target"], L)
        kc, vc = commit_kv(kc, vc, x["k_tree"], x["v_tree"], walk["acc_nodes"], walk["accept_len"])
        a = int(walk["accept_len"])
        emitted = [int(tree["tree_tok"][n]) for n in walk["acc_nodes"][:a]] + [int(walk["bonus"])]
        records.append(dict(context=list(g), topk_tok=tok, topk_logq=lq, mask=mask, pos_ids=pos,
                            prefix_len=P, o=o, lse=lse, emitted=emitted, k_cache=kc, v_cache=vc,
                            **tree, **walk))
        g.extend(emitted)
    return g, records
