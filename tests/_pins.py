"""Independent checkers used as pins of the oracle's tree builder.

Neither calls into the oracle's heap: one enumerates every valid tree, the other
solves the budgeted tree problem by dynamic programming over the factorised draft
(the DDTree page, 理論基礎: each position's marginal depends on the context before
the block only, so all subtrees rooted at one depth face the same marginals).
"""
from typing import List, Tuple

import numpy as np


def candidate_tree(L: int, K: int) -> Tuple[List[tuple], List[int]]:
    """Rank paths of the K-ary depth-L candidate tree in breadth-first order, and
    each one's parent index (-1 for depth-1 nodes, whose parent is the root)."""
    paths: List[tuple] = []
    parents: List[int] = []
    level = [((), -1)]
    for _ in range(L):
        nxt = []
        for p, _pi in level:
            pidx = paths.index(p) if p else -1
            for r in range(K):
                paths.append(p + (r,))
                parents.append(pidx)
                nxt.append((p + (r,), None))
        level = nxt
    return paths, parents


def brute_force_best(prob: np.ndarray, parents: List[int], B: int):
    """Every prefix-closed set of exactly B candidates; returns (best value, the
    maximising sets, number of sets).  Sets are grown in increasing breadth-first
    index, each new node's parent already present, so each set is visited once."""
    n = len(parents)
    children = [[] for _ in range(n + 1)]  # slot n = the root
    for i, p in enumerate(parents):
        children[n if p < 0 else p].append(i)
    best = [-1.0, [], 0]
    chosen: List[int] = []

    def rec(avail: List[int], last: int, value: float):
        if len(chosen) == B:
            best[2] += 1
            if value > best[0] + 1e-12:
                best[0], best[1] = value, [tuple(chosen)]
            elif abs(value - best[0]) <= 1e-12:
                best[1].append(tuple(chosen))
            return
        for j, i in enumerate(avail):
            if i <= last:
                continue
            chosen.append(i)
            rec(sorted(avail[j + 1:] + children[i]), i, value + prob[i])
            chosen.pop()

    rec(sorted(children[n]), -1, 0.0)
    return best[0], best[1], best[2]


def dp_optimum(q: np.ndarray, B: int) -> float:
    """max over prefix-closed trees with <= B non-root nodes of the sum of prefix
    probabilities, q [L, K] the per-position candidate probabilities.

    f_L(b) = 0; a node at depth d with b descendants to place splits them among its
    K children: f_d(b) = max over b_0+..+b_{K-1} = b of sum over children with
    b_r >= 1 of q[d, r] * (1 + f_{d+1}(b_r - 1)).  Returns f_0(B).
    """
    L, K = q.shape
    f_next = np.zeros(B + 1)
    cc, bb = np.meshgrid(np.arange(B + 1), np.arange(B + 1))  # bb: total, cc: given to child
    valid = cc <= bb
    for d in range(L - 1, -1, -1):
        g = np.zeros(B + 1)
        for r in range(K):
            gain = np.zeros(B + 1)
            gain[1:] = q[d, r] * (1.0 + f_next[:B])
            tot = np.where(valid, g[np.clip(bb - cc, 0, B)] + gain[cc], -np.inf)
            g = tot.max(axis=1)
        f_next = g
    return float(f_next[B])
