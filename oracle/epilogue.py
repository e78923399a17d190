"""Plain CPU fp64 oracle of the verifier epilogue: the target's LM head and its greedy
token at every tree node, and the tree walk driven by those tokens.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the bench's CPU-baseline
leg may import this module.  It shares no code with the HIP path.

Source: the DDTree page ("策展 · X (Twitter)", easyvibecoding.app/curated/665).  The
target scores the whole tree in one forward (運作流程 step 3) and the walk follows its
greedy choice at each node (step 4).  The page says nothing of the target's last
layer; the reading here ([R26], kept with the design notes) is the standard one: a
node's next-token logits are its final hidden state h [d] times the LM-head
(output-embedding) weight W [V, d], logit_v = h . w_v, and the greedy token is their
arg-max, equal logits to the smaller id ([R11]).

Precision.  The operands are bfloat16 values.  A product of two of them has at most
16 significant bits, so every product is exact in fp64, and a sum of d <= 2^16 such
products carries a relative error below d * 2^-53 (1e-12 at d = 8192): the values
returned are the exact logits to far better than the fp32 the kernel decides in.
"""
from typing import Dict, List, Tuple

import numpy as np

U32 = 2.0 ** -24  # unit roundoff of fp32


def lm_head_logits(hidden, weight, chunk: int = 4096) -> np.ndarray:
    """Logits [M, V] in fp64: hidden [M, d] times weight [V, d] transposed.

    ``weight`` is anything that slices by vocabulary rows into float arrays (a
    [V, d] array, or a view that decodes bfloat16 rows on demand); it is read
    ``chunk`` rows at a time so that a full-size weight never needs an fp64 copy."""
    h = np.asarray(hidden, dtype=np.float64)
    V = weight.shape[0]
    out = np.empty((h.shape[0], V), dtype=np.float64)
    for lo in range(0, V, chunk):
        w = np.asarray(weight[lo:lo + chunk], dtype=np.float64)
        out[:, lo:lo + w.shape[0]] = h @ w.T
    return out


def lm_head_argmax(hidden, weight, chunk: int = 4096) -> Tuple[np.ndarray, np.ndarray]:
    """Greedy token [M] (int64) and its logit [M] (fp64) per row: the arg-max of the
    row's logits, equal logits to the smaller id."""
    x = lm_head_logits(hidden, weight, chunk)
    tok = np.argmax(x, axis=1)  # the first (smallest) index among equal maxima
    return tok, x[np.arange(x.shape[0]), tok]


def top_two(logits_row: np.ndarray) -> Tuple[int, float, float]:
    """(arg-max, max, largest value at any other index) of one row; the second value
    equals the first when the maximum is attained twice."""
    x = np.asarray(logits_row, dtype=np.float64)
    t = int(np.argmax(x))
    rest = np.delete(x, t)
    return t, float(x[t]), float(rest.max()) if rest.size else -np.inf


def fp32_accumulation_bound(hidden, weight, chunk: int = 4096) -> np.ndarray:
    """Per row, a bound on |fp32 logit - exact logit| that holds for every vocabulary
    entry and any order of summation: the d products are exact in fp32 (bfloat16
    times bfloat16), and d - 1 additions each rounded to fp32 err by at most
    gamma_{d-1} * sum_i |h_i w_vi| (the standard recursive-summation bound), which
    is at most gamma_d * sum_i |h_i| * max_v |w_vi|."""
    h = np.abs(np.asarray(hidden, dtype=np.float64))
    d = h.shape[1]
    wmax = np.zeros(d, dtype=np.float64)
    for lo in range(0, weight.shape[0], chunk):
        w = np.abs(np.asarray(weight[lo:lo + chunk], dtype=np.float64))
        wmax = np.maximum(wmax, w.max(axis=0))
    gamma = d * U32 / (1.0 - d * U32)
    return gamma * (h @ wmax)


def tree_walk_tokens(tree_tok: np.ndarray, parent: np.ndarray, num_nodes: int,
                     node_tok: np.ndarray, L: int) -> Dict[str, np.ndarray]:
    """The tree walk of 運作流程 step 4 with the target's token at every node given
    (node_tok[n], e.g. from the LM-head arg-max): from the root, while a child of the
    current node carries the current node's token, accept it and move there; the
    token at the node where the walk stops is the next round's bonus.  Children are
    searched in index order ([R12], [R13] as in the logits walk)."""
    cur = 0
    acc: List[int] = []
    while True:
        want = int(node_tok[cur])
        nxt = -1
        for c in range(num_nodes):
            if int(parent[c]) == cur and int(tree_tok[c]) == want:
                nxt = c
                break
        if nxt < 0:
            break
        acc.append(nxt)
        cur = nxt
    acc_nodes = np.full(L, -1, dtype=np.int32)
    acc_tok = np.full(L, -1, dtype=np.int32)
    acc_nodes[:len(acc)] = acc
    acc_tok[:len(acc)] = [int(tree_tok[n]) for n in acc]
    return {"accept_len": np.int32(len(acc)), "acc_nodes": acc_nodes, "acc_tok": acc_tok,
            "bonus": np.int32(int(node_tok[cur]))}
