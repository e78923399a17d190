"""One whole verification round in the oracle, over a batch of sequences.

TEST INFRASTRUCTURE (see ``oracle/ddtree.py``).  Inputs arrive in the library's
layouts; bfloat16 operands arrive as their uint16 encodings and are widened here
(a bfloat16 is the upper half of an IEEE fp32).
"""
from typing import Callable, Dict, Optional, Sequence, Union

import numpy as np

from . import ddtree


def widen(x: np.ndarray) -> np.ndarray:
    """uint16 bfloat16 encodings or fp32 values -> fp64."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def verify_round(draft_logits: np.ndarray, bonus: np.ndarray, K: int, B: int,
                 q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                 cu_prefix: np.ndarray, k_tree: np.ndarray, v_tree: np.ndarray,
                 scale: float,
                 target: Union[np.ndarray, Callable[[int, Dict[str, np.ndarray]], np.ndarray]],
                 seqs: Optional[Sequence[int]] = None,
                 attention_rows: Optional[Dict[int, Sequence]] = None) -> Dict[int, Dict]:
    """Run top-K, tree build, mask, tree attention and walk for each sequence.

    draft_logits [S,L,V]; bonus [S]; q [S,N,Hq,D]; k_cache/v_cache [sum P,Hkv,D];
    cu_prefix [S+1]; k_tree/v_tree [S,N,Hkv,D].  ``target`` is [S,N,V] target logits
    or a function (s, tree) -> [N,V] (the target is evaluated at the built tree).
    ``attention_rows[s]`` restricts attention to the listed (node, head) rows.
    Returns {s: {topk_tok, topk_logq, tree..., mask, pos_ids, o, lse, walk...}}.
    """
    S, L, V = draft_logits.shape
    N = B + 1
    out = {}
    for s in (range(S) if seqs is None else seqs):
        tok, lq = ddtree.topk(draft_logits[s], K)
        tree = ddtree.build_tree(tok, lq, int(bonus[s]), B)
        nn = int(tree["num_nodes"])
        P0, P1 = int(cu_prefix[s]), int(cu_prefix[s + 1])
        mask = ddtree.tree_mask(tree["parent"], nn, N)
        pos = ddtree.position_ids(tree["depth"], nn, P1 - P0)
        rows = None if attention_rows is None else attention_rows.get(s)
        o, lse = ddtree.tree_attention(widen(q[s]), widen(k_cache[P0:P1]), widen(v_cache[P0:P1]),
                                       widen(k_tree[s]), widen(v_tree[s]), mask, nn, scale, rows)
        tl = target(s, tree) if callable(target) else target[s]
        walk = ddtree.tree_walk(tree["tree_tok"], tree["parent"], nn, tl, L)
        out[s] = dict(topk_tok=tok, topk_logq=lq, mask=mask, pos_ids=pos, o=o, lse=lse, **tree, **walk)
    return out
