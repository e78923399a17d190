"""Pins of the oracle's tree walk.

Losslessness (DDTree page, 核心創新: verification keeps the target's output
distribution): under greedy decoding, the accepted tokens plus the bonus must be
exactly the first accept_len + 1 tokens that the synthetic target produces when
decoded one token at a time from the bonus token, and the walk must stop at the
first step whose token is not in the tree.
"""
import numpy as np
import pytest

import oracle
from ddt_synthetic import configs, gen

from _cases import attempts


def _greedy_decode(cfg, s, a, chain, keep, steps):
    y = []
    for _ in range(steps):
        row = gen.target_row(cfg, s, a, tuple(y), chain, keep)
        y.append(int(np.argmax(row)))   # numpy: first index of the maximum
    return y


def _check_lossless(cfg, s, a):
    d = gen.draft(cfg, s, a)
    keep = gen.keep_flags(cfg, s, a)
    tok, lq = oracle.topk(d["logits"], cfg.K)
    tree = oracle.build_tree(tok, lq, d["bonus"], cfg.B)
    nn = int(tree["num_nodes"])
    tl = gen.target_logits(cfg, s, a, tree["tree_tok"], tree["parent"], nn, d["chain"], keep)
    w = oracle.tree_walk(tree["tree_tok"], tree["parent"], nn, tl, cfg.L)
    acc = int(w["accept_len"])
    y = _greedy_decode(cfg, s, a, d["chain"], keep, acc + 1)
    assert w["acc_tok"][:acc].tolist() == y[:acc]
    assert int(w["bonus"]) == y[acc]
    assert np.all(w["acc_nodes"][acc:] == -1) and np.all(w["acc_tok"][acc:] == -1)
    paths = {tuple(int(tree["tree_tok"][m]) for m in oracle.ancestors(tree["parent"], n)[1:])
             for n in range(nn)}
    assert tuple(y[:acc]) in paths
    assert tuple(y[:acc + 1]) not in paths          # the walk stops at the first miss
    return acc


def test_lossless_tiny_workload():
    cfg = configs.C0
    accs = [_check_lossless(cfg, 0, a) for a in range(40)]
    assert max(accs) >= 3       # the planted chain is accepted deep on some draws


@pytest.mark.parametrize("seed", range(6))
def test_lossless_deeper(seed):
    cfg = configs.custom("t", L=8, V=16, K=4, B=40)
    _check_lossless(cfg, seed, 0)


def test_lossless_32k_vocab():
    cfg = configs.C1
    _check_lossless(cfg, 0, attempts(cfg)[0])


def test_depth_L_stops_walk():
    """A chain that the target follows all the way: accept L, bonus from node L."""
    L, V = 3, 5
    parent = np.array([-1, 0, 1, 2], dtype=np.int32)
    tree_tok = np.array([4, 1, 2, 3], dtype=np.int32)
    tl = np.zeros((4, V), dtype=np.float32)
    for n, want in enumerate([1, 2, 3, 0]):
        tl[n, want] = 1.0
    w = oracle.tree_walk(tree_tok, parent, 4, tl, L)
    assert int(w["accept_len"]) == 3 and w["acc_nodes"].tolist() == [1, 2, 3] and int(w["bonus"]) == 0


def test_k1_walk_is_single_path_verification():
    """K = 1: the walk accepts the longest prefix of the draft chain that matches
    the target's greedy tokens (single-path drafting, 核心創新)."""
    cfg = configs.custom("t", L=4, V=12, K=1, B=4)
    for s in range(10):
        d = gen.draft(cfg, s, 0)
        keep = gen.keep_flags(cfg, s, 0)
        tok, lq = oracle.topk(d["logits"], 1)
        tree = oracle.build_tree(tok, lq, d["bonus"], cfg.B)
        tl = gen.target_logits(cfg, s, 0, tree["tree_tok"], tree["parent"], 5, d["chain"], keep)
        w = oracle.tree_walk(tree["tree_tok"], tree["parent"], 5, tl, cfg.L)
        draft_path = np.argmax(d["logits"], axis=1).tolist()
        y = _greedy_decode(cfg, s, 0, d["chain"], keep, cfg.L + 1)
        match = 0
        while match < cfg.L and draft_path[match] == y[match]:
            match += 1
        assert int(w["accept_len"]) == match and int(w["bonus"]) == y[match]
