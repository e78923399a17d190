"""Proposition 1 (DDTree page, 理論基礎), checked by simulation.

Draw a continuation y_1..y_L with y_i ~ q_i independently (the factorised draft),
walk it down the tree, and count the accepted depth.  The mean over many draws
must match the sum of the tree's prefix probabilities, which is what the oracle's
tree maximises.
"""
import numpy as np
import pytest
from scipy.special import softmax

import oracle
from ddt_synthetic import configs, gen


@pytest.mark.parametrize("name,seed", [("C0", 0), ("C0", 1), ("mid", 2)])
def test_expected_acceptance_by_simulation(name, seed):
    cfg = configs.C0 if name == "C0" else configs.custom("mid", L=6, V=20, K=4, B=30)
    d = gen.draft(cfg, seed, 0)
    tok, lq = oracle.topk(d["logits"], cfg.K)
    tree = oracle.build_tree(tok, lq, d["bonus"], cfg.B)
    nn = int(tree["num_nodes"])
    paths = set()
    for n in range(1, nn):
        paths.add(tuple(int(tree["tree_tok"][m]) for m in oracle.ancestors(tree["parent"], n)[1:]))

    rng = np.random.default_rng(1234 + seed)
    M = 200_000
    q = softmax(d["logits"].astype(np.float64), axis=1)           # full-vocabulary marginals
    y = np.stack([rng.choice(cfg.V, size=M, p=q[i]) for i in range(cfg.L)], axis=1)
    acc = np.zeros(M, dtype=np.int64)
    alive = np.ones(M, dtype=bool)
    for dpt in range(1, cfg.L + 1):
        pref = [tuple(r) for r in y[:, :dpt]]
        hit = np.array([p in paths for p in pref]) & alive
        acc += hit
        alive = hit
    mean, sd = acc.mean(), acc.std() / np.sqrt(M)
    want = oracle.expected_acceptance(tree["node_logq"], nn)
    assert abs(mean - want) < 5 * sd + 1e-9, (mean, want, sd)
