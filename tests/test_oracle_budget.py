"""Pins of the oracle's adaptive budget (oracle.choose_budget, oracle.prune_tree),
independent of their own code:
  * the tree cut to b nodes is the tree built directly at budget b (Proposition 2: the
    top-b prefixes form a tree; the heap's first b pops are those prefixes), for every
    b up to B, canonical order included;
  * E[accept](b) of the cut tree equals the exact dynamic-programming optimum at b
    (Proposition 1 and optimality);
  * the chosen budget maximises (E + 1) / cost over trees built one budget at a time;
  * closed cases: a constant cost takes the whole tree, a steep cost takes none.
"""
import numpy as np
import pytest

import oracle
from ddt_synthetic import configs, gen

from _pins import dp_optimum


def _tree(L, K, B, seed, boost=0.0, V=120):
    cfg = configs.custom("budget", cfg_id=800, L=L, V=V, K=K, B=B, chain_boost=boost)
    d = gen.draft(cfg, seed, 0)
    tok, lq = oracle.topk(d["logits"], K)
    return tok, lq, d["bonus"], oracle.build_tree(tok, lq, d["bonus"], B)


def _gap_ok(tree):
    nn = int(tree["num_nodes"])
    lp = np.sort(tree["node_logq"][1:nn])
    return np.all(np.diff(lp) >= 1e-9)


@pytest.mark.parametrize("L,K,B,seed,boost", [(4, 4, 30, 0, 0.0), (5, 3, 60, 1, 3.0), (6, 2, 40, 2, 8.0),
                                              (3, 8, 100, 3, 0.0), (8, 1, 8, 4, 2.0)])
def test_cut_tree_is_the_tree_built_at_that_budget(L, K, B, seed, boost):
    tok, lq, bonus, tree = _tree(L, K, B, seed, boost)
    assert _gap_ok(tree)
    nn = int(tree["num_nodes"])
    for b in range(0, nn):
        cut = oracle.prune_tree(tree, b)
        ref = oracle.build_tree(tok, lq, bonus, b)
        assert int(cut["num_nodes"]) == int(ref["num_nodes"]) == b + 1
        for k in ("tree_tok", "parent", "depth"):
            assert np.array_equal(cut[k][:b + 1], ref[k]), (b, k)
        assert np.all(cut["parent"][b + 1:] == -1)
        e = oracle.expected_acceptance(cut["node_logq"], b + 1)
        assert abs(e - dp_optimum(np.exp(lq), b)) <= 1e-9 * max(1.0, e)


@pytest.mark.parametrize("seed", range(5))
def test_chosen_budget_maximises_tokens_per_cost(seed):
    L, K, B = 5, 4, 40
    tok, lq, bonus, tree = _tree(L, K, B, seed, boost=2.0)
    nn = int(tree["num_nodes"])
    rng = np.random.default_rng(seed)
    cost = 30.0 + 0.9 * np.arange(B + 1) + rng.uniform(0, 2, B + 1)   # a noisy linear cost
    b, e = oracle.choose_budget(tree["node_logq"], nn, cost)
    # brute force: every budget's own tree, its expected acceptance from scratch
    vals = []
    for bb in range(nn):
        t = oracle.build_tree(tok, lq, bonus, bb)
        vals.append((oracle.expected_acceptance(t["node_logq"], bb + 1) + 1.0) / cost[bb])
    assert b == int(np.argmax(vals))
    assert abs(e - oracle.expected_acceptance(oracle.prune_tree(tree, b)["node_logq"], b + 1)) <= 1e-12


def test_closed_cases():
    tok, lq, bonus, tree = _tree(4, 4, 30, 0, 2.0)
    nn = int(tree["num_nodes"])
    assert oracle.choose_budget(tree["node_logq"], nn, np.ones(31))[0] == nn - 1     # constant cost
    steep = 1.0 + 1e6 * np.arange(31)
    assert oracle.choose_budget(tree["node_logq"], nn, steep) == (0, 0.0)          # steep cost
    cut = oracle.prune_tree(tree, 0)
    assert int(cut["num_nodes"]) == 1 and cut["tree_tok"][0] == tree["tree_tok"][0]
