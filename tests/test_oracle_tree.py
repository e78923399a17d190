"""Pins of the oracle's best-first tree builder.

* Proposition 2 (DDTree page, 理論基礎): the selected prefixes form a valid tree.
* Brute force: on tiny shapes, no prefix-closed tree of B nodes has a larger sum of
  prefix probabilities, and the maximiser is unique and is the oracle's tree.
* Dynamic programming over the factorised draft gives the same optimum on every
  workload shape.
* K = 1 reduces to single-path drafting: the chain of each position's best token.
"""
import numpy as np
import pytest

import oracle
from ddt_synthetic import configs, gen

from _cases import attempts
from _pins import brute_force_best, candidate_tree, dp_optimum


def _tree(cfg, s, a, B=None, K=None):
    d = gen.draft(cfg, s, a)
    tok, lq = oracle.topk(d["logits"], K or cfg.K)
    return tok, lq, oracle.build_tree(tok, lq, d["bonus"], cfg.B if B is None else B)


def _check_valid(tree, tok, B, L):
    nn = int(tree["num_nodes"])
    par, dep, rank = tree["parent"], tree["depth"], tree["rank"]
    assert par[0] == -1 and dep[0] == 0
    for n in range(1, nn):
        p = par[n]
        assert 0 <= p < n                      # parents precede children
        assert dep[n] == dep[p] + 1 <= L
        assert tree["tree_tok"][n] == tok[dep[n] - 1, rank[n]]
        assert tree["node_logq"][n] <= tree["node_logq"][p]
    # a parent's children are contiguous and in rank order 0, 1, 2, ...
    for p in range(nn):
        kids = [n for n in range(nn) if par[n] == p]
        assert kids == list(range(kids[0], kids[0] + len(kids))) if kids else True
        assert [rank[k] for k in kids] == list(range(len(kids)))
    # canonical: depths non-decreasing, parents non-decreasing within a depth
    assert np.all(np.diff(dep[:nn]) >= 0)
    assert np.all(tree["tree_tok"][nn:] == -1) and np.all(par[nn:] == -1)
    assert nn == min(B, sum(tok.shape[1] ** d for d in range(1, L + 1))) + 1


@pytest.mark.parametrize("seed", range(12))
def test_prop2_closure_and_canonical_order(seed):
    cfg = configs.custom("t", L=5, V=40, K=3, B=20)
    tok, lq, tree = _tree(cfg, seed, 0)
    _check_valid(tree, tok, cfg.B, cfg.L)


@pytest.mark.parametrize("L,K,B,seed", [(3, 3, 5, s) for s in range(6)] + [(2, 4, 6, 7), (4, 2, 7, 8)])
def test_brute_force_small(L, K, B, seed):
    cfg = configs.custom("t", L=L, V=24, K=K, B=B)
    tok, lq, tree = _tree(cfg, seed, 0)
    paths, parents = candidate_tree(L, K)
    prob = np.array([np.exp(sum(lq[i, r] for i, r in enumerate(p))) for p in paths])
    best, sets, _ = brute_force_best(prob, parents, B)
    assert len(sets) == 1
    got = {tuple(int(tree["rank"][m]) for m in oracle.ancestors(tree["parent"], n)[1:])
           for n in range(1, int(tree["num_nodes"]))}
    assert got == {paths[i] for i in sets[0]}
    assert oracle.expected_acceptance(tree["node_logq"], int(tree["num_nodes"])) == pytest.approx(best, rel=1e-12)


def test_brute_force_tiny_workload():
    """All 1,165,524 prefix-closed 8-node trees of the 4-ary depth-4 candidate tree."""
    cfg = configs.C0
    a = attempts(cfg)[0]
    tok, lq, tree = _tree(cfg, 0, a)
    paths, parents = candidate_tree(cfg.L, cfg.K)
    prob = np.array([np.exp(sum(lq[i, r] for i, r in enumerate(p))) for p in paths])
    best, sets, count = brute_force_best(prob, parents, cfg.B)
    assert count == 1165524
    assert len(sets) == 1
    got = {tuple(int(tree["rank"][m]) for m in oracle.ancestors(tree["parent"], n)[1:])
           for n in range(1, int(tree["num_nodes"]))}
    assert got == {paths[i] for i in sets[0]}
    assert oracle.expected_acceptance(tree["node_logq"], cfg.N) == pytest.approx(best, rel=1e-12)


@pytest.mark.parametrize("name,nseq", [("C0", 1), ("C1", 1), ("C2", 2), ("C3-B16", 1), ("C3-B64", 1),
                                       ("C3-B512", 1), ("C4", 2)])
def test_dp_optimum_on_workloads(name, nseq):
    cfg = configs.get(name)
    at = attempts(cfg)
    for s in range(nseq):
        tok, lq, tree = _tree(cfg, s, at[s])
        _check_valid(tree, tok, cfg.B, cfg.L)
        val = oracle.expected_acceptance(tree["node_logq"], int(tree["num_nodes"]))
        assert val == pytest.approx(dp_optimum(np.exp(lq), cfg.B), rel=1e-12)


def test_acceptance_concave_in_budget():
    """Adding a node adds its prefix probability, and pops come out in
    non-increasing probability: the optimum grows with B with shrinking steps."""
    cfg = configs.custom("t", L=6, V=50, K=4, B=60)
    d = gen.draft(cfg, 3, 0)
    tok, lq = oracle.topk(d["logits"], cfg.K)
    vals = [oracle.expected_acceptance(t["node_logq"], int(t["num_nodes"]))
            for t in (oracle.build_tree(tok, lq, 0, b) for b in range(0, 61))]
    inc = np.diff(vals)
    assert np.all(inc > 0)
    assert np.all(np.diff(inc) <= 1e-15)


@pytest.mark.parametrize("B", [1, 3, 4, 9])
def test_k1_is_single_path(B):
    cfg = configs.custom("t", L=4, V=30, K=1, B=B)
    d = gen.draft(cfg, 1, 0)
    tok, lq, tree = _tree(cfg, 1, 0)
    depth = min(B, cfg.L)
    assert int(tree["num_nodes"]) == depth + 1
    assert tree["tree_tok"][1:depth + 1].tolist() == np.argmax(d["logits"], axis=1)[:depth].tolist()
    assert tree["parent"][:depth + 1].tolist() == [-1] + list(range(depth))


def test_budget_zero_and_shortfall():
    cfg = configs.custom("t", L=2, V=10, K=2, B=0)
    tok, lq, tree = _tree(cfg, 0, 0)
    assert int(tree["num_nodes"]) == 1 and tree["tree_tok"][0] == gen.draft(cfg, 0, 0)["bonus"]
    tok, lq, tree = _tree(cfg, 0, 0, B=10)   # only 2 + 4 candidates exist
    assert int(tree["num_nodes"]) == 7
    assert np.all(tree["parent"][7:] == -1) and np.all(tree["depth"][7:] == -1)
