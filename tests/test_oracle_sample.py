"""Pins of the oracle's walk at temperature > 0 (oracle.sample_token,
oracle.tree_walk_sample): the sampling rule against the distribution it must draw
from, and the walk against plain one-token-at-a-time sampling of the same target with
the same noise (losslessness: DDTree page, 核心創新; 運作流程 step 4)."""
import numpy as np
import pytest
from scipy import stats

import oracle
from ddt_synthetic import configs, gen


def _softmax(z):
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - z.max())
    return e / e.sum()


@pytest.mark.parametrize("T", [0.6, 1.0, 2.5])
def test_sampling_rule_draws_from_softmax_over_temperature(T):
    """Chi-squared goodness of fit of 20000 draws, each with its own noise row from the
    generator, against softmax(x / T)."""
    cfg = configs.custom("gumbel", cfg_id=700, L=1, V=7, K=1, B=1)
    x = np.array([1.0, -0.5, 0.3, 2.0, 0.0, -2.0, 1.2], dtype=np.float32)
    t = np.float32(1.0 / T)
    M = 20000
    counts = np.zeros(cfg.V)
    for i in range(M):
        counts[oracle.sample_token(x, gen.gumbel_noise(cfg, i)[0], t)] += 1
    p = _softmax(x.astype(np.float64) / T)
    res = stats.chisquare(counts, M * p)
    assert res.pvalue > 1e-3, (counts / M, p, res)


def test_zero_inverse_temperature_is_uniform_and_zero_noise_is_greedy():
    cfg = configs.custom("gumbel", cfg_id=701, L=1, V=5, K=1, B=1)
    x = np.array([3.0, -1.0, 0.5, 7.0, 2.0], dtype=np.float32)
    M = 10000
    counts = np.bincount([oracle.sample_token(x, gen.gumbel_noise(cfg, i)[0], 0.0) for i in range(M)],
                         minlength=5)
    assert stats.chisquare(counts, np.full(5, M / 5)).pvalue > 1e-3
    rng = np.random.default_rng(0)
    for _ in range(200):
        row = np.round(rng.standard_normal(50) * 2).astype(np.float32)   # ties included
        assert oracle.sample_token(row, np.zeros(50, np.float32), 1.0) == oracle.greedy_token(row)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("T", [0.5, 1.0])
def test_sampling_walk_is_plain_sampling(seed, T):
    """Accepted tokens and the bonus equal the first a + 1 tokens of plain sampling
    (token k + 1 drawn from the target after tokens 1..k with noise row k), computed
    here from the path-keyed target without the tree."""
    cfg = configs.custom("sample-walk", cfg_id=702, L=5, V=300, K=4, B=30, chain_boost=4.0)
    d = gen.draft(cfg, seed, 0)
    keep = gen.keep_flags(cfg, seed, 0)
    tok, lq = oracle.topk(d["logits"], cfg.K)
    tree = oracle.build_tree(tok, lq, d["bonus"], cfg.B)
    nn = int(tree["num_nodes"])
    tl = gen.target_logits(cfg, seed, 0, tree["tree_tok"], tree["parent"], nn, d["chain"], keep)
    noise = gen.gumbel_noise(cfg, seed)
    t = np.float32(1.0 / T)
    w = oracle.tree_walk_sample(tree["tree_tok"], tree["parent"], tree["depth"], nn, tl, noise, t, cfg.L)
    a = int(w["accept_len"])
    plain, path = [], ()
    for k in range(a + 1):
        y = oracle.sample_token(gen.target_row(cfg, seed, 0, path, d["chain"], keep), noise[k], t)
        plain.append(y)
        path = path + (y,)
    assert [int(v) for v in w["acc_tok"][:a]] + [int(w["bonus"])] == plain
    # the walk stops exactly where plain sampling leaves the tree (or at depth L)
    node = int(w["acc_nodes"][a - 1]) if a > 0 else 0
    kids = [int(tree["tree_tok"][c]) for c in range(nn) if tree["parent"][c] == node]
    assert a == cfg.L or plain[-1] not in kids


def test_sampling_walk_accepts_on_confident_paths():
    """The tests above are not vacuous: across seeds the sampling walk accepts tokens."""
    cfg = configs.custom("sample-walk", cfg_id=702, L=5, V=300, K=4, B=30, chain_boost=4.0)
    total = 0
    for seed in range(6):
        d = gen.draft(cfg, seed, 0)
        keep = gen.keep_flags(cfg, seed, 0)
        tok, lq = oracle.topk(d["logits"], cfg.K)
        tree = oracle.build_tree(tok, lq, d["bonus"], cfg.B)
        nn = int(tree["num_nodes"])
        tl = gen.target_logits(cfg, seed, 0, tree["tree_tok"], tree["parent"], nn, d["chain"], keep)
        w = oracle.tree_walk_sample(tree["tree_tok"], tree["parent"], tree["depth"], nn, tl,
                                    gen.gumbel_noise(cfg, seed), np.float32(1.0), cfg.L)
        total += int(w["accept_len"])
    assert total >= 6


def test_noise_row_follows_depth_not_node_index():
    """Hand-built tree: root 0 -> nodes 1 (token 5) and 2 (token 7); node 2 -> node 3
    (token 9).  Flat target logits; noise row 0 favours 7, row 1 favours 9, row 2
    favours 4, row 3 favours 5.  Sampling goes root -> 7 (node 2, depth 1) -> 9 (node
    3, depth 2) -> 4, not a child: accept [2, 3], bonus 4."""
    tree_tok = np.array([11, 5, 7, 9], dtype=np.int32)
    parent = np.array([-1, 0, 0, 2], dtype=np.int32)
    depth = np.array([0, 1, 1, 2], dtype=np.int32)
    V, L = 12, 3
    target = np.zeros((4, V), dtype=np.float32)
    noise = np.zeros((L + 1, V), dtype=np.float32)
    for d, t in enumerate([7, 9, 4, 5]):
        noise[d, t] = 3.0
    w = oracle.tree_walk_sample(tree_tok, parent, depth, 4, target, noise, 1.0, L)
    assert int(w["accept_len"]) == 2
    assert w["acc_nodes"].tolist() == [2, 3, -1] and w["acc_tok"].tolist() == [7, 9, -1]
    assert int(w["bonus"]) == 4


def test_sampling_walk_deep_acceptance_is_plain_sampling():
    """A confident draft and a cool target: walks accept several tokens, through nodes
    whose indices differ from their depths."""
    cfg = configs.custom("sample-deep", cfg_id=703, L=6, V=200, K=3, B=40, chain_boost=9.0)
    deepest = 0
    for seed in range(5):
        d = gen.draft(cfg, seed, 0)
        keep = np.ones(cfg.L + 1, dtype=bool)   # the target follows the planted chain
        tok, lq = oracle.topk(d["logits"], cfg.K)
        tree = oracle.build_tree(tok, lq, d["bonus"], cfg.B)
        nn = int(tree["num_nodes"])
        tl = gen.target_logits(cfg, seed, 0, tree["tree_tok"], tree["parent"], nn, d["chain"], keep)
        noise = gen.gumbel_noise(cfg, seed)
        t = np.float32(1.0 / 0.3)
        w = oracle.tree_walk_sample(tree["tree_tok"], tree["parent"], tree["depth"], nn, tl, noise, t, cfg.L)
        a = int(w["accept_len"])
        plain, path = [], ()
        for k in range(a + 1):
            y = oracle.sample_token(gen.target_row(cfg, seed, 0, path, d["chain"], keep), noise[k], t)
            plain.append(y)
            path = path + (y,)
        assert [int(v) for v in w["acc_tok"][:a]] + [int(w["bonus"])] == plain
        deepest = max(deepest, a)
    assert deepest >= 3
