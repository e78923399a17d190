"""Pins of the oracle's softmax + top-K against library routines and invariants."""
import numpy as np
import pytest
from scipy.special import logsumexp

import oracle
from ddt_synthetic import configs, gen


def _ref_order(x):
    # Python's own sort, independent of numpy's lexsort: logit desc, id asc
    return sorted(range(len(x)), key=lambda v: (-float(x[v]), v))


@pytest.mark.parametrize("V,k,seed", [(64, 4, 0), (64, 64, 1), (1000, 8, 2), (32000, 8, 3)])
def test_topk_matches_library(V, k, seed):
    rng = np.random.default_rng(seed)
    x = (2 * rng.standard_normal((3, V))).astype(np.float32)
    tok, lq = oracle.topk(x, k)
    for r in range(3):
        assert tok[r].tolist() == _ref_order(x[r])[:k]
        lse = logsumexp(x[r].astype(np.float64))
        np.testing.assert_allclose(lq[r], x[r, tok[r]].astype(np.float64) - lse, rtol=0, atol=1e-12)


def test_ties_go_to_smaller_id():
    x = np.array([[1.0, 3.0, 3.0, -2.0, 3.0, 0.0, 0.0, 3.0]], dtype=np.float32)
    tok, _ = oracle.topk(x, 6)
    assert tok[0].tolist() == [1, 2, 4, 7, 0, 5]
    x = np.array([[-0.0, 0.0, -0.0]], dtype=np.float32)  # signed zeros compare equal
    tok, _ = oracle.topk(x, 3)
    assert tok[0].tolist() == [0, 1, 2]


def test_full_k_is_a_distribution():
    x = (3 * np.random.default_rng(5).standard_normal((2, 300))).astype(np.float32)
    tok, lq = oracle.topk(x, 300)
    for r in range(2):
        assert sorted(tok[r].tolist()) == list(range(300))
        assert np.sum(np.exp(lq[r])) == pytest.approx(1.0, abs=1e-12)
        assert np.all(np.diff(lq[r]) <= 0)


def test_planted_chain_is_top1_on_tiny_workload():
    # +6 - 0.4 i over N(0, 4) noise on 64 tokens: the chain token is usually, not
    # always, the argmax; check the oracle agrees with numpy's argmax every time.
    cfg = configs.C0
    for a in range(10):
        d = gen.draft(cfg, 0, a)
        tok, _ = oracle.topk(d["logits"], 1)
        assert tok[:, 0].tolist() == np.argmax(d["logits"], axis=1).tolist()
