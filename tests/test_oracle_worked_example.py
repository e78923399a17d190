"""The oracle against a round worked by hand (tests/golden/worked_example.json)."""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


@pytest.fixture(scope="module")
def ex():
    with open(GOLDEN) as f:
        return json.load(f)


def _logits(ex):
    return np.log(np.array(ex["q"], dtype=np.float64)).astype(np.float32)


def test_topk(ex):
    tok, lq = oracle.topk(_logits(ex), ex["K"])
    assert tok.tolist() == ex["topk_tok"]
    np.testing.assert_allclose(np.exp(lq), ex["topk_q"], rtol=1e-6)


@pytest.mark.parametrize("B", ["2", "3", "5"])
def test_tree(ex, B):
    tok, lq = oracle.topk(_logits(ex), ex["K"])
    tree = oracle.build_tree(tok, lq, ex["bonus"], int(B))
    want = ex["trees"][B]
    assert int(tree["num_nodes"]) == int(B) + 1
    assert tree["tree_tok"].tolist() == want["tree_tok"]
    assert tree["parent"].tolist() == want["parent"]
    assert tree["depth"].tolist() == want["depth"]
    assert oracle.expected_acceptance(tree["node_logq"], int(tree["num_nodes"])) == pytest.approx(
        want["expected_acceptance"], rel=1e-6)
    if "mask" in want:
        m = oracle.tree_mask(tree["parent"], int(tree["num_nodes"]), int(B) + 1)
        assert m[:, 0].tolist() == want["mask"]


def test_walk(ex):
    w = ex["walk"]
    tok, lq = oracle.topk(_logits(ex), ex["K"])
    tree = oracle.build_tree(tok, lq, ex["bonus"], w["B"])
    r = oracle.tree_walk(tree["tree_tok"], tree["parent"], int(tree["num_nodes"]),
                         np.array(w["target_logits"], dtype=np.float32), ex["L"])
    assert int(r["accept_len"]) == w["accept_len"]
    assert r["acc_nodes"][:w["accept_len"]].tolist() == w["acc_nodes"]
    assert r["acc_tok"][:w["accept_len"]].tolist() == w["acc_tok"]
    assert int(r["bonus"]) == w["bonus"]
