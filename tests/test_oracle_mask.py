"""Pins of the oracle's ancestor bitmask and position ids (DDTree page, 核心創新 and
運作流程 step 3: every node attends to its ancestors only)."""
import numpy as np
import pytest

import oracle
from ddt_synthetic import configs, gen


def _popcount(words):
    return sum(bin(int(w)).count("1") for w in words)


@pytest.mark.parametrize("L,K,B,seed", [(4, 4, 8, 0), (5, 3, 40, 1), (3, 8, 70, 2), (16, 1, 16, 3)])
def test_mask_closed_forms(L, K, B, seed):
    cfg = configs.custom("t", L=L, V=64, K=K, B=B)
    d = gen.draft(cfg, seed, 0)
    tok, lq = oracle.topk(d["logits"], K)
    tree = oracle.build_tree(tok, lq, d["bonus"], B)
    nn, N = int(tree["num_nodes"]), B + 1
    m = oracle.tree_mask(tree["parent"], nn, N)
    assert m.shape == (N, (N + 31) // 32)
    for n in range(nn):
        assert _popcount(m[n]) == tree["depth"][n] + 1
        assert (int(m[n, n // 32]) >> (n % 32)) & 1
        p = tree["parent"][n]
        if p >= 0:
            assert np.all((m[n] & m[p]) == m[p])      # superset of the parent's row
            assert _popcount(m[n] ^ m[p]) == 1        # exactly one new bit: n itself
        # no later node is ever visible (parents precede children)
        for j in range(n + 1, N):
            assert not (int(m[n, j // 32]) >> (j % 32)) & 1
    assert not np.any(m[nn:])
    # a node's position is where its token lands when its root-to-node path is laid
    # out after the prefix as one plain sequence: the prefix holds P tokens and the
    # path holds popcount(mask row) tokens (the root b included), so the node's token
    # is the last of P + popcount entries (運作流程 step 3 scores each node as the
    # continuation of the context by its path)
    P = 100
    pos = oracle.position_ids(tree["depth"], nn, P)
    for n in range(nn):
        assert pos[n] == P + _popcount(m[n]) - 1
        assert pos[n] == P + len(oracle.ancestors(tree["parent"], n)) - 1
    assert np.all(pos[nn:] == -1)


@pytest.mark.parametrize("P", [0, 1, 37, 4096])
def test_positions_of_a_chain_are_plain_decoding(P):
    """K = 1 makes the tree a single path (the single-path verification the DDTree
    page's 核心創新 contrasts with): the positions must then be those plain
    one-token-at-a-time decoding gives b, c_1, c_2, ...: P, P + 1, P + 2, ..."""
    L = 9
    cfg = configs.custom("chain", L=L, V=50, K=1, B=L)
    d = gen.draft(cfg, 4, 0)
    tok, lq = oracle.topk(d["logits"], 1)
    tree = oracle.build_tree(tok, lq, d["bonus"], L)
    assert int(tree["num_nodes"]) == L + 1
    pos = oracle.position_ids(tree["depth"], L + 1, P)
    assert pos.tolist() == list(range(P, P + L + 1))


def test_word_boundaries():
    # a chain of 70 nodes crosses two word boundaries
    parent = np.array([-1] + list(range(69)), dtype=np.int32)
    m = oracle.tree_mask(parent, 70, 70)
    assert m.shape == (70, 3)
    assert m[31].tolist() == [0xFFFFFFFF, 0, 0]
    assert m[32].tolist() == [0xFFFFFFFF, 1, 0]
    assert m[69].tolist() == [0xFFFFFFFF, 0xFFFFFFFF, 0x3F]
