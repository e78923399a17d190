"""Pins of the oracle's verifier epilogue (LM head + greedy token) and of the tree walk
driven by per-node tokens.

Each pin checks the oracle against something other than itself: a hand-worked
example, exact rational arithmetic with a brute-force arg-max, one-hot rows that
reduce the product to a column lookup, exact ties from duplicated weight rows,
permutation equivariance, the fp32 bound against actual fp32 sums in several
orders, the generator's planted margins, and losslessness of the token-driven walk
(DDTree page, 核心創新: verification keeps the target's greedy output) against
one-token-at-a-time greedy decoding of the synthetic target.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from ddt_synthetic import configs, gen

from _cases import attempts


def _bf16(x):
    return gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(np.asarray(x, dtype=np.float32)))


def test_hand_example():
    # W rows: e0, e1, e0 + e1, 0.5 e0 (V = 4, d = 2)
    W = np.array([[1, 0], [0, 1], [1, 1], [0.5, 0]], dtype=np.float32)
    H = np.array([[2, 1],      # logits 2, 1, 3, 1      -> token 2, value 3
                  [1, 1],      # logits 1, 1, 2, 0.5    -> token 2, value 2
                  [1, -1],     # logits 1, -1, 0, 0.5   -> token 0, value 1
                  [0, 0],      # all zero: a four-way tie -> token 0
                  [-1, -1]],   # logits -1, -1, -2, -0.5 -> token 3, value -0.5
                 dtype=np.float32)
    tok, val = oracle.lm_head_argmax(H, W)
    assert tok.tolist() == [2, 2, 0, 0, 3]
    assert val.tolist() == [3.0, 2.0, 1.0, 0.0, -0.5]
    # a tie between the two largest goes to the smaller id
    tok, _ = oracle.lm_head_argmax(np.array([[1, 1]], np.float32), np.array([[0, 2], [2, 0]], np.float32))
    assert tok.tolist() == [0]


def test_exact_rational_brute_force():
    r = np.random.default_rng(7)
    M, V, d = 5, 37, 64
    H = _bf16(r.standard_normal((M, d)))
    W = _bf16(r.standard_normal((V, d)) / 8)
    tok, val = oracle.lm_head_argmax(H, W)
    x = oracle.lm_head_logits(H, W, chunk=5)
    for m in range(M):
        exact = [sum(Fraction(float(H[m, i])) * Fraction(float(W[v, i])) for i in range(d))
                 for v in range(V)]
        best = 0
        for v in range(1, V):
            if exact[v] > exact[best]:
                best = v
        assert tok[m] == best
        for v in range(V):
            assert abs(x[m, v] - float(exact[v])) <= 1e-12 * (1 + abs(float(exact[v])))
        assert val[m] == x[m, best]


def test_one_hot_rows_read_a_column():
    r = np.random.default_rng(3)
    V, d = 200, 48
    W = _bf16(r.standard_normal((V, d)))
    cols = [0, 5, 47, 13]
    H = np.zeros((len(cols), d), dtype=np.float32)
    for m, j in enumerate(cols):
        H[m, j] = 2.0 if m % 2 == 0 else -3.0
    tok, val = oracle.lm_head_argmax(H, W)
    for m, j in enumerate(cols):
        c = H[m, j]
        best = max(range(V), key=lambda v: (float(c) * float(W[v, j]), -v))
        assert tok[m] == best
        assert val[m] == float(c) * float(W[best, j])


def test_duplicate_rows_tie_to_smallest_id():
    r = np.random.default_rng(11)
    V, d = 300, 64
    W = _bf16(r.standard_normal((V, d)) / 8)
    h = _bf16(r.standard_normal((1, d)))
    t, _ = oracle.lm_head_argmax(h, W)
    t = int(t[0])
    # copies of the winning row placed before and after it: the first copy wins
    for pos in (0, t // 2, V - 1):
        W2 = W.copy()
        W2[pos] = W[t]
        tok, _ = oracle.lm_head_argmax(h, W2)
        assert int(tok[0]) == min(pos, t)


def test_permutation_equivariance():
    r = np.random.default_rng(5)
    M, V, d = 6, 500, 64
    H = _bf16(r.standard_normal((M, d)))
    W = _bf16(r.standard_normal((V, d)) / 8)
    perm = r.permutation(V)
    tok, val = oracle.lm_head_argmax(H, W)
    tok_p, val_p = oracle.lm_head_argmax(H, W[perm])
    # W[perm][j] = W[perm[j]]: the winner's new index j satisfies perm[j] = tok
    assert perm[tok_p].tolist() == tok.tolist()
    assert np.array_equal(val, val_p)


def test_bound_covers_fp32_sums_in_several_orders():
    r = np.random.default_rng(9)
    M, V, d = 4, 40, 512
    H = _bf16(r.standard_normal((M, d)))
    W = _bf16(r.standard_normal((V, d)) / np.sqrt(d))
    x = oracle.lm_head_logits(H, W)
    bound = oracle.fp32_accumulation_bound(H, W)
    for m in range(M):
        for v in range(V):
            p = (H[m].astype(np.float32) * W[v].astype(np.float32)).astype(np.float32)  # exact
            sums = []
            for order in (p, p[::-1], r.permutation(p)):
                acc = np.float32(0)
                for t in order:
                    acc = np.float32(acc + t)
                sums.append(acc)
            # blocked: 16-term partial sums, then the running total (the MFMA's shape)
            acc = np.float32(0)
            for b in range(0, d, 16):
                part = np.float32(0)
                for t in p[b:b + 16]:
                    part = np.float32(part + t)
                acc = np.float32(acc + part)
            sums.append(acc)
            for s_ in sums:
                assert abs(float(s_) - x[m, v]) <= bound[m]
    assert np.all(bound > 0)


def test_bound_is_nearly_reached_by_an_adversarial_sum():
    # one product of 1, then d - 1 products of 2^-25: each is below half an ulp of 1,
    # so a sequential fp32 sum rounds every one of them away and ends at 1, while the
    # exact sum is 1 + (d - 1) 2^-25.  The error is about half of gamma_d * sum|h||w|:
    # a bound smaller by a factor of two or more (a dropped factor d, a wrong unit
    # roundoff) would fail here.
    d = 512
    H = np.full((1, d), 2.0 ** -12, dtype=np.float32)
    W = np.full((1, d), 2.0 ** -13, dtype=np.float32)
    H[0, 0] = W[0, 0] = 1.0
    x = oracle.lm_head_logits(H, W)[0, 0]
    assert x == 1.0 + (d - 1) * 2.0 ** -25
    acc = np.float32(0)
    for t in (H[0] * W[0]).astype(np.float32):
        acc = np.float32(acc + t)
    assert acc == np.float32(1.0)
    bound = oracle.fp32_accumulation_bound(H, W)[0]
    err = x - float(acc)
    assert 0.45 * bound <= err <= bound


def test_planted_tokens_lead_by_a_margin():
    cfg = configs.custom("lm", V=5000, K=4, B=8, Hq=4, D=64)   # d = 256
    W = gen.lm_head_weight(cfg)
    toks = [0, 4999, 17, 2500, 17, 3]
    Hb = gen.hidden_states(cfg, 0, W, toks)
    H = gen.bf16_bits_to_f32(Hb)
    Wf = gen.bf16_bits_to_f32(W)
    tok, val = oracle.lm_head_argmax(H, Wf)
    bound = oracle.fp32_accumulation_bound(H, Wf)
    x = oracle.lm_head_logits(H, Wf)
    assert tok.tolist() == toks
    for m in range(len(toks)):
        t, top, second = oracle.top_two(x[m])
        assert top - second > 3.0 and top - second > 100 * bound[m]
    # an unplanted row has no such lead: its top two sit within ~1 of each other
    Hz = gen.bf16_bits_to_f32(gen.hidden_states(cfg, 0, W, [-1]))
    _, top, second = oracle.top_two(oracle.lm_head_logits(Hz, Wf)[0])
    assert top - second < 3.0


def _greedy_decode(cfg, s, a, chain, keep, steps):
    y = []
    for _ in range(steps):
        row = gen.target_row(cfg, s, a, tuple(y), chain, keep)
        y.append(int(np.argmax(row)))
    return y


def _check_token_walk_lossless(cfg, s, a, d):
    dr = gen.draft(cfg, s, a)
    keep = gen.keep_flags(cfg, s, a)
    tok, lq = oracle.topk(dr["logits"], cfg.K)
    tree = oracle.build_tree(tok, lq, dr["bonus"], cfg.B)
    nn = int(tree["num_nodes"])
    W = gen.lm_head_weight(cfg, d)
    b = {"chain": dr["chain"][None], "keep": keep[None], "attempts": np.array([a])}
    one = configs.custom("one", S=1, L=cfg.L, V=cfg.V, K=cfg.K, B=cfg.B, cfg_id=cfg.cfg_id)
    tr = {"tree_tok": tree["tree_tok"][None], "parent": tree["parent"][None],
          "num_nodes": np.array([nn])}
    H = gen.bf16_bits_to_f32(gen.tree_hidden_states(one, b, tr, W)[0])
    node_tok, _ = oracle.lm_head_argmax(H[:nn], gen.bf16_bits_to_f32(W))
    w = oracle.tree_walk_tokens(tree["tree_tok"], tree["parent"], nn, node_tok, cfg.L)
    acc = int(w["accept_len"])
    y = _greedy_decode(cfg, s, a, dr["chain"], keep, acc + 1)
    assert w["acc_tok"][:acc].tolist() == y[:acc]
    assert int(w["bonus"]) == y[acc]
    assert np.all(w["acc_nodes"][acc:] == -1) and np.all(w["acc_tok"][acc:] == -1)
    paths = {tuple(int(tree["tree_tok"][m]) for m in oracle.ancestors(tree["parent"], n)[1:])
             for n in range(nn)}
    assert tuple(y[:acc]) in paths and tuple(y[:acc + 1]) not in paths
    return acc


@pytest.mark.parametrize("seed", range(4))
def test_token_walk_lossless(seed):
    cfg = configs.custom("lmw", cfg_id=100 + seed, L=8, V=64, K=4, B=40)
    _check_token_walk_lossless(cfg, 0, 0, d=128)


def test_token_walk_lossless_deep():
    cfg = configs.C0
    accs = [_check_token_walk_lossless(cfg, 0, a, d=64) for a in range(12)]
    assert max(accs) >= 3


def test_token_walk_lossless_32k_vocab():
    cfg = configs.C1
    _check_token_walk_lossless(cfg, 0, attempts(cfg)[0], d=128)


def test_token_walk_hand_built():
    # root 0 (token 7) with children 1 (token 3) and 2 (token 5); node 1 has child 3
    # (token 9), node 2 has child 4 (token 3).
    tree_tok = np.array([7, 3, 5, 9, 3])
    parent = np.array([-1, 0, 0, 1, 2])
    # the root's token is 5 -> node 2; node 2's token 3 -> node 4; node 4's token 8 stops
    w = oracle.tree_walk_tokens(tree_tok, parent, 5, np.array([5, 0, 3, 0, 8]), L=3)
    assert int(w["accept_len"]) == 2
    assert w["acc_nodes"].tolist() == [2, 4, -1] and w["acc_tok"].tolist() == [5, 3, -1]
    assert int(w["bonus"]) == 8
    # the root's token is in no child: nothing accepted, the bonus is the root's token
    w = oracle.tree_walk_tokens(tree_tok, parent, 5, np.array([1, 0, 0, 0, 0]), L=3)
    assert int(w["accept_len"]) == 0 and int(w["bonus"]) == 1
    # nodes past num_nodes are not searched
    w = oracle.tree_walk_tokens(tree_tok, parent, 2, np.array([5, 0, 3, 0, 8]), L=3)
    assert int(w["accept_len"]) == 0 and int(w["bonus"]) == 5
