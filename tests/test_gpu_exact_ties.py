"""Draft trees under exact ties (quantised draft logits), through the C ABI.

When prefix probabilities tie exactly at the budget boundary, several trees are
optimal, and the pages fix no tie order (DDTree page "策展 · X (Twitter)",
section 核心創新: a best-first heap; section 理論基礎: Proposition 2, the top-B
prefixes form a tree).  The builder takes equal scores in its own node order, the
oracle shallower first and then by rank path, so the selected sets may differ.  What
is unique is compared exactly; the rest is checked for validity:
  * top-K tokens (equal logits to the smaller id, on both sides): bit-exact;
  * num_nodes, and the sorted multiset of the selected prefixes' log-probabilities;
  * the GPU tree is prefix-closed, in canonical order (depth, parent, sibling rank),
    its tokens are the top-K tokens of its rank paths, and its expected acceptance
    (Proposition 1) equals the oracle's and the dynamic-programming optimum;
  * mask, position ids and the walk on the GPU's own tree equal the oracle's on it.
Quantisation levels are chosen so that the cuts over at most 64, at most 256 and
more candidates all meet boundary ties.
"""
import numpy as np
import pytest
import torch

import block_diffusion_draft_position_amd as ddt
import oracle
from ddt_synthetic import configs, gen

from _gpu import dev_tensor
from _pins import dp_optimum

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ddt.load()


def _quantised(S, L, V, step, rng):
    return (np.round(rng.standard_normal((S, L, V)) * 2.0 / step) * step).astype(np.float32)


CASES = {
    # name: (S, L, V, K, B, quantisation step (0 = all logits equal))
    "cut64": (4, 4, 300, 8, 30, 1.0),
    "cut256": (3, 4, 500, 16, 100, 1.0),
    "radix": (2, 3, 2000, 32, 500, 0.5),
    "all-equal": (2, 4, 64, 4, 12, 0.0),
    "all-equal-wide": (1, 3, 100, 64, 1023, 0.0),
    "levels-deep": (2, 8, 40, 3, 200, 2.0),
}


@pytest.mark.parametrize("fused", [False, True], ids=["calls", "fused"])
@pytest.mark.parametrize("name", list(CASES))
def test_exact_ties(name, fused):
    S, L, V, K, B, step = CASES[name]
    print(f"[case] exact ties {name}: S={S} L={L} V={V} K={K} B={B} step={step} fused={fused}", flush=True)
    rng = np.random.default_rng(11 + len(name))
    x = np.zeros((S, L, V), dtype=np.float32) if step == 0 else _quantised(S, L, V, step, rng)
    bonus = rng.integers(0, V, size=S).astype(np.int32)
    N = B + 1
    P = np.array([5 + 3 * s for s in range(S)], dtype=np.int64)
    cu = np.concatenate([[0], np.cumsum(P)]).astype(np.int64)
    d_x, d_b, d_cu = dev_tensor(x), dev_tensor(bonus), dev_tensor(cu)
    if fused:
        r = ddt.ddt_draft_tree(d_x, d_b, d_cu, K, B)
        tok, lq, mask, pos = r["topk_tok"], r["topk_logq"], r["mask"], r["pos_ids"]
        tree = {k: r[k] for k in ("tree_tok", "parent", "depth", "node_logq", "num_nodes")}
    else:
        tok, lq = ddt.ddt_topk(d_x, K)
        tree = ddt.ddt_build_tree(tok, lq, d_b, B)
        mask, pos = ddt.ddt_tree_mask(tree["parent"], tree["depth"], tree["num_nodes"], d_cu)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in tree.items()}
    gtok, gmask, gpos = tok.cpu().numpy(), mask.cpu().numpy().view(np.uint32), pos.cpu().numpy()
    ties_seen = 0
    for s in range(S):
        rt, rl = oracle.topk(x[s], K)
        assert np.array_equal(gtok[s], rt), f"seq {s}: top-K tokens"
        ref = oracle.build_tree(rt, rl, int(bonus[s]), B)
        nn = int(ref["num_nodes"])
        assert int(g["num_nodes"][s]) == nn, f"seq {s}: num_nodes"
        par, dep, tt = g["parent"][s], g["depth"][s], g["tree_tok"][s]
        # structure: root, prefix closure, canonical order, tokens from the rank paths
        assert par[0] == -1 and dep[0] == 0 and tt[0] == bonus[s]
        score = np.zeros(nn)
        rank = np.full(nn, -1)
        for n in range(1, nn):
            p = int(par[n])
            assert 0 <= p < n, f"seq {s}: parent of {n}"
            assert dep[n] == dep[p] + 1 and dep[n] <= L
            row = list(rt[dep[n] - 1])
            assert int(tt[n]) in row, f"seq {s}: node {n} token not a top-K token"
            rank[n] = row.index(int(tt[n]))
            score[n] = score[p] + rl[dep[n] - 1, rank[n]]
            if n > 1:
                a = (int(dep[n - 1]), int(par[n - 1]), int(rank[n - 1]) if n - 1 > 0 else -1)
                assert a < (int(dep[n]), p, int(rank[n])), f"seq {s}: canonical order at {n}"
        # siblings hold ranks 0..c-1 (a stream is consumed from its best candidate)
        for p in range(nn):
            kids = sorted(int(rank[c]) for c in range(1, nn) if par[c] == p)
            assert kids == list(range(len(kids))), f"seq {s}: children of {p}"
        assert np.all(par[nn:] == -1) and np.all(tt[nn:] == -1) and np.all(dep[nn:] == -1)
        # what is unique: the multiset of selected log-probabilities, hence Prop. 1's value
        ref_lp = np.sort(ref["node_logq"][1:nn])
        got_lp = np.sort(score[1:])
        np.testing.assert_allclose(got_lp, ref_lp, rtol=0, atol=1e-9)
        np.testing.assert_allclose(g["node_logq"][s][:nn], score.astype(np.float32), rtol=0, atol=1e-4)
        ea = float(np.sum(np.exp(score[1:])))
        opt = dp_optimum(np.exp(rl), B)
        assert abs(ea - opt) <= 1e-6 * max(1.0, opt), (ea, opt)
        assert abs(ea - oracle.expected_acceptance(ref["node_logq"], nn)) <= 1e-9 * max(1.0, ea)
        # the boundary tie this test is about: the B-th and the next candidate score equal
        ties_seen += oracle.selection_gap(rl, B) == 0.0
        # mask, positions and walk on the GPU's tree
        m_ref = oracle.tree_mask(par, nn, N)
        assert np.array_equal(gmask[s], m_ref), f"seq {s}: mask"
        assert np.array_equal(gpos[s], oracle.position_ids(dep, nn, int(P[s]))), f"seq {s}: pos"
    assert ties_seen > 0, "no boundary tie in this case: quantisation too fine"
    # the walk on the GPU's own trees
    target = rng.standard_normal((S, N, V)).astype(np.float32)
    for s in range(S):
        nn = int(g["num_nodes"][s])
        for n in range(nn):   # follow the first child where there is one
            kids = [c for c in range(nn) if g["parent"][s][c] == n]
            if kids and rng.random() < 0.8:
                target[s, n, int(g["tree_tok"][s][kids[-1]])] += 20.0
    w = ddt.ddt_tree_walk(tree["tree_tok"], tree["parent"], tree["num_nodes"], dev_tensor(target), L)
    gw = {k: v.cpu().numpy() for k, v in w.items()}
    for s in range(S):
        ref = oracle.tree_walk(g["tree_tok"][s], g["parent"][s], int(g["num_nodes"][s]), target[s], L)
        for k in ("accept_len", "acc_nodes", "acc_tok", "bonus"):
            assert np.array_equal(gw[k][s], ref[k]), f"seq {s}: walk {k}"
