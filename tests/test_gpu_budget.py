"""Adaptive node budget (ddt_adapt_budget) through the C ABI against the oracle
(oracle.choose_budget, oracle.prune_tree): the chosen budget, the cut tree (tokens,
parents, depths, num_nodes) bit-exact, its log-probabilities and expected acceptance
within the fp32 tolerance, and the cut tree's mask from ddt_tree_mask.

The GPU ranks fp32 node log-probabilities and the oracle fp64 ones, so draws are kept
only when the decision has a margin: sorted scores at least 1e-3 apart
(the fp32 scores are within 1e-4 of the fp64 ones) and the best ratio at least 1e-4
(relative) above the next; ``attempt`` re-draws otherwise."""
import numpy as np
import pytest
import torch

import block_diffusion_draft_position_amd as ddt
import oracle
from ddt_synthetic import configs, gen

from _gpu import NODE_LOGQ_ATOL, dev_tensor

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ddt.load()


def _ratios(tree, cost):
    nn = int(tree["num_nodes"])
    order = oracle.score_order(tree["node_logq"], nn)
    e = np.concatenate([[0.0], np.cumsum(np.exp(tree["node_logq"][order]))])
    return (e + 1.0) / cost[:nn]


def _margins_ok(tree, cost):
    """The cut boundary at the chosen budget is at least 1e-3 wide, and the best ratio
    beats by 1e-3 (relative) every budget whose cost differs from the chosen one's:
    scores swapped by rounding move a ratio by at most a few 1e-4.  Among budgets of
    equal cost the ratio grows with b on both sides alike."""
    nn = int(tree["num_nodes"])
    lp = np.sort(tree["node_logq"][1:nn])[::-1]
    j = _ratios(tree, cost)
    b = int(np.argmax(j))
    if 0 < b < nn - 1 and lp[b - 1] - lp[b] < 1e-3:
        return False
    others = j[cost[:nn] != cost[b]]
    return others.size == 0 or j[b] >= np.max(others) * (1 + 1e-3)


def _draw(cfg, cost):
    """Per sequence, the first attempt whose oracle tree clears the margins."""
    att, trees = [], []
    for s in range(cfg.S):
        for a in range(200):
            d = gen.draft(cfg, s, a)
            tok, lq = oracle.topk(d["logits"], cfg.K)
            t = oracle.build_tree(tok, lq, d["bonus"], cfg.B)
            if oracle.selection_gap(lq, cfg.B) >= 1e-4 and _margins_ok(t, cost):
                break
        else:
            raise RuntimeError(f"{cfg.name} seq {s}: no draw clears the margins")
        att.append(a)
        trees.append(t)
    return att, trees


def _linear(B, c0, c1):
    return (c0 + c1 * np.arange(B + 1)).astype(np.float32)


def _cost(B, spec):
    if spec[0] == "step":      # flat up to a knee, then ten times dearer
        _, c0, knee = spec
        c = np.full(B + 1, c0, dtype=np.float32)
        c[knee + 1:] *= 10.0
        return c
    return _linear(B, *spec)


CASES = {
    "confident": (dict(S=4, L=8, V=3000, K=6, B=120, chain_boost=4.0), (40.0, 0.5)),
    "confident-steep": (dict(S=3, L=6, V=2000, K=4, B=60, chain_boost=6.0), (10.0, 2.0)),
    "sweep-shape": (dict(S=1, L=16, V=128256, K=32, B=512), (55.0, 0.33)),
    "flat-cost": (dict(S=2, L=5, V=500, K=4, B=40, chain_boost=3.0), (50.0, 0.0)),
    "prohibitive": (dict(S=2, L=5, V=500, K=4, B=40, chain_boost=3.0), (1.0, 1e6)),
    "shortfall": (dict(S=2, L=2, V=400, K=3, B=30, chain_boost=3.0), (20.0, 0.1)),
    "large-B": (dict(S=1, L=6, V=4000, K=16, B=1023, chain_boost=5.0), ("step", 60.0, 700)),
    "large-B-flat": (dict(S=1, L=6, V=4000, K=16, B=1023, chain_boost=5.0), (60.0, 0.0)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_adapt_budget_matches_oracle(name):
    kw, spec = CASES[name]
    cfg = configs.custom(f"budget-{name}", cfg_id=900 + len(name), **kw)
    cost = _cost(cfg.B, spec)
    att, trees = _draw(cfg, cost)
    print(f"[case] adapt budget {name}: attempts {att}", flush=True)
    b = gen.batch(cfg, att, with_qkv=False)
    tok, lq = ddt.ddt_topk(dev_tensor(b["draft_logits"]), cfg.K)
    tree = ddt.ddt_build_tree(tok, lq, dev_tensor(b["bonus"].astype(np.int32)), cfg.B)
    torch.cuda.synchronize()
    for s in range(cfg.S):   # the GPU's tree is the oracle's before the cut
        for k in ("tree_tok", "parent", "depth"):
            assert np.array_equal(tree[k][s].cpu().numpy(), trees[s][k]), f"seq {s}: {k}"
    budget, expected = ddt.ddt_adapt_budget(tree, dev_tensor(cost))
    mask, _ = ddt.ddt_tree_mask(tree["parent"], tree["depth"], tree["num_nodes"], None)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in tree.items()}
    gm = mask.cpu().numpy().view(np.uint32)
    chosen = []
    for s in range(cfg.S):
        t = trees[s]
        bs, es = oracle.choose_budget(t["node_logq"], int(t["num_nodes"]), cost.astype(np.float64))
        chosen.append(bs)
        assert int(budget[s]) == bs, f"seq {s}: budget"
        assert abs(float(expected[s]) - es) <= 1e-5 * max(1.0, es)
        cut = oracle.prune_tree(t, bs)
        assert int(got["num_nodes"][s]) == bs + 1
        for k in ("tree_tok", "parent", "depth"):
            assert np.array_equal(got[k][s], cut[k]), f"seq {s}: cut {k}"
        np.testing.assert_allclose(got["node_logq"][s][:bs + 1], cut["node_logq"][:bs + 1], rtol=0,
                                   atol=NODE_LOGQ_ATOL)
        assert np.all(np.isneginf(got["node_logq"][s][bs + 1:]))
        assert np.array_equal(gm[s], oracle.tree_mask(cut["parent"], bs + 1, cfg.N)), f"seq {s}: mask"
    print(f"[case] {name}: budgets {chosen} of {cfg.B}", flush=True)
    if name == "flat-cost":
        assert all(c == int(trees[s]["num_nodes"]) - 1 for s, c in enumerate(chosen))
    if name == "prohibitive":
        assert chosen == [0] * cfg.S
    if name in ("confident", "confident-steep"):
        assert any(0 < c < cfg.B for c in chosen)   # an intermediate budget
    if name == "large-B":
        assert chosen == [700]
