"""The walk at temperature > 0 (ddt_tree_walk_sample) through the C ABI against the
oracle's (oracle.tree_walk_sample), bit-exact on accept lengths, accepted nodes and
tokens and bonus tokens, on the workloads' shapes at full size and on small shapes;
plus exact ties of the sampling score (equal scores go to the smaller id) and the
greedy limit (zero noise, inverse temperature 1: ddt_tree_walk's result)."""
import numpy as np
import pytest
import torch

import block_diffusion_draft_position_amd as ddt
import oracle
from ddt_synthetic import configs, gen

from _cases import attempts
from _gpu import dev_tensor, target_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ddt.load()


def _trees(cfg, b):
    trees = {}
    for s in range(cfg.S):
        tok, lq = oracle.topk(b["draft_logits"][s], cfg.K)
        trees[s] = oracle.build_tree(tok, lq, int(b["bonus"][s]), cfg.B)
    return trees


def _run(cfg, b, trees, tl, noise, inv_t):
    st = lambda k: dev_tensor(np.stack([trees[s][k] for s in range(cfg.S)]).astype(np.int32))
    nn = dev_tensor(np.array([trees[s]["num_nodes"] for s in range(cfg.S)], dtype=np.int32))
    w = ddt.ddt_tree_walk_sample(st("tree_tok"), st("parent"), st("depth"), nn, dev_tensor(tl),
                                 dev_tensor(noise), inv_t, cfg.L)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in w.items()}
    acc = 0
    for s in range(cfg.S):
        t = trees[s]
        ref = oracle.tree_walk_sample(t["tree_tok"], t["parent"], t["depth"], int(t["num_nodes"]), tl[s],
                                      noise[s], inv_t, cfg.L)
        for k in ("accept_len", "acc_nodes", "acc_tok", "bonus"):
            assert np.array_equal(got[k][s], ref[k]), f"{cfg.name} seq {s}: {k}"
        acc += int(ref["accept_len"])
    return acc


@pytest.mark.parametrize("inv_t", [1.0, np.float32(1 / 0.7), np.float32(1 / 1.6)])
@pytest.mark.parametrize("name", ["C0", "C1", "C2", "C3-B512", "C4"])
def test_sampling_walk_full_workloads(name, inv_t):
    cfg = configs.get(name)
    print(f"[case] sampling walk {name} inv_t={float(inv_t):.4f}", flush=True)
    b = gen.batch(cfg, attempts(cfg), with_qkv=False)
    trees = _trees(cfg, b)
    tl = target_for(cfg, b, trees)
    noise = np.stack([gen.gumbel_noise(cfg, s) for s in range(cfg.S)])
    _run(cfg, b, trees, tl, noise, np.float32(inv_t))


@pytest.mark.parametrize("inv_t", [1.0, 3.0, 0.0])
def test_sampling_walk_confident_shapes(inv_t):
    """Confident drafts (acceptance of several tokens), a ragged vocabulary (4099: the
    scalar tail of the row loads) and inverse temperature 0 (uniform draws)."""
    cfg = configs.custom("sample-mid", cfg_id=710, S=6, L=6, V=4099, K=4, B=40, chain_boost=5.0)
    b = gen.batch(cfg, with_qkv=False)
    b["keep"][:] = True
    trees = _trees(cfg, b)
    tl = target_for(cfg, b, trees)
    noise = np.stack([gen.gumbel_noise(cfg, s) for s in range(cfg.S)])
    acc = _run(cfg, b, trees, tl, noise, np.float32(inv_t))
    if inv_t >= 1.0:
        assert acc >= cfg.S   # the walk accepts tokens: the comparison is not vacuous


def test_sampling_score_ties_and_greedy_limit():
    """Scores equal in fp32 go to the smaller id (including -0 against +0); with zero
    noise and inverse temperature 1 the sampling walk is the greedy walk."""
    S, L, V, B = 2, 3, 3000, 10
    cfg = configs.custom("sample-ties", cfg_id=711, S=S, L=L, V=V, K=3, B=B)
    b = gen.batch(cfg, with_qkv=False)
    trees = _trees(cfg, b)
    rng = np.random.default_rng(9)
    tl = np.round(rng.standard_normal((S, B + 1, V)) * 2).astype(np.float32) * 0.5
    noise = np.round(rng.standard_normal((S, L + 1, V))).astype(np.float32)
    for s in range(S):          # planted exact ties at the top, one pair of signed zeros
        for n in range(B + 1):
            lo, hi = sorted(rng.choice(V, 2, replace=False))
            tl[s, n, lo] = tl[s, n, hi] = 40.0
        tl[s, 0, :] = np.minimum(tl[s, 0, :], 1.0)
        tl[s, 0, 17], noise[s, 0, 17] = -0.0, 50.0
        tl[s, 0, 9], noise[s, 0, 9] = 0.0, 50.0
    _run(cfg, b, trees, tl, noise, np.float32(1.0))
    zero = np.zeros_like(noise)
    _run(cfg, b, trees, tl, zero, np.float32(1.0))
    st = lambda k: dev_tensor(np.stack([trees[s][k] for s in range(S)]).astype(np.int32))
    nn = dev_tensor(np.array([trees[s]["num_nodes"] for s in range(S)], dtype=np.int32))
    g1 = ddt.ddt_tree_walk(st("tree_tok"), st("parent"), nn, dev_tensor(tl), L)
    g2 = ddt.ddt_tree_walk_sample(st("tree_tok"), st("parent"), st("depth"), nn, dev_tensor(tl),
                                  dev_tensor(zero), 1.0, L)
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k
