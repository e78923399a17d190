"""The tree walk's three strategies through the C ABI (ddt_tree_walk_strategy): the row
scan (every node's arg-max by many workgroups, then the walk), the path walk (one
workgroup per sequence scans only the rows of the nodes it visits) and the hybrid (the
path walk for up to three accepted tokens, then the scan over the reached node's
subtree).  Each is forced in turn and compared with the oracle's walk, bit-exact on
accept lengths, accepted nodes and tokens and bonus tokens: ragged and 4-aligned
vocabularies, rows longer than one pass of the path walk's loads, the interface's
largest trees, long accepted paths (which the hybrid hands over), exact ties, the
sampling walk and the allocation-free entry point.  The planner's own choice is
covered by every other walk test."""
import numpy as np
import pytest
import torch

import block_diffusion_draft_position_amd as ddt
import oracle
from ddt_synthetic import configs, gen

from _cases import attempts
from _gpu import dev_tensor, target_for

pytestmark = pytest.mark.gpu

STRATEGIES = {"scan": ddt.WALK_SCAN, "path": ddt.WALK_PATH, "hybrid": ddt.WALK_HYBRID}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ddt.load()


@pytest.fixture(params=sorted(STRATEGIES))
def strategy(request):
    prev = ddt.walk_strategy(STRATEGIES[request.param])
    assert prev == ddt.WALK_AUTO
    yield request.param
    ddt.walk_strategy(ddt.WALK_AUTO)


def _trees(cfg, b):
    trees = {}
    for s in range(cfg.S):
        tok, lq = oracle.topk(b["draft_logits"][s], cfg.K)
        trees[s] = oracle.build_tree(tok, lq, int(b["bonus"][s]), cfg.B)
    return trees


def _stack(cfg, trees, k):
    return dev_tensor(np.stack([trees[s][k] for s in range(cfg.S)]).astype(np.int32))


def _num_nodes(cfg, trees):
    return dev_tensor(np.array([trees[s]["num_nodes"] for s in range(cfg.S)], dtype=np.int32))


def _greedy(cfg, trees, tl, noalloc=False):
    fn = ddt.ddt_tree_walk_noalloc if noalloc else ddt.ddt_tree_walk
    w = fn(_stack(cfg, trees, "tree_tok"), _stack(cfg, trees, "parent"), _num_nodes(cfg, trees),
           dev_tensor(tl), cfg.L)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in w.items()}


def _check(cfg, trees, tl, got, what):
    acc = []
    for s in range(cfg.S):
        t = trees[s]
        ref = oracle.tree_walk(t["tree_tok"], t["parent"], int(t["num_nodes"]), tl[s], cfg.L)
        for k in ("accept_len", "acc_nodes", "acc_tok", "bonus"):
            assert np.array_equal(got[k][s], ref[k]), f"{what} seq {s}: {k}"
        acc.append(int(ref["accept_len"]))
    return acc


def _batch(cfg, confident):
    b = gen.batch(cfg, with_qkv=False)
    if confident:
        b["keep"][:] = True   # the target agrees with the draft's chain: long accepted paths
    return b


SHAPES = [
    # (name, config keywords, confident)
    ("ragged-257", dict(S=3, L=4, V=257, K=4, B=12), False),
    ("ragged-4099", dict(S=4, L=6, V=4099, K=4, B=40, chain_boost=5.0), True),
    ("aligned-3000", dict(S=3, L=5, V=3000, K=4, B=40, chain_boost=5.0), True),
    # 70000 logits: more than one pass of 1024 threads x 16 float4 loads
    ("long-70000", dict(S=2, L=8, V=70000, K=4, B=60, chain_boost=5.0), True),
    ("B0", dict(S=2, L=4, V=500, K=4, B=0), False),
    ("L1", dict(S=2, L=1, V=500, K=6, B=6, chain_boost=5.0), True),
    ("deep-64", dict(S=2, L=64, V=40, K=2, B=150, chain_boost=200.0), True),
    ("widest", dict(S=1, L=3, V=5000, K=64, B=1023), False),
    ("wide-deep", dict(S=2, L=16, V=300, K=4, B=1023, chain_boost=200.0), True),
    # every position accepted with L = 3: the hybrid hands over at a node of depth L,
    # whose subtree is itself, and the scan only takes the bonus there
    ("L3-full", dict(S=3, L=3, V=4096, K=4, B=40, chain_boost=200.0), True),
    # a shortfall tree (31 nodes for a budget of 50: rows past num_nodes are padding)
    # whose walk of 4 tokens the hybrid hands over
    ("shortfall-deep", dict(S=2, L=4, V=600, K=2, B=50, chain_boost=200.0), True),
]


@pytest.mark.parametrize("name,kw,confident", SHAPES, ids=[s[0] for s in SHAPES])
def test_walk_strategies_match_oracle(strategy, name, kw, confident):
    cfg = configs.custom(f"walk-{name}", cfg_id=730 + [s[0] for s in SHAPES].index(name), **kw)
    print(f"[case] walk {strategy} {name}", flush=True)
    b = _batch(cfg, confident)
    trees = _trees(cfg, b)
    tl = target_for(cfg, b, trees)
    acc = _check(cfg, trees, tl, _greedy(cfg, trees, tl), f"{strategy} {name}")
    if confident:
        assert max(acc) >= min(cfg.L, 3), acc   # paths of several nodes are walked


@pytest.mark.parametrize("name", ["C2", "C4"])
def test_walk_strategies_full_workloads(strategy, name):
    cfg = configs.get(name)
    print(f"[case] walk {strategy} {name}", flush=True)
    b = gen.batch(cfg, attempts(cfg), with_qkv=False)
    trees = _trees(cfg, b)
    tl = target_for(cfg, b, trees)
    _check(cfg, trees, tl, _greedy(cfg, trees, tl), f"{strategy} {name}")


@pytest.mark.parametrize("kind", ["all-equal", "levels"])
def test_walk_strategies_exact_ties(strategy, kind):
    """Rows of equal logits: the arg-max is the smallest id among the row's maxima, and a
    child carrying it is searched for in index order."""
    cfg = configs.custom(f"walk-ties-{kind}", cfg_id=745, S=3, L=5, V=6000, K=4, B=50)
    b = gen.batch(cfg, with_qkv=False)
    trees = _trees(cfg, b)
    rng = np.random.default_rng(31)
    if kind == "all-equal":
        tl = np.full((cfg.S, cfg.N, cfg.V), 0.25, dtype=np.float32)
    else:
        tl = (np.round(rng.standard_normal((cfg.S, cfg.N, cfg.V)) * 2.0) / 2.0).astype(np.float32)
    # lead each tree's first chain with the lowest-id maximum so that the walk moves
    for s in range(cfg.S):
        t = trees[s]
        cur = 0
        for _ in range(cfg.L):
            kids = [c for c in range(int(t["num_nodes"])) if t["parent"][c] == cur]
            if not kids:
                break
            tok = int(t["tree_tok"][kids[0]])
            top = tl[s, cur].max()
            tl[s, cur, tok] = top
            tl[s, cur, :tok][tl[s, cur, :tok] == top] = top - 0.5
            cur = kids[0]
    acc = _check(cfg, trees, tl, _greedy(cfg, trees, tl), f"{strategy} ties {kind}")
    assert max(acc) >= 2, acc


@pytest.mark.parametrize("name,inv_t", [("C4", 1.0), ("C4", np.float32(1 / 0.7)), ("C2", 1.0),
                                        ("C0", 1.0)])
def test_sampling_walk_strategies(strategy, name, inv_t):
    cfg = configs.get(name)
    print(f"[case] sampling walk {strategy} {name} inv_t={float(inv_t):.4f}", flush=True)
    b = gen.batch(cfg, attempts(cfg), with_qkv=False)
    trees = _trees(cfg, b)
    tl = target_for(cfg, b, trees)
    noise = np.stack([gen.gumbel_noise(cfg, s) for s in range(cfg.S)])
    w = ddt.ddt_tree_walk_sample(_stack(cfg, trees, "tree_tok"), _stack(cfg, trees, "parent"),
                                 _stack(cfg, trees, "depth"), _num_nodes(cfg, trees), dev_tensor(tl),
                                 dev_tensor(noise), np.float32(inv_t), cfg.L)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in w.items()}
    for s in range(cfg.S):
        t = trees[s]
        ref = oracle.tree_walk_sample(t["tree_tok"], t["parent"], t["depth"], int(t["num_nodes"]),
                                      tl[s], noise[s], np.float32(inv_t), cfg.L)
        for k in ("accept_len", "acc_nodes", "acc_tok", "bonus"):
            assert np.array_equal(got[k][s], ref[k]), f"{strategy} {name} seq {s}: {k}"


def test_path_walk_noalloc_and_workspace_untouched():
    """The allocation-free entry point under each strategy in turn, hybrid walks with
    hand-overs (accepted paths of 4-6 tokens) among them: same outputs as the oracle
    every time, so each call left the array zero for the next (the scan relies on it)."""
    cfg = configs.custom("walk-na", cfg_id=750, S=4, L=6, V=4096, K=4, B=40, chain_boost=5.0)
    b = _batch(cfg, True)
    trees = _trees(cfg, b)
    tl = target_for(cfg, b, trees)
    try:
        for mode in (ddt.WALK_PATH, ddt.WALK_SCAN, ddt.WALK_HYBRID, ddt.WALK_HYBRID, ddt.WALK_SCAN):
            ddt.walk_strategy(mode)
            acc = _check(cfg, trees, tl, _greedy(cfg, trees, tl, noalloc=True), f"noalloc mode {mode}")
        assert max(acc) > 3, acc   # the hybrid handed over
    finally:
        ddt.walk_strategy(ddt.WALK_AUTO)


@pytest.mark.parametrize("inv_t", [1.0, 3.0])
def test_sampling_walk_strategies_long_paths(strategy, inv_t):
    """The sampling walk on confident drafts (accepted paths of several tokens, so the
    hybrid hands its walks over to the scan with the noise rows of the later depths)."""
    cfg = configs.custom("walk-sample-long", cfg_id=760, S=6, L=8, V=4099, K=4, B=60, chain_boost=5.0)
    b = _batch(cfg, True)
    trees = _trees(cfg, b)
    tl = target_for(cfg, b, trees)
    noise = np.stack([gen.gumbel_noise(cfg, s) for s in range(cfg.S)])
    w = ddt.ddt_tree_walk_sample(_stack(cfg, trees, "tree_tok"), _stack(cfg, trees, "parent"),
                                 _stack(cfg, trees, "depth"), _num_nodes(cfg, trees), dev_tensor(tl),
                                 dev_tensor(noise), np.float32(inv_t), cfg.L)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in w.items()}
    acc = []
    for s in range(cfg.S):
        t = trees[s]
        ref = oracle.tree_walk_sample(t["tree_tok"], t["parent"], t["depth"], int(t["num_nodes"]),
                                      tl[s], noise[s], np.float32(inv_t), cfg.L)
        for k in ("accept_len", "acc_nodes", "acc_tok", "bonus"):
            assert np.array_equal(got[k][s], ref[k]), f"{strategy} inv_t={inv_t} seq {s}: {k}"
        acc.append(int(ref["accept_len"]))
    assert max(acc) > 3, acc   # at least one walk goes past the hybrid's three path steps
