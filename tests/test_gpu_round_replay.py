"""The benchmarked path: VerifyRound (ddt_draft_tree -> ddt_tree_attention ->
ddt_tree_walk on preallocated buffers and workspaces) over rotated input copies,
eagerly and replayed from HIP graphs, as bench.py runs it.

Each copy holds a different batch (its own seeds: different trees, one of them a
shortfall tree with num_nodes < B + 1).  The eager round of each copy must match the
oracle; every graph replay, interleaved with the other copies' replays and with eager
work and synchronisations in between, must reproduce that copy's eager outputs bit for
bit.  All copies share one walk workspace, which every call must leave zero-filled
(include/ddt.h), and one attention workspace.  Also: repeated ddt_tree_walk calls on
one workspace with changes of shape in between.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import block_diffusion_draft_position_amd as ddt
import oracle
from ddt_synthetic import configs, gen

from _gpu import check_attention_rows, dev_tensor, target_for, upload, widen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ddt.load()


# V = 40000 gives the walk several batches per row; the third copy's L = 2, K = 3
# candidate tree holds only 12 prefixes for B = 40 (shortfall)
BASE = dict(S=3, L=6, V=40000, K=6, B=40, prefix=(300, 1500), Hq=16, Hkv=2, D=128, dtype="bf16")


def _copies():
    cfgs = [configs.custom("replay-a", cfg_id=201, **BASE),
            configs.custom("replay-b", cfg_id=202, **BASE),
            configs.custom("replay-c", cfg_id=203, **{**BASE, "L": 2, "K": 3})]
    return cfgs


def _oracle_round(cfg, b):
    trees = {}
    for s in range(cfg.S):
        tok, lq = oracle.topk(b["draft_logits"][s], cfg.K)
        trees[s] = (tok, lq, oracle.build_tree(tok, lq, int(b["bonus"][s]), cfg.B))
    tl = target_for(cfg, b, {s: t[2] for s, t in trees.items()})
    return trees, tl


def _snapshot(res):
    return {k: v.clone() for k, v in res.items() if v is not None}


def test_verify_round_graph_replay_matches_eager_and_oracle():
    cfgs = _copies()
    # one round object per (L, K); the copies of one shape share it, as in the benchmark
    sh = ddt.Shape(S=BASE["S"], L=BASE["L"], V=BASE["V"], K=BASE["K"], B=BASE["B"], Hq=BASE["Hq"],
                   Hkv=BASE["Hkv"], D=BASE["D"], dtype=torch.bfloat16, max_prefix=BASE["prefix"][1])
    copies = []
    for cfg in cfgs:
        b = gen.batch(cfg)
        trees, tl = _oracle_round(cfg, b)
        d = upload(b)
        d["target"] = dev_tensor(tl)
        copies.append((cfg, b, d, trees, tl))
    assert int(copies[2][3][0][2]["num_nodes"]) < cfgs[2].N, "the third copy must be a shortfall tree"
    rounds = {}
    for cfg, *_ in copies:
        key = (cfg.L, cfg.K)
        if key not in rounds:
            rounds[key] = ddt.VerifyRound(dataclasses.replace(sh, L=cfg.L, K=cfg.K), "cuda")
    # all round objects share one walk workspace and one attention workspace
    ws_walk = max((r.ws_walk for r in rounds.values()), key=lambda t: t.numel())
    ws_attn = max((r.ws_attn for r in rounds.values()), key=lambda t: t.numel())
    for r in rounds.values():
        r.ws_walk, r.ws_attn = ws_walk, ws_attn

    def step(i):
        cfg, b, d, _, _ = copies[i]
        r = rounds[(cfg.L, cfg.K)]
        return r(d["draft_logits"], d["bonus"], d["q"], d["k_cache"], d["v_cache"], d["cu_prefix"],
                 d["k_tree"], d["v_tree"], d["target"])

    eager = []
    for i, (cfg, b, d, trees, tl) in enumerate(copies):
        print(f"[case] eager round of copy {cfg.name}", flush=True)
        res = step(i)
        torch.cuda.synchronize()
        snap = _snapshot(res)
        eager.append(snap)
        _check_oracle(cfg, b, trees, tl, snap)
    assert not torch.any(ws_walk), "walk workspace not left zero-filled"
    # capture one graph per copy, then replay them in rotation
    graphs = []
    for i in range(len(copies)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(i)
        graphs.append(g)
    torch.cuda.synchronize()
    order = [0, 1, 2, 2, 0, 1, 0, 0, 2, 1]
    for it, i in enumerate(order):
        print(f"[case] replay {it} of copy {copies[i][0].name}", flush=True)
        graphs[i].replay()
        if it % 3 == 1:   # the program's own eager work between replays
            torch.cuda.synchronize()
            _ = (copies[i][2]["draft_logits"] * 2.0).sum().item()
        torch.cuda.synchronize()
        cfg = copies[i][0]
        got = rounds[(cfg.L, cfg.K)].results()
        for k, v in eager[i].items():
            assert torch.equal(got[k], v), f"replay {it} (copy {i}): {k} differs from the eager round"
        assert not torch.any(ws_walk), f"replay {it}: walk workspace not left zero-filled"
    del graphs


def _check_oracle(cfg, b, trees, tl, got):
    scale = 1.0 / math.sqrt(cfg.D)
    mask = got["mask"].cpu().numpy().view(np.uint32)
    for s in range(cfg.S):
        tok, lq, t = trees[s]
        nn = int(t["num_nodes"])
        assert np.array_equal(got["topk_tok"][s].cpu().numpy(), tok)
        assert int(got["num_nodes"][s]) == nn
        for k in ("tree_tok", "parent", "depth"):
            assert np.array_equal(got[k][s].cpu().numpy(), t[k]), f"seq {s}: {k}"
        m_ref = oracle.tree_mask(t["parent"], nn, cfg.N)
        assert np.array_equal(mask[s], m_ref)
        w = oracle.tree_walk(t["tree_tok"], t["parent"], nn, tl[s], cfg.L)
        for k, gk in (("accept_len", "accept_len"), ("acc_nodes", "acc_nodes"), ("acc_tok", "acc_tok"),
                      ("bonus", "bonus")):
            assert np.array_equal(got[gk][s].cpu().numpy(), w[k]), f"seq {s}: {k}"
        rows = [(n, h) for n in range(cfg.N) for h in range(cfg.Hq)][::5]
        p0, p1 = int(b["cu_prefix"][s]), int(b["cu_prefix"][s + 1])
        W = oracle.round.widen
        ref_o, _ = oracle.tree_attention(W(b["q"][s]), W(b["k_cache"][p0:p1]), W(b["v_cache"][p0:p1]),
                                         W(b["k_tree"][s]), W(b["v_tree"][s]), m_ref, nn, scale, rows)
        go = widen(got["out"][s])
        check_attention_rows(go[[r[0] for r in rows], [r[1] for r in rows]], ref_o, cfg.dtype,
                             f"{cfg.name} seq {s}")


@pytest.mark.parametrize("strategy", ["auto", "scan", "hybrid"])
def test_walk_workspace_reuse_across_shapes(strategy):
    """ddt_tree_walk on one workspace, sized for the largest call, several calls in a
    row with different S, B and V (one row batch and several), a shortfall tree and a
    confident draft whose walk the hybrid hands over to the scan; every call must match
    the oracle and leave the workspace zero-filled, under the planner's choice and under
    the two strategies that use the workspace."""
    shapes = [dict(S=2, L=5, V=70000, K=4, B=30), dict(S=1, L=3, V=900, K=2, B=50),
              dict(S=4, L=4, V=128256, K=8, B=64), dict(S=3, L=6, V=5000, K=5, B=20),
              dict(S=3, L=8, V=4099, K=4, B=60, chain_boost=5.0),
              dict(S=2, L=5, V=70000, K=4, B=30)]
    need = max(ddt.load().ddt_tree_walk_workspace_size(sh["S"], sh["B"], sh["V"]) for sh in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    mode = {"auto": ddt.WALK_AUTO, "scan": ddt.WALK_SCAN, "hybrid": ddt.WALK_HYBRID}[strategy]
    ddt.walk_strategy(mode)
    try:
        _reuse_calls(shapes, ws, strategy)
    finally:
        ddt.walk_strategy(ddt.WALK_AUTO)


def _reuse_calls(shapes, ws, strategy):
    for i, sh in enumerate(shapes):
        print(f"[case] walk {strategy} call {i}: {sh}", flush=True)
        cfg = configs.custom(f"walk-reuse-{i}", cfg_id=300 + i, prefix=(1, 1), Hq=1, Hkv=1, D=32,
                             dtype="f32", **sh)
        b = gen.batch(cfg, with_qkv=False)
        confident = "chain_boost" in sh
        if confident:
            b["keep"][:] = True
        trees = {}
        for s in range(cfg.S):
            tok, lq = oracle.topk(b["draft_logits"][s], cfg.K)
            trees[s] = oracle.build_tree(tok, lq, int(b["bonus"][s]), cfg.B)
        tl = target_for(cfg, b, trees)
        tt = dev_tensor(np.stack([trees[s]["tree_tok"] for s in range(cfg.S)]))
        par = dev_tensor(np.stack([trees[s]["parent"] for s in range(cfg.S)]))
        nn = dev_tensor(np.array([trees[s]["num_nodes"] for s in range(cfg.S)], dtype=np.int32))
        w = ddt.ddt_tree_walk(tt, par, nn, dev_tensor(tl), cfg.L, ws=ws)
        torch.cuda.synchronize()
        acc = []
        for s in range(cfg.S):
            ref = oracle.tree_walk(trees[s]["tree_tok"], trees[s]["parent"], int(trees[s]["num_nodes"]),
                                   tl[s], cfg.L)
            for k in ("accept_len", "acc_nodes", "acc_tok", "bonus"):
                assert np.array_equal(w[k][s].cpu().numpy(), ref[k]), f"call {i} seq {s}: {k}"
            acc.append(int(ref["accept_len"]))
        assert not torch.any(ws), f"call {i}: workspace not left zero-filled"
        if confident:
            assert max(acc) > 3, acc   # a walk longer than the hybrid's three path steps
        if i == 1:
            assert int(trees[0]["num_nodes"]) < cfg.N, "call 1 must be a shortfall tree"
