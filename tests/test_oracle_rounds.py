"""Pins of the oracle's multi-round loop (oracle/rounds.py) against what the
mathematics fixes, independently of the loop's own code:
  * losslessness over rounds (DDTree page, 核心創新: the target's output is preserved;
    運作流程 step 4: the first mismatch is carried as the next bonus): the tokens
    emitted by R rounds equal plain one-token-at-a-time greedy decoding of the same
    target, computed here without trees;
  * the committed cache equals the cache plain decoding builds: row P0 + i holds the
    K/V of generated token i in its context, drawn directly from the synthetic model;
  * every round's root attention equals plain causal attention of the root's query
    over the whole sequence so far (the initial prefix, every earlier generated token,
    then the root itself), assembled here from the synthetic model;
  * positions continue the sequence: the root of a round sits at P0 + (tokens
    generated before it).
"""
import math

import numpy as np
import pytest

import oracle
from ddt_synthetic import configs, gen


def _setup(cfg, s):
    P0 = gen.prefix_len(cfg, s)
    x = gen.qkv(cfg, s, P0)
    b0 = gen.seq_first_bonus(cfg, s)
    draft = lambda g: gen.seq_draft(cfg, s, g)
    inputs = lambda g, t: gen.seq_tree_inputs(cfg, s, g, t["tree_tok"], t["parent"], int(t["num_nodes"]))
    return P0, x["k_prefix"], x["v_prefix"], b0, draft, inputs


CASES = [
    # confident drafter: several tokens accepted per round
    dict(name="confident", S=2, L=6, V=300, K=4, B=20, prefix=(40, 90), Hq=4, Hkv=2, D=32,
         dtype="f32", chain_boost=6.0),
    # weak drafter: mostly one token per round
    dict(name="weak", S=1, L=4, V=2000, K=3, B=10, prefix=(20, 20), Hq=2, Hkv=1, D=32, dtype="bf16"),
    # tiny budget: chains of one
    dict(name="B1", S=1, L=5, V=200, K=2, B=1, prefix=(10, 10), Hq=2, Hkv=2, D=32, dtype="f32",
         chain_boost=8.0),
]


@pytest.mark.parametrize("kw", CASES, ids=[c["name"] for c in CASES])
def test_rounds_equal_plain_greedy_decoding(kw):
    kw = dict(kw)
    cfg = configs.custom(kw.pop("name"), cfg_id=500, **kw)
    rounds = 6
    total_accepted = 0
    for s in range(cfg.S):
        P0, kp, vp, b0, draft, inputs = _setup(cfg, s)
        g, rec = oracle.run_rounds(draft, inputs, kp, vp, b0, cfg.K, cfg.B, rounds,
                                   1.0 / math.sqrt(cfg.D), attention_rows=[(0, h) for h in range(cfg.Hq)])
        target_fn = lambda ctx: gen.seq_target_row(cfg, s, ctx)
        assert g[1:] == oracle.greedy_decode(target_fn, [b0], len(g) - 1)
        assert len(g) - 1 == sum(int(r["accept_len"]) + 1 for r in rec)
        total_accepted += sum(int(r["accept_len"]) for r in rec)
        # the committed cache is the sequential cache
        kc, vc = rec[-1]["k_cache"], rec[-1]["v_cache"]
        assert kc.shape[0] == P0 + len(g) - 1     # every generated token but the pending bonus
        assert np.array_equal(kc[:P0], kp) and np.array_equal(vc[:P0], vp)
        for i in range(len(g) - 1):
            x = gen.seq_node_qkv(cfg, s, g[:i + 1])
            assert np.array_equal(kc[P0 + i], x["k"]), f"seq {s}: K row of generated token {i}"
            assert np.array_equal(vc[P0 + i], x["v"]), f"seq {s}: V row of generated token {i}"
        # each round's root: positions and plain causal attention over the whole sequence
        W = oracle.round.widen
        done = 0
        for r in rec:
            assert r["prefix_len"] == P0 + done and r["pos_ids"][0] == P0 + done
            assert r["context"] == g[:done + 1]
            seq_k = [W(kp)] + [W(gen.seq_node_qkv(cfg, s, g[:i + 1])["k"])[None] for i in range(done + 1)]
            seq_v = [W(vp)] + [W(gen.seq_node_qkv(cfg, s, g[:i + 1])["v"])[None] for i in range(done + 1)]
            keys, vals = np.concatenate(seq_k), np.concatenate(seq_v)
            q_root = W(gen.seq_node_qkv(cfg, s, g[:done + 1])["q"])
            G = cfg.Hq // cfg.Hkv
            for h in range(cfg.Hq):
                o, lse = oracle.attend(q_root[h], keys[:, h // G], vals[:, h // G], 1.0 / math.sqrt(cfg.D))
                np.testing.assert_allclose(r["o"][h], o, rtol=0, atol=1e-12)
                assert abs(r["lse"][h] - lse) <= 1e-12 * max(1.0, abs(lse))
            done += int(r["accept_len"]) + 1
    if kw.get("chain_boost", 0) >= 6.0 and cfg.B > 1:
        assert total_accepted >= 2 * rounds * cfg.S, total_accepted   # several per round


def test_commit_appends_root_then_accepted_path():
    kp = np.arange(2 * 3 * 4, dtype=np.float32).reshape(2, 3, 4)
    kt = 100 + np.arange(5 * 3 * 4, dtype=np.float32).reshape(5, 3, 4)
    k, v = oracle.commit_kv(kp, -kp, kt, -kt, np.array([2, 4, -1, -1]), 2)
    assert k.shape == (5, 3, 4)
    assert np.array_equal(k[:2], kp) and np.array_equal(k[2], kt[0])
    assert np.array_equal(k[3], kt[2]) and np.array_equal(k[4], kt[4])
    assert np.array_equal(v, -k)
    k0, _ = oracle.commit_kv(kp, kp, kt, kt, np.array([-1, -1, -1, -1]), 0)
    assert k0.shape[0] == 3 and np.array_equal(k0[2], kt[0])
