"""Several verification rounds on the GPU with the KV cache carried between them
(DDTree page "策展 · X (Twitter)", section 運作流程: each round starts from the bonus
token the previous one emitted), against the oracle's loop (oracle/rounds.py), whose
output is pinned to plain greedy decoding.

Per round, through the C ABI: ddt_draft_tree (with prefix_len), ddt_tree_attention
(with prefix_len), ddt_tree_walk, ddt_commit_kv.  The next round's bonus is the
previous walk's bonus_out tensor, passed on the device.  The cache has room for every
round: sequence s owns rows cu[s] .. cu[s+1] and its length advances in place.  Each
round is compared with the oracle's: tree, mask and positions bit-exact, attention
within the bf16/fp32 tolerances, walk bit-exact, the committed cache bit for bit and
the new lengths exactly; the tokens emitted over all rounds must be the oracle's.
"""
import math

import numpy as np
import pytest
import torch

import block_diffusion_draft_position_amd as ddt
import oracle
from ddt_synthetic import configs, gen
from ddt_synthetic.configs import TIE_GAP

from _gpu import check_attention_rows, dev_tensor, widen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ddt.load()


CASES = {
    "bf16": dict(S=3, L=6, V=2000, K=4, B=24, prefix=(100, 700), Hq=8, Hkv=2, D=128, dtype="bf16",
                 chain_boost=5.0),
    "f32": dict(S=2, L=5, V=500, K=3, B=12, prefix=(30, 80), Hq=4, Hkv=2, D=64, dtype="f32",
                chain_boost=6.0),
    "long-vocab": dict(S=2, L=8, V=40000, K=8, B=40, prefix=(1000, 1300), Hq=16, Hkv=2, D=128,
                       dtype="bf16", chain_boost=7.0),
}
ROUNDS = 5


class Drafts:
    """The round's draft logits for context g: the first attempt whose selection
    boundary clears the near-tie gap (the GPU accumulates in fp32, the oracle in fp64)."""

    def __init__(self, cfg, s):
        self.cfg, self.s, self.cache = cfg, s, {}

    def __call__(self, g):
        key = tuple(g)
        if key not in self.cache:
            for a in range(64):
                x = gen.seq_draft(self.cfg, self.s, g, a)
                _, lq = oracle.topk(x, self.cfg.K)
                if oracle.selection_gap(lq, self.cfg.B) >= TIE_GAP:
                    break
            self.cache[key] = x
        return self.cache[key]


@pytest.mark.parametrize("name", list(CASES))
def test_rounds_match_oracle(name):
    cfg = configs.custom(f"rounds-{name}", cfg_id=600 + len(name), **CASES[name])
    S, N, L = cfg.S, cfg.N, cfg.L
    scale = 1.0 / math.sqrt(cfg.D)
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    # ---- oracle loop, one sequence at a time
    drafts = [Drafts(cfg, s) for s in range(S)]
    ref, P0, pre = [], [], []
    for s in range(S):
        P = gen.prefix_len(cfg, s)
        x = gen.qkv(cfg, s, P)
        P0.append(P)
        pre.append(x)
        inputs = lambda g, t, s=s: gen.seq_tree_inputs(cfg, s, g, t["tree_tok"], t["parent"], int(t["num_nodes"]))
        rows = [(n, h) for n in range(N) for h in range(cfg.Hq)][::3]
        ref.append(oracle.run_rounds(drafts[s], inputs, x["k_prefix"], x["v_prefix"],
                                     gen.seq_first_bonus(cfg, s), cfg.K, cfg.B, ROUNDS, scale, rows))
    # ---- the GPU's cache: room for every round
    cap = [P0[s] + ROUNDS * (L + 1) for s in range(S)]
    cu = np.concatenate([[0], np.cumsum(cap)]).astype(np.int64)
    et = np.uint16 if cfg.dtype == "bf16" else np.float32
    kc = np.zeros((int(cu[-1]), cfg.Hkv, cfg.D), dtype=et)
    vc = np.zeros_like(kc)
    for s in range(S):
        kc[cu[s]:cu[s] + P0[s]] = pre[s]["k_prefix"]
        vc[cu[s]:cu[s] + P0[s]] = pre[s]["v_prefix"]
    d_kc, d_vc, d_cu = dev_tensor(kc), dev_tensor(vc), dev_tensor(cu)
    d_len = dev_tensor(np.array(P0, dtype=np.int64))
    bonus = dev_tensor(np.array([gen.seq_first_bonus(cfg, s) for s in range(S)], dtype=np.int32))
    g = [[gen.seq_first_bonus(cfg, s)] for s in range(S)]
    W = oracle.round.widen
    for r in range(ROUNDS):
        print(f"[case] {cfg.name} round {r}", flush=True)
        logits = dev_tensor(np.stack([drafts[s](g[s]) for s in range(S)]))
        dt = ddt.ddt_draft_tree(logits, bonus, d_cu, cfg.K, cfg.B, prefix_len=d_len)
        torch.cuda.synchronize()
        tt, par, nn = (dt[k].cpu().numpy() for k in ("tree_tok", "parent", "num_nodes"))
        xs = [gen.seq_tree_inputs(cfg, s, g[s], tt[s], par[s], int(nn[s])) for s in range(S)]
        q = dev_tensor(np.stack([x["q"] for x in xs]))
        kt = dev_tensor(np.stack([x["k_tree"] for x in xs]))
        vt = dev_tensor(np.stack([x["v_tree"] for x in xs]))
        tgt = dev_tensor(np.stack([x["target"] for x in xs]))
        out, lse = ddt.ddt_tree_attention(q, d_kc, d_vc, d_cu, kt, vt, dt["mask"], dt["num_nodes"], scale,
                                          max_prefix=max(cap), prefix_len=d_len)
        w = ddt.ddt_tree_walk(dt["tree_tok"], dt["parent"], dt["num_nodes"], tgt, L)
        app = ddt.ddt_commit_kv(d_kc, d_vc, d_cu, d_len, kt, vt, w["acc_nodes"], w["accept_len"])
        torch.cuda.synchronize()
        gmask = dt["mask"].cpu().numpy().view(np.uint32)
        gpos = dt["pos_ids"].cpu().numpy()
        gw = {k: v.cpu().numpy() for k, v in w.items()}
        glen = d_len.cpu().numpy()
        gkc = d_kc.cpu().view(torch.int16 if cfg.dtype == "bf16" else torch.int32).numpy()
        gvc = d_vc.cpu().view(torch.int16 if cfg.dtype == "bf16" else torch.int32).numpy()
        go = widen(out)
        for s in range(S):
            rec = ref[s][1][r]
            nn_s = int(rec["num_nodes"])
            assert rec["context"] == g[s], f"seq {s} round {r}: context"
            assert int(nn[s]) == nn_s
            for k in ("tree_tok", "parent"):
                assert np.array_equal(dt[k][s].cpu().numpy(), rec[k]), f"seq {s} round {r}: {k}"
            assert np.array_equal(gmask[s], rec["mask"]), f"seq {s} round {r}: mask"
            assert np.array_equal(gpos[s], rec["pos_ids"]), f"seq {s} round {r}: positions"
            rows = [(n, h) for n in range(N) for h in range(cfg.Hq)][::3]
            check_attention_rows(go[s][[a for a, _ in rows], [b for _, b in rows]], rec["o"], cfg.dtype,
                                 f"seq {s} round {r}")
            for k in ("accept_len", "acc_nodes", "acc_tok", "bonus"):
                assert np.array_equal(gw[k][s], rec[k]), f"seq {s} round {r}: walk {k}"
            a = int(rec["accept_len"])
            assert int(app[s]) == a + 1 and int(glen[s]) == rec["k_cache"].shape[0]
            lo = int(cu[s])
            n_rows = rec["k_cache"].shape[0]
            view = np.int16 if cfg.dtype == "bf16" else np.int32
            assert np.array_equal(gkc[lo:lo + n_rows], np.ascontiguousarray(rec["k_cache"]).view(view)), \
                f"seq {s} round {r}: K cache"
            assert np.array_equal(gvc[lo:lo + n_rows], np.ascontiguousarray(rec["v_cache"]).view(view)), \
                f"seq {s} round {r}: V cache"
            g[s].extend(rec["emitted"])
        bonus = w["bonus"]   # carried on the device into the next round
    for s in range(S):
        assert g[s] == ref[s][0], f"seq {s}: emitted tokens"
    print("accepted per sequence:", [sum(int(x["accept_len"]) for x in ref[s][1]) for s in range(S)])


def test_commit_refuses_a_full_region():
    """A sequence whose room cannot take the round's rows is left unchanged (appended
    -1); the others commit."""
    S, N, L, Hkv, D = 2, 6, 4, 2, 64
    rng = np.random.default_rng(3)
    cu = np.array([0, 12, 20], dtype=np.int64)
    lens = np.array([5, 6], dtype=np.int64)       # sequence 1: 2 rows of room
    kc = rng.standard_normal((20, Hkv, D)).astype(np.float32)
    vc = rng.standard_normal((20, Hkv, D)).astype(np.float32)
    kt = rng.standard_normal((S, N, Hkv, D)).astype(np.float32)
    vt = rng.standard_normal((S, N, Hkv, D)).astype(np.float32)
    acc = np.array([[1, 3, 5, -1], [2, 4, -1, -1]], dtype=np.int32)
    alen = np.array([3, 2], dtype=np.int32)
    d_kc, d_vc, d_len = dev_tensor(kc), dev_tensor(vc), dev_tensor(lens)
    app = ddt.ddt_commit_kv(d_kc, d_vc, dev_tensor(cu), d_len, dev_tensor(kt), dev_tensor(vt),
                            dev_tensor(acc), dev_tensor(alen))
    torch.cuda.synchronize()
    assert app.cpu().tolist() == [4, -1]
    assert d_len.cpu().tolist() == [9, 6]
    k_new = d_kc.cpu().numpy()
    ref0, _ = oracle.commit_kv(kc[0:5], vc[0:5], kt[0], vt[0], acc[0], 3)
    assert np.array_equal(k_new[0:9], ref0)
    assert np.array_equal(k_new[9:], kc[9:])        # sequence 0's spare room and sequence 1
