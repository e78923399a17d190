"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Integers (top-K tokens, tree, mask, positions, walk) must match exactly; floats
within the tolerances of tests/_gpu.py.  Small shapes span several key tiles,
several splits and ragged tails; the full workloads compare every integer output
and a sample of attention rows that the oracle computes one by one.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import block_diffusion_draft_position_amd as ddt
import oracle
from ddt_synthetic import configs, gen

from _cases import attempts
from _gpu import (NODE_LOGQ_ATOL, TOPK_ATOL, check_attention_rows, dev_tensor, target_for, upload,
                  widen)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ddt.load()


def _say(*a):
    print(*a, flush=True)


def run_case(cfg, att=None, rows_per_seq=None, sharp=False, seed_rows=0, fused=False):
    """Full round on the GPU and in the oracle; compare everything.  fused: steps 1-3
    through ddt_draft_tree instead of ddt_topk, ddt_build_tree and ddt_tree_mask."""
    _say(f"[case] {cfg.name} S={cfg.S} L={cfg.L} V={cfg.V} K={cfg.K} B={cfg.B} P={cfg.prefix} "
         f"Hq={cfg.Hq} Hkv={cfg.Hkv} D={cfg.D} {cfg.dtype} sharp={sharp} fused={fused}")
    if att is None:
        att = attempts(cfg)
    b = gen.batch(cfg, att)
    if sharp:
        _sharpen(cfg, b)
    scale = 1.0 / math.sqrt(cfg.D)
    # ---- oracle: steps 1-3 for every sequence
    trees, tk = {}, {}
    for s in range(cfg.S):
        tok, lq = oracle.topk(b["draft_logits"][s], cfg.K)
        tk[s] = (tok, lq)
        trees[s] = oracle.build_tree(tok, lq, int(b["bonus"][s]), cfg.B)
    tl = target_for(cfg, b, trees)
    # ---- GPU
    d = upload(b)
    d["target"] = dev_tensor(tl)
    if fused:
        dt = ddt.ddt_draft_tree(d["draft_logits"], d["bonus"], d["cu_prefix"], cfg.K, cfg.B)
        tok, lq, mask, pos = dt["topk_tok"], dt["topk_logq"], dt["mask"], dt["pos_ids"]
        tree = {k: dt[k] for k in ("tree_tok", "parent", "depth", "node_logq", "num_nodes")}
    else:
        tok, lq = ddt.ddt_topk(d["draft_logits"], cfg.K)
        tree = ddt.ddt_build_tree(tok, lq, d["bonus"], cfg.B)
        mask, pos = ddt.ddt_tree_mask(tree["parent"], tree["depth"], tree["num_nodes"], d["cu_prefix"])
    out, lse = ddt.ddt_tree_attention(d["q"], d["k_cache"], d["v_cache"], d["cu_prefix"], d["k_tree"],
                                      d["v_tree"], mask, tree["num_nodes"], scale)
    walk = ddt.ddt_tree_walk(tree["tree_tok"], tree["parent"], tree["num_nodes"], d["target"], cfg.L)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in tree.items() if v is not None}
    gw = {k: v.cpu().numpy() for k, v in walk.items()}
    gtok, glq = tok.cpu().numpy(), lq.cpu().numpy()
    gmask = mask.cpu().numpy().view(np.uint32)
    gpos = pos.cpu().numpy()
    rng = np.random.default_rng(1000 + seed_rows)
    for s in range(cfg.S):
        t = trees[s]
        nn = int(t["num_nodes"])
        assert np.array_equal(gtok[s], tk[s][0]), f"seq {s}: top-K tokens"
        np.testing.assert_allclose(glq[s], tk[s][1], rtol=0, atol=TOPK_ATOL, err_msg=f"seq {s}: logq")
        assert int(g["num_nodes"][s]) == nn, f"seq {s}: num_nodes"
        for k in ("tree_tok", "parent", "depth"):
            assert np.array_equal(g[k][s], t[k]), f"seq {s}: {k}"
        np.testing.assert_allclose(g["node_logq"][s][:nn], t["node_logq"][:nn], rtol=0,
                                   atol=NODE_LOGQ_ATOL)
        assert np.all(np.isneginf(g["node_logq"][s][nn:]))
        P = int(b["prefix_lens"][s])
        m_ref = oracle.tree_mask(t["parent"], nn, cfg.N)
        assert np.array_equal(gmask[s], m_ref), f"seq {s}: mask"
        assert np.array_equal(gpos[s], oracle.position_ids(t["depth"], nn, P)), f"seq {s}: pos"
        w = oracle.tree_walk(t["tree_tok"], t["parent"], nn, tl[s], cfg.L)
        assert int(gw["accept_len"][s]) == int(w["accept_len"]), f"seq {s}: accept_len"
        assert np.array_equal(gw["acc_nodes"][s], w["acc_nodes"]) and np.array_equal(gw["acc_tok"][s], w["acc_tok"])
        assert int(gw["bonus"][s]) == int(w["bonus"]), f"seq {s}: bonus"
        # attention: all rows, or a sample
        all_rows = [(n, h) for n in range(cfg.N) for h in range(cfg.Hq)]
        if rows_per_seq is None or rows_per_seq >= len(all_rows):
            rows = all_rows
        else:
            deep = int(np.argmax(t["depth"][:nn]))
            pick = set(map(tuple, [all_rows[i] for i in rng.choice(len(all_rows), rows_per_seq, replace=False)]))
            pick |= {(deep, h) for h in range(min(cfg.Hq, 4))} | {(0, 0), (nn - 1, cfg.Hq - 1)}
            if nn < cfg.N:
                pick |= {(cfg.N - 1, 0)}
            rows = sorted(pick)
        p0, p1 = int(b["cu_prefix"][s]), int(b["cu_prefix"][s + 1])
        ref_o, ref_l = oracle.tree_attention(oracle.round.widen(b["q"][s]), oracle.round.widen(b["k_cache"][p0:p1]),
                                             oracle.round.widen(b["v_cache"][p0:p1]), oracle.round.widen(b["k_tree"][s]),
                                             oracle.round.widen(b["v_tree"][s]), m_ref, nn, scale, rows)
        go = widen(out[s])
        gl = lse[s].cpu().numpy().astype(np.float64)
        idx_n = np.array([r[0] for r in rows])
        idx_h = np.array([r[1] for r in rows])
        check_attention_rows(go[idx_n, idx_h], ref_o, cfg.dtype, f"{cfg.name} seq {s}")
        valid = idx_n < nn
        np.testing.assert_allclose(gl[idx_n[valid], idx_h[valid]], ref_l[valid], rtol=0,
                                   atol=1e-5 if cfg.dtype == "f32" else 4e-3)
        assert np.all(np.isneginf(gl[idx_n[~valid], idx_h[~valid]]))
    return gw


def _sharpen(cfg, b):
    """Make the tree keys dominate the softmax so that a mask error cannot hide under a
    long prefix: every query and tree key leans on one direction u per (seq, KV head)."""
    rng = np.random.default_rng(77)
    a = math.sqrt(10.0 * math.sqrt(cfg.D))
    enc = (lambda x: gen.f32_to_bf16_bits(x)) if cfg.dtype == "bf16" else (lambda x: x.astype(np.float32))
    dec = (lambda x: gen.bf16_bits_to_f32(x)) if cfg.dtype == "bf16" else (lambda x: x)
    G = cfg.Hq // cfg.Hkv
    q = dec(b["q"]).copy()
    kt = dec(b["k_tree"]).copy()
    for s in range(cfg.S):
        for g in range(cfg.Hkv):
            u = rng.standard_normal(cfg.D)
            u /= np.linalg.norm(u)
            q[s, :, g * G:(g + 1) * G, :] += (a * u).astype(np.float32)
            kt[s, :, g, :] = (a * u).astype(np.float32) + 0.3 * rng.standard_normal((cfg.N, cfg.D))
    b["q"] = enc(q)
    b["k_tree"] = enc(kt)


# ----------------------------------------------------------------------------- small shapes
MID = dict(S=3, L=5, V=3000, K=4, B=40, prefix=(0, 700), Hq=8, Hkv=2)


@pytest.mark.parametrize("D", [128, 64, 32])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_mid_shapes(D, dtype):
    cfg = configs.custom(f"mid-{dtype}-D{D}", D=D, dtype=dtype, **MID)
    run_case(cfg)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_sharp_tree_keys(dtype):
    cfg = configs.custom(f"sharp-{dtype}", S=2, L=6, V=500, K=3, B=50, prefix=(2000, 2600),
                         Hq=8, Hkv=2, D=128, dtype=dtype)
    run_case(cfg, sharp=True)


@pytest.mark.parametrize("name,kw", [
    ("B0", dict(B=0)), ("B1", dict(B=1)), ("K1", dict(K=1, B=7)), ("L1", dict(L=1, K=6, B=6)),
    ("P0", dict(prefix=(0, 0))), ("P1", dict(prefix=(1, 1))), ("P7", dict(prefix=(7, 7))),
    ("shortfall", dict(L=2, K=3, B=20)), ("wide", dict(K=64, B=200, L=3, V=400)),
    ("deep", dict(L=64, K=2, B=150, V=40)), ("gqa8", dict(Hq=16, Hkv=2)), ("mha", dict(Hq=4, Hkv=4)),
    # confident drafts: chain log-probabilities of exactly 0 (boost 200) or ~1e-12 (boost 30),
    # which the tree builder meets one depth per round
    ("sure", dict(B=12, chain_boost=200.0)), ("sure-deep", dict(L=16, K=4, B=60, V=300, chain_boost=200.0)),
    ("near-sure", dict(L=8, B=30, chain_boost=30.0)),
])
@pytest.mark.parametrize("fused", [False, True], ids=["calls", "fused"])
def test_edge_cases(name, kw, fused):
    base = dict(S=2, L=4, V=257, K=4, B=12, prefix=(5, 150), Hq=8, Hkv=2, D=128, dtype="bf16")
    base.update(kw)
    cfg = configs.custom(f"edge-{name}", **base)
    run_case(cfg, fused=fused)


def _tie_rows(kind, rows, V, rng):
    if kind == "all-equal":
        return np.full((rows, V), 0.5, dtype=np.float32)
    if kind == "levels":        # a few distinct values: hundreds of ties in every chunk
        return (np.round(rng.standard_normal((rows, V)) * 2.0) / 2.0).astype(np.float32)
    if kind == "top-level":     # one value shared by a third of the row, the rest below it
        x = rng.uniform(-8.0, -1.0, (rows, V)).astype(np.float32)
        x[rng.random((rows, V)) < 1 / 3] = 2.0
        return x
    if kind == "neg-inf":       # mostly -inf, a few finite values, ties among them
        x = np.full((rows, V), -np.inf, dtype=np.float32)
        for r in range(rows):
            idx = rng.choice(V, size=200, replace=False)
            x[r, idx] = np.round(rng.standard_normal(200)).astype(np.float32)
        return x
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["all-equal", "levels", "top-level", "neg-inf"])
@pytest.mark.parametrize("rows,V,k", [(3, 4099, 8), (2, 3000, 64), (20, 70000, 32), (20, 110000, 16)])
def test_topk_ties(kind, rows, V, k):
    """Top-K of rows with heavy ties: chunks whose candidates exceed what the rank
    count holds take the wave-maximum fallback.  Equal logits go to the smaller id;
    tokens must match exactly.  V = 4099 leaves a ragged tail (scalar loads); 20 rows of
    70000 use the 16-per-lane chunks, 20 rows of 110000 the 32-per-lane chunks."""
    rng = np.random.default_rng(7 + rows + k)
    x = _tie_rows(kind, rows, V, rng)
    rt, rl = oracle.topk(x, k)
    gt, gl = ddt.ddt_topk(dev_tensor(x), k)
    torch.cuda.synchronize()
    assert np.array_equal(gt.cpu().numpy(), rt), kind
    assert np.max(np.abs(gl.cpu().numpy().astype(np.float64) - rl)) <= TOPK_ATOL, kind


def test_narrow_attention_groups():
    """A grid too large for one workgroup per CU: 4-wave row groups, two per CU, the last
    group of each (sequence, KV head) holding only the remainder rows (its other waves
    idle), ragged prefixes cut into many splits."""
    cfg = configs.custom("narrow", S=6, L=4, V=500, K=4, B=64, prefix=(900, 3000), Hq=16, Hkv=4,
                         D=128, dtype="bf16")
    run_case(cfg, rows_per_seq=240)


@pytest.mark.parametrize("name,kw", [
    # 152 rows per KV head: a full 128-row group and 24 rows left, so each of the two
    # streams of the remainder group computes both 16-row query blocks
    ("rem24", dict(S=4, B=18, prefix=(1500, 3000), Hq=16, Hkv=2)),
    # 4 rows left and prefixes cut into one-tile splits: the second stream gets no tile
    ("rem4-one-tile", dict(S=6, B=64, prefix=(5, 500), Hq=16, Hkv=4)),
    # 8 rows left, three tiles per split (two for one stream, one for the other) and a
    # ragged last tile in each sequence's last split
    ("rem8-odd", dict(S=3, B=16, prefix=(2000, 4100), Hq=16, Hkv=2)),
    # 1028 rows per KV head: eight full groups and 4 rows, the remainder groups dispatched
    # after every full group
    ("rem4-last", dict(S=2, B=256, prefix=(300, 700), Hq=32, Hkv=8)),
])
def test_remainder_group_streams(name, kw):
    """Remainder row groups of at most 32 rows: two waves stream alternate key tiles for
    the same rows and merge their partial softmax states; every row is checked."""
    cfg = configs.custom(name, L=4, V=500, K=4, D=128, dtype="bf16", **kw)
    run_case(cfg)


def test_signed_zero_ties():
    """-0.0 and +0.0 compare equal, so a tie between them goes to the smaller token id,
    in the top-K and in the walk's arg-max, as in the oracle."""
    S, L, V, K, B = 2, 3, 96, 4, 6
    rng = np.random.default_rng(5)
    logits = np.full((S, L, V), -4.0, dtype=np.float32)
    logits += rng.uniform(-0.5, 0.0, size=logits.shape).astype(np.float32)
    for s in range(S):
        for i in range(L):
            ids = rng.choice(V, 3, replace=False)
            lo, mid, hi = np.sort(ids)
            logits[s, i, lo] = -0.0
            logits[s, i, hi] = 0.0
            logits[s, i, mid] = -0.0
    bonus = np.array([1, 2], dtype=np.int32)
    d = dev_tensor(logits)
    tok, lq = ddt.ddt_topk(d, K)
    gtok, glq = tok.cpu().numpy(), lq.cpu().numpy()
    for s in range(S):
        rt, rl = oracle.topk(logits[s], K)
        assert np.array_equal(gtok[s], rt), s
        np.testing.assert_allclose(glq[s], rl, rtol=0, atol=TOPK_ATOL)
    # the zeros tie exactly, so the tree may order them either way (a tie the synthetic
    # workloads exclude); the walk is checked on the GPU's own tree on both sides
    tree = ddt.ddt_build_tree(tok, lq, dev_tensor(bonus), B)
    gt = {k: v.cpu().numpy() for k, v in tree.items() if v is not None}
    N = B + 1
    target = np.full((S, N, V), -3.0, dtype=np.float32)
    for s in range(S):
        for n in range(int(gt["num_nodes"][s])):
            kids = [c for c in range(N) if gt["parent"][s][c] == n]
            want = int(gt["tree_tok"][s][kids[0]]) if kids else int(rng.integers(V))
            other = (want + 7) % V
            lo, hi = min(want, other), max(want, other)
            target[s, n, lo] = -0.0   # the smaller id holds -0: it must win the tie
            target[s, n, hi] = 0.0
    walk = ddt.ddt_tree_walk(tree["tree_tok"], tree["parent"], tree["num_nodes"], dev_tensor(target), L)
    gw = {k: v.cpu().numpy() for k, v in walk.items()}
    for s in range(S):
        w = oracle.tree_walk(gt["tree_tok"][s], gt["parent"][s], int(gt["num_nodes"][s]), target[s], L)
        assert int(gw["accept_len"][s]) == int(w["accept_len"]), s
        assert int(gw["bonus"][s]) == int(w["bonus"]), s
        assert np.array_equal(gw["acc_nodes"][s], w["acc_nodes"]), s


@pytest.mark.parametrize("fused", [False, True], ids=["calls", "fused"])
def test_large_budget_multi_word_mask(fused):
    cfg = configs.custom("bigB", S=1, L=8, V=1000, K=16, B=700, prefix=(300, 300), Hq=4, Hkv=1,
                         D=64, dtype="bf16")
    run_case(cfg, fused=fused)


@pytest.mark.parametrize("fused", [False, True], ids=["calls", "fused"])
def test_widest_round(fused):
    """K = 64 and B = 1023 over three positions: the third round has 3369 candidates for
    809 places, more than the 2048 whose keys the radix select keeps in LDS, so each of
    its passes recomputes the keys stream by stream (the earlier rounds take 45 and 169
    candidates: all of them, then a ranked cut)."""
    cfg = configs.custom("widest", S=1, L=3, V=5000, K=64, B=1023, prefix=(64, 64), Hq=4, Hkv=1,
                         D=64, dtype="bf16")
    run_case(cfg, rows_per_seq=64, fused=fused)


@pytest.mark.parametrize("fused", [False, True], ids=["calls", "fused"])
def test_size_limits(fused):
    """L, K and B at the interface's limits (64, 64, 1023): the tree builder's LDS table
    (about 90 KB) is above the default dynamic-LDS limit of a launch."""
    cfg = configs.custom("limits", S=1, L=64, V=200, K=64, B=1023, prefix=(40, 40), Hq=2, Hkv=1,
                         D=32, dtype="bf16")
    run_case(cfg, fused=fused)


def test_fused_matches_calls_bitwise():
    """ddt_draft_tree equals ddt_topk -> ddt_build_tree -> ddt_tree_mask bit for bit,
    including the fp32 log-probabilities, on a long-vocabulary batch."""
    cfg = configs.custom("fused-eq", S=3, L=12, V=40000, K=8, B=90, prefix=(10, 900), Hq=8,
                         Hkv=2, D=128, dtype="bf16")
    b = gen.batch(cfg, attempts(cfg), with_qkv=False)
    d = upload(b)
    dt = ddt.ddt_draft_tree(d["draft_logits"], d["bonus"], d["cu_prefix"], cfg.K, cfg.B)
    tok, lq = ddt.ddt_topk(d["draft_logits"], cfg.K)
    tree = ddt.ddt_build_tree(tok, lq, d["bonus"], cfg.B)
    mask, pos = ddt.ddt_tree_mask(tree["parent"], tree["depth"], tree["num_nodes"], d["cu_prefix"])
    ref = dict(topk_tok=tok, topk_logq=lq, mask=mask, pos_ids=pos, **tree)
    for k, v in ref.items():
        assert torch.equal(dt[k], v), k


def test_tiny_workload_many_draws():
    cfg = dataclasses.replace(configs.C0, S=16)   # sequences 0..15 of the tiny workload
    w = run_case(cfg)
    _say("tiny accept lengths", w["accept_len"].tolist())


def test_deterministic():
    cfg = configs.custom("det", S=2, L=6, V=5000, K=8, B=60, prefix=(900, 1300), Hq=8, Hkv=2,
                         D=128, dtype="bf16")
    b = gen.batch(cfg)
    d = upload(b)
    outs = []
    for _ in range(2):
        tok, lq = ddt.ddt_topk(d["draft_logits"], cfg.K)
        tree = ddt.ddt_build_tree(tok, lq, d["bonus"], cfg.B)
        mask, _ = ddt.ddt_tree_mask(tree["parent"], tree["depth"], tree["num_nodes"], None)
        out, lse = ddt.ddt_tree_attention(d["q"], d["k_cache"], d["v_cache"], d["cu_prefix"],
                                          d["k_tree"], d["v_tree"], mask, tree["num_nodes"])
        outs.append([x.cpu() for x in (tok, lq, tree["tree_tok"], mask, out.view(torch.int16), lse)])
    for a, b2 in zip(*outs):
        assert torch.equal(a, b2)


# ----------------------------------------------------------------------------- full workloads
@pytest.mark.parametrize("name,rows", [("C0", None), ("C1", 200), ("C2", 48), ("C3-B16", 64),
                                       ("C3-B32", 64), ("C3-B64", 64), ("C3-B128", 64),
                                       ("C3-B256", 64), ("C3-B512", 64), ("C4", 12)])
@pytest.mark.parametrize("fused", [False, True], ids=["calls", "fused"])
def test_full_workloads(name, rows, fused):
    run_case(configs.get(name), rows_per_seq=rows, fused=fused)
