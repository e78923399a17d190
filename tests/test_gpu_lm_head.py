"""The fused verifier epilogue (ddt_lm_head_argmax) and the token-driven walk
(ddt_tree_walk_tokens) through the C ABI against the oracle.

The kernel decides each node's arg-max on fp32 logits (bf16 products, fp32 sums);
the oracle's logits are exact.  Reading R26 of the design notes: where the exact top
two differ by more than twice the fp32 accumulation bound the tokens must be equal;
elsewhere the kernel's token must be within twice the bound of the exact maximum.
The returned maximum must be within the bound of the exact logit of the returned
token.  Exact ties (duplicated weight rows) must go to the smaller id.  The walk is
integer work: bit-exact.
"""
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


class _Rows:
    """bfloat16 weight rows decoded on slicing (the oracle reads a full-size weight in
    chunks without an fp32 copy of the whole)."""

    def __init__(self, bits):
        self.bits = bits
        self.shape = bits.shape

    def __getitem__(self, sl):
        return gen.bf16_bits_to_f32(self.bits[sl])


def _check(Hf, Wr, tok, mx, rows, what):
    """Hf [M, d] fp32 hidden rows, Wr weight rows, tok/mx [M] from the kernel; checks
    the given rows.  Returns the number of rows whose arg-max is decided."""
    x = oracle.lm_head_logits(Hf[rows], Wr)
    bound = oracle.fp32_accumulation_bound(Hf[rows], Wr)
    V = x.shape[1]
    decided = 0
    for k, m in enumerate(rows):
        t, top, second = oracle.top_two(x[k])
        g = int(tok[m])
        assert 0 <= g < V, f"{what}: row {m} token {g}"
        if top - second > 2 * bound[k]:
            assert g == t, f"{what}: row {m}: token {g}, oracle {t} (gap {top - second:.3g}, bound {bound[k]:.3g})"
            decided += 1
        else:
            assert x[k, g] >= top - 2 * bound[k], f"{what}: row {m}: token {g} logit {x[k, g]} < max {top}"
        assert abs(float(mx[m]) - x[k, g]) <= bound[k], f"{what}: row {m}: max {mx[m]} vs {x[k, g]}"
    return decided


def _run(H_bits, W_bits, num_nodes=None):
    S, N, d = H_bits.shape
    hid = dev_tensor(H_bits.reshape(S, N, d))
    w = dev_tensor(W_bits)
    nn = None if num_nodes is None else dev_tensor(np.asarray(num_nodes, dtype=np.int32))
    tok, mx = ddt.ddt_lm_head_argmax(hid, w, nn)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), mx.cpu().numpy()


def _planted(cfg, W, S, N, r, frac_unplanted=0.15):
    toks = r.integers(0, cfg.V, size=(S, N))
    toks[r.random((S, N)) < frac_unplanted] = -1
    H = np.stack([gen.hidden_states(cfg, s, W, toks[s]) for s in range(S)])
    return H, toks


# shapes: every tile height (32, 64, 128 rows), ragged vocabulary and row tiles,
# vocabularies below one tile, one row, several row tiles, K from one step to many
SMALL = [
    dict(S=1, B=16, V=3001, d=320),     # 17 rows
    dict(S=2, B=20, V=1000, d=128),     # 42 rows
    dict(S=3, B=22, V=3001, d=320),     # 69 rows: 256 x 128 tile, the second wave's rows ragged
    dict(S=4, B=63, V=5000, d=64),      # 256 rows: one full 256 x 256 tile
    dict(S=1, B=0, V=1, d=64),          # one row, one vocabulary entry
    dict(S=2, B=5, V=255, d=64),        # below one vocabulary tile
    dict(S=1, B=200, V=257, d=192),     # 201 rows (the last wave holds 9); one entry in the
                                        # second vocabulary tile
    dict(S=2, B=100, V=4096, d=1024),   # exact tiles, 16 K-steps
    # above 256 rows: several 256 x 256 row tiles (eight waves of 64 rows), the last ragged
    dict(S=1, B=256, V=3001, d=320),    # 257 rows: the second row tile holds one
    dict(S=3, B=100, V=1000, d=128),    # 303 rows: 47 in the last tile (two blocks of one wave)
    dict(S=2, B=300, V=4099, d=192),    # 602 rows: 90 in the last tile (two waves, three blocks)
    dict(S=4, B=127, V=513, d=256),     # 512 rows: two full row tiles; one entry in the third
                                        # vocabulary tile
]


@pytest.mark.parametrize("shape", SMALL, ids=[f"S{s['S']}B{s['B']}V{s['V']}d{s['d']}" for s in SMALL])
def test_small_shapes(shape):
    S, B, V, d = shape["S"], shape["B"], shape["V"], shape["d"]
    N = B + 1
    cfg = configs.custom("lmh", V=V, B=max(B, 1), S=S)
    r = np.random.default_rng(S * 1000 + N * 7 + V)
    W = gen.lm_head_weight(cfg, d)
    H, toks = _planted(cfg, W, S, N, r)
    tok, mx = _run(H, W)
    Hf = gen.bf16_bits_to_f32(H.reshape(S * N, d))
    dec = _check(Hf, gen.bf16_bits_to_f32(W), tok.reshape(-1), mx.reshape(-1), list(range(S * N)),
                 f"S{S} B{B} V{V} d{d}")
    planted = int((toks.reshape(-1) >= 0).sum())
    assert V == 1 or dec >= planted   # every planted row is decided


@pytest.mark.parametrize("N", [40, 300])
def test_exact_ties_go_to_the_smaller_id(N):
    # copies of a row's planted weight row placed at other ids: in the same wave's
    # block, the other lane half (ids 4 apart), another wave, another vocabulary tile,
    # and after the original; equal weight rows give equal fp32 sums.  40 rows take the
    # narrow tile (64 vocabulary entries per wave), 300 the 256 x 256 tile (128 per wave)
    V, d, S = 1024, 128, 1
    cfg = configs.custom("lmt", V=V, B=N - 1, S=S)
    W = gen.lm_head_weight(cfg, d).copy()
    toks = np.full(N, -1, dtype=np.int64)
    expect = {}
    # (planted id, copy id), all ids distinct.  The tile is 256 entries wide: 701 sits
    # in 700's 32-entry block; 706 and 710 are in the two lane halves of one block; 590
    # is in another wave than 650 at 64 entries per wave; 20, 255 and 900 are in other
    # vocabulary tiles; the copies 701, 900 and 1 come after the original.
    cases = [(700, 701), (710, 706), (650, 590), (300, 20), (500, 900), (1023, 255),
             (812, 808), (100, 99), (880, 879), (0, 1)]
    used = set()
    for m, (t, c) in enumerate(cases):
        assert t not in used and c not in used
        used.update((t, c))
    # with 300 rows the tied rows sit in the last, partly filled row tile (rows 260 on)
    first = 0 if N <= 256 else 260
    for k, (t, c) in enumerate(cases):
        W[c] = W[t]
        toks[first + k] = t
        expect[first + k] = (k, min(t, c))
    H = gen.hidden_states(cfg, 0, W, toks)[None]
    tok, mx = _run(H, W)
    for m, (k, want) in expect.items():
        assert int(tok[0, m]) == want, (m, cases[k], int(tok[0, m]))
        assert mx[0, m] == mx[0, m]  # finite
    # the rest of the rows still satisfy the oracle
    Hf = gen.bf16_bits_to_f32(H[0])
    _check(Hf, gen.bf16_bits_to_f32(W), tok[0], mx[0], list(range(N)), "ties")


def test_padding_rows():
    V, d, S, B = 2000, 192, 3, 30
    N = B + 1
    cfg = configs.custom("lmp", V=V, B=B, S=S)
    r = np.random.default_rng(4)
    W = gen.lm_head_weight(cfg, d)
    H, _ = _planted(cfg, W, S, N, r, frac_unplanted=0.0)
    nn = np.array([N, 5, 1], dtype=np.int32)
    for s in range(S):
        H[s, nn[s]:] = 0x7FC0   # NaN bit patterns in the padding rows: they are not used
    tok, mx = _run(H, W, nn)
    for s in range(S):
        assert np.all(tok[s, nn[s]:] == -1) and np.all(np.isneginf(mx[s, nn[s]:]))
        Hf = gen.bf16_bits_to_f32(H[s, :nn[s]])
        _check(Hf, gen.bf16_bits_to_f32(W), tok[s], mx[s], list(range(nn[s])), f"padding seq {s}")


@pytest.mark.parametrize("name,sample", [("C1", None), ("C2", 24), ("C3-B512", 16), ("C4", 8)])
def test_full_size(name, sample):
    """Workload shapes at full size (d = Hq * D): every row is planted, so its token must
    be the planted one (the construction's margin is about 7 against a bound below
    0.2); sampled rows (all rows for C1) against the exact oracle."""
    cfg = configs.get(name)
    d = gen.d_model(cfg)
    S, N = cfg.S, cfg.N
    W = gen.lm_head_weight(cfg, workers=16)
    r = np.random.default_rng(cfg.cfg_id)
    toks = r.integers(0, cfg.V, size=(S, N))
    H = np.stack([gen.hidden_states(cfg, s, W, toks[s]) for s in range(S)])
    tok, mx = _run(H, W)
    assert np.array_equal(tok, toks.astype(np.int32))
    M = S * N
    rows = list(range(M)) if sample is None else sorted(set(r.choice(M, size=sample, replace=False).tolist()) | {0, M - 1})
    Hf = gen.bf16_bits_to_f32(H.reshape(M, d)[rows])
    dec = _check(np.asarray(Hf), _Rows(W), tok.reshape(-1)[rows], mx.reshape(-1)[rows],
                 list(range(len(rows))), name)
    assert dec == len(rows)


def _walk_case(S, B, L, V, seed):
    """Oracle trees from random drafts, node tokens that follow a child with
    probability 0.8 (deep walks), random otherwise."""
    cfg = configs.custom("wt", S=S, L=L, V=V, K=min(8, V), B=B, cfg_id=300 + seed)
    r = np.random.default_rng(seed)
    N = B + 1
    tt = np.zeros((S, N), np.int32)
    pp = np.full((S, N), -1, np.int32)
    nn = np.zeros(S, np.int32)
    nt = np.zeros((S, N), np.int32)
    for s in range(S):
        d = gen.draft(cfg, s)
        tok, lq = oracle.topk(d["logits"], cfg.K)
        tree = oracle.build_tree(tok, lq, d["bonus"], B)
        n = int(tree["num_nodes"])
        tt[s], pp[s], nn[s] = tree["tree_tok"], tree["parent"], n
        for v in range(N):
            kids = [c for c in range(n) if tree["parent"][c] == v]
            nt[s, v] = int(tree["tree_tok"][r.choice(kids)]) if kids and r.random() < 0.8 else int(r.integers(0, V))
    return cfg, tt, pp, nn, nt


@pytest.mark.parametrize("S,B,L,V,seed", [(4, 8, 4, 64, 0), (8, 64, 16, 500, 1), (3, 300, 16, 50, 2),
                                          (2, 1023, 16, 40, 3), (5, 0, 1, 10, 4)])
def test_walk_tokens(S, B, L, V, seed):
    cfg, tt, pp, nn, nt = _walk_case(S, B, L, V, seed)
    w = ddt.ddt_tree_walk_tokens(dev_tensor(tt), dev_tensor(pp), dev_tensor(nn), dev_tensor(nt), L)
    torch.cuda.synchronize()
    for s in range(S):
        ref = oracle.tree_walk_tokens(tt[s], pp[s], int(nn[s]), nt[s], L)
        assert int(w["accept_len"][s]) == int(ref["accept_len"]), s
        assert w["acc_nodes"][s].cpu().numpy().tolist() == ref["acc_nodes"].tolist()
        assert w["acc_tok"][s].cpu().numpy().tolist() == ref["acc_tok"].tolist()
        assert int(w["bonus"][s]) == int(ref["bonus"])


@pytest.mark.parametrize("name", ["C1", "C2"])
def test_fused_epilogue_walk_equals_logits_walk(name):
    """A round's walk from the fused epilogue equals the walk over the target logits:
    each node's hidden state plants the token its synthetic target logits lift."""
    cfg = configs.get(name)
    b = gen.batch(cfg, attempts=attempts(cfg), with_qkv=False)
    trees = {}
    for s in range(cfg.S):
        tok, lq = oracle.topk(b["draft_logits"][s], cfg.K)
        trees[s] = oracle.build_tree(tok, lq, int(b["bonus"][s]), cfg.B)
    st = lambda k: np.stack([trees[s][k] for s in range(cfg.S)]).astype(np.int32)
    tr = {"tree_tok": st("tree_tok"), "parent": st("parent"),
          "num_nodes": np.array([trees[s]["num_nodes"] for s in range(cfg.S)], dtype=np.int32)}
    W = gen.lm_head_weight(cfg, workers=16)
    H = gen.tree_hidden_states(cfg, b, tr, W, workers=8)
    tok, _ = ddt.ddt_lm_head_argmax(dev_tensor(H), dev_tensor(W), dev_tensor(tr["num_nodes"]))
    w = ddt.ddt_tree_walk_tokens(dev_tensor(tr["tree_tok"]), dev_tensor(tr["parent"]),
                                 dev_tensor(tr["num_nodes"]), tok, cfg.L)
    torch.cuda.synchronize()
    tl = target_for(cfg, b, trees)
    for s in range(cfg.S):
        ref = oracle.tree_walk(trees[s]["tree_tok"], trees[s]["parent"], int(trees[s]["num_nodes"]),
                               tl[s], cfg.L)
        assert int(w["accept_len"][s]) == int(ref["accept_len"]), s
        assert w["acc_nodes"][s].cpu().numpy().tolist() == ref["acc_nodes"].tolist()
        assert int(w["bonus"][s]) == int(ref["bonus"])
