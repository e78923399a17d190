"""Tree attention through one reused workspace and replayed from a HIP graph (as the
benchmark runs it): every call and every replay must give the first eager call's
bits, and that call must match the oracle.  Two shapes are grids small enough to sit
on the GPU at once (the latency-bound plan: wide row groups, one-tile splits); two take
the narrow plan, whose last row group of each (sequence, KV head) holds 4 rows and runs
as two streams, dispatched among the full groups or after all of them."""
import math

import numpy as np
import pytest
import torch

import block_diffusion_draft_position_amd as ddt
import oracle
from ddt_synthetic import configs, gen

from _gpu import check_attention_rows, upload, widen

pytestmark = pytest.mark.gpu

# (1) two row groups of 8 waves per (sequence, KV head), twelve prefix splits and the
# tree split; (2) ragged prefixes (686, 253 and 190 keys): the sequences of one launch
# hold 11, 4 and 3 prefix splits, and the splits past a sequence's prefix exit at once
SHAPES = {
    "two-row-groups": dict(S=1, L=8, V=1000, K=4, B=63, prefix=(768, 768), Hq=16, Hkv=2),
    "ragged": dict(S=3, L=5, V=800, K=4, B=30, prefix=(0, 700), Hq=8, Hkv=2),
    # (3) 260 rows per KV head in groups of 128: two full groups and 4 rows
    "remainder-streams": dict(S=6, L=4, V=500, K=4, B=64, prefix=(900, 3000), Hq=16, Hkv=4),
    # (4) 1028 rows per KV head: eight full groups, the 4-row groups dispatched last
    "remainder-last": dict(S=2, L=4, V=500, K=4, B=256, prefix=(300, 700), Hq=32, Hkv=8),
}


def _setup(name):
    cfg = configs.custom(f"merge-{name}", D=128, dtype="bf16", **SHAPES[name])
    b = gen.batch(cfg)
    d = upload(b)
    tok, lq = ddt.ddt_topk(d["draft_logits"], cfg.K)
    tree = ddt.ddt_build_tree(tok, lq, d["bonus"], cfg.B)
    mask, _ = ddt.ddt_tree_mask(tree["parent"], tree["depth"], tree["num_nodes"], None)
    maxp = int(np.max(b["prefix_lens"]))
    need = ddt.attention_workspace_size(cfg.S, cfg.B, cfg.Hq, cfg.Hkv, cfg.D, 1, maxp)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(d["q"])
    lse = torch.empty(cfg.S, cfg.N, cfg.Hq, dtype=torch.float32, device="cuda")

    def call():
        ddt.ddt_tree_attention(d["q"], d["k_cache"], d["v_cache"], d["cu_prefix"], d["k_tree"],
                               d["v_tree"], mask, tree["num_nodes"], 1.0 / math.sqrt(cfg.D),
                               max_prefix=maxp, out=out, lse=lse, ws=ws)

    return cfg, b, d, tree, mask, out, lse, call


def _check_oracle(cfg, b, tree, mask, out, lse):
    go = widen(out)
    gl = lse.cpu().numpy().astype(np.float64)
    gm = mask.cpu().numpy().view(np.uint32)
    par = tree["parent"].cpu().numpy()
    nn = tree["num_nodes"].cpu().numpy()
    rows = [(n, h) for n in range(cfg.N) for h in range(cfg.Hq)][::7]
    idx_n = np.array([r[0] for r in rows])
    idx_h = np.array([r[1] for r in rows])
    for s in range(cfg.S):
        m_ref = oracle.tree_mask(par[s], int(nn[s]), cfg.N)
        assert np.array_equal(gm[s], m_ref), f"seq {s}: mask"
        p0, p1 = int(b["cu_prefix"][s]), int(b["cu_prefix"][s + 1])
        ref_o, ref_l = oracle.tree_attention(widen(b["q"][s]), widen(b["k_cache"][p0:p1]),
                                             widen(b["v_cache"][p0:p1]), widen(b["k_tree"][s]),
                                             widen(b["v_tree"][s]), m_ref, int(nn[s]),
                                             1.0 / math.sqrt(cfg.D), rows)
        check_attention_rows(go[s][idx_n, idx_h], ref_o, "bf16", f"{cfg.name} seq {s}")
        valid = idx_n < nn[s]
        np.testing.assert_allclose(gl[s][idx_n[valid], idx_h[valid]], ref_l[valid], rtol=0, atol=4e-3)


@pytest.mark.parametrize("name", sorted(SHAPES))
def test_workspace_reuse(name):
    cfg, b, d, tree, mask, out, lse, call = _setup(name)
    print(f"[case] {cfg.name} workspace reuse", flush=True)
    call()
    torch.cuda.synchronize()
    first = (out.view(torch.int16).clone(), lse.clone())
    _check_oracle(cfg, b, tree, mask, out, lse)
    for _ in range(4):
        out.zero_()
        lse.zero_()
        call()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), first[0])
        assert torch.equal(lse, first[1])


@pytest.mark.parametrize("name", sorted(SHAPES))
def test_graph_replay(name):
    cfg, b, d, tree, mask, out, lse, call = _setup(name)
    print(f"[case] {cfg.name} graph replay", flush=True)
    call()
    torch.cuda.synchronize()
    first = (out.view(torch.int16).clone(), lse.clone())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for i in range(5):
        out.zero_()
        lse.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), first[0]), i
        assert torch.equal(lse, first[1]), i
        call()  # eager work between the replays, on the same workspace
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), first[0]), i
