"""ddt_tree_walk_noalloc (the walk on the library's static scratch, no allocation in
the call) through the C ABI, against ddt_tree_walk on a caller workspace and against
the oracle: two calls in a row, the second with a smaller problem, then the first
shape again (the scratch keeps the last call's contents, which must be zero)."""
import ctypes

import numpy as np
import pytest
import torch

import block_diffusion_draft_position_amd as ddt
import oracle
from ddt_synthetic import configs, gen

from _gpu import dev_tensor, target_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ddt.load()


SHAPES = [dict(S=4, L=6, V=128256, K=8, B=64), dict(S=2, L=4, V=3000, K=4, B=12),
          dict(S=4, L=6, V=128256, K=8, B=64)]


def test_noalloc_walk_matches_workspace_walk():
    lib = ddt.load()
    assert lib.ddt_tree_walk_noalloc_max_bytes() == 1 << 20
    for i, sh in enumerate(SHAPES):
        print(f"[case] noalloc walk call {i}: {sh}", flush=True)
        cfg = configs.custom(f"noalloc-{i}", cfg_id=400 + i, prefix=(1, 1), Hq=1, Hkv=1, D=32,
                             dtype="f32", **sh)
        assert lib.ddt_tree_walk_workspace_size(cfg.S, cfg.B, cfg.V) <= lib.ddt_tree_walk_noalloc_max_bytes()
        b = gen.batch(cfg, with_qkv=False)
        trees = {}
        for s in range(cfg.S):
            tok, lq = oracle.topk(b["draft_logits"][s], cfg.K)
            trees[s] = oracle.build_tree(tok, lq, int(b["bonus"][s]), cfg.B)
        tl = target_for(cfg, b, trees)
        tt = dev_tensor(np.stack([trees[s]["tree_tok"] for s in range(cfg.S)]))
        par = dev_tensor(np.stack([trees[s]["parent"] for s in range(cfg.S)]))
        nn = dev_tensor(np.array([trees[s]["num_nodes"] for s in range(cfg.S)], dtype=np.int32))
        tgt = dev_tensor(tl)
        ref = ddt.ddt_tree_walk(tt, par, nn, tgt, cfg.L)
        # the entry point itself, called through ctypes with raw pointers
        got = {k: torch.full_like(v, -7) for k, v in ref.items()}
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        p = lambda t: ctypes.c_void_p(t.data_ptr())
        rc = lib.ddt_tree_walk_noalloc(p(tt), p(par), p(nn), p(tgt), cfg.S, cfg.B, cfg.L, cfg.V,
                                       p(got["accept_len"]), p(got["acc_nodes"]), p(got["acc_tok"]),
                                       p(got["bonus"]), st)
        assert rc == 0, lib.ddt_status_string(rc)
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(got[k], ref[k]), f"call {i}: {k}"
        for s in range(cfg.S):
            w = oracle.tree_walk(trees[s]["tree_tok"], trees[s]["parent"], int(trees[s]["num_nodes"]),
                                 tl[s], cfg.L)
            for k in ("accept_len", "acc_nodes", "acc_tok", "bonus"):
                assert np.array_equal(got[k][s].cpu().numpy(), w[k]), f"call {i} seq {s}: {k}"
