"""Pins of the oracle's tree attention against torch's scaled_dot_product_attention
(CPU, fp64), a library routine independent of the oracle.

* every node's output equals plain attention of that node's query over the prefix
  followed by its root-to-node path (DDTree page, 核心創新 and 運作流程 step 3:
  ancestor-only masking scores every branch in one forward as if it were alone);
* a chain tree equals causal attention over prefix + chain;
* grouped-query heads read KV head h // (Hq / Hkv) (torch's enable_gqa convention);
* the log-sum-exp equals torch.logsumexp of the scaled scores.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from ddt_synthetic import configs, gen


def _case(L, K, B, P, Hq, Hkv, D, seed):
    cfg = configs.custom("t", L=L, V=50, K=K, B=B, prefix=(P, P), Hq=Hq, Hkv=Hkv, D=D)
    d = gen.draft(cfg, seed, 0)
    tok, lq = oracle.topk(d["logits"], K)
    tree = oracle.build_tree(tok, lq, d["bonus"], B)
    x = gen.qkv(cfg, seed)
    nn = int(tree["num_nodes"])
    mask = oracle.tree_mask(tree["parent"], nn, cfg.N)
    return cfg, tree, x, nn, mask


def _path(parent, n):
    out = [n]
    while parent[out[-1]] >= 0:
        out.append(int(parent[out[-1]]))
    return out[::-1]


@pytest.mark.parametrize("L,K,B,P,Hq,Hkv,D,seed", [
    (4, 4, 8, 32, 1, 1, 32, 0), (5, 3, 30, 7, 8, 2, 16, 1), (3, 6, 40, 0, 4, 4, 8, 2),
    (6, 2, 20, 1, 6, 3, 64, 3), (2, 8, 50, 65, 4, 1, 32, 4)])
def test_each_node_equals_attention_over_its_path(L, K, B, P, Hq, Hkv, D, seed):
    cfg, tree, x, nn, mask = _case(L, K, B, P, Hq, Hkv, D, seed)
    scale = 1 / math.sqrt(D)
    o, lse = oracle.tree_attention(x["q"], x["k_prefix"], x["v_prefix"], x["k_tree"], x["v_tree"],
                                   mask, nn, scale)
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    for n in range(nn):
        path = _path(tree["parent"], n)
        k = torch.cat([t(x["k_prefix"]), t(x["k_tree"][path])], 0).permute(1, 0, 2)[None]   # [1,Hkv,T,D]
        v = torch.cat([t(x["v_prefix"]), t(x["v_tree"][path])], 0).permute(1, 0, 2)[None]
        q = t(x["q"][n])[None, :, None, :]                                                  # [1,Hq,1,D]
        ref = F.scaled_dot_product_attention(q, k, v, scale=scale, enable_gqa=True)[0, :, 0]
        np.testing.assert_allclose(o[n], ref.numpy(), rtol=1e-12, atol=1e-12)
        kr = k.repeat_interleave(Hq // Hkv, dim=1)[0]                                       # [Hq,T,D]
        ref_lse = torch.logsumexp(scale * torch.einsum("hd,htd->ht", q[0, :, 0], kr), dim=-1)
        np.testing.assert_allclose(lse[n], ref_lse.numpy(), rtol=1e-12, atol=1e-12)
    assert not np.any(o[nn:]) and np.all(np.isneginf(lse[nn:]))


def test_chain_equals_causal_attention():
    cfg, tree, x, nn, mask = _case(L=8, K=1, B=8, P=13, Hq=4, Hkv=2, D=32, seed=5)
    assert nn == 9
    scale = 0.3
    o, _ = oracle.tree_attention(x["q"], x["k_prefix"], x["v_prefix"], x["k_tree"], x["v_tree"],
                                 mask, nn, scale)
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    k = torch.cat([t(x["k_prefix"]), t(x["k_tree"])], 0).permute(1, 0, 2)[None]
    v = torch.cat([t(x["v_prefix"]), t(x["v_tree"])], 0).permute(1, 0, 2)[None]
    q = t(x["q"]).permute(1, 0, 2)[None]                                                    # [1,Hq,N,D]
    allowed = torch.ones(nn, 13 + nn, dtype=torch.bool)
    allowed[:, 13:] = torch.tril(torch.ones(nn, nn, dtype=torch.bool))
    ref = F.scaled_dot_product_attention(q, k, v, attn_mask=allowed, scale=scale, enable_gqa=True)
    np.testing.assert_allclose(o, ref[0].permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_root_only_is_decode_attention():
    cfg, tree, x, nn, mask = _case(L=3, K=3, B=0, P=40, Hq=8, Hkv=2, D=16, seed=6)
    assert nn == 1
    o, _ = oracle.tree_attention(x["q"], x["k_prefix"], x["v_prefix"], x["k_tree"], x["v_tree"],
                                 mask, nn, 0.25)
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    k = torch.cat([t(x["k_prefix"]), t(x["k_tree"][:1])], 0).permute(1, 0, 2)[None]
    v = torch.cat([t(x["v_prefix"]), t(x["v_tree"][:1])], 0).permute(1, 0, 2)[None]
    ref = F.scaled_dot_product_attention(t(x["q"][0])[None, :, None], k, v, scale=0.25, enable_gqa=True)
    np.testing.assert_allclose(o[0], ref[0, :, 0].numpy(), rtol=1e-12, atol=1e-12)
