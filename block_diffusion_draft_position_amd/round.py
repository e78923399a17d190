"""One DDTree verification round on the GPU, with every buffer allocated up front.

The library calls run back to back on the current stream:
  ddt_draft_tree (= ddt_topk -> ddt_build_tree -> ddt_tree_mask, fused)
  -> ddt_tree_attention -> ddt_tree_walk
(DDTree page "策展 · X (Twitter)", section 運作流程 steps 1-4); fused=False makes
the three separate calls instead, with identical results.  The object holds
its outputs and workspaces, so a round allocates nothing and can be captured in a
HIP graph.  Target logits are an input here: in a real verifier they come out of
the target model's forward over the tree, which this library does not contain.
"""
import math
from dataclasses import dataclass
from typing import Dict, Optional

import torch

from . import _lib


@dataclass
class Shape:
    S: int
    L: int
    V: int
    K: int
    B: int
    Hq: int
    Hkv: int
    D: int
    dtype: torch.dtype
    max_prefix: int

    @property
    def N(self):
        return self.B + 1


class VerifyRound:
    def __init__(self, shape: Shape, device="cuda", fused: bool = True):
        self.shape = sh = shape
        self.fused = fused
        dev = torch.device(device)
        self.device = dev
        S, L, K, N = sh.S, sh.L, sh.K, sh.N
        i32 = dict(dtype=torch.int32, device=dev)
        self.topk_tok = torch.empty(S, L, K, **i32)
        self.topk_logq = torch.empty(S, L, K, dtype=torch.float32, device=dev)
        self.tree = {"tree_tok": torch.empty(S, N, **i32), "parent": torch.empty(S, N, **i32),
                     "depth": torch.empty(S, N, **i32),
                     "node_logq": torch.empty(S, N, dtype=torch.float32, device=dev),
                     "num_nodes": torch.empty(S, **i32)}
        self.mask = torch.empty(S, N, (N + 31) // 32, **i32)
        self.pos_ids = torch.empty(S, N, **i32)
        self.out = torch.empty(S, N, sh.Hq, sh.D, dtype=sh.dtype, device=dev)
        self.lse = torch.empty(S, N, sh.Hq, dtype=torch.float32, device=dev)
        self.walk = {"accept_len": torch.empty(S, **i32), "acc_nodes": torch.empty(S, L, **i32),
                     "acc_tok": torch.empty(S, L, **i32), "bonus": torch.empty(S, **i32)}
        lib = _lib.load()
        dt = _lib.DDT_BF16 if sh.dtype == torch.bfloat16 else _lib.DDT_F32
        self.ws_topk = _lib._ws(lib.ddt_topk_workspace_size(S * L, sh.V, K), dev)
        self.ws_attn = _lib._ws(lib.ddt_tree_attention_workspace_size(
            S, sh.B, sh.Hq, sh.Hkv, sh.D, dt, sh.max_prefix), dev)
        self.ws_walk = _lib._ws(lib.ddt_tree_walk_workspace_size(S, sh.B, sh.V), dev)
        self.scale = 1.0 / math.sqrt(sh.D)

    def draft_tree(self, draft_logits, bonus, cu_prefix):
        """Steps 1-3: top-K, tree, mask and position ids."""
        sh = self.shape
        if self.fused:
            out = dict(topk_tok=self.topk_tok, topk_logq=self.topk_logq, mask=self.mask,
                       pos_ids=self.pos_ids, **self.tree)
            _lib.ddt_draft_tree(draft_logits, bonus, cu_prefix, sh.K, sh.B, out, self.ws_topk)
            return
        _lib.ddt_topk(draft_logits, sh.K, self.topk_tok, self.topk_logq, self.ws_topk)
        _lib.ddt_build_tree(self.topk_tok, self.topk_logq, bonus, sh.B, self.tree)
        _lib.ddt_tree_mask(self.tree["parent"], self.tree["depth"], self.tree["num_nodes"],
                           cu_prefix, self.mask, self.pos_ids)

    def attention(self, q, k_cache, v_cache, cu_prefix, k_tree, v_tree):
        _lib.ddt_tree_attention(q, k_cache, v_cache, cu_prefix, k_tree, v_tree, self.mask,
                                self.tree["num_nodes"], self.scale, self.shape.max_prefix,
                                True, self.out, self.lse, self.ws_attn)

    def walk_tree(self, target_logits):
        _lib.ddt_tree_walk(self.tree["tree_tok"], self.tree["parent"], self.tree["num_nodes"],
                           target_logits, self.shape.L, self.walk, self.ws_walk)

    def __call__(self, draft_logits, bonus, q, k_cache, v_cache, cu_prefix, k_tree, v_tree,
                 target_logits) -> Dict[str, torch.Tensor]:
        self.draft_tree(draft_logits, bonus, cu_prefix)
        self.attention(q, k_cache, v_cache, cu_prefix, k_tree, v_tree)
        self.walk_tree(target_logits)
        return self.results()

    def results(self) -> Dict[str, torch.Tensor]:
        return dict(topk_tok=self.topk_tok, topk_logq=self.topk_logq, mask=self.mask,
                    pos_ids=self.pos_ids, out=self.out, lse=self.lse, **self.tree, **self.walk)
