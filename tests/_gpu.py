"""Helpers for the GPU tests: upload generator batches, run the library, compare
against the oracle with the stated tolerances."""
import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

import oracle
from ddt_synthetic import gen
from ddt_synthetic.configs import Config

# Tolerances (derivations in the design notes):
#   topk logq: fp32 x - lse with lse accumulated in fp64 -> ~1e-6; bound 2e-5, five
#     times below the 1e-4 near-tie gap the generator keeps.
#   node logq: fp32 rounding of an fp64 sum of <= 64 fp32 logq values -> 1e-4.
#   attention fp32: per row max|d| <= 1e-5 * max|ref|.
#   attention bf16: |d| <= 2e-2 + 1e-2 |ref| elementwise, and per row
#     ||d||_2 <= 1e-2 ||ref||_2 (an all-zero output would pass the first alone).
#   lse: 1e-5 (fp32 inputs); 4e-3 for bf16 inputs, whose row sums are formed from the
#     bf16-rounded softmax weights (relative error <= 2^-8 in the sum).
TOPK_ATOL = 2e-5
NODE_LOGQ_ATOL = 1e-4
F32_ROW_RTOL = 1e-5
BF16_ATOL, BF16_RTOL, BF16_ROW_L2 = 2e-2, 1e-2, 1e-2


def dev_tensor(x: np.ndarray, device="cuda") -> torch.Tensor:
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def upload(b: Dict[str, np.ndarray], device="cuda") -> Dict[str, torch.Tensor]:
    out = {}
    for k in ("draft_logits", "q", "k_cache", "v_cache", "k_tree", "v_tree", "cu_prefix"):
        if k in b:
            out[k] = dev_tensor(b[k], device)
    out["bonus"] = dev_tensor(b["bonus"].astype(np.int32), device)
    return out


def widen(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu()
        if x.dtype == torch.bfloat16:
            return x.float().double().numpy()
        return x.double().numpy()
    return oracle.round.widen(x)


def check_attention_rows(got: np.ndarray, ref: np.ndarray, dtype: str, what: str):
    """got/ref [rows, D] (fp64 views)."""
    assert got.shape == ref.shape, (got.shape, ref.shape)
    d = np.abs(got - ref)
    if dtype == "f32":
        scale = np.maximum(np.max(np.abs(ref), axis=-1), 1e-30)
        bad = np.max(d, axis=-1) > F32_ROW_RTOL * scale
        assert not np.any(bad), f"{what}: fp32 rows off: {np.flatnonzero(bad)[:8]} max rel {np.max(np.max(d, -1) / scale):.3g}"
    else:
        el = d > BF16_ATOL + BF16_RTOL * np.abs(ref)
        assert not np.any(el), f"{what}: {el.sum()} bf16 elements off, worst {d.max():.3g}"
        rn = np.linalg.norm(d, axis=-1) / np.maximum(np.linalg.norm(ref, axis=-1), 1e-30)
        assert np.all(rn <= BF16_ROW_L2), f"{what}: row L2 rel {rn.max():.3g}"


def target_for(cfg: Config, b: Dict[str, np.ndarray], trees: Dict[int, Dict]) -> np.ndarray:
    """[S,N,V] target logits evaluated at the oracle's trees (path-keyed)."""
    S = cfg.S
    out = np.zeros((S, cfg.N, cfg.V), dtype=np.float32)
    for s in range(S):
        t = trees[s]
        gen.target_logits(cfg, s, int(b["attempts"][s]), t["tree_tok"], t["parent"],
                          int(t["num_nodes"]), b["chain"][s], b["keep"][s], out=out[s])
    return out
