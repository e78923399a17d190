"""ctypes binding of libddt.so (include/ddt.h).

Argument marshalling only: every step runs in the library's HIP kernels.  PyTorch
supplies device memory and the current stream.  If the library is missing the
import of this module succeeds but every call raises, naming the build command.
"""
import ctypes
import math
import os
from typing import Dict, Optional, Tuple

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libddt.so")

DDT_F32, DDT_BF16 = 0, 1
MAX_K, MAX_L, MAX_B = 64, 64, 1023

_lib = None


class DDTError(RuntimeError):
    pass


def _p(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def load() -> ctypes.CDLL:
    """Load libddt.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise DDTError(f"{LIB_PATH} is missing: build it with "
                       "`python -m block_diffusion_draft_position_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    sig = {
        "ddt_status_string": (ctypes.c_char_p, [i32]),
        "ddt_topk_workspace_size": (sz, [i64, i64, i32]),
        "ddt_topk": (i32, [vp, i64, i64, i64, i32, vp, vp, vp, sz, vp]),
        "ddt_build_tree": (i32, [vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp]),
        "ddt_tree_mask": (i32, [vp, vp, vp, vp, vp, i32, i32, vp, vp, vp]),
        "ddt_draft_tree_workspace_size": (sz, [i32, i32, i64, i32]),
        "ddt_draft_tree": (i32, [vp, i64, vp, vp, vp, i32, i32, i64, i32, i32, vp, vp, vp, vp, vp,
                                 vp, vp, vp, vp, vp, sz, vp]),
        "ddt_tree_attention_workspace_size": (sz, [i32, i32, i32, i32, i32, i32, i64]),
        "ddt_tree_attention": (i32, [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                     i32, f32, i64, vp, vp, vp, sz, vp]),
        "ddt_adapt_budget": (i32, [vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp]),
        "ddt_commit_kv": (i32, [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp]),
        "ddt_tree_walk_workspace_size": (sz, [i32, i32, i64]),
        "ddt_tree_walk": (i32, [vp, vp, vp, vp, i32, i32, i32, i64, vp, vp, vp, vp, vp, sz, vp]),
        "ddt_tree_walk_sample": (i32, [vp, vp, vp, vp, vp, vp, f32, i32, i32, i32, i64, vp, vp, vp, vp,
                                       vp, sz, vp]),
        "ddt_tree_walk_noalloc_max_bytes": (sz, []),
        "ddt_tree_walk_noalloc": (i32, [vp, vp, vp, vp, i32, i32, i32, i64, vp, vp, vp, vp, vp]),
        "ddt_lm_head_argmax_workspace_size": (sz, [i32, i32, i64, i32]),
        "ddt_lm_head_argmax": (i32, [vp, vp, vp, i32, i32, i32, i64, vp, vp, vp, sz, vp]),
        "ddt_tree_walk_tokens": (i32, [vp, vp, vp, vp, i32, i32, i32, vp, vp, vp, vp, vp]),
        "ddt_tree_walk_strategy": (i32, [i32]),
        "ddt_tree_walk_mode": (i32, [i32, i32, i32, i64]),
        "ddt_lm_head_profiling": (i32, [i32]),
        "ddt_lm_head_timing": (i32, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int)]),
        "ddt_attention_profiling": (i32, [i32]),
        "ddt_attention_timing": (i32, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(ctypes.c_int)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


EXPORTS = ("ddt_status_string", "ddt_topk_workspace_size", "ddt_topk", "ddt_build_tree",
           "ddt_tree_mask", "ddt_draft_tree_workspace_size", "ddt_draft_tree",
           "ddt_adapt_budget", "ddt_tree_attention_workspace_size", "ddt_tree_attention",
           "ddt_commit_kv",
           "ddt_tree_walk_workspace_size", "ddt_tree_walk", "ddt_tree_walk_sample",
           "ddt_tree_walk_noalloc_max_bytes", "ddt_tree_walk_strategy", "ddt_tree_walk_mode",
           "ddt_tree_walk_noalloc", "ddt_lm_head_argmax_workspace_size", "ddt_lm_head_argmax",
           "ddt_tree_walk_tokens", "ddt_lm_head_profiling", "ddt_lm_head_timing",
           "ddt_attention_profiling", "ddt_attention_timing")


def _check(status: int, what: str):
    if status != 0:
        msg = load().ddt_status_string(status).decode()
        raise DDTError(f"{what}: {msg} (status {status})")


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _ws(nbytes: int, device) -> torch.Tensor:
    # zero-filled: the completion counters at the front of a workspace start at zero
    return torch.zeros(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# ----------------------------------------------------------------------------- entry points
def ddt_topk(logits: torch.Tensor, k: int, out_tok=None, out_logq=None, ws=None):
    """logits [..., V] fp32 -> (tok [..., k] int32, logq [..., k] fp32)."""
    lib = load()
    _dev(logits, "logits", torch.float32)
    V = logits.shape[-1]
    rows = logits.numel() // V
    lead = tuple(logits.shape[:-1])
    if out_tok is None:
        out_tok = torch.empty(lead + (k,), dtype=torch.int32, device=logits.device)
    if out_logq is None:
        out_logq = torch.empty(lead + (k,), dtype=torch.float32, device=logits.device)
    need = lib.ddt_topk_workspace_size(rows, V, k)
    if ws is None:
        ws = _ws(need, logits.device)
    _check(lib.ddt_topk(_p(logits), rows, V, V, k, _p(out_tok), _p(out_logq), _p(ws), ws.numel(),
                        _stream(logits.device)), "ddt_topk")
    return out_tok, out_logq


def ddt_build_tree(topk_tok: torch.Tensor, topk_logq: torch.Tensor, bonus: torch.Tensor, B: int,
                   out: Optional[Dict[str, torch.Tensor]] = None, with_logq: bool = True):
    """[S,L,K] top-K tokens/logq + bonus [S] -> canonical tree dict ([S,B+1] arrays)."""
    lib = load()
    S, L, K = topk_tok.shape
    _dev(topk_tok, "topk_tok", torch.int32)
    _dev(topk_logq, "topk_logq", torch.float32, (S, L, K))
    _dev(bonus, "bonus", torch.int32, (S,))
    dev = topk_tok.device
    N = B + 1
    if out is None:
        out = {"tree_tok": torch.empty(S, N, dtype=torch.int32, device=dev),
               "parent": torch.empty(S, N, dtype=torch.int32, device=dev),
               "depth": torch.empty(S, N, dtype=torch.int32, device=dev),
               "node_logq": torch.empty(S, N, dtype=torch.float32, device=dev) if with_logq else None,
               "num_nodes": torch.empty(S, dtype=torch.int32, device=dev)}
    _check(lib.ddt_build_tree(_p(topk_tok), _p(topk_logq), _p(bonus), S, L, K, B,
                              _p(out["tree_tok"]), _p(out["parent"]), _p(out["depth"]),
                              _p(out.get("node_logq")), _p(out["num_nodes"]), _stream(dev)),
           "ddt_build_tree")
    return out


def _prefix_len(prefix_len, S):
    if prefix_len is not None:
        _dev(prefix_len, "prefix_len", torch.int64, (S,))
    return prefix_len


def ddt_tree_mask(parent: torch.Tensor, depth: torch.Tensor, num_nodes: torch.Tensor,
                  cu_prefix: Optional[torch.Tensor], mask=None, pos_ids=None, prefix_len=None):
    """-> (mask [S,N,W] int32 view of uint32 bits, pos_ids [S,N] or None)."""
    lib = load()
    S, N = parent.shape
    _dev(parent, "parent", torch.int32)
    _dev(depth, "depth", torch.int32, (S, N))
    _dev(num_nodes, "num_nodes", torch.int32, (S,))
    if cu_prefix is not None:
        _dev(cu_prefix, "cu_prefix", torch.int64, (S + 1,))
    W = (N + 31) // 32
    dev = parent.device
    if mask is None:
        mask = torch.empty(S, N, W, dtype=torch.int32, device=dev)
    if pos_ids is None and cu_prefix is not None:
        pos_ids = torch.empty(S, N, dtype=torch.int32, device=dev)
    _prefix_len(prefix_len, S)
    _check(lib.ddt_tree_mask(_p(parent), _p(depth), _p(num_nodes), _p(cu_prefix), _p(prefix_len),
                             S, N - 1, _p(mask), _p(pos_ids), _stream(dev)), "ddt_tree_mask")
    return mask, pos_ids


def ddt_draft_tree(logits: torch.Tensor, bonus: torch.Tensor, cu_prefix: Optional[torch.Tensor],
                   K: int, B: int, out: Optional[Dict[str, torch.Tensor]] = None, ws=None,
                   prefix_len=None):
    """logits [S,L,V] fp32, bonus [S], cu_prefix [S+1] or None -> dict with topk_tok,
    topk_logq, tree_tok, parent, depth, node_logq, num_nodes, mask (int32 view of
    uint32 bits) and pos_ids (None without cu_prefix): steps 1-3 in two launches."""
    lib = load()
    _dev(logits, "logits", torch.float32)
    S, L, V = logits.shape
    _dev(bonus, "bonus", torch.int32, (S,))
    if cu_prefix is not None:
        _dev(cu_prefix, "cu_prefix", torch.int64, (S + 1,))
    dev = logits.device
    N = B + 1
    W = (N + 31) // 32
    if out is None:
        i32 = dict(dtype=torch.int32, device=dev)
        out = {"topk_tok": torch.empty(S, L, K, **i32),
               "topk_logq": torch.empty(S, L, K, dtype=torch.float32, device=dev),
               "tree_tok": torch.empty(S, N, **i32), "parent": torch.empty(S, N, **i32),
               "depth": torch.empty(S, N, **i32),
               "node_logq": torch.empty(S, N, dtype=torch.float32, device=dev),
               "num_nodes": torch.empty(S, **i32), "mask": torch.empty(S, N, W, **i32),
               "pos_ids": torch.empty(S, N, **i32) if cu_prefix is not None else None}
    need = lib.ddt_draft_tree_workspace_size(S, L, V, K)
    if ws is None:
        ws = _ws(need, dev)
    _prefix_len(prefix_len, S)
    _check(lib.ddt_draft_tree(_p(logits), V, _p(bonus), _p(cu_prefix), _p(prefix_len), S, L, V, K, B,
                              _p(out.get("topk_tok")), _p(out.get("topk_logq")),
                              _p(out["tree_tok"]), _p(out["parent"]), _p(out["depth"]),
                              _p(out.get("node_logq")), _p(out["num_nodes"]), _p(out["mask"]),
                              _p(out.get("pos_ids")), _p(ws), ws.numel(), _stream(dev)),
           "ddt_draft_tree")
    return out


def ddt_adapt_budget(tree: Dict[str, torch.Tensor], cost: torch.Tensor):
    """Cut each sequence's tree (a ddt_build_tree dict, modified in place) to the budget
    that maximises (E[accept] + 1) / cost[b]; cost [B+1] fp32 on the device.
    Returns (budget [S] int32, expected acceptance [S] fp32)."""
    lib = load()
    S, N = tree["tree_tok"].shape
    for k in ("tree_tok", "parent", "depth"):
        _dev(tree[k], k, torch.int32, (S, N))
    _dev(tree["node_logq"], "node_logq", torch.float32, (S, N))
    _dev(tree["num_nodes"], "num_nodes", torch.int32, (S,))
    _dev(cost, "cost", torch.float32, (N,))
    dev = cost.device
    budget = torch.empty(S, dtype=torch.int32, device=dev)
    expected = torch.empty(S, dtype=torch.float32, device=dev)
    _check(lib.ddt_adapt_budget(_p(cost), S, N - 1, _p(tree["tree_tok"]), _p(tree["parent"]),
                                _p(tree["depth"]), _p(tree["node_logq"]), _p(tree["num_nodes"]),
                                _p(budget), _p(expected), _stream(dev)), "ddt_adapt_budget")
    return budget, expected


def attention_workspace_size(S, B, Hq, Hkv, D, dtype, max_prefix) -> int:
    return int(load().ddt_tree_attention_workspace_size(S, B, Hq, Hkv, D, dtype, max_prefix))


def ddt_tree_attention(q, k_cache, v_cache, cu_prefix, k_tree, v_tree, mask, num_nodes,
                       scale: Optional[float] = None, max_prefix: Optional[int] = None,
                       with_lse: bool = True, out=None, lse=None, ws=None, prefix_len=None):
    """q [S,N,Hq,D]; k/v_cache [T,Hkv,D]; k/v_tree [S,N,Hkv,D] (fp32 or bf16) ->
    (out [S,N,Hq,D], lse [S,N,Hq] fp32 or None)."""
    lib = load()
    S, N, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    dt = {torch.float32: DDT_F32, torch.bfloat16: DDT_BF16}.get(q.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {q.dtype}")
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("k_tree", k_tree),
                    ("v_tree", v_tree)):
        _dev(t, name, q.dtype)
    if k_cache.shape != v_cache.shape or k_cache.shape[2] != D:
        raise ValueError("k_cache/v_cache must be [T, Hkv, D]")
    _dev(k_tree, "k_tree", q.dtype, (S, N, Hkv, D))
    _dev(v_tree, "v_tree", q.dtype, (S, N, Hkv, D))
    _dev(cu_prefix, "cu_prefix", torch.int64, (S + 1,))
    _dev(mask, "mask", None, (S, N, (N + 31) // 32))
    _dev(num_nodes, "num_nodes", torch.int32, (S,))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    _prefix_len(prefix_len, S)
    if max_prefix is None:
        cu = cu_prefix.cpu()
        lens = prefix_len.cpu() if prefix_len is not None else cu[1:] - cu[:-1]
        max_prefix = int(lens.max())
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    if with_lse and lse is None:
        lse = torch.empty(S, N, Hq, dtype=torch.float32, device=dev)
    need = lib.ddt_tree_attention_workspace_size(S, N - 1, Hq, Hkv, D, dt, max_prefix)
    if ws is None:
        ws = _ws(need, dev)
    _check(lib.ddt_tree_attention(_p(q), _p(k_cache), _p(v_cache), _p(cu_prefix), _p(prefix_len), _p(k_tree),
                                  _p(v_tree), _p(mask), _p(num_nodes), S, N - 1, Hq, Hkv, D, dt,
                                  float(scale), int(max_prefix), _p(out), _p(lse if with_lse else None),
                                  _p(ws), ws.numel(), _stream(dev)), "ddt_tree_attention")
    return out, (lse if with_lse else None)


def ddt_commit_kv(k_cache, v_cache, cu_prefix, prefix_len, k_tree, v_tree, acc_nodes, accept_len,
                  appended=None):
    """Append each sequence's root and accepted nodes' tree K/V to its cache region
    and advance prefix_len, in place; returns appended [S] int32 (-1: no room)."""
    lib = load()
    S, N, Hkv, D = k_tree.shape
    dt = {torch.float32: DDT_F32, torch.bfloat16: DDT_BF16}.get(k_tree.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {k_tree.dtype}")
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache), ("v_tree", v_tree)):
        _dev(t, name, k_tree.dtype)
    if k_cache.shape != v_cache.shape or tuple(k_cache.shape[1:]) != (Hkv, D):
        raise ValueError("k_cache/v_cache must be [rows, Hkv, D]")
    _dev(v_tree, "v_tree", k_tree.dtype, (S, N, Hkv, D))
    _dev(cu_prefix, "cu_prefix", torch.int64, (S + 1,))
    _dev(prefix_len, "prefix_len", torch.int64, (S,))
    _dev(accept_len, "accept_len", torch.int32, (S,))
    _dev(acc_nodes, "acc_nodes", torch.int32)
    L = acc_nodes.shape[1]
    if appended is None:
        appended = torch.empty(S, dtype=torch.int32, device=k_tree.device)
    _check(lib.ddt_commit_kv(_p(k_cache), _p(v_cache), _p(cu_prefix), _p(prefix_len), _p(k_tree),
                             _p(v_tree), _p(acc_nodes), _p(accept_len), S, N - 1, L, Hkv, D, dt,
                             _p(appended), _stream(k_tree.device)), "ddt_commit_kv")
    return appended


def ddt_tree_walk(tree_tok, parent, num_nodes, target_logits, L: int, out=None, ws=None):
    """target_logits [S,N,V] fp32 -> dict(accept_len [S], acc_nodes [S,L], acc_tok [S,L], bonus [S])."""
    lib = load()
    S, N = tree_tok.shape
    _dev(tree_tok, "tree_tok", torch.int32)
    _dev(parent, "parent", torch.int32, (S, N))
    _dev(num_nodes, "num_nodes", torch.int32, (S,))
    _dev(target_logits, "target_logits", torch.float32)
    if target_logits.shape[:2] != (S, N):
        raise ValueError("target_logits must be [S, N, V]")
    V = target_logits.shape[2]
    dev = tree_tok.device
    if out is None:
        out = {"accept_len": torch.empty(S, dtype=torch.int32, device=dev),
               "acc_nodes": torch.empty(S, L, dtype=torch.int32, device=dev),
               "acc_tok": torch.empty(S, L, dtype=torch.int32, device=dev),
               "bonus": torch.empty(S, dtype=torch.int32, device=dev)}
    need = lib.ddt_tree_walk_workspace_size(S, N - 1, V)
    if ws is None:
        ws = _ws(need, dev)
    _check(lib.ddt_tree_walk(_p(tree_tok), _p(parent), _p(num_nodes), _p(target_logits), S, N - 1,
                             L, V, _p(out["accept_len"]), _p(out["acc_nodes"]), _p(out["acc_tok"]),
                             _p(out["bonus"]), _p(ws), ws.numel(), _stream(dev)), "ddt_tree_walk")
    return out


def ddt_tree_walk_sample(tree_tok, parent, depth, num_nodes, target_logits, gumbel,
                         inv_temperature: float, L: int, out=None, ws=None):
    """Walk at temperature 1 / inv_temperature by the Gumbel-max rule; gumbel [S, L+1, V]
    fp32 noise, row d for depth d -> dict(accept_len, acc_nodes, acc_tok, bonus)."""
    lib = load()
    S, N = tree_tok.shape
    _dev(tree_tok, "tree_tok", torch.int32)
    _dev(parent, "parent", torch.int32, (S, N))
    _dev(depth, "depth", torch.int32, (S, N))
    _dev(num_nodes, "num_nodes", torch.int32, (S,))
    _dev(target_logits, "target_logits", torch.float32)
    if target_logits.shape[:2] != (S, N):
        raise ValueError("target_logits must be [S, N, V]")
    V = target_logits.shape[2]
    _dev(gumbel, "gumbel", torch.float32, (S, L + 1, V))
    dev = tree_tok.device
    if out is None:
        out = {"accept_len": torch.empty(S, dtype=torch.int32, device=dev),
               "acc_nodes": torch.empty(S, L, dtype=torch.int32, device=dev),
               "acc_tok": torch.empty(S, L, dtype=torch.int32, device=dev),
               "bonus": torch.empty(S, dtype=torch.int32, device=dev)}
    need = lib.ddt_tree_walk_workspace_size(S, N - 1, V)
    if ws is None:
        ws = _ws(need, dev)
    _check(lib.ddt_tree_walk_sample(_p(tree_tok), _p(parent), _p(depth), _p(num_nodes),
                                    _p(target_logits), _p(gumbel), float(inv_temperature), S, N - 1,
                                    L, V, _p(out["accept_len"]), _p(out["acc_nodes"]),
                                    _p(out["acc_tok"]), _p(out["bonus"]), _p(ws), ws.numel(),
                                    _stream(dev)), "ddt_tree_walk_sample")
    return out


def ddt_tree_walk_noalloc(tree_tok, parent, num_nodes, target_logits, L: int, out=None):
    """ddt_tree_walk on the library's static workspace (no allocation in the call)."""
    lib = load()
    S, N = tree_tok.shape
    _dev(tree_tok, "tree_tok", torch.int32)
    _dev(parent, "parent", torch.int32, (S, N))
    _dev(num_nodes, "num_nodes", torch.int32, (S,))
    _dev(target_logits, "target_logits", torch.float32)
    if target_logits.shape[:2] != (S, N):
        raise ValueError("target_logits must be [S, N, V]")
    V = target_logits.shape[2]
    dev = tree_tok.device
    if out is None:
        out = {"accept_len": torch.empty(S, dtype=torch.int32, device=dev),
               "acc_nodes": torch.empty(S, L, dtype=torch.int32, device=dev),
               "acc_tok": torch.empty(S, L, dtype=torch.int32, device=dev),
               "bonus": torch.empty(S, dtype=torch.int32, device=dev)}
    _check(lib.ddt_tree_walk_noalloc(_p(tree_tok), _p(parent), _p(num_nodes), _p(target_logits), S,
                                     N - 1, L, V, _p(out["accept_len"]), _p(out["acc_nodes"]),
                                     _p(out["acc_tok"]), _p(out["bonus"]), _stream(dev)),
           "ddt_tree_walk_noalloc")
    return out


def ddt_lm_head_argmax(hidden, weight, num_nodes=None, out_tok=None, out_max=None, ws=None,
                       with_max: bool = True):
    """hidden [S, N, d] bf16, weight [V, d] bf16 -> (node_tok [S, N] int32, node_max [S, N]
    fp32 or None): the LM-head arg-max per node, equal logits to the smaller id."""
    lib = load()
    _dev(hidden, "hidden", torch.bfloat16)
    _dev(weight, "weight", torch.bfloat16)
    if hidden.dim() != 3 or weight.dim() != 2 or hidden.shape[2] != weight.shape[1]:
        raise ValueError("hidden must be [S, N, d] and weight [V, d]")
    S, N, d = hidden.shape
    V = weight.shape[0]
    dev = hidden.device
    if num_nodes is not None:
        _dev(num_nodes, "num_nodes", torch.int32, (S,))
    if out_tok is None:
        out_tok = torch.empty(S, N, dtype=torch.int32, device=dev)
    _dev(out_tok, "out_tok", torch.int32, (S, N))
    if out_max is None and with_max:
        out_max = torch.empty(S, N, dtype=torch.float32, device=dev)
    if out_max is not None:
        _dev(out_max, "out_max", torch.float32, (S, N))
    need = lib.ddt_lm_head_argmax_workspace_size(S, N - 1, V, d)
    if ws is None:
        ws = torch.empty(max(int(need), 1), dtype=torch.uint8, device=dev)
    _check(lib.ddt_lm_head_argmax(_p(hidden), _p(weight), _p(num_nodes), S, N - 1, d, V,
                                  _p(out_tok), _p(out_max), _p(ws), ws.numel(), _stream(dev)),
           "ddt_lm_head_argmax")
    return out_tok, out_max


def ddt_tree_walk_tokens(tree_tok, parent, num_nodes, node_tok, L: int, out=None):
    """node_tok [S, N] int32 (each node's target token) -> dict(accept_len [S],
    acc_nodes [S, L], acc_tok [S, L], bonus [S])."""
    lib = load()
    S, N = tree_tok.shape
    _dev(tree_tok, "tree_tok", torch.int32)
    _dev(parent, "parent", torch.int32, (S, N))
    _dev(num_nodes, "num_nodes", torch.int32, (S,))
    _dev(node_tok, "node_tok", torch.int32, (S, N))
    dev = tree_tok.device
    if out is None:
        out = {"accept_len": torch.empty(S, dtype=torch.int32, device=dev),
               "acc_nodes": torch.empty(S, L, dtype=torch.int32, device=dev),
               "acc_tok": torch.empty(S, L, dtype=torch.int32, device=dev),
               "bonus": torch.empty(S, dtype=torch.int32, device=dev)}
    _check(lib.ddt_tree_walk_tokens(_p(tree_tok), _p(parent), _p(num_nodes), _p(node_tok), S, N - 1,
                                    L, _p(out["accept_len"]), _p(out["acc_nodes"]), _p(out["acc_tok"]),
                                    _p(out["bonus"]), _stream(dev)), "ddt_tree_walk_tokens")
    return out


WALK_AUTO, WALK_SCAN, WALK_PATH, WALK_HYBRID = 0, 1, 2, 3


def walk_strategy(mode: int) -> int:
    """Set the tree walk's strategy for the process (WALK_AUTO, WALK_SCAN, WALK_PATH,
    WALK_HYBRID); returns the previous one."""
    prev = load().ddt_tree_walk_strategy(int(mode))
    if prev < 0:
        _check(prev, "ddt_tree_walk_strategy")
    return prev


def walk_mode(S: int, B: int, L: int, vocab: int) -> int:
    """The strategy a walk of this shape would use now (WALK_SCAN, WALK_PATH or
    WALK_HYBRID)."""
    m = load().ddt_tree_walk_mode(S, B, L, vocab)
    if m < 0:
        _check(m, "ddt_tree_walk_mode")
    return m


def lm_head_profiling(enable: bool):
    _check(load().ddt_lm_head_profiling(1 if enable else 0), "ddt_lm_head_profiling")


def lm_head_timing() -> Tuple[float, int]:
    """(summed milliseconds of the epilogue's tile kernel, calls) since the last read."""
    tm, n = ctypes.c_double(0.0), ctypes.c_int(0)
    _check(load().ddt_lm_head_timing(ctypes.byref(tm), ctypes.byref(n)), "ddt_lm_head_timing")
    return tm.value, n.value


def attention_profiling(enable: bool):
    _check(load().ddt_attention_profiling(1 if enable else 0), "ddt_attention_profiling")


def attention_timing() -> Tuple[float, float, int]:
    """(summed milliseconds of the main kernel, summed milliseconds of the whole
    attention step, calls) since the last read."""
    tm, ts, n = ctypes.c_double(0.0), ctypes.c_double(0.0), ctypes.c_int(0)
    _check(load().ddt_attention_timing(ctypes.byref(tm), ctypes.byref(ts), ctypes.byref(n)),
           "ddt_attention_timing")
    return tm.value, ts.value, n.value
