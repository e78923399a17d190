"""Seeded synthetic inputs for one DDTree verification round.

Both the CPU oracle and the HIP path consume exactly these arrays.  The module
draws random numbers and plants structure; it computes nothing of the method
itself (no softmax, no top-K, no tree selection, no attention, no argmax).

What is synthesised, and why:
  * the drafter's per-position logits.  The DDTree page ("策展 · X (Twitter)",
    easyvibecoding.app/curated/665), section 運作流程 step 1, has one
    block-diffusion forward emit a marginal distribution for each of the next L
    positions; with no trained drafter available, logits are N(0, 2^2) noise with
    a planted chain token c_i lifted by 6 - 0.4*i at position i (i = 1..L).
  * the bonus token b (section 運作流程, opening paragraph): uniform.
  * the verifier's attention operands: post-RoPE Q, K, V drawn N(0, 1) in fp32,
    rounded to bfloat16 (round to nearest even) for the bf16 workloads.
  * the target model's next-token logits at every tree node (section 運作流程,
    step 4 walks them): N(0, 1) noise plus +10 on one token.  On the planted chain
    that token is the chain's next token, kept with probability 0.85 per depth;
    elsewhere it is uniform.  All target randomness is keyed by the node's token
    path, so the target is a deterministic function of the path, as a real model
    conditioned on the same context would be.

Seeds: numpy SeedSequence keyed by (workload id, sequence, [attempt], stream tag,
...).  ``attempt`` re-draws the draft side only; callers bump it to reject draws
whose prefix probabilities come within a stated gap of each other.
"""
from typing import Dict, List, Optional, Sequence

import numpy as np

from .configs import Config

# stream tags inside one (workload, sequence) key
_T_DRAFT, _T_KEEP, _T_PREFIX, _T_QKV, _T_TARGET = 0, 1, 2, 3, 4
KEEP_PROB = 0.85
TARGET_BOOST = 10.0


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


# ----------------------------------------------------------------------------- dtypes
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bfloat16 (nearest, ties to even); returns the uint16 encodings.
    Inputs are finite."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((b + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------- draft side
def draft(cfg: Config, seq: int, attempt: int = 0) -> Dict[str, np.ndarray]:
    """Draft logits [L, V] fp32, planted chain c_1..c_{L+1} and the bonus token."""
    r = _rng(cfg.cfg_id, seq, attempt, _T_DRAFT)
    chain = r.integers(0, cfg.V, size=cfg.L + 1, dtype=np.int64)
    bonus = int(r.integers(0, cfg.V))
    z = r.standard_normal((cfg.L, cfg.V), dtype=np.float32)
    logits = (np.float32(2.0) * z).astype(np.float32)
    for i in range(1, cfg.L + 1):  # position i holds c_i
        t = chain[i - 1]
        logits[i - 1, t] = np.float32(np.float64(logits[i - 1, t]) + (6.0 - 0.4 * i) + cfg.chain_boost)
    return {"logits": logits, "chain": chain, "bonus": bonus}


def keep_flags(cfg: Config, seq: int, attempt: int = 0) -> np.ndarray:
    """keep[d] (d = 0..L): does the on-chain target at depth d continue the chain?"""
    r = _rng(cfg.cfg_id, seq, attempt, _T_KEEP)
    return r.random(cfg.L + 1) < KEEP_PROB


def prefix_len(cfg: Config, seq: int) -> int:
    lo, hi = cfg.prefix
    if lo == hi:
        return lo
    return int(_rng(cfg.cfg_id, seq, _T_PREFIX).integers(lo, hi + 1))


# ----------------------------------------------------------------------------- attention operands
def qkv(cfg: Config, seq: int, P: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Q [N,Hq,D], prefix K/V [P,Hkv,D], tree K/V [N,Hkv,D].

    fp32 workloads return float32 arrays; bf16 workloads return uint16 bfloat16
    encodings.  Prefix K/V are drawn first so they do not depend on the budget B.
    """
    if P is None:
        P = prefix_len(cfg, seq)
    r = _rng(cfg.cfg_id, seq, _T_QKV)
    N = cfg.N
    shapes = [("k_prefix", (P, cfg.Hkv, cfg.D)), ("v_prefix", (P, cfg.Hkv, cfg.D)),
              ("q", (N, cfg.Hq, cfg.D)), ("k_tree", (N, cfg.Hkv, cfg.D)),
              ("v_tree", (N, cfg.Hkv, cfg.D))]
    out = {}
    for name, shp in shapes:
        x = r.standard_normal(shp, dtype=np.float32)
        out[name] = f32_to_bf16_bits(x) if cfg.dtype == "bf16" else x
    return out


# ----------------------------------------------------------------------------- target side
def node_paths(tree_tok: np.ndarray, parent: np.ndarray, num_nodes: int) -> List[tuple]:
    """Token path (t_1..t_d) of every node, root excluded (the root is the bonus)."""
    paths: List[tuple] = []
    for n in range(num_nodes):
        p = int(parent[n])
        if p < 0:
            paths.append(())
        else:
            if p >= n:
                raise ValueError("parents must precede their children")
            paths.append(paths[p] + (int(tree_tok[n]),))
    return paths


def target_row(cfg: Config, seq: int, attempt: int, path: Sequence[int],
               chain: np.ndarray, keep: np.ndarray) -> np.ndarray:
    """The synthetic target's next-token logits [V] fp32 after context b, *path."""
    d = len(path)
    r = _rng(cfg.cfg_id, seq, attempt, _T_TARGET, d, *[int(t) for t in path])
    row = r.standard_normal(cfg.V, dtype=np.float32)
    on_chain = d <= cfg.L and all(int(path[j]) == int(chain[j]) for j in range(d))
    if on_chain and bool(keep[d]):
        tok = int(chain[d])
    else:
        tok = int(r.integers(0, cfg.V))
    row[tok] = np.float32(np.float64(row[tok]) + TARGET_BOOST)
    return row


def target_logits(cfg: Config, seq: int, attempt: int, tree_tok: np.ndarray, parent: np.ndarray,
                  num_nodes: int, chain: np.ndarray, keep: np.ndarray,
                  out: Optional[np.ndarray] = None) -> np.ndarray:
    """Target logits [N, V] fp32 for the nodes of one tree; rows >= num_nodes are 0."""
    if out is None:
        out = np.zeros((cfg.N, cfg.V), dtype=np.float32)
    else:
        out[num_nodes:] = 0
    for n, path in enumerate(node_paths(tree_tok, parent, num_nodes)):
        out[n] = target_row(cfg, seq, attempt, path, chain, keep)
    return out


# ----------------------------------------------------------------------------- batches
def batch(cfg: Config, attempts: Optional[Sequence[int]] = None,
          with_qkv: bool = True) -> Dict[str, np.ndarray]:
    """All S sequences of one workload, stacked in the layouts the library takes.

    draft_logits [S,L,V] f32; bonus [S] i32; chain [S,L+1]; keep [S,L+1];
    prefix_lens [S]; cu_prefix [S+1] i64; q [S,N,Hq,D]; k_cache/v_cache
    [sum P, Hkv, D] (sequences packed back to back); k_tree/v_tree [S,N,Hkv,D].
    """
    S = cfg.S
    if attempts is None:
        attempts = [0] * S
    logits = np.empty((S, cfg.L, cfg.V), dtype=np.float32)
    bonus = np.empty(S, dtype=np.int32)
    chain = np.empty((S, cfg.L + 1), dtype=np.int64)
    keep = np.empty((S, cfg.L + 1), dtype=bool)
    for s in range(S):
        dr = draft(cfg, s, attempts[s])
        logits[s] = dr["logits"]
        bonus[s] = dr["bonus"]
        chain[s] = dr["chain"]
        keep[s] = keep_flags(cfg, s, attempts[s])
    P = np.array([prefix_len(cfg, s) for s in range(S)], dtype=np.int64)
    cu = np.zeros(S + 1, dtype=np.int64)
    cu[1:] = np.cumsum(P)
    out = {"draft_logits": logits, "bonus": bonus, "chain": chain, "keep": keep,
           "prefix_lens": P, "cu_prefix": cu, "attempts": np.asarray(attempts, dtype=np.int64)}
    if with_qkv:
        et = np.uint16 if cfg.dtype == "bf16" else np.float32
        T = int(cu[-1])
        q = np.empty((S, cfg.N, cfg.Hq, cfg.D), dtype=et)
        kc = np.empty((T, cfg.Hkv, cfg.D), dtype=et)
        vc = np.empty_like(kc)
        kt = np.empty((S, cfg.N, cfg.Hkv, cfg.D), dtype=et)
        vt = np.empty_like(kt)
        for s in range(S):
            x = qkv(cfg, s, int(P[s]))
            q[s] = x["q"]
            kc[cu[s]:cu[s + 1]] = x["k_prefix"]
            vc[cu[s]:cu[s + 1]] = x["v_prefix"]
            kt[s] = x["k_tree"]
            vt[s] = x["v_tree"]
        out.update(q=q, k_cache=kc, v_cache=vc, k_tree=kt, v_tree=vt)
    return out
