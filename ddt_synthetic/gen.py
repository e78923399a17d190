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
  * the target's last layer for the fused verifier epilogue: an LM-head weight
    N(0, 1/d) and per-node final hidden states that plant the node's target token
    (section "verifier epilogue" below).

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


def _target_draw(cfg: Config, seq: int, attempt: int, path: Sequence[int],
                 chain: np.ndarray, keep: np.ndarray):
    d = len(path)
    r = _rng(cfg.cfg_id, seq, attempt, _T_TARGET, d, *[int(t) for t in path])
    row = r.standard_normal(cfg.V, dtype=np.float32)
    on_chain = d <= cfg.L and all(int(path[j]) == int(chain[j]) for j in range(d))
    if on_chain and bool(keep[d]):
        tok = int(chain[d])
    else:
        tok = int(r.integers(0, cfg.V))
    return row, tok


def target_row(cfg: Config, seq: int, attempt: int, path: Sequence[int],
               chain: np.ndarray, keep: np.ndarray) -> np.ndarray:
    """The synthetic target's next-token logits [V] fp32 after context b, *path."""
    row, tok = _target_draw(cfg, seq, attempt, path, chain, keep)
    row[tok] = np.float32(np.float64(row[tok]) + TARGET_BOOST)
    return row


def target_token(cfg: Config, seq: int, attempt: int, path: Sequence[int],
                 chain: np.ndarray, keep: np.ndarray) -> int:
    """The token target_row lifts by TARGET_BOOST after context b, *path (the same
    draws): the synthetic target's planted choice there."""
    return _target_draw(cfg, seq, attempt, path, chain, keep)[1]


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
          with_qkv: bool = True, workers: int = 1) -> Dict[str, np.ndarray]:
    """All S sequences of one workload, stacked in the layouts the library takes.

    draft_logits [S,L,V] f32; bonus [S] i32; chain [S,L+1]; keep [S,L+1];
    prefix_lens [S]; cu_prefix [S+1] i64; q [S,N,Hq,D]; k_cache/v_cache
    [sum P, Hkv, D] (sequences packed back to back); k_tree/v_tree [S,N,Hkv,D].
    ``workers`` > 1 draws the sequences' attention operands on that many threads
    (each sequence has its own seed, so the arrays are the same either way).
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
        def fill(s):
            x = qkv(cfg, s, int(P[s]))
            q[s] = x["q"]
            kc[cu[s]:cu[s + 1]] = x["k_prefix"]
            vc[cu[s]:cu[s + 1]] = x["v_prefix"]
            kt[s] = x["k_tree"]
            vt[s] = x["v_tree"]

        if workers > 1 and S > 1:
            from concurrent.futures import ThreadPoolExecutor
            with ThreadPoolExecutor(max_workers=min(workers, S)) as ex:
                list(ex.map(fill, range(S)))
        else:
            for s in range(S):
                fill(s)
        out.update(q=q, k_cache=kc, v_cache=vc, k_tree=kt, v_tree=vt)
    return out


# ----------------------------------------------------------------------------- several rounds
# A synthetic model keyed by the whole generated sequence, for loops of verification
# rounds (the DDTree page, section 運作流程: each round starts from the bonus token the
# previous one emitted, and the target's output carries over from round to round).
# ``g`` is the list of generated tokens of a sequence: the first bonus token b_0 and
# every token emitted after it; the initial context (the prefix) is fixed per
# sequence.  Everything below is drawn from seeds keyed by (workload, sequence, tag,
# *g), so each quantity is a function of its context, as a real model's would be:
#   planted_next(g)   the target's planted next token after g (uniform draw)
#   seq_target_row(g) target logits after g: N(0, 1) noise plus 10 on planted_next(g)
#   seq_draft(g)      a round's draft logits [L, V] from context g (g ends with the
#                     round's bonus token): N(0, 2^2) noise; position i's planted token
#                     is the target's i-th planted continuation c_i (c_1 =
#                     planted_next(g), c_{i+1} = planted_next(g + c_1..c_i)) with
#                     probability 0.85, else a uniform token, lifted by 6 - 0.4 i plus
#                     cfg.chain_boost.  ``attempt`` re-draws the noise and the errors.
#   seq_node_qkv(g)   Q [Hq, D], K and V [Hkv, D] of the last token of g in context
_T_SEQ_FIRST, _T_SEQ_NEXT, _T_SEQ_TARGET, _T_SEQ_DRAFT, _T_SEQ_ERR, _T_SEQ_QKV = 20, 21, 22, 23, 24, 25
DRAFT_HIT_PROB = 0.85


def seq_first_bonus(cfg: Config, seq: int) -> int:
    """b_0: the bonus token the first round starts from."""
    return int(_rng(cfg.cfg_id, seq, _T_SEQ_FIRST).integers(0, cfg.V))


def planted_next(cfg: Config, seq: int, g: Sequence[int]) -> int:
    return int(_rng(cfg.cfg_id, seq, _T_SEQ_NEXT, *[int(t) for t in g]).integers(0, cfg.V))


def seq_target_row(cfg: Config, seq: int, g: Sequence[int]) -> np.ndarray:
    """The synthetic target's next-token logits [V] fp32 after generated tokens g."""
    r = _rng(cfg.cfg_id, seq, _T_SEQ_TARGET, *[int(t) for t in g])
    row = r.standard_normal(cfg.V, dtype=np.float32)
    t = planted_next(cfg, seq, g)
    row[t] = np.float32(np.float64(row[t]) + TARGET_BOOST)
    return row


def seq_draft(cfg: Config, seq: int, g: Sequence[int], attempt: int = 0) -> np.ndarray:
    """Draft logits [L, V] fp32 of a round whose context is g (ending in its bonus)."""
    key = [int(t) for t in g]
    r = _rng(cfg.cfg_id, seq, _T_SEQ_DRAFT, attempt, *key)
    logits = (np.float32(2.0) * r.standard_normal((cfg.L, cfg.V), dtype=np.float32)).astype(np.float32)
    e = _rng(cfg.cfg_id, seq, _T_SEQ_ERR, attempt, *key)
    hit = e.random(cfg.L) < DRAFT_HIT_PROB
    wrong = e.integers(0, cfg.V, size=cfg.L)
    ctx = list(key)
    for i in range(1, cfg.L + 1):
        c = planted_next(cfg, seq, ctx)
        t = c if hit[i - 1] else int(wrong[i - 1])
        logits[i - 1, t] = np.float32(np.float64(logits[i - 1, t]) + (6.0 - 0.4 * i) + cfg.chain_boost)
        ctx.append(c)
    return logits


def seq_node_qkv(cfg: Config, seq: int, g: Sequence[int]) -> Dict[str, np.ndarray]:
    """Q [Hq, D] and K, V [Hkv, D] of the last token of g (bf16 encodings for the bf16
    workloads, fp32 otherwise)."""
    r = _rng(cfg.cfg_id, seq, _T_SEQ_QKV, *[int(t) for t in g])
    out = {}
    for name, shp in (("q", (cfg.Hq, cfg.D)), ("k", (cfg.Hkv, cfg.D)), ("v", (cfg.Hkv, cfg.D))):
        x = r.standard_normal(shp, dtype=np.float32)
        out[name] = f32_to_bf16_bits(x) if cfg.dtype == "bf16" else x
    return out


def seq_tree_inputs(cfg: Config, seq: int, g: Sequence[int], tree_tok: np.ndarray,
                    parent: np.ndarray, num_nodes: int) -> Dict[str, np.ndarray]:
    """A round's verifier inputs at a tree whose root is the last token of g: Q
    [N,Hq,D], tree K/V [N,Hkv,D] and target logits [N,V] of every node, each from the
    node's context g + (its path); rows past num_nodes are zero."""
    et = np.uint16 if cfg.dtype == "bf16" else np.float32
    q = np.zeros((cfg.N, cfg.Hq, cfg.D), dtype=et)
    kt = np.zeros((cfg.N, cfg.Hkv, cfg.D), dtype=et)
    vt = np.zeros_like(kt)
    tl = np.zeros((cfg.N, cfg.V), dtype=np.float32)
    base = [int(t) for t in g]
    for n, path in enumerate(node_paths(tree_tok, parent, num_nodes)):
        ctx = base + list(path)
        x = seq_node_qkv(cfg, seq, ctx)
        q[n], kt[n], vt[n] = x["q"], x["k"], x["v"]
        tl[n] = seq_target_row(cfg, seq, ctx)
    return {"q": q, "k_tree": kt, "v_tree": vt, "target": tl}


# ----------------------------------------------------------------------------- sampling noise
_T_GUMBEL = 30


def gumbel_noise(cfg: Config, seq: int, rnd: int = 0) -> np.ndarray:
    """Standard Gumbel draws [L + 1, V] fp32 for one sequence's round ``rnd``: row d is
    the noise of the target's sampling step at depth d (shared by every node of that
    depth).  These are the random numbers the sampling rule consumes; both the oracle
    and the library take them as an input."""
    r = _rng(cfg.cfg_id, seq, _T_GUMBEL, rnd)
    return r.gumbel(size=(cfg.L + 1, cfg.V)).astype(np.float32)


# ----------------------------------------------------------------------------- verifier epilogue
# The target's last layer at every tree node: a final hidden state h [d] and the LM
# head (output embedding) W [V, d], both bfloat16, with d = Hq * D (the model width of
# the workload's attention shape).  W is drawn N(0, 1/d), so an unplanted logit h . w_v
# is about N(0, 1) for h ~ N(0, I).  A node's hidden state is z + beta * w_t with
# z ~ N(0, I_d) and t a planted token: its logit for t is then about beta (|w_t|^2 is
# about 1) against N(0, 1 + beta^2 / d) elsewhere, so with beta = 12 the planted
# token leads the rest of a 128K vocabulary (whose maximum is about 4.9) by about 7.
# A token < 0 plants nothing (h = z).  Rounded to bfloat16 (nearest even).
_T_LMHEAD, _T_HIDDEN = 40, 41
HIDDEN_BETA = 12.0
LMHEAD_CHUNK = 4096  # vocabulary rows per seed chunk, so that threads can share the draw


def d_model(cfg: Config) -> int:
    return cfg.Hq * cfg.D


def lm_head_weight(cfg: Config, d: Optional[int] = None, workers: int = 1) -> np.ndarray:
    """LM-head weight [V, d] as bfloat16 encodings (uint16), N(0, 1/d), drawn in chunks
    of LMHEAD_CHUNK vocabulary rows each with its own seed (the same array for any
    ``workers``)."""
    d = d_model(cfg) if d is None else int(d)
    out = np.empty((cfg.V, d), dtype=np.uint16)
    sd = np.float32(1.0 / np.sqrt(d))

    def fill(c):
        lo, hi = c * LMHEAD_CHUNK, min(cfg.V, (c + 1) * LMHEAD_CHUNK)
        r = _rng(cfg.cfg_id, _T_LMHEAD, d, c)
        out[lo:hi] = f32_to_bf16_bits(r.standard_normal((hi - lo, d), dtype=np.float32) * sd)

    chunks = range((cfg.V + LMHEAD_CHUNK - 1) // LMHEAD_CHUNK)
    if workers > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(fill, chunks))
    else:
        for c in chunks:
            fill(c)
    return out


def hidden_states(cfg: Config, seq: int, weight_bits: np.ndarray, tokens: Sequence[int],
                  beta: float = HIDDEN_BETA, rnd: int = 0) -> np.ndarray:
    """Final hidden states [len(tokens), d] (bfloat16 encodings) of one sequence's
    nodes: row n is z_n + beta * w_{tokens[n]} (z_n ~ N(0, I_d) keyed by the
    sequence, round and node), or z_n where tokens[n] < 0."""
    d = weight_bits.shape[1]
    n = len(tokens)
    r = _rng(cfg.cfg_id, seq, _T_HIDDEN, rnd, d)
    h = r.standard_normal((n, d), dtype=np.float32)
    for i, t in enumerate(tokens):
        if int(t) >= 0:
            h[i] += np.float32(beta) * bf16_bits_to_f32(weight_bits[int(t)])
    return f32_to_bf16_bits(h)


def tree_hidden_states(cfg: Config, b: Dict[str, np.ndarray], tree: Dict[str, np.ndarray],
                       weight_bits: np.ndarray, beta: float = HIDDEN_BETA,
                       workers: int = 1) -> np.ndarray:
    """Hidden states [S, N, d] for the trees of a batch: node n of sequence s plants
    the synthetic target's token after n's path (target_token), so the argmax of the
    LM head at every node is the token the target logits of ``target_logits`` lift.
    ``tree`` holds tree_tok / parent / num_nodes [S, N] / [S]; padding rows plant
    nothing."""
    S, N, d = cfg.S, cfg.N, weight_bits.shape[1]
    out = np.empty((S, N, d), dtype=np.uint16)
    att = b.get("attempts", np.zeros(S, dtype=np.int64))

    def fill(s):
        nn = int(tree["num_nodes"][s])
        toks = [-1] * N
        for n, path in enumerate(node_paths(tree["tree_tok"][s], tree["parent"][s], nn)):
            toks[n] = target_token(cfg, s, int(att[s]), path, b["chain"][s], b["keep"][s])
        out[s] = hidden_states(cfg, s, weight_bits, toks, beta)

    if workers > 1 and S > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=min(workers, S)) as ex:
            list(ex.map(fill, range(S)))
    else:
        for s in range(S):
            fill(s)
    return out
