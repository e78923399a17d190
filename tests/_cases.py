"""Input selection for the tests: seeded draws with the near-tie rejection rule.

The GPU accumulates prefix log-probabilities from fp32 log-probabilities; the
oracle works in fp64.  Only the selection boundary can change a tree (the output
order is canonical), so the tests keep draws whose prefix log-probabilities are
separated by at least ``TIE_GAP``: every candidate pair for the tiny workload,
the selection boundary (B-th selected against best unselected) elsewhere.
``attempt`` re-draws the draft side until the rule holds.
"""
import functools
import json
import os
from typing import List

import numpy as np

import oracle
from ddt_synthetic import configs, gen
from ddt_synthetic.configs import TIE_GAP, Config

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
ATTEMPTS_FILE = os.path.join(GOLDEN, "attempts.json")


def draw_ok(cfg: Config, logq: np.ndarray, budgets=None) -> bool:
    if cfg.near_tie == "all":
        lp = np.sort(oracle.candidate_logprobs(logq))
        return bool(np.all(np.diff(lp) >= TIE_GAP))
    for B in (budgets or [cfg.B]):
        k = min(B, cfg.K) if budgets else cfg.K  # the sweep keeps K = min(B, 32)
        if oracle.selection_gap(logq[:, :k], B) < TIE_GAP:
            return False
    return True


def pick_attempt(cfg: Config, seq: int, max_attempts: int = 64) -> int:
    budgets = None
    if cfg.name.startswith("C3-"):
        budgets = list(configs.C3_BUDGETS)  # one draw must serve every budget
        cfg = configs.C3[max(budgets)]
    for a in range(max_attempts):
        dr = gen.draft(cfg, seq, a)
        _, lq = oracle.topk(dr["logits"], cfg.K)
        if draw_ok(cfg, lq, budgets):
            return a
    raise RuntimeError(f"{cfg.name} seq {seq}: no draw passes the near-tie rule")


@functools.lru_cache(maxsize=None)
def _table():
    if os.path.exists(ATTEMPTS_FILE):
        with open(ATTEMPTS_FILE) as f:
            return json.load(f)
    return {}


def attempts(cfg: Config) -> List[int]:
    """Accepted attempt per sequence: the committed table when it covers the
    workload (written by tests/golden/make_attempts.py from the oracle), else a
    fresh search."""
    key = "C3" if cfg.name.startswith("C3-") else cfg.name
    t = _table().get(key)
    if t is not None and len(t) >= cfg.S:
        return list(t[:cfg.S])
    return [pick_attempt(cfg, s) for s in range(cfg.S)]
