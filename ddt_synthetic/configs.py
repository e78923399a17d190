"""Workload shapes for one DDTree verification round.

Notation follows the DDTree page ("策展 · X (Twitter)", easyvibecoding.app/curated/665,
Liran Ringel's DDTree post): L draft positions produced by one block-diffusion
forward (section 運作流程, step 1), node budget B (section 核心創新), bonus token b
(section 運作流程, opening paragraph).  Shapes beyond those symbols (vocabulary,
top-K width, prefix length, head counts) are workload choices of this repository:
a tiny fp32 case, a 32k-vocabulary single sequence, a Llama-3-8B-shaped batch, a
node-budget sweep and a 70B-shaped long-context batch.

This module holds sizes only; it does no arithmetic of the method.
"""
from dataclasses import dataclass, replace
from typing import Tuple


@dataclass(frozen=True)
class Config:
    name: str
    cfg_id: int              # seed namespace; the node-budget sweep shares one id
    S: int                   # sequences in the batch
    L: int                   # draft positions per round
    V: int                   # vocabulary size
    K: int                   # candidates kept per position (top-K)
    B: int                   # node budget (non-root nodes)
    prefix: Tuple[int, int]  # inclusive range of prefix lengths P_s
    Hq: int
    Hkv: int
    D: int
    dtype: str               # "f32" or "bf16" for Q/K/V and the attention output
    near_tie: str            # "all": every candidate pair; "boundary": selection boundary
    chain_boost: float = 0.0  # extra logit on the planted chain token (confident drafts)

    @property
    def N(self) -> int:
        """Tree nodes including the root (the bonus token)."""
        return self.B + 1

    @property
    def W(self) -> int:
        """32-bit words per node in the ancestor bitmask."""
        return (self.N + 31) // 32


TIE_GAP = 1e-4  # minimum separation of prefix log-probabilities kept by the generator

C0 = Config("C0", 0, S=1, L=4, V=64, K=4, B=8, prefix=(32, 32), Hq=1, Hkv=1, D=32,
            dtype="f32", near_tie="all")
C1 = Config("C1", 1, S=1, L=16, V=32000, K=8, B=32, prefix=(1024, 1024), Hq=32, Hkv=8,
            D=128, dtype="bf16", near_tie="boundary")
C2 = Config("C2", 2, S=8, L=16, V=128256, K=8, B=64, prefix=(4096, 4096), Hq=32, Hkv=8,
            D=128, dtype="bf16", near_tie="boundary")
_C3 = Config("C3", 3, S=1, L=16, V=128256, K=32, B=64, prefix=(8192, 8192), Hq=32, Hkv=8,
             D=128, dtype="bf16", near_tie="boundary")
C3_BUDGETS = (16, 32, 64, 128, 256, 512)
C3 = {b: replace(_C3, name=f"C3-B{b}", B=b, K=min(b, 32)) for b in C3_BUDGETS}
C4 = Config("C4", 4, S=32, L=16, V=128256, K=8, B=64, prefix=(16384, 32768), Hq=64, Hkv=8,
            D=128, dtype="bf16", near_tie="boundary")

CONFIGS = {"C0": C0, "C1": C1, "C2": C2, "C4": C4}
CONFIGS.update({c.name: c for c in C3.values()})


def get(name: str) -> Config:
    try:
        return CONFIGS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(CONFIGS)}") from None


def custom(name: str, **kw) -> Config:
    """A test shape: C0's fields overridden by ``kw`` (cfg_id defaults to 100)."""
    base = dict(cfg_id=100, near_tie="boundary")
    base.update(kw)
    return replace(C0, name=name, **base)
