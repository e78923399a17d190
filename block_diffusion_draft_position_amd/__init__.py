"""MI355X-native DDTree verification round.

The work happens in libddt.so (include/ddt.h): hand-written HIP kernels for gfx950.
This package is its thin Python binding (PyTorch supplies device memory and streams)
and its build script.
"""
from ._lib import (  # noqa: F401
    DDT_BF16, DDT_F32, DDTError, EXPORTS, LIB_PATH, attention_profiling, attention_timing,
    attention_workspace_size, ddt_adapt_budget, ddt_build_tree, ddt_commit_kv, ddt_draft_tree,
    ddt_lm_head_argmax, ddt_topk, ddt_tree_attention, ddt_tree_mask, ddt_tree_walk,
    ddt_tree_walk_noalloc, ddt_tree_walk_sample, ddt_tree_walk_tokens, lm_head_profiling,
    lm_head_timing, load, WALK_AUTO, WALK_HYBRID, WALK_PATH, WALK_SCAN, walk_mode, walk_strategy,
)
from .round import Shape, VerifyRound  # noqa: F401
