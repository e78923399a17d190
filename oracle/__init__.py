"""CPU fp64 oracle of one DDTree verification round.

TEST INFRASTRUCTURE: imported only by the tests, the smoke check and the bench's
CPU-baseline leg, never by the library's product path.
"""
from .ddtree import (  # noqa: F401
    ancestors, attend, best_first_prefixes, build_tree, candidate_logprobs, choose_budget,
    expected_acceptance, greedy_token, position_ids, prune_tree, sample_token, score_order,
    selection_gap, softmax_topk_row,
    topk, tree_attention, tree_mask, tree_walk, tree_walk_sample, visible_nodes,
)
from .epilogue import (  # noqa: F401
    fp32_accumulation_bound, lm_head_argmax, lm_head_logits, top_two, tree_walk_tokens,
)
from .round import verify_round  # noqa: F401
from .rounds import commit_kv, greedy_decode, run_rounds  # noqa: F401
