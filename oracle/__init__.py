"""CPU fp64 oracle of one DDTree verification round.

TEST INFRASTRUCTURE: imported only by the tests, the smoke check and the bench's
CPU-baseline leg, never by the library's product path.
"""
from .ddtree import (  # noqa: F401
    ancestors, attend, best_first_prefixes, build_tree, candidate_logprobs,
    expected_acceptance, greedy_token, position_ids, selection_gap, softmax_topk_row,
    topk, tree_attention, tree_mask, tree_walk, visible_nodes,
)
from .round import verify_round  # noqa: F401
