"""CPU oracle for tree verification — TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct NumPy (fp64) definitions of what the hot path
computes: tree metadata, tree-masked attention over a paged prefix, the
multi-step speculative-sampling walk with siblings drawn without replacement,
longest-accepted-path selection, the commit of the accepted path's K/V, and
the draw of a node's children without replacement (Gumbel-top-k), and
the draft-tree constructions (EAGLE-2 expansion and rerank; TreeSpark's
best-first expansion with the calibrated theta stop). Each function cites the passage of the
source pages it follows:

  [survey]    "Tree-based speculative decoding: draft trees win latency, lose
              batches, return cost-aware" (speculative-decoding.pages.dev)
  [TreeSpark] TreeSpark: Markov-conditioned draft trees (paperpeel 2609.22098)
  [explainer] tree-vs-chain interview explainer (zenaique, io-tree-spec-decoding)

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package. The HIP library shares no code with it, and the product path
never calls it.
"""
from .tree import (check_tree, depths, ancestors_or_self, children,
                   ancestor_bitsets, first_child_next_sibling)
from .attention import tree_attention, tree_attention_rows, decode_values
from .sampler import (softmax_T, proposal_without, proposal_with, residual_update,
                      acceptance_ratio, inverse_cdf, greedy_request,
                      greedy_walk_request, walk_request, tree_spec_sample)
from .path import accept_path_request, tree_accept_path
from .commit import BadKeepList, check_keep, kv_commit_layer, kv_commit
from .siblings import philox4x32_10, draw_children, tree_draw_siblings
from .enumerate import enumerate_node_laws
from . import construct
from . import treespark

__all__ = [
    "check_tree", "depths", "ancestors_or_self", "children", "ancestor_bitsets",
    "first_child_next_sibling", "tree_attention", "tree_attention_rows",
    "decode_values", "softmax_T", "proposal_without", "proposal_with", "residual_update",
    "acceptance_ratio", "inverse_cdf", "greedy_request", "greedy_walk_request", "walk_request",
    "tree_spec_sample", "accept_path_request", "tree_accept_path",
    "BadKeepList", "check_keep", "kv_commit_layer", "kv_commit",
    "philox4x32_10", "draw_children", "tree_draw_siblings",
    "enumerate_node_laws", "construct", "treespark",
]
