"""Longest accepted path, emitted tokens and the KV keep-list.

[TreeSpark §3.2 step 3]: commit the longest surviving root path, then one
correction or bonus token. [TreeSpark §5.1]: tau = accepted draft length + 1
tokens per target forward. [explainer, Red flags]: exactly one path is
accepted. [survey, Systems]: the accepted slots feed a compaction gather
(EAGLE's retrieve_indices), so the path's logical KV positions are exported.
"""
import numpy as np

from .tree import children, check_tree


class TwoAcceptedSiblings(ValueError):
    pass


def accept_path_request(parent, tokens, flags, next_token, prefix_len):
    """Follow flags from the root through the unique flagged child.

    Returns (path_nodes, out_tokens, kv_keep): path_nodes starts at the root;
    out_tokens = tokens of the path's non-root nodes, then next_token at the
    stop node; kv_keep = prefix_len + node for every path node.
    """
    check_tree(parent)
    ch = children(parent)
    v = 0
    path = [0]
    while True:
        fl = [c for c in ch[v] if int(flags[c]) == 1]
        if len(fl) > 1:
            raise TwoAcceptedSiblings(f"node {v} has accepted children {fl}")
        if not fl:
            break
        v = fl[0]
        path.append(v)
    out = [int(tokens[c]) for c in path[1:]] + [int(next_token[v])]
    keep = [int(prefix_len) + c for c in path]
    return path, out, keep


def tree_accept_path(node_indptr, parent, tokens, flags, next_token, prefix_len, max_depth):
    """Batched form with the boundary's [B][max_depth+1] layouts (-1 padded)."""
    B = len(node_indptr) - 1
    W = max_depth + 1
    path_nodes = np.full((B, W), -1, dtype=np.int32)
    out_tokens = np.full((B, W), -1, dtype=np.int32)
    kv_keep = np.full((B, W), -1, dtype=np.int32)
    out_len = np.zeros(B, dtype=np.int32)
    for r in range(B):
        a, b = int(node_indptr[r]), int(node_indptr[r + 1])
        path, out, keep = accept_path_request(parent[a:b], tokens[a:b], flags[a:b],
                                              next_token[a:b], prefix_len[r])
        n = len(path)
        path_nodes[r, :n] = path
        out_tokens[r, :n] = out
        kv_keep[r, :n] = keep
        out_len[r] = n
    return path_nodes, out_tokens, out_len, kv_keep
