"""Tree metadata: the flattened draft tree as a parent array.

[survey, Timeline]: SpecInfer stores the tree's tokens in the KV cache in
topological order and masks each token's attention to its ancestors.
[TreeSpark §3.2 step 3, §4]: per-depth position ids and a per-step
ancestor-bitmask mask. Siblings are ordered by draw order ([TreeSpark §1]),
which is ascending row index here.
"""
import numpy as np


def check_tree(parent):
    """Raise ValueError unless parent[0] == -1 and 0 <= parent[i] < i."""
    parent = np.asarray(parent)
    if len(parent) == 0:
        return
    if parent[0] != -1:
        raise ValueError("root must have parent -1")
    for i in range(1, len(parent)):
        if not (0 <= parent[i] < i):
            raise ValueError(f"parent[{i}] = {parent[i]} is not in [0, {i})")


def ancestors_or_self(parent):
    """anc(i) = {i} U anc(parent[i]); anc(0) = {0}."""
    check_tree(parent)
    anc = []
    for i in range(len(parent)):
        s = {i}
        if i > 0:
            s |= anc[parent[i]]
        anc.append(s)
    return anc


def depths(parent):
    """depth[i] = depth[parent[i]] + 1, depth[root] = 0."""
    check_tree(parent)
    d = [0] * len(parent)
    for i in range(1, len(parent)):
        d[i] = d[parent[i]] + 1
    return np.asarray(d, dtype=np.int32)


def children(parent):
    """children(v) = [i : parent[i] == v] in ascending i (= draw order)."""
    out = [[] for _ in range(len(parent))]
    for i in range(1, len(parent)):
        out[int(parent[i])].append(i)
    return out


def ancestor_bitsets(parent, words=None):
    """Bit j of word j//32 of row i is set iff j is in anc(i)."""
    n = len(parent)
    if words is None:
        words = (n + 31) // 32
    out = np.zeros((n, words), dtype=np.uint32)
    for i, s in enumerate(ancestors_or_self(parent)):
        for j in s:
            out[i, j // 32] |= np.uint32(1) << np.uint32(j % 32)
    return out


def first_child_next_sibling(parent):
    """Children lists in draw order as (first_child, next_sibling), -1 = none."""
    n = len(parent)
    fc = np.full(n, -1, dtype=np.int32)
    ns = np.full(n, -1, dtype=np.int32)
    for v, ch in enumerate(children(parent)):
        if ch:
            fc[v] = ch[0]
            for a, b in zip(ch[:-1], ch[1:]):
                ns[a] = b
    return fc, ns
