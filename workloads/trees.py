"""Draft-tree shapes as parent arrays.

A tree of N rows is a parent array ``parent[N]`` with ``parent[0] == -1`` (the
root, i.e. the last committed token) and ``0 <= parent[i] < i`` for i > 0
(topological order, as the survey page's Timeline describes SpecInfer storing
tree tokens "by topology"). Siblings appear in ascending index in the order in
which they were drawn (the sibling draw order of the TreeSpark paper, §1/§3.3).
Node counts include the root.
"""
import numpy as np


def tree_depths(parent):
    """Depth (edges from the root) of every row; a generator-side helper."""
    parent = np.asarray(parent)
    d = np.zeros(len(parent), dtype=np.int64)
    for i in range(1, len(parent)):
        d[i] = d[parent[i]] + 1
    return d


def bfs_renumber(parent_creation):
    """Renumber a tree given in creation order into BFS order.

    Children of a node are visited in creation order, which is their draw
    order. Returns (parent_bfs, new_index_of_creation_node).
    """
    parent_creation = np.asarray(parent_creation, dtype=np.int64)
    n = len(parent_creation)
    children = [[] for _ in range(n)]
    for i in range(1, n):
        children[parent_creation[i]].append(i)
    order = [0]
    head = 0
    while head < len(order):
        v = order[head]
        head += 1
        order.extend(children[v])
    assert len(order) == n, "not a tree rooted at node 0"
    new_of_old = np.empty(n, dtype=np.int64)
    new_of_old[np.asarray(order)] = np.arange(n)
    parent_bfs = np.full(n, -1, dtype=np.int32)
    for old in range(1, n):
        parent_bfs[new_of_old[old]] = new_of_old[parent_creation[old]]
    return parent_bfs, new_of_old


def expansion_vector_tree(vec):
    """Static tree from an expansion vector <k1..km> (SpecInfer, survey page
    Timeline): every node at depth i-1 gets k_i children. <1,1,3,1,1> gives
    1+1+1+3+3+3 = 12 rows including the root."""
    parent = [-1]
    level = [0]
    for k in vec:
        nxt = []
        for v in level:
            for _ in range(int(k)):
                parent.append(v)
                nxt.append(len(parent) - 1)
        level = nxt
    p, _ = bfs_renumber(np.asarray(parent))
    return p


def chain_tree(n):
    """A chain (linear tree, K = 1) of n rows."""
    return np.asarray([-1] + list(range(n - 1)), dtype=np.int32)


def star_tree(n):
    """Root plus n-1 children of the root."""
    return np.asarray([-1] + [0] * (n - 1), dtype=np.int32)


def random_tree(rng, n, depth_cap, spine_depth=None):
    """Random tree of n rows: a spine from the root to ``spine_depth`` (default
    min(depth_cap, n-1)); every further node picks a uniform parent among the
    nodes at depth < depth_cap created so far. Returned in BFS order with
    siblings in creation order."""
    if spine_depth is None:
        spine_depth = min(depth_cap, n - 1)
    assert spine_depth <= n - 1 and spine_depth <= depth_cap
    parent = [-1]
    depth = [0]
    for d in range(1, spine_depth + 1):
        parent.append(d - 1)
        depth.append(d)
    while len(parent) < n:
        cand = [i for i in range(len(parent)) if depth[i] < depth_cap]
        p = int(cand[rng.integers(len(cand))])
        parent.append(p)
        depth.append(depth[p] + 1)
    pb, _ = bfs_renumber(np.asarray(parent))
    return pb


def _relabel(parent, order):
    parent = np.asarray(parent)
    n = len(parent)
    new_of_old = np.empty(n, dtype=np.int64)
    new_of_old[np.asarray(order)] = np.arange(n)
    out = np.full(n, -1, dtype=np.int32)
    for old in range(1, n):
        out[new_of_old[old]] = new_of_old[parent[old]]
    return out, new_of_old


def relabel_dfs(parent):
    """Relabel into DFS preorder, keeping each node's children in their order."""
    parent = np.asarray(parent)
    n = len(parent)
    children = [[] for _ in range(n)]
    for i in range(1, n):
        children[parent[i]].append(i)
    order, stack = [], [0]
    while stack:
        v = stack.pop()
        order.append(v)
        stack.extend(reversed(children[v]))
    return _relabel(parent, order)


def relabel_random_topological(rng, parent):
    """A uniformly-chosen-step random topological order that keeps the
    relative order of siblings (so the sibling draw order is unchanged)."""
    parent = np.asarray(parent)
    n = len(parent)
    children = [[] for _ in range(n)]
    for i in range(1, n):
        children[parent[i]].append(i)
    nxt_child = [0] * n
    avail = [0]
    order = []
    while avail:
        j = int(rng.integers(len(avail)))
        v = avail.pop(j)
        order.append(v)
        if children[v]:
            avail.append(children[v][0])
            nxt_child[v] = 1
        p = parent[v]
        if p >= 0 and nxt_child[p] < len(children[p]):
            avail.append(children[p][nxt_child[p]])
            nxt_child[p] += 1
    assert len(order) == n
    return _relabel(parent, order)


def _log_softmax(x):
    m = x.max()
    return x - m - np.log(np.exp(x - m).sum())


def eagle2_tree(rng, depth=6, topk=8, rows=60, vocab=151936, sigma=1.5,
                return_stats=False):
    """EAGLE-2-shaped dynamic tree (survey page, Timeline and Dynamic trees):
    per layer the top-k frontier nodes by path product are expanded, each into
    its top-k children under N(0, sigma) draft logits; at the end the kept set
    is reranked by path value.

    A plain global rerank of flat N(0,1.5) logits never keeps a depth-6 node
    (path products fall too fast), so the kept set is seeded with the root
    path of the best depth-``depth`` candidate and then filled by value with
    root-connected nodes (OPT-Tree Thm 3.1: top path-product nodes are
    root-connected), up to ``rows`` rows including the root.
    Returns the parent array in BFS order (siblings in rank order).
    """
    par = [-1]
    val = [0.0]
    dep = [0]
    tok = [-1]
    frontier = [0]
    for d in range(1, depth + 1):
        new = []
        for f in frontier:
            lp = _log_softmax(rng.normal(0.0, sigma, vocab))
            top = np.argpartition(-lp, topk)[:topk]
            top = top[np.argsort(-lp[top], kind="stable")]
            for t in top:
                par.append(f)
                val.append(val[f] + float(lp[t]))
                dep.append(d)
                tok.append(int(t))
                new.append(len(par) - 1)
        new.sort(key=lambda i: -val[i])
        frontier = new[:topk]
    val = np.asarray(val)
    dep = np.asarray(dep)
    deepest = [i for i in range(len(par)) if dep[i] == depth]
    best = max(deepest, key=lambda i: val[i])
    keep = set()
    v = best
    while v >= 0:
        keep.add(v)
        v = par[v]
    order = np.argsort(-val, kind="stable")
    while len(keep) < rows:
        added = False
        for i in order:
            i = int(i)
            if i not in keep and par[i] in keep:
                keep.add(i)
                added = True
                break
        assert added
    kept = sorted(keep)  # creation order: parents precede children
    remap = {old: new for new, old in enumerate(kept)}
    parent_c = np.asarray([-1] + [remap[par[o]] for o in kept[1:]])
    pb, _ = bfs_renumber(parent_c)
    if return_stats:
        hist = np.bincount(tree_depths(pb), minlength=depth + 1)
        return pb, hist
    return pb
