"""Move generated inputs to another topological numbering of the same trees.

The boundary accepts any topological parent array (the survey page's Timeline:
tree tokens are stored in the KV cache "by topology"), not only BFS order. A
relabelling maps old row i of request r to new row new_of_old[r][i]; every
per-row input moves with its row (queries, the tree's own K/V at logical
positions P_r + i, logits rows, tokens, uniforms), so the relabelled problem
is the same problem and its outputs are the old ones, permuted. Row
permutation only: no verification arithmetic lives here.
"""
import numpy as np

from .trees import relabel_dfs, relabel_random_topological
from .inputs import AttentionInputs, SamplerInputs, PAGE


def relabel_trees(trees, kind, rng=None):
    """[(new_parent, new_of_old)] per tree; kind "dfs" or "random" (a random
    topological order that keeps each node's children in draw order)."""
    out = []
    for t in trees:
        if kind == "dfs":
            out.append(relabel_dfs(t))
        elif kind == "random":
            out.append(relabel_random_topological(rng, t))
        else:
            raise ValueError(kind)
    return out


def relabel_attention(inp, maps):
    """AttentionInputs with every request's tree renumbered by maps[r] =
    (new_parent, new_of_old): query row a+i moves to a+new_of_old[i], and the
    K/V at logical position P_r+i to P_r+new_of_old[i] (same pages)."""
    q = np.empty_like(inp.q)
    k = inp.k_pages.copy()
    v = inp.v_pages.copy()
    parent = np.empty_like(inp.parent)
    for r, (newp, new_of_old) in enumerate(maps):
        a, b = int(inp.node_indptr[r]), int(inp.node_indptr[r + 1])
        n = b - a
        assert len(newp) == n
        q[a + np.asarray(new_of_old)] = inp.q[a:b]
        parent[a:b] = newp
        P = int(inp.prefix_len[r])
        base = int(inp.page_indptr[r])
        for i in range(n):
            src, dst = P + i, P + int(new_of_old[i])
            ps, ss = inp.page_indices[base + src // PAGE], src % PAGE
            pd, sd = inp.page_indices[base + dst // PAGE], dst % PAGE
            k[pd, :, sd, :] = inp.k_pages[ps, :, ss, :]
            v[pd, :, :, sd] = inp.v_pages[ps, :, :, ss]
    out = AttentionInputs(**{**inp.__dict__})
    out.q, out.k_pages, out.v_pages, out.parent = q, k, v, parent
    return out


def relabel_sampler(inp, maps):
    """SamplerInputs renumbered by maps[r] = (new_parent, new_of_old): logits
    rows, tokens and uniforms move with their node."""
    T = int(inp.node_indptr[-1])
    perm = np.empty(T, dtype=np.int64)   # new global row of old global row
    parent = np.empty_like(inp.parent)
    for r, (newp, new_of_old) in enumerate(maps):
        a, b = int(inp.node_indptr[r]), int(inp.node_indptr[r + 1])
        perm[a:b] = a + np.asarray(new_of_old)
        parent[a:b] = newp

    def move(x):
        if x is None:
            return None
        y = np.empty_like(x)
        y[perm] = x
        return y

    return SamplerInputs(vocab=inp.vocab, target_logits=move(inp.target_logits),
                         draft_logits=move(inp.draft_logits), tokens=move(inp.tokens),
                         node_indptr=inp.node_indptr.copy(), parent=parent,
                         temperature=inp.temperature.copy(), uniforms=move(inp.uniforms),
                         extra=dict(inp.extra))


def global_perm(node_indptr, maps):
    """new global row of every old global row."""
    T = int(node_indptr[-1])
    perm = np.empty(T, dtype=np.int64)
    for r, (_, new_of_old) in enumerate(maps):
        a = int(node_indptr[r])
        perm[a:a + len(new_of_old)] = a + np.asarray(new_of_old)
    return perm
