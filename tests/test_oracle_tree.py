"""Pins for the oracle's tree metadata and for the tree generators."""
import os

import numpy as np
import pytest

import oracle
from workloads import (expansion_vector_tree, random_tree, chain_tree, star_tree,
                       eagle2_tree, relabel_dfs, relabel_random_topological,
                       make_config)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _reachability_ancestors(parent):
    """Ancestors-or-self by transitive closure of the child->parent relation
    (boolean matrix powers), an algorithm independent of the oracle's
    recursive definition."""
    n = len(parent)
    A = np.eye(n, dtype=bool)
    for i in range(1, n):
        A[i, parent[i]] = True
    R = A.copy()
    while True:
        R2 = (R.astype(np.int64) @ R.astype(np.int64)) > 0
        if (R2 == R).all():
            break
        R = R2
    return [set(np.nonzero(R[i])[0].tolist()) for i in range(n)]


def _golden_tree():
    lines = [l for l in open(os.path.join(GOLDEN, "expansion_vector_1_1_3_1_1.txt"))
             if l.strip() and not l.startswith("#")]
    return (np.array(lines[0].split(), dtype=np.int64),
            np.array(lines[1].split(), dtype=np.int64))


def test_expansion_vector_golden():
    parent, depth = _golden_tree()
    got = expansion_vector_tree([1, 1, 3, 1, 1])
    assert len(got) == 12
    np.testing.assert_array_equal(got, parent)
    np.testing.assert_array_equal(oracle.depths(parent), depth)


@pytest.mark.parametrize("seed", range(6))
def test_ancestors_match_transitive_closure(seed):
    rng = np.random.default_rng(seed)
    for parent in (random_tree(rng, 40, depth_cap=6), chain_tree(17), star_tree(9),
                   expansion_vector_tree([2, 1, 3])):
        anc = oracle.ancestors_or_self(parent)
        assert anc == _reachability_ancestors(parent)
        d = oracle.depths(parent)
        assert all(len(s) - 1 == d[i] for i, s in enumerate(anc))
        bits = oracle.ancestor_bitsets(parent)
        for i, s in enumerate(anc):
            got = {j for j in range(len(parent)) if (bits[i, j // 32] >> (j % 32)) & 1}
            assert got == s


def test_first_child_next_sibling_lists_children_in_draw_order():
    rng = np.random.default_rng(3)
    parent = random_tree(rng, 50, depth_cap=5)
    fc, ns = oracle.first_child_next_sibling(parent)
    for v in range(len(parent)):
        lst, c = [], fc[v]
        while c >= 0:
            lst.append(int(c))
            c = ns[c]
        assert lst == [i for i in range(len(parent)) if parent[i] == v]


@pytest.mark.parametrize("bad", [[0, 0], [-1, 1], [-1, 0, 3, 1], [-1, -1], [-1, 0, 2]])
def test_check_tree_rejects(bad):
    with pytest.raises(ValueError):
        oracle.check_tree(np.asarray(bad))


def test_random_tree_invariants():
    rng = np.random.default_rng(7)
    for n, cap in ((768, 12), (32, 8), (16, 8), (9, 8)):
        p = random_tree(rng, n, depth_cap=cap)
        oracle.check_tree(p)
        d = oracle.depths(p)
        assert len(p) == n and d.max() == min(cap, n - 1)
        assert (np.diff(d) >= 0).all(), "BFS order"


def test_relabels_are_topological_and_keep_sibling_order():
    rng = np.random.default_rng(11)
    p = random_tree(rng, 60, depth_cap=6)
    for q, new_of_old in (relabel_dfs(p), relabel_random_topological(rng, p)):
        oracle.check_tree(q)
        for v in range(len(p)):
            old_ch = [i for i in range(len(p)) if p[i] == v]
            new_ch = [i for i in range(len(q)) if q[i] == new_of_old[v]]
            assert [int(new_of_old[c]) for c in old_ch] == new_ch


def test_eagle2_tree_shape():
    rng = np.random.default_rng(0)
    p, hist = eagle2_tree(rng, vocab=4096, return_stats=True)
    oracle.check_tree(p)
    assert len(p) == 60 and oracle.depths(p).max() == 6
    assert hist.sum() == 60


def test_config_shapes():
    c = make_config("tiny")
    assert c.attn.total_nodes == 12 and c.attn.max_kv_len == 140
    assert c.sampler.vocab == 512
    c = make_config("batched", sampler=False)
    assert c.attn.batch == 16 and all(len(t) == 32 for t in c.trees)
    assert all(1024 <= p <= 4096 for p in c.prefix_lens)
    assert max(oracle.depths(t).max() for t in c.trees) <= 8
