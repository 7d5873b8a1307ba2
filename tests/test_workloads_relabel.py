"""The relabel helpers move every per-row input with its row: the oracle's
outputs on a relabelled problem are the original outputs, permuted (P4 for
attention; for the walk, the same decisions at the same nodes)."""
import numpy as np
import pytest

import oracle
from workloads import make_attention_inputs, make_sampler_inputs, random_tree, chain_tree
from workloads.relabel import relabel_trees, relabel_attention, relabel_sampler, global_perm


@pytest.mark.parametrize("kind", ["dfs", "random"])
def test_attention_rows_permute(kind):
    rng = np.random.default_rng(3)
    trees = [random_tree(rng, 23, depth_cap=5), chain_tree(6), random_tree(rng, 40, depth_cap=9)]
    inp = make_attention_inputs(rng, rng, trees, [17, 0, 35], 4, 2, 16, dtype="fp32")
    maps = relabel_trees(trees, kind, rng)
    rel = relabel_attention(inp, maps)
    for r, (newp, _) in enumerate(maps):
        oracle.check_tree(newp)
    perm = global_perm(inp.node_indptr, maps)
    np.testing.assert_allclose(oracle.tree_attention(rel)[perm], oracle.tree_attention(inp),
                               rtol=1e-12, atol=1e-12)
    if kind == "dfs":   # a non-BFS order really moved rows
        assert (perm != np.arange(len(perm))).any()


@pytest.mark.parametrize("kind", ["dfs", "random"])
def test_walk_decisions_permute(kind):
    rng = np.random.default_rng(4)
    trees = [random_tree(rng, int(rng.integers(2, 30)), depth_cap=6) for _ in range(12)]
    temps = rng.choice([0.0, 0.5, 1.0], size=12)
    inp = make_sampler_inputs(rng, rng, rng, trees, 64, temps, mode="correlated")
    maps = relabel_trees(trees, kind, rng)
    rel = relabel_sampler(inp, maps)
    perm = global_perm(inp.node_indptr, maps)
    f0, n0, _ = oracle.tree_spec_sample(inp)
    f1, n1, _ = oracle.tree_spec_sample(rel)
    np.testing.assert_array_equal(f1[perm], f0)
    np.testing.assert_array_equal(n1[perm], n0)
