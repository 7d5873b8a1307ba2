"""GPU parity on trees numbered in non-BFS topological orders.

The boundary accepts any topological parent array ([survey] Timeline: tree
tokens sit in the KV cache by topology). BFS numbering keeps every sibling set
contiguous and ancestor bits packed near the low words; DFS preorder and
random topological orders (siblings still in draw order) scatter both. Each
relabelled problem carries its rows along (queries, tree K/V, logits rows,
tokens, uniforms), so it is the same problem: the HIP path must match the
oracle on the relabelled inputs, and its outputs must be the BFS outputs
permuted (bit-exact for the sampler's integer outputs).
"""
import numpy as np
import pytest

import oracle
from workloads import make_config, make_attention_inputs, make_sampler_inputs, random_tree
from workloads.relabel import relabel_trees, relabel_attention, relabel_sampler, global_perm

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "fp32": 1e-5}
EPS = 1e-6   # the near-threshold band of the specification


def _attn(inp):
    from gpu_run import run_attention
    got, st, bits = run_attention(inp)
    assert st == 0, (st, bits)
    return got


@pytest.mark.parametrize("kind", ["dfs", "random"])
@pytest.mark.parametrize("name,batch", [("eagle2", None), ("batched", None), ("highload", 24),
                                        ("sequoia", None)])
def test_attention_relabelled(name, batch, kind):
    cfg = make_config(name, sampler=False, batch=batch)
    maps = relabel_trees(cfg.trees, kind, np.random.default_rng(11))
    rel = relabel_attention(cfg.attn, maps)
    got = _attn(rel)
    err = np.abs(got - oracle.tree_attention(rel)).max()
    assert err <= TOL[rel.dtype], err
    base = _attn(cfg.attn)
    perm = global_perm(cfg.attn.node_indptr, maps)
    assert np.abs(got[perm] - base).max() <= TOL[rel.dtype]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("kind", ["dfs", "random"])
def test_attention_relabelled_random_small(dtype, kind):
    """Ragged tails, G in {1, 4}, trees up to 200 rows (7 bitset words)."""
    rng = np.random.default_rng(5 + (dtype == "bf16"))
    trees = [random_tree(rng, int(rng.integers(2, 200)), depth_cap=int(rng.integers(2, 30)))
             for _ in range(6)]
    prefixes = [int(x) for x in rng.integers(0, 500, size=6)]
    for Hq, Hkv, D in ((8, 8, 64), (32, 8, 128)):
        inp = make_attention_inputs(rng, rng, trees, prefixes, Hq, Hkv, D, dtype=dtype)
        rel = relabel_attention(inp, relabel_trees(trees, kind, rng))
        err = np.abs(_attn(rel) - oracle.tree_attention(rel)).max()
        assert err <= TOL[dtype], err


def _sample(inp, md, prefix_lens, greedy_path=False):
    from gpu_run import run_sampler
    got = run_sampler(inp, max_depth=md, prefix_lens=prefix_lens, greedy_path=greedy_path)
    assert got["status"] == 0, (got["status"], got["bits"])
    return got


def _check_sampler(inp, got, prefix_lens, greedy_path=False):
    from test_gpu_sampler import compare_walk
    flags, nts, logs = oracle.tree_spec_sample(inp, greedy_path=greedy_path)
    pn, ot, ol, kk = oracle.tree_accept_path(inp.node_indptr, inp.parent, inp.tokens, flags,
                                             nts, prefix_lens, got["max_depth"])
    skipped, _ = compare_walk(inp, got, flags, nts, logs, pn, ot, ol, kk)
    assert skipped == 0, skipped


@pytest.mark.parametrize("kind", ["dfs", "random"])
@pytest.mark.parametrize("temp", ["mixed", 1.0])
def test_sampler_and_path_relabelled(kind, temp):
    """The highload sampler workload (V = 151936) renumbered: flags, next
    tokens, paths, emitted tokens and keep-lists equal the oracle's on the
    relabelled inputs, and equal the BFS run's after mapping the rows."""
    cfg = make_config("highload", attention=False, temperature=temp)
    maps = relabel_trees(cfg.trees, kind, np.random.default_rng(12))
    rel = relabel_sampler(cfg.sampler, maps)
    got = _sample(rel, 8, cfg.prefix_lens)
    _check_sampler(rel, got, cfg.prefix_lens)
    base = _sample(cfg.sampler, 8, cfg.prefix_lens)
    perm = global_perm(cfg.sampler.node_indptr, maps)
    # the same decisions at the same nodes: the GPU's arithmetic does not
    # depend on the numbering
    np.testing.assert_array_equal(got["flag"][perm], base["flag"])
    np.testing.assert_array_equal(got["next_token"][perm], base["next_token"])
    np.testing.assert_array_equal(got["out_len"], base["out_len"])
    np.testing.assert_array_equal(got["out_tokens"], base["out_tokens"])
    for r in range(rel.batch):
        a = int(rel.node_indptr[r])
        n = base["out_len"][r]
        mapped = perm[a + base["path_nodes"][r, :n]] - a
        np.testing.assert_array_equal(got["path_nodes"][r, :n], mapped)


@pytest.mark.parametrize("kind", ["dfs", "random"])
def test_greedy_walk_relabelled(kind):
    """Greedy requests verified along the walk only, on the renumbered
    highload trees (T = 0): equal to the oracle on the relabelled inputs and
    to the BFS run after mapping the rows."""
    cfg = make_config("highload", attention=False, temperature=0.0)
    maps = relabel_trees(cfg.trees, kind, np.random.default_rng(13))
    rel = relabel_sampler(cfg.sampler, maps)
    got = _sample(rel, 8, cfg.prefix_lens, greedy_path=True)
    _check_sampler(rel, got, cfg.prefix_lens, greedy_path=True)
    base = _sample(cfg.sampler, 8, cfg.prefix_lens, greedy_path=True)
    perm = global_perm(cfg.sampler.node_indptr, maps)
    np.testing.assert_array_equal(got["flag"][perm], base["flag"])
    np.testing.assert_array_equal(got["next_token"][perm], base["next_token"])
    np.testing.assert_array_equal(got["out_tokens"], base["out_tokens"])


@pytest.mark.parametrize("kind", ["dfs", "random"])
def test_sampler_relabelled_random_small(kind):
    rng = np.random.default_rng(21)
    trees = [random_tree(rng, int(rng.integers(2, 60)), depth_cap=int(rng.integers(1, 12)))
             for _ in range(20)]
    temps = rng.choice([0.0, 0.5, 1.0, 2.0], size=20)
    inp = make_sampler_inputs(rng, rng, rng, trees, 1000, temps, mode="correlated")
    rel = relabel_sampler(inp, relabel_trees(trees, kind, rng))
    _check_sampler(rel, _sample(rel, 12, None), [0] * 20)
