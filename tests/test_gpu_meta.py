"""GPU parity: tv_tree_meta (depth, ancestor-or-self bitsets, children in
draw order; [TreeSpark] §3.2 step 3 and §4: per-depth positions and an
ancestor-bitmask mask) against the oracle's tree functions, on BFS, DFS and
random topological numberings, row counts that are not multiples of 32,
max_nodes above every tree, and batches of several requests."""
import numpy as np
import pytest

import oracle
from workloads import random_tree, chain_tree, star_tree, relabel_dfs, relabel_random_topological

pytestmark = pytest.mark.gpu


def _run(trees, max_nodes, outputs=("depth", "anc", "fc", "ns")):
    import torch
    import tree_verification_verify_amd as tv
    counts = [len(t) for t in trees]
    indptr = np.zeros(len(trees) + 1, np.int32)
    indptr[1:] = np.cumsum(counts)
    T = int(indptr[-1])
    parent = np.concatenate([np.asarray(t, np.int32) for t in trees])
    words = (max_nodes + 31) // 32
    dev = "cuda"
    ni = torch.from_numpy(indptr).to(dev)
    pa = torch.from_numpy(parent).to(dev)
    depth = torch.full((T,), -7, dtype=torch.int32, device=dev) if "depth" in outputs else None
    anc = torch.full((T, words), 0x5A5A5A5A, dtype=torch.int32, device=dev) if "anc" in outputs else None
    fc = torch.full((T,), -7, dtype=torch.int32, device=dev) if "fc" in outputs else None
    ns = torch.full((T,), -7, dtype=torch.int32, device=dev) if "ns" in outputs else None
    ws = tv.alloc_workspace(256)
    tv.tv_tree_meta(len(trees), max_nodes, ni, pa, depth, anc, fc, ns, ws)
    st, bits = tv.device_status(ws)
    cpu = lambda x: None if x is None else x.cpu().numpy()
    a = cpu(anc)
    return dict(depth=cpu(depth), anc=None if a is None else a.view(np.uint32), fc=cpu(fc),
                ns=cpu(ns), indptr=indptr, st=st, bits=bits, words=words)


def _check(trees, got):
    assert got["st"] == 0, (got["st"], got["bits"])
    for r, t in enumerate(trees):
        a, b = int(got["indptr"][r]), int(got["indptr"][r + 1])
        if got["depth"] is not None:
            np.testing.assert_array_equal(got["depth"][a:b], oracle.depths(t), err_msg=f"depth {r}")
        if got["anc"] is not None:
            np.testing.assert_array_equal(got["anc"][a:b], oracle.ancestor_bitsets(t, got["words"]),
                                          err_msg=f"anc {r}")
        fc, ns = oracle.first_child_next_sibling(t)
        if got["fc"] is not None:
            np.testing.assert_array_equal(got["fc"][a:b], fc, err_msg=f"first child {r}")
        if got["ns"] is not None:
            np.testing.assert_array_equal(got["ns"][a:b], ns, err_msg=f"next sibling {r}")


def _orders(rng, t):
    return [np.asarray(t), relabel_dfs(t)[0], relabel_random_topological(rng, t)[0]]


@pytest.mark.parametrize("order", [0, 1, 2])
def test_batch_of_trees(order):
    rng = np.random.default_rng(31 + order)
    base = [random_tree(rng, n, depth_cap=d) for n, d in ((45, 6), (100, 12), (33, 4), (7, 7))]
    base += [np.array([-1]), chain_tree(64), star_tree(65)]
    trees = [_orders(rng, t)[order] for t in base]
    _check(trees, _run(trees, 200))         # max_nodes above every tree: 7 words


@pytest.mark.parametrize("order", [0, 1, 2])
def test_largest_tree(order):
    rng = np.random.default_rng(41)
    t = _orders(rng, random_tree(rng, 1024, depth_cap=30))[order]
    _check([t], _run([t], 1024))            # 32 words, every bit position used


def test_outputs_may_be_null():
    rng = np.random.default_rng(5)
    trees = [random_tree(rng, 70, depth_cap=9), random_tree(rng, 20, depth_cap=3)]
    _check(trees, _run(trees, 70, outputs=("depth",)))
    _check(trees, _run(trees, 70, outputs=("anc", "ns")))


def test_bad_parent_sets_the_tree_bit():
    t = np.array([-1, 0, 0, 1, 2, 7, 3, 4], np.int32)   # row 5's parent is after it
    got = _run([t], 8)
    assert got["bits"] & 1 and got["st"] != 0
    t2 = np.array([3, 0, 0, 1], np.int32)               # root without parent -1
    got = _run([t2], 4)
    assert got["bits"] & 1


def test_tree_above_max_nodes_sets_the_shape_bit():
    t = random_tree(np.random.default_rng(2), 40, depth_cap=5)
    got = _run([t], 32)                                # 40 rows do not fit 1 word
    assert got["bits"] & (1 << 5)
