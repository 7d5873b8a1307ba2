"""GPU parity: tree_expand_step + tree_rerank (EAGLE-2 construction, HIP,
via the C ABI) against the fp64 oracle. Tokens, parents, frontiers and the
final tree are compared exactly; values within 1e-5. A request whose oracle
has a frontier or rerank cut within EPS (a choice fp32 may take either way)
is excluded and counted."""
import numpy as np
import pytest

import oracle.construct as C
from workloads import make_construct_inputs

pytestmark = pytest.mark.gpu

EPS = 1e-4


def _run(*a, **kw):
    from gpu_run import run_construct
    return run_construct(*a, **kw)


def _compare(root, rows, k, m, got, requests=None, allow_near=0):
    assert got["status"] == 0, (got["status"], got["bits"])
    B = root.shape[0]
    R = rows.shape[1] + 1
    near = 0
    for b in (range(B) if requests is None else requests):
        parent, token, cands, frontiers = C.eagle2_tree(root[b], list(rows[b]), k, m)
        if C.near_ties(cands, frontiers, k, m, EPS):
            near += 1
            continue
        n = len(cands.value)
        assert got["num_cand"] == n
        np.testing.assert_array_equal(got["token"][b, :n], cands.token, err_msg=f"request {b}")
        np.testing.assert_array_equal(got["parent"][b, :n], cands.parent, err_msg=f"request {b}")
        np.testing.assert_allclose(got["value"][b, :n], cands.value, rtol=0, atol=1e-5)
        for d in range(R):
            np.testing.assert_array_equal(got["frontiers"][d][b], frontiers[d], err_msg=f"{b} {d}")
        cnt = len(parent)
        assert got["out_count"][b] == cnt
        np.testing.assert_array_equal(got["out_parent"][b, :cnt], parent)
        np.testing.assert_array_equal(got["out_token"][b, :cnt], token)
        assert (got["out_parent"][b, cnt:] == -1).all() and (got["out_token"][b, cnt:] == -1).all()
    assert near <= allow_near, near
    total = B if requests is None else len(requests)
    assert total - near >= total - allow_near >= 1
    return near


# near: requests the oracle itself finds within EPS of a tie (counted on the
# CPU from the oracle alone); the rest are compared.
@pytest.mark.parametrize("V,k,R,m,near", [(7, 3, 3, 8, 0), (64, 4, 4, 20, 0), (1000, 10, 6, 60, 0),
                                          (4099, 16, 3, 100, 1), (4096, 1, 5, 10, 0),
                                          (300, 8, 2, 1000, 0), (50, 2, 6, 1, 0)])
def test_random_shapes(V, k, R, m, near):
    """Scalar (V % 4 != 0) and vector rows, k from 1 to 16, m below, at and
    above the candidate count."""
    rng = np.random.default_rng(V + 7 * k + R)
    root, rows = make_construct_inputs(rng, 6, V, k, R)
    _compare(root, rows, k, m, _run(root, rows, k, m), allow_near=near)


@pytest.mark.parametrize("V,k,R", [(151936, 10, 3), (4099, 16, 2), (7, 3, 3)])
def test_split_rounds_match_unsplit(V, k, R):
    """Rows split over several workgroups (the workspace given) and unsplit
    rows take the same decisions; values differ only in the log-sum-exp's
    summation order."""
    rng = np.random.default_rng(V + k)
    root, rows = make_construct_inputs(rng, 8, V, k, R)
    a = _run(root, rows, k, 30, split=True)
    b = _run(root, rows, k, 30, split=False)
    assert a["status"] == 0 and b["status"] == 0
    for key in ("token", "parent", "out_parent", "out_token", "out_count"):
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)
    for fa, fb in zip(a["frontiers"], b["frontiers"]):
        np.testing.assert_array_equal(fa, fb)
    np.testing.assert_allclose(a["value"], b["value"], rtol=0, atol=1e-5)
    _compare(root, rows, k, 30, a, allow_near=0)


def test_integer_logits_with_ties():
    """Integer logits: many exact ties inside rows (lower token id first) and
    between sibling values (lower candidate id first)."""
    rng = np.random.default_rng(3)
    root, rows = make_construct_inputs(rng, 8, 257, 6, 4, integer_levels=5)
    _compare(root, rows, 6, 40, _run(root, rows, 6, 40), allow_near=1)


def test_eagle2_shape_full_vocab():
    """The EAGLE-2 shape (top-k 10, depth 6, 60 kept nodes) over V = 151936 for
    a 64-request batch; every request is compared with the oracle (4 of the
    64 have a near tie and are excluded) and checked for shape."""
    rng = np.random.default_rng(2024)
    B, V, k, R, m = 64, 151936, 10, 6, 60
    root, rows = make_construct_inputs(rng, B, V, k, R)
    got = _run(root, rows, k, m)
    _compare(root, rows, k, m, got, allow_near=4)
    for b in range(B):
        par = got["out_parent"][b]
        assert got["out_count"][b] == m + 1 and par[0] == -1
        assert all(0 <= par[i] < i for i in range(1, m + 1))
        assert ((got["out_token"][b, 1:] >= 0) & (got["out_token"][b, 1:] < V)).all()


def test_bad_frontier_and_nonfinite_logits_are_reported():
    rng = np.random.default_rng(4)
    root, rows = make_construct_inputs(rng, 3, 128, 4, 3)
    got = _run(root, rows, 4, 10, bad_frontier=999)
    assert got["status"] != 0 and got["bits"] & 1      # TV_DEV_TREE
    root[1, 5] = np.nan
    got = _run(root, rows, 4, 10)
    assert got["bits"] & 4                             # TV_DEV_LOGITS


def test_construct_then_greedy_verify_matches_the_oracle():
    """The rows composed: the GPU builds EAGLE-2 trees, and its parent and
    token arrays feed greedy verification (tree_spec_sample at T = 0) and
    tree_accept_path on the GPU; the oracle runs its own construction, walk
    and path. Target rows are the expanded nodes' draft rows plus noise, so
    paths of several tokens are accepted."""
    import oracle
    from gpu_run import run_sampler
    from workloads.inputs import SamplerInputs
    rng = np.random.default_rng(77)
    B, V, k, R, m = 8, 4096, 4, 4, 20
    root, rows = make_construct_inputs(rng, B, V, k, R)
    got = _run(root, rows, k, m)
    assert got["status"] == 0
    n = m + 1
    target = np.empty((B * n, V), dtype=np.float32)
    for b in range(B):
        parent, token, cands, frontiers = C.eagle2_tree(root[b], list(rows[b]), k, m)
        assert not C.near_ties(cands, frontiers, k, m, EPS)
        np.testing.assert_array_equal(got["out_parent"][b], parent)
        np.testing.assert_array_equal(got["out_token"][b], token)
        _, _, keep = C.rerank(cands, m)
        row_of = {-1: root[b]}
        for d, fr in enumerate(frontiers[:-1]):
            for s, f in enumerate(fr):
                row_of[f] = rows[b, d, s]
        for j, c in enumerate([-1] + list(keep)):
            base = row_of.get(c)
            if base is None:  # a leaf: its row only decides a bonus token
                base = (rng.standard_normal(V) * 2).astype(np.float32)
            target[b * n + j] = base + (rng.standard_normal(V) * 0.3).astype(np.float32)
    inp = SamplerInputs(vocab=V, target_logits=target, draft_logits=None,
                        tokens=got["out_token"].reshape(-1).astype(np.int32),
                        node_indptr=(np.arange(B + 1) * n).astype(np.int32),
                        parent=got["out_parent"].reshape(-1).astype(np.int32),
                        temperature=np.zeros(B, np.float32),
                        uniforms=np.zeros((B * n, 2), np.float32))
    ver = run_sampler(inp, max_depth=R)
    assert ver["status"] == 0, (ver["status"], ver["bits"])
    flags, nts, _ = oracle.tree_spec_sample(inp)
    pn, ot, ol, kk = oracle.tree_accept_path(inp.node_indptr, inp.parent, inp.tokens, flags, nts,
                                             [0] * B, R)
    np.testing.assert_array_equal(ver["flag"], flags)
    np.testing.assert_array_equal(ver["next_token"], nts)
    np.testing.assert_array_equal(ver["out_len"], ol)
    np.testing.assert_array_equal(ver["out_tokens"], ot)
    np.testing.assert_array_equal(ver["path_nodes"], pn)
    assert ol.max() >= 3  # some request accepts at least two drafted tokens
