"""Pins for the oracle's tree-masked attention (library routine: torch SDPA on
the CPU in float64, given explicit key sets)."""
import numpy as np
import pytest
import torch

import oracle
from workloads import (chain_tree, star_tree, random_tree, make_attention_inputs,
                       relabel_random_topological, relabel_dfs)
from workloads.inputs import repage


def _sdpa_rows(q_rows, K, V, scale):
    """q_rows [n][D]; K, V [L][D] -> SDPA outputs [n][D] (no mask)."""
    q = torch.from_numpy(q_rows)[None, None]
    k = torch.from_numpy(np.ascontiguousarray(K))[None, None]
    v = torch.from_numpy(np.ascontiguousarray(V))[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale)
    return o[0, 0].numpy()


def _logical(inp, r, which):
    """[L][Hkv][D] logical K or V of request r, read slot by slot (K pages
    are [page][g][slot][d], V pages [page][g][d][slot])."""
    L = inp.kv_len(r)
    base = int(inp.page_indptr[r])
    if which == "k":
        pool = oracle.decode_values(inp.k_pages, inp.dtype)
        return np.stack([pool[inp.page_indices[base + t // 16], :, t % 16, :] for t in range(L)])
    pool = oracle.decode_values(inp.v_pages, inp.dtype)
    return np.stack([pool[inp.page_indices[base + t // 16], :, :, t % 16] for t in range(L)])


def _make(trees, prefixes, Hq=4, Hkv=2, D=32, dtype="fp32", seed=0):
    g = np.random.default_rng(seed)
    return make_attention_inputs(g, g, trees, prefixes, Hq, Hkv, D, dtype=dtype)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_chain_equals_causal_attention(dtype):
    """P1: a chain tree is causal attention over prefix + chain."""
    N, P = 11, 37
    inp = _make([chain_tree(N)], [P], dtype=dtype)
    out = oracle.tree_attention(inp)
    Q = oracle.decode_values(inp.q, inp.dtype)
    K, V = _logical(inp, 0, "k"), _logical(inp, 0, "v")
    G = inp.num_q_heads // inp.num_kv_heads
    L = P + N
    mask = np.tril(np.ones((L, L), dtype=bool))[P:]          # last N query positions
    for h in range(inp.num_q_heads):
        q = torch.from_numpy(Q[:, h, :])[None, None]
        k = torch.from_numpy(np.ascontiguousarray(K[:, h // G]))[None, None]
        v = torch.from_numpy(np.ascontiguousarray(V[:, h // G]))[None, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            q, k, v, attn_mask=torch.from_numpy(mask), scale=inp.sm_scale)[0, 0].numpy()
        np.testing.assert_allclose(out[:, h], ref, rtol=1e-12, atol=1e-12)


def test_single_node_is_decode_attention():
    """P2: a 1-row tree is plain single-query decode attention."""
    inp = _make([np.array([-1])], [53])
    out = oracle.tree_attention(inp)
    Q = oracle.decode_values(inp.q, inp.dtype)
    K, V = _logical(inp, 0, "k"), _logical(inp, 0, "v")
    for h in range(inp.num_q_heads):
        ref = _sdpa_rows(Q[:, h], K[:, h // 2], V[:, h // 2], inp.sm_scale)
        np.testing.assert_allclose(out[:, h], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", range(3))
def test_row_is_decode_over_prefix_plus_path(seed):
    """P3: row i equals decode attention over the linear sequence
    prefix + (root .. i) (SpecInfer's equivalence to incremental decoding)."""
    rng = np.random.default_rng(seed)
    trees = [random_tree(rng, 23, depth_cap=5), random_tree(rng, 9, depth_cap=3)]
    prefixes = [int(rng.integers(1, 60)), int(rng.integers(1, 60))]
    inp = _make(trees, prefixes, Hq=6, Hkv=3, D=16, seed=seed)
    out = oracle.tree_attention(inp)
    Q = oracle.decode_values(inp.q, inp.dtype)
    G = 2
    for r, parent in enumerate(trees):
        K, V = _logical(inp, r, "k"), _logical(inp, r, "v")
        P = prefixes[r]
        a = int(inp.node_indptr[r])
        for i in range(len(parent)):
            path, j = [], i
            while j >= 0:
                path.append(j)
                j = parent[j]
            keys = list(range(P)) + [P + j for j in reversed(path)]
            for h in range(inp.num_q_heads):
                ref = _sdpa_rows(Q[a + i:a + i + 1, h], K[keys, h // G], V[keys, h // G], inp.sm_scale)
                np.testing.assert_allclose(out[a + i, h], ref[0], rtol=1e-12, atol=1e-12)


def test_star_tree_closed_form():
    """P5: in a star every row sees prefix + root + itself."""
    inp = _make([star_tree(7)], [20], Hq=2, Hkv=2)
    out = oracle.tree_attention(inp)
    Q = oracle.decode_values(inp.q, inp.dtype)
    K, V = _logical(inp, 0, "k"), _logical(inp, 0, "v")
    for i in range(7):
        keys = list(range(20)) + sorted({20, 20 + i})
        for h in range(2):
            ref = _sdpa_rows(Q[i:i + 1, h], K[keys, h], V[keys, h], inp.sm_scale)
            np.testing.assert_allclose(out[i, h], ref[0], rtol=1e-12, atol=1e-12)


def test_relabel_permutes_rows_and_repaging_changes_nothing():
    """P4: relabelling to another topological order permutes rows (with the
    tree K/V and Q permuted alike); a new page placement changes nothing;
    GQA equals MHA with repeated KV heads."""
    rng = np.random.default_rng(5)
    parent = random_tree(rng, 19, depth_cap=4)
    P = 29
    inp = _make([parent], [P], Hq=4, Hkv=2, D=16, seed=9)
    base = oracle.tree_attention(inp)
    # page placement
    moved = repage(inp, np.random.default_rng(1), spare_pages=5)
    np.testing.assert_array_equal(oracle.tree_attention(moved), base)
    # relabel: new row new_of_old[i] holds old row i's query and K/V
    for newp, new_of_old in (relabel_dfs(parent), relabel_random_topological(rng, parent)):
        rel = make_attention_inputs(np.random.default_rng(0), np.random.default_rng(0),
                                    [newp], [P], 4, 2, 16, dtype="fp32", shuffle=False)
        Kl, Vl = _logical(inp, 0, "k"), _logical(inp, 0, "v")
        Kn, Vn = Kl.copy(), Vl.copy()
        Kn[P + new_of_old] = Kl[P:]
        Vn[P + new_of_old] = Vl[P:]
        L = P + 19
        kp = np.zeros_like(rel.k_pages)
        vp = np.zeros_like(rel.v_pages)
        for t in range(L):
            kp[rel.page_indices[t // 16], :, t % 16] = Kn[t]
            vp[rel.page_indices[t // 16], :, :, t % 16] = Vn[t]
        rel.k_pages, rel.v_pages = kp, vp
        rel.q = np.empty_like(inp.q)
        rel.q[new_of_old] = inp.q
        got = oracle.tree_attention(rel)
        np.testing.assert_allclose(got[new_of_old], base, rtol=1e-13, atol=1e-13)
    # GQA == MHA with repeated KV heads
    mha = make_attention_inputs(np.random.default_rng(0), np.random.default_rng(0),
                                [parent], [P], 4, 4, 16, dtype="fp32", shuffle=False)
    mha.q = inp.q.copy()
    mha.page_indices = inp.page_indices.copy()
    mha.k_pages = np.repeat(inp.k_pages, 2, axis=1)
    mha.v_pages = np.repeat(inp.v_pages, 2, axis=1)
    np.testing.assert_allclose(oracle.tree_attention(mha), base, rtol=1e-13, atol=1e-13)


def test_rows_api_matches_full():
    rng = np.random.default_rng(2)
    trees = [random_tree(rng, 12, depth_cap=4), chain_tree(5)]
    inp = _make(trees, [40, 17], Hq=4, Hkv=1, D=16)
    full = oracle.tree_attention(inp)
    picks = [(1, 3), (0, 11), (0, 0)]
    rows = oracle.tree_attention_rows(inp, picks)
    for n, (r, i) in enumerate(picks):
        np.testing.assert_array_equal(rows[n], full[int(inp.node_indptr[r]) + i])
