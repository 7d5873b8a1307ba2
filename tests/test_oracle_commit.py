"""Pins for the oracle's commit of the accepted path's K/V.

The main pin goes through attention: after committing a root path that ends at
node v, plain causal decode attention of v's query over the first P + n logical
positions of the committed cache (torch SDPA on the CPU, float64) must equal
the oracle's tree-attention row of v before the commit (SpecInfer's
equivalence of tree attention and incremental decoding, [survey, Timeline]);
every other logical position must keep its old K/V.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.commit import PAGE
from workloads import chain_tree, random_tree, make_attention_inputs
from workloads.inputs import repage


def _logical(k_pages, v_pages, inp, r, L, dtype):
    base = int(inp.page_indptr[r])
    K = oracle.decode_values(k_pages, dtype)
    V = oracle.decode_values(v_pages, dtype)
    Kl = np.stack([K[inp.page_indices[base + t // PAGE], :, t % PAGE, :] for t in range(L)])
    Vl = np.stack([V[inp.page_indices[base + t // PAGE], :, :, t % PAGE] for t in range(L)])
    return Kl, Vl  # [L][Hkv][D]


def _root_path(parent, v):
    path = [v]
    while parent[path[-1]] >= 0:
        path.append(int(parent[path[-1]]))
    return sorted(path)


def _case(seed, dtype="fp32", B=3, N=24, Hq=4, Hkv=2, D=32):
    g = np.random.default_rng(seed)
    trees = [random_tree(g, N, depth_cap=6) for _ in range(B)]
    prefixes = [int(x) for x in g.integers(5, 60, size=B)]  # not page aligned
    inp = make_attention_inputs(g, g, trees, prefixes, Hq, Hkv, D, dtype=dtype)
    ends = [int(g.integers(0, N)) for _ in range(B)]
    paths = [_root_path(t, v) for t, v in zip(trees, ends)]
    W = max(len(p) for p in paths) + 2
    kv_keep = np.full((B, W), -1, dtype=np.int32)
    out_len = np.zeros(B, dtype=np.int32)
    for r, path in enumerate(paths):
        kv_keep[r, :len(path)] = prefixes[r] + np.asarray(path)
        out_len[r] = len(path)
    return inp, ends, kv_keep, out_len


def _decode(q_heads, Kl, Vl, G, scale):
    """q_heads [Hq][D]; Kl, Vl [L][Hkv][D] -> [Hq][D] by SDPA per kv head."""
    Hq = q_heads.shape[0]
    out = np.zeros_like(q_heads)
    for h in range(Hq):
        g = h // G
        q = torch.from_numpy(q_heads[h][None, None, None])
        k = torch.from_numpy(np.ascontiguousarray(Kl[:, g, :]))[None, None]
        v = torch.from_numpy(np.ascontiguousarray(Vl[:, g, :]))[None, None]
        out[h] = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale)[0, 0, 0].numpy()
    return out


def _check_commit(inp, ends, kv_keep, out_len, commit=oracle.kv_commit_layer):
    k_new, v_new = commit(inp.k_pages, inp.v_pages, inp.page_indptr, inp.page_indices,
                          inp.prefix_len, kv_keep, out_len)
    Q = oracle.decode_values(inp.q, inp.dtype)
    G = inp.num_q_heads // inp.num_kv_heads
    worst = 0.0
    for r, v in enumerate(ends):
        P, n, L = int(inp.prefix_len[r]), int(out_len[r]), inp.kv_len(r)
        K0, V0 = _logical(inp.k_pages, inp.v_pages, inp, r, L, inp.dtype)
        K1, V1 = _logical(k_new, v_new, inp, r, L, inp.dtype)
        # positions outside the committed run keep their K/V
        keep = np.r_[0:P, P + n:L]
        assert np.array_equal(K0[keep], K1[keep]) and np.array_equal(V0[keep], V1[keep])
        a = int(inp.node_indptr[r])
        dec = _decode(Q[a + v], K1[:P + n], V1[:P + n], G, inp.sm_scale)
        tree_row = oracle.tree_attention_rows(inp, [(r, v)])[0]
        worst = max(worst, float(np.abs(dec - tree_row).max()))
    assert worst < 1e-12, worst
    return worst


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_commit_then_decode_equals_tree_row(seed, dtype):
    inp, ends, kv_keep, out_len = _case(seed, dtype)
    _check_commit(inp, ends, kv_keep, out_len)


def test_planted_destination_shift_is_caught():
    """A commit that writes the path one slot too far must fail the pin."""
    def shifted(k_pages, v_pages, page_indptr, page_indices, prefix_len, kv_keep, out_len):
        k_new, v_new = k_pages.copy(), v_pages.copy()
        for r in range(len(prefix_len)):
            base, P = int(page_indptr[r]), int(prefix_len[r])
            for j in range(int(out_len[r])):
                s, d = int(kv_keep[r][j]), P + j + 1
                ps, ss = int(page_indices[base + s // PAGE]), s % PAGE
                pd, sd = int(page_indices[base + d // PAGE]), d % PAGE
                k_new[pd, :, sd, :] = k_pages[ps, :, ss, :]
                v_new[pd, :, :, sd] = v_pages[ps, :, :, ss]
        return k_new, v_new
    inp, ends, kv_keep, out_len = _case(5, N=12)
    with pytest.raises(AssertionError):
        _check_commit(inp, ends, kv_keep, out_len, commit=shifted)


def test_planted_v_layout_mistake_is_caught():
    """Reading V pages as if they were laid out like K ([g][slot][d]) must
    fail the pin."""
    def wrong_v(k_pages, v_pages, page_indptr, page_indices, prefix_len, kv_keep, out_len):
        k_new, v_new = oracle.kv_commit_layer(k_pages, v_pages, page_indptr, page_indices,
                                              prefix_len, kv_keep, out_len)
        Hkv, D = v_pages.shape[1], v_pages.shape[2]
        for r in range(len(prefix_len)):
            base, P = int(page_indptr[r]), int(prefix_len[r])
            for j in range(int(out_len[r])):
                s, d = int(kv_keep[r][j]), P + j
                if s == d:
                    continue
                ps, ss = int(page_indices[base + s // PAGE]), s % PAGE
                pd, sd = int(page_indices[base + d // PAGE]), d % PAGE
                v_new[pd, :, :, sd] = v_pages[ps].reshape(Hkv, PAGE, D)[:, ss, :]
        return k_new, v_new
    inp, ends, kv_keep, out_len = _case(6, N=12)
    with pytest.raises(AssertionError):
        _check_commit(inp, ends, kv_keep, out_len, commit=wrong_v)


def test_chain_fully_accepted_and_root_only_are_identity():
    g = np.random.default_rng(3)
    inp = make_attention_inputs(g, g, [chain_tree(8), random_tree(g, 10, depth_cap=4)],
                                [33, 16], 4, 2, 16, dtype="fp32")
    kv_keep = np.array([[33 + j for j in range(8)], [16] + [-1] * 7], dtype=np.int32)
    out_len = np.array([8, 1], dtype=np.int32)
    k_new, v_new = oracle.kv_commit_layer(inp.k_pages, inp.v_pages, inp.page_indptr,
                                          inp.page_indices, inp.prefix_len, kv_keep, out_len)
    assert np.array_equal(k_new, inp.k_pages) and np.array_equal(v_new, inp.v_pages)


def test_skipped_requests_and_page_placement_invariance():
    inp, ends, kv_keep, out_len = _case(7)
    out_len[1] = 0  # skipped
    g = np.random.default_rng(11)
    moved = repage(inp, g, spare_pages=3)
    a = oracle.kv_commit_layer(inp.k_pages, inp.v_pages, inp.page_indptr, inp.page_indices,
                               inp.prefix_len, kv_keep, out_len)
    b = oracle.kv_commit_layer(moved.k_pages, moved.v_pages, moved.page_indptr,
                               moved.page_indices, moved.prefix_len, kv_keep, out_len)
    for r in range(inp.batch):
        L = inp.kv_len(r)
        Ka, Va = _logical(a[0], a[1], inp, r, L, inp.dtype)
        Kb, Vb = _logical(b[0], b[1], moved, r, L, moved.dtype)
        assert np.array_equal(Ka, Kb) and np.array_equal(Va, Vb)
    K0, V0 = _logical(inp.k_pages, inp.v_pages, inp, 1, inp.kv_len(1), inp.dtype)
    K1, V1 = _logical(a[0], a[1], inp, 1, inp.kv_len(1), inp.dtype)
    assert np.array_equal(K0, K1) and np.array_equal(V0, V1)


def test_bad_keep_lists_raise():
    inp, ends, kv_keep, out_len = _case(8)
    for mutate in ("root", "order", "past"):
        kk = kv_keep.copy()
        r = int(np.argmax(out_len))
        n = int(out_len[r])
        if mutate == "root":
            kk[r, 0] += 1
        elif mutate == "order":
            if n < 3:
                continue
            kk[r, 1], kk[r, 2] = kk[r, 2], kk[r, 1]
        else:
            kk[r, n - 1] = (int(inp.page_indptr[r + 1]) - int(inp.page_indptr[r])) * PAGE
        with pytest.raises(oracle.BadKeepList):
            oracle.kv_commit_layer(inp.k_pages, inp.v_pages, inp.page_indptr, inp.page_indices,
                                   inp.prefix_len, kk, out_len)


def test_multi_layer_commit_is_per_layer():
    inp, ends, kv_keep, out_len = _case(9, B=2, N=10)
    k2 = np.stack([inp.k_pages, inp.k_pages[::-1].copy()])
    v2 = np.stack([inp.v_pages, inp.v_pages[::-1].copy()])
    ko, vo = oracle.kv_commit(k2, v2, inp.page_indptr, inp.page_indices, inp.prefix_len,
                              kv_keep, out_len)
    for layer in range(2):
        a = oracle.kv_commit_layer(k2[layer], v2[layer], inp.page_indptr, inp.page_indices,
                                   inp.prefix_len, kv_keep, out_len)
        assert np.array_equal(ko[layer], a[0]) and np.array_equal(vo[layer], a[1])
