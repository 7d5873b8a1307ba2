"""GPU parity: tree_kv_commit (HIP, via the C ABI) against the oracle's commit.

The commit moves bytes only, so the comparison is bit-exact over the whole
page pools of every layer (untouched positions included).
"""
import numpy as np
import pytest

import oracle
from workloads import make_config, make_attention_inputs, random_tree, chain_tree

pytestmark = pytest.mark.gpu


def _root_path(parent, v):
    path = [v]
    while parent[path[-1]] >= 0:
        path.append(int(parent[path[-1]]))
    return sorted(path)


def _keep_lists(inp, trees, rng, W=None, special=None):
    B = inp.batch
    paths = []
    for r, t in enumerate(trees):
        v = int(rng.integers(0, len(t)))
        # end at the deepest node sometimes, so long paths occur
        if rng.random() < 0.5:
            d = oracle.depths(np.asarray(t))
            v = int(np.argmax(d))
        paths.append(_root_path(t, v))
    W = W or max(len(p) for p in paths) + 1
    kv_keep = np.full((B, W), -1, dtype=np.int32)
    out_len = np.zeros(B, dtype=np.int32)
    for r, p in enumerate(paths):
        kv_keep[r, :len(p)] = int(inp.prefix_len[r]) + np.asarray(p)
        out_len[r] = len(p)
    if special:
        special(kv_keep, out_len)
    return kv_keep, out_len, W


def _layers(inp, L, rng, stride_pad=0):
    """[L] copies of the pools with different contents (+ stride padding)."""
    def noise(a):
        if inp.dtype == "bf16":
            return rng.integers(0, 1 << 16, size=a.shape, dtype=np.uint16) & 0x7f7f
        return rng.standard_normal(a.shape).astype(np.float32)
    ks = [inp.k_pages] + [noise(inp.k_pages) for _ in range(L - 1)]
    vs = [inp.v_pages] + [noise(inp.v_pages) for _ in range(L - 1)]
    return np.stack(ks), np.stack(vs)


def _run(inp, k_layers, v_layers, kv_keep, out_len, max_depth, stride_pad=0):
    import torch
    import tree_verification_verify_amd as tv
    from workloads.device import attention_tensors
    t = attention_tensors(inp)
    L = k_layers.shape[0]
    per = int(np.prod(k_layers.shape[1:]))
    tdt = torch.bfloat16 if inp.dtype == "bf16" else torch.float32
    ndt = np.int16 if inp.dtype == "bf16" else np.float32

    def dev(a):
        flat = np.zeros(L * (per + stride_pad), dtype=a.dtype)
        for layer in range(L):
            flat[layer * (per + stride_pad): layer * (per + stride_pad) + per] = a[layer].ravel()
        return torch.from_numpy(flat.view(ndt)).to("cuda").view(tdt)

    kd, vd = dev(k_layers), dev(v_layers)
    desc = tv.attn_desc(inp.batch, inp.num_q_heads, inp.num_kv_heads, inp.head_dim,
                        inp.max_nodes, inp.max_depth, inp.max_kv_len, inp.num_pages, inp.dtype)
    ws = tv.alloc_workspace(4096)
    keep_d = torch.from_numpy(kv_keep).to("cuda")
    len_d = torch.from_numpy(out_len).to("cuda")
    tv.tree_kv_commit(desc, kd, vd, t["page_indptr"], t["page_indices"], t["prefix_len"], keep_d,
                      len_d, max_depth, num_layers=L, layer_stride=per + stride_pad,
                      status_workspace=ws)
    st, bits = tv.device_status(ws)

    def host(d):
        a = d.view(torch.int16 if inp.dtype == "bf16" else torch.float32).cpu().numpy()
        a = a.view(k_layers.dtype)
        return np.stack([a[layer * (per + stride_pad): layer * (per + stride_pad) + per]
                         for layer in range(L)])
    return host(kd).reshape(k_layers.shape), host(vd).reshape(v_layers.shape), st, bits


def _compare(inp, k_layers, v_layers, kv_keep, out_len, max_depth, stride_pad=0):
    kg, vg, st, bits = _run(inp, k_layers, v_layers, kv_keep, out_len, max_depth, stride_pad)
    assert st == 0, bits
    ko, vo = oracle.kv_commit(k_layers, v_layers, inp.page_indptr, inp.page_indices,
                              inp.prefix_len, kv_keep, out_len)
    assert np.array_equal(kg.view(np.uint8), ko.view(np.uint8))
    assert np.array_equal(vg.view(np.uint8), vo.view(np.uint8))


def test_highload_shape_three_layers():
    cfg = make_config("highload", sampler=False)
    rng = np.random.default_rng(0)
    kv_keep, out_len, W = _keep_lists(cfg.attn, cfg.trees, rng, W=17)
    k, v = _layers(cfg.attn, 3, rng)
    _compare(cfg.attn, k, v, kv_keep, out_len, W - 1)


@pytest.mark.parametrize("dtype,D", [("fp32", 64), ("bf16", 64), ("fp32", 128)])
def test_dtypes_head_dims_and_layer_stride(dtype, D):
    rng = np.random.default_rng(1)
    trees = [random_tree(rng, int(n), depth_cap=8) for n in rng.integers(2, 40, size=9)]
    prefixes = [int(x) for x in rng.integers(0, 300, size=9)]
    inp = make_attention_inputs(rng, rng, trees, prefixes, 8, 2, D, dtype=dtype, spare_pages=5)
    kv_keep, out_len, W = _keep_lists(inp, trees, rng)
    k, v = _layers(inp, 2, rng)
    _compare(inp, k, v, kv_keep, out_len, W - 1, stride_pad=64)


def test_long_paths_span_several_chunks():
    rng = np.random.default_rng(2)
    trees = [random_tree(rng, 300, depth_cap=90, spine_depth=90) for _ in range(3)]
    inp = make_attention_inputs(rng, rng, trees, [7, 64, 1000], 4, 1, 128, dtype="bf16")
    kv_keep, out_len, W = _keep_lists(inp, trees, rng)
    assert out_len.max() > 64
    k, v = _layers(inp, 2, rng)
    _compare(inp, k, v, kv_keep, out_len, W - 1)


def test_skipped_root_only_and_in_place_requests():
    rng = np.random.default_rng(3)
    trees = [chain_tree(8), random_tree(rng, 20, depth_cap=5), random_tree(rng, 20, depth_cap=5),
             chain_tree(40)]
    inp = make_attention_inputs(rng, rng, trees, [16, 33, 0, 5], 4, 2, 128, dtype="bf16")

    def special(kv_keep, out_len):
        kv_keep[0, :8] = 16 + np.arange(8)       # fully accepted chain: nothing moves
        out_len[0] = 8
        out_len[1] = 0                            # skipped
        kv_keep[2, 0] = 0                         # root only
        out_len[2] = 1
        kv_keep[3, :40] = 5 + np.arange(40)       # chain longer than one chunk
        out_len[3] = 40
    kv_keep, out_len, W = _keep_lists(inp, trees, rng, W=41, special=special)
    k, v = _layers(inp, 2, rng)
    _compare(inp, k, v, kv_keep, out_len, W - 1)


@pytest.mark.parametrize("mutation,bit", [("root", 8), ("order", 8), ("past", 8), ("length", 32)])
def test_bad_keep_lists_are_reported_and_untouched(mutation, bit):
    rng = np.random.default_rng(4)
    trees = [random_tree(rng, 24, depth_cap=6) for _ in range(4)]
    inp = make_attention_inputs(rng, rng, trees, [10, 20, 30, 40], 4, 2, 64, dtype="bf16")
    kv_keep, out_len, W = _keep_lists(inp, trees, rng, W=10)
    r = int(np.argmax(out_len))
    n = int(out_len[r])
    bad_k, bad_o = kv_keep.copy(), out_len.copy()
    if mutation == "root":
        bad_k[r, 0] += 1
    elif mutation == "order":
        bad_k[r, n - 1] = bad_k[r, n - 2]
    elif mutation == "past":
        bad_k[r, n - 1] = (int(inp.page_indptr[r + 1]) - int(inp.page_indptr[r])) * 16
    else:
        bad_o[r] = W + 1
    k, v = _layers(inp, 1, rng)
    kg, vg, st, bits = _run(inp, k, v, bad_k, bad_o, W - 1)
    assert bits & bit
    # the bad request is untouched, the others are committed
    good_o = bad_o.copy()
    good_o[r] = 0
    ko, vo = oracle.kv_commit(k, v, inp.page_indptr, inp.page_indices, inp.prefix_len,
                              kv_keep, good_o)
    assert np.array_equal(kg.view(np.uint8), ko.view(np.uint8))
    assert np.array_equal(vg.view(np.uint8), vo.view(np.uint8))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_attend_commit_then_decode_matches_tree_row(dtype):
    """End to end on the GPU: tree attention over a tree, commit of a root
    path's K/V, then a one-row tree at the committed position (prefix
    P + n - 1, the row's own key at P + n - 1) must give the tree row of the
    path's last node (SpecInfer's equivalence; [survey, Timeline])."""
    import torch
    import tree_verification_verify_amd as tv
    from workloads.device import attention_tensors
    from workloads.inputs import AttentionInputs
    from gpu_run import run_attention
    rng = np.random.default_rng(11)
    trees = [random_tree(rng, int(n), depth_cap=7) for n in rng.integers(8, 33, size=6)]
    prefixes = [int(x) for x in rng.integers(200, 900, size=6)]
    D = 128 if dtype == "bf16" else 64
    inp = make_attention_inputs(rng, rng, trees, prefixes, 8, 2, D, dtype=dtype)
    kv_keep, out_len, W = _keep_lists(inp, trees, rng)
    ends = []
    for r in range(inp.batch):
        n = int(out_len[r])
        ends.append(int(kv_keep[r, n - 1]) - prefixes[r])
    tree_out, st, _ = run_attention(inp)
    assert st == 0
    # commit on the GPU (one layer: the pools themselves)
    t = attention_tensors(inp)
    desc = tv.attn_desc(inp.batch, inp.num_q_heads, inp.num_kv_heads, inp.head_dim,
                        inp.max_nodes, inp.max_depth, inp.max_kv_len, inp.num_pages, dtype)
    ws = tv.alloc_workspace(4096)
    tv.tree_kv_commit(desc, t["k_pages"], t["v_pages"], t["page_indptr"], t["page_indices"],
                      t["prefix_len"], torch.from_numpy(kv_keep).cuda(),
                      torch.from_numpy(out_len).cuda(), W - 1, num_layers=1, status_workspace=ws)
    assert tv.device_status(ws)[0] == 0
    bits = (lambda x: x.view(torch.int16).cpu().numpy().view(np.uint16)) if dtype == "bf16" else \
        (lambda x: x.cpu().numpy())
    k_new, v_new = bits(t["k_pages"]), bits(t["v_pages"])
    # one-row trees at P + n - 1 with the queries of the paths' last nodes
    q_rows = np.stack([inp.q[int(inp.node_indptr[r]) + ends[r]] for r in range(inp.batch)])
    one = AttentionInputs(
        dtype=dtype, num_q_heads=inp.num_q_heads, num_kv_heads=inp.num_kv_heads, head_dim=D,
        q=q_rows, k_pages=k_new, v_pages=v_new, page_indptr=inp.page_indptr,
        page_indices=inp.page_indices,
        prefix_len=np.array([prefixes[r] + int(out_len[r]) - 1 for r in range(inp.batch)],
                            dtype=np.int32),
        node_indptr=np.arange(inp.batch + 1, dtype=np.int32),
        parent=np.full(inp.batch, -1, dtype=np.int32), sm_scale=inp.sm_scale)
    dec_out, st, _ = run_attention(one)
    assert st == 0
    tol = 2e-2 if dtype == "bf16" else 1e-5
    ref = oracle.tree_attention_rows(inp, [(r, ends[r]) for r in range(inp.batch)])
    for r in range(inp.batch):
        assert np.abs(dec_out[r] - ref[r]).max() <= tol
        assert np.abs(tree_out[int(inp.node_indptr[r]) + ends[r]] - ref[r]).max() <= tol


def test_walk_path_commit_on_the_gpu_matches_the_oracle():
    """The next-step chain on the GPU: sampling walk and accepted path on a
    highload sub-batch, then the commit of the GPU's own keep-lists over two
    layers; the keep-lists equal the oracle's and the pools are bit-exact
    with the oracle's commit."""
    import torch
    import tree_verification_verify_amd as tv
    from workloads.device import sampler_tensors
    cfg = make_config("highload", batch=12, vocab=4096)
    s, inp = cfg.sampler, cfg.attn
    st = sampler_tensors(s)
    md = 16
    sdesc = tv.sample_desc(s.batch, s.vocab, s.max_nodes, md)
    sws = tv.alloc_workspace(tv.sample_workspace_size(sdesc))
    T = int(s.node_indptr[-1])
    flag = torch.empty(T, dtype=torch.int8, device="cuda")
    nt = torch.empty(T, dtype=torch.int32, device="cuda")
    tv.tree_spec_sample(sdesc, st["target_logits"], st["draft_logits"], st["tokens"],
                        st["node_indptr"], st["parent"], st["temperature"], st["uniforms"],
                        flag, nt, sws)
    B = s.batch
    pn = torch.empty(B * (md + 1), dtype=torch.int32, device="cuda")
    ot, kk = torch.empty_like(pn), torch.empty_like(pn)
    ol = torch.empty(B, dtype=torch.int32, device="cuda")
    prefix = torch.from_numpy(np.asarray(inp.prefix_len, dtype=np.int32)).cuda()
    tv.tree_accept_path(B, md, st["node_indptr"], st["parent"], st["tokens"], flag, nt, prefix,
                        pn, ot, ol, kk, sws)
    assert tv.device_status(sws)[0] == 0
    keep = kk.cpu().numpy().reshape(B, md + 1)
    olen = ol.cpu().numpy()
    rf, rn, logs = oracle.tree_spec_sample(s)
    _, _, rol, rkeep = oracle.tree_accept_path(s.node_indptr, s.parent, s.tokens, rf, rn,
                                               cfg.prefix_lens, md)
    # requests whose walk met a near-threshold decision may differ; none expected here
    assert np.array_equal(olen, rol) and np.array_equal(keep, rkeep)
    rng = np.random.default_rng(21)
    k, v = _layers(inp, 2, rng)
    _compare(inp, k, v, keep, olen, md)
