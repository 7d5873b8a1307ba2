"""Run the HIP path through the C ABI on generated inputs (GPU tests only)."""
import numpy as np


def run_attention(inp, repeat=1, sm_scale=0.0):
    import torch
    import tree_verification_verify_amd as tv
    from workloads.device import attention_tensors
    t = attention_tensors(inp)
    desc = tv.attn_desc(inp.batch, inp.num_q_heads, inp.num_kv_heads, inp.head_dim,
                        max(1, inp.max_nodes), inp.max_depth, max(inp.max_kv_len, inp.max_nodes),
                        inp.num_pages, inp.dtype, sm_scale)
    ws = tv.alloc_workspace(tv.attn_workspace_size(desc))
    outs = []
    for _ in range(repeat):
        out = torch.full_like(t["q"], float("nan"))
        tv.tree_verify_attn(desc, t["q"], t["k_pages"], t["v_pages"], t["page_indptr"],
                            t["page_indices"], t["prefix_len"], t["node_indptr"],
                            t["parent"], out, ws)
        outs.append(out)
    st, bits = tv.device_status(ws)
    res = [o.float().cpu().numpy().astype(np.float64) for o in outs]
    return (res if repeat > 1 else res[0]), st, bits


def run_sampler(inp, max_depth=None, prefix_lens=None, ws=None, replacement=False, greedy_path=False):
    """ws: a workspace to reuse (sized for at least this batch); a fresh
    zero-filled one when None. replacement: the with-replacement rule;
    greedy_path: greedy requests read only the rows their walk visits."""
    import torch
    import tree_verification_verify_amd as tv
    from workloads.device import sampler_tensors
    t = sampler_tensors(inp)
    md = max_depth if max_depth is not None else inp.max_nodes
    desc = tv.sample_desc(inp.batch, inp.vocab, inp.max_nodes, md, replacement=replacement,
                          greedy_path=greedy_path)
    if ws is None:
        ws = tv.alloc_workspace(tv.sample_workspace_size(desc))
    else:
        assert ws.numel() >= tv.sample_workspace_size(desc)
    T = int(inp.node_indptr[-1])
    flag = torch.full((T,), -7, dtype=torch.int8, device="cuda")
    nt = torch.full((T,), -7, dtype=torch.int32, device="cuda")
    tv.tree_spec_sample(desc, t["target_logits"], t["draft_logits"], t["tokens"],
                        t["node_indptr"], t["parent"], t["temperature"], t["uniforms"],
                        flag, nt, ws)
    B, W = inp.batch, md + 1
    pn = torch.empty(B * W, dtype=torch.int32, device="cuda")
    ot = torch.empty_like(pn)
    kk = torch.empty_like(pn)
    ol = torch.empty(B, dtype=torch.int32, device="cuda")
    if prefix_lens is None:
        prefix_lens = [0] * B
    prefix = torch.tensor(prefix_lens, dtype=torch.int32, device="cuda")
    tv.tree_accept_path(B, md, t["node_indptr"], t["parent"], t["tokens"], flag, nt, prefix,
                        pn, ot, ol, kk, ws)
    st, bits = tv.device_status(ws)
    return dict(flag=flag.cpu().numpy(), next_token=nt.cpu().numpy(),
                path_nodes=pn.cpu().numpy().reshape(B, W), out_tokens=ot.cpu().numpy().reshape(B, W),
                out_len=ol.cpu().numpy(), kv_keep=kk.cpu().numpy().reshape(B, W),
                status=st, bits=bits, max_depth=md)


def run_construct(root, rows, k, m, num_rounds=None, bad_frontier=None, split=True):
    """EAGLE-2 construction on the GPU: rounds of tree_expand_step, then
    tree_rerank. root [B][V], rows [B][R-1][k][V] (numpy fp32). split: give
    tree_expand_step the workspace with which it splits rounds of few rows."""
    import torch
    import tree_verification_verify_amd as tv
    B, V = root.shape
    R = rows.shape[1] + 1 if num_rounds is None else num_rounds
    cap = k + (R - 1) * k * k
    ws = tv.alloc_workspace(tv.expand_workspace_size(B, k, k) if split else 256)
    cv = torch.full((B, cap), float("nan"), dtype=torch.float32, device="cuda")
    ct = torch.full((B, cap), -7, dtype=torch.int32, device="cuda")
    cp = torch.full((B, cap), -7, dtype=torch.int32, device="cuda")
    frontiers = []
    nxt = torch.full((B, k), -7, dtype=torch.int32, device="cuda")
    tv.tree_expand_step(torch.from_numpy(root).cuda().view(B, 1, V), None, 0, cv, ct, cp, nxt, ws)
    frontiers.append(nxt)
    off = k
    for d in range(R - 1):
        fr = frontiers[-1]
        if bad_frontier is not None and d == 0:
            fr = fr.clone()
            fr[0, 0] = bad_frontier
        nxt = torch.full((B, k), -7, dtype=torch.int32, device="cuda")
        tv.tree_expand_step(torch.from_numpy(np.ascontiguousarray(rows[:, d])).cuda(), fr, off,
                            cv, ct, cp, nxt, ws)
        frontiers.append(nxt)
        off += k * k
    op = torch.full((B, m + 1), -7, dtype=torch.int32, device="cuda")
    ot = torch.full_like(op, -7)
    oc = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    tv.tree_rerank(off, m, cv, ct, cp, op, ot, oc, ws)
    st, bits = tv.device_status(ws)
    return dict(value=cv.cpu().numpy(), token=ct.cpu().numpy(), parent=cp.cpu().numpy(),
                frontiers=[f.cpu().numpy() for f in frontiers], out_parent=op.cpu().numpy(),
                out_token=ot.cpu().numpy(), out_count=oc.cpu().numpy(), status=st, bits=bits,
                num_cand=off)


def run_spark(inp, N, K, stream_id=0, seed=0, ws=None, repeat=1, a=0.67, b=-0.46):
    """TreeSpark construction on the GPU; returns dict of numpy outputs."""
    import torch
    import tree_verification_verify_amd as tv
    dev = "cuda"
    B = inp.batch
    desc = tv.spark_desc(B, inp.vocab, inp.rank, inp.depths, N, K, a, b)
    if ws is None:
        ws = tv.alloc_workspace(tv.spark_workspace_size(desc))
    U = torch.from_numpy(np.ascontiguousarray(inp.base_logits)).to(dev)
    w1 = torch.from_numpy(inp.w1.view(np.int16)).to(dev).view(torch.bfloat16)
    w2 = torch.from_numpy(inp.w2.view(np.int16)).to(dev).view(torch.bfloat16)
    anchor = torch.from_numpy(inp.anchor).to(dev)
    temp = torch.from_numpy(inp.temperature).to(dev)
    theta = torch.from_numpy(inp.theta).to(dev)
    outs = []
    for _ in range(repeat):
        par = torch.full((B, N + 1), -7, dtype=torch.int32, device=dev)
        tok = torch.full_like(par, -7)
        cnt = torch.full((B,), -7, dtype=torch.int32, device=dev)
        logs = torch.full((B, N + 1), float("nan"), dtype=torch.float32, device=dev)
        tv.tree_spark_build(desc, U, w1, w2, anchor, temp, theta, par, tok, cnt, ws,
                            out_logsurv=logs, stream_id=stream_id, seed=seed)
        outs.append(dict(parent=par.cpu().numpy(), token=tok.cpu().numpy(),
                         count=cnt.cpu().numpy(), logS=logs.cpu().numpy()))
    st, bits = tv.device_status(ws)
    res = outs if repeat > 1 else outs[0]
    return res, st, bits
