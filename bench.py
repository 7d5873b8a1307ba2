"""Tree-verification benchmark on one MI355X.

One step = one pass of the whole hot path over one batch:
  tree_verify_attn (one attention layer, every tree row of every request)
  -> tree_spec_sample (greedy / rejection walk without or with replacement; greedy
     requests read only the rows their walk visits unless --greedy every)
  -> tree_accept_path (longest accepted path, emitted tokens, KV keep-list).
Workload (default): "highload" — 64 requests, prefixes U{512..8192}, per-request
budget from {8-row chain, 16-row tree, 32-row tree}, 32 q / 8 kv heads, D 128,
bf16 paged KV; sampler over V = 151936 with per-request T in {0, 0.5, 1}.
Inputs are synthetic, seeded, and resident in HBM before timing starts.

Prints ONE JSON line: value = tree nodes verified per second (whole step),
plus the attention kernel's roofline and the CPU oracle's rate on a sample.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "tree-verify nodes/s per layer + achieved HBM GB/s (% of MI355X peak), 1 GPU"
HBM_PEAK_GBS = 8000.0
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "tree_verify_attn_highload_counters.md")
ATTN_SOURCE = os.path.join(ROOT, "tree_verification_verify_amd", "csrc", "tree_attn.hip")


def attn_algorithmic_bytes(inp):
    """KV read once per kv head + Q in + O out (bf16: 2 bytes/element)."""
    s = 2 if inp.dtype == "bf16" else 4
    total = 0
    for r in range(inp.batch):
        L = inp.kv_len(r)
        N = inp.nodes(r)
        total += L * inp.num_kv_heads * inp.head_dim * 2 * s
        total += 2 * N * inp.num_q_heads * inp.head_dim * s
    return total


def attn_algorithmic_flops(cfg):
    import oracle
    inp = cfg.attn
    f = 0
    for r, parent in enumerate(cfg.trees):
        d = oracle.depths(parent)
        P = int(inp.prefix_len[r])
        f += sum(4 * inp.num_q_heads * inp.head_dim * (P + int(di) + 1) for di in d)
    return f


def sampler_algorithmic_bytes(sinp, out_len, greedy_path=False):
    """Rows the walk must read: at T = 0 every target row (the every-node
    form) or the target row of each visited node (the walk-only form); the
    target and draft row of each visited node at T > 0."""
    V = sinp.vocab
    total = 0
    for r in range(sinp.batch):
        n = int(sinp.node_indptr[r + 1] - sinp.node_indptr[r])
        if float(sinp.temperature[r]) == 0.0:
            total += (int(out_len[r]) if greedy_path else n) * V * 4
        else:
            total += int(out_len[r]) * V * 4 * 2
    return total


def read_traffic():
    """HBM bytes per attention launch from the committed counter summary,
    or None when the kernel source changed since the counters were taken."""
    if not os.path.exists(PROFILE_COUNTERS):
        return None
    text = open(PROFILE_COUNTERS).read()
    m_sha = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_sha or not m_b:
        return None
    sha = hashlib.sha256(open(ATTN_SOURCE, "rb").read()).hexdigest()
    if sha != m_sha.group(1):
        return None
    return float(m_b.group(1))


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, budget_s=12.0, replacement=False, requests=32, repeats=3, greedy_path=False):
    """The oracle as it stands (fp64 NumPy attention + sampling walk + path)
    on a fixed sample of the workload's requests (the first `requests`),
    timed with perf_counter, median of `repeats` runs, once with the BLAS
    pools limited to every core in this process's affinity set and once
    with one thread. Returns nodes/s of the all-core run, with the one-thread
    figure, the CPU model and every run's time beside it."""
    import oracle
    from workloads.inputs import SamplerInputs
    from threadpoolctl import threadpool_limits
    inp, s = cfg.attn, cfg.sampler
    sample = list(range(min(requests, inp.batch)))
    nodes = sum(inp.nodes(r) for r in sample)

    def run():
        t0 = time.perf_counter()
        for r in sample:
            n = inp.nodes(r)
            oracle.tree_attention_rows(inp, [(r, i) for i in range(n)])
            a, b = int(s.node_indptr[r]), int(s.node_indptr[r + 1])
            one = SamplerInputs(vocab=s.vocab, target_logits=s.target_logits[a:b],
                                draft_logits=None if s.draft_logits is None else s.draft_logits[a:b],
                                tokens=s.tokens[a:b], node_indptr=np.array([0, b - a], np.int32),
                                parent=s.parent[a:b], temperature=s.temperature[r:r + 1],
                                uniforms=s.uniforms[a:b])
            f, nt, _ = oracle.tree_spec_sample(one, replacement=replacement, greedy_path=greedy_path)
            oracle.tree_accept_path(one.node_indptr, one.parent, one.tokens, f, nt,
                                    [int(inp.prefix_len[r])], 16)
        return time.perf_counter() - t0

    cores = len(os.sched_getaffinity(0))
    times = {}
    for label, limit in (("all", cores), ("one", 1)):
        with threadpool_limits(limits=limit):
            times[label] = [run() for _ in range(repeats)]
    med = {k: float(np.median(v)) for k, v in times.items()}
    return {"value": nodes / med["all"], "unit": "nodes/s", "cores": cores, "kind": "oracle",
            "sample": f"first {len(sample)} of {inp.batch} requests ({nodes} tree rows): fp64 "
                      f"NumPy attention + sampling walk + path; median of {repeats} runs",
            "cpu_model": _cpu_model(), "one_thread_value": nodes / med["one"],
            "runs_s": {k: [round(x, 3) for x in v] for k, v in times.items()}}


def attn_sweep(names, rotate_bytes, reps):
    """Attention alone on each named workload, launched back to back over
    distinct copies of Q, K/V pages and outputs totalling >= rotate_bytes, so
    the 256 MB Infinity Cache cannot serve a small layer from an earlier
    launch. The launches of one pass over the copies are captured in one HIP
    graph (host launch cost out of the way) and replayed `reps` times; the
    output of the first copy is checked against an eager call after the
    replays. Prints one JSON line per workload."""
    import ctypes
    import torch
    import tree_verification_verify_amd as tv
    from tree_verification_verify_amd import _lib
    from workloads import make_config
    from workloads.device import attention_tensors
    lib = _lib.load()
    stream = torch.cuda.Stream()
    for name in names:
        cfg = make_config(name, sampler=False)
        inp = cfg.attn
        a = attention_tensors(inp, "cuda")
        desc = tv.attn_desc(inp.batch, inp.num_q_heads, inp.num_kv_heads, inp.head_dim,
                            inp.max_nodes, inp.max_depth, inp.max_kv_len, inp.num_pages,
                            inp.dtype)
        abytes = attn_algorithmic_bytes(inp)
        flops = attn_algorithmic_flops(cfg)
        copy_bytes = (a["k_pages"].numel() + a["v_pages"].numel() + 2 * a["q"].numel()) * 2
        n = max(1, -(-rotate_bytes // copy_bytes))
        copies = []
        for i in range(n):
            k = a["k_pages"] if i == 0 else a["k_pages"].clone()
            v = a["v_pages"] if i == 0 else a["v_pages"].clone()
            q = a["q"] if i == 0 else a["q"].clone()
            o = torch.empty_like(q)
            ws = tv.alloc_workspace(tv.attn_workspace_size(desc))
            copies.append((q, k, v, o, ws))
        ref = torch.empty_like(a["q"])
        tv.tree_verify_attn(desc, a["q"], a["k_pages"], a["v_pages"], a["page_indptr"],
                            a["page_indices"], a["prefix_len"], a["node_indptr"], a["parent"],
                            ref, copies[0][4])
        torch.cuda.synchronize()
        P = ctypes.c_void_p
        calls = [(ctypes.byref(desc), P(q.data_ptr()), P(k.data_ptr()), P(v.data_ptr()),
                  P(a["page_indptr"].data_ptr()), P(a["page_indices"].data_ptr()),
                  P(a["prefix_len"].data_ptr()), P(a["node_indptr"].data_ptr()),
                  P(a["parent"].data_ptr()), P(o.data_ptr()), P(ws.data_ptr()), ws.numel())
                 for (q, k, v, o, ws) in copies]
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            for c in calls:  # warm-up outside the graph
                st = lib.tree_verify_attn(*c, P(stream.cuda_stream))
                if st != 0:
                    raise SystemExit(f"{name}: tree_verify_attn returned {st}")
            stream.synchronize()
            with torch.cuda.graph(graph, stream=stream):
                for c in calls:
                    lib.tree_verify_attn(*c, P(stream.cuda_stream))
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):  # replay() launches on the current stream
            graph.replay()
            e0.record(stream)
            for _ in range(reps):
                graph.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        per_us = e0.elapsed_time(e1) * 1e3 / (reps * n)
        err = (copies[0][3].float() - ref.float()).abs().max().item()
        st, bits = tv.device_status(copies[0][4])
        if st != 0 or err != 0.0:
            raise SystemExit(f"{name}: graph replay differs from eager (max {err}) or status {st}/{bits}")
        gbs = abytes / (per_us * 1e-6) / 1e9
        tfl = flops / (per_us * 1e-6) / 1e12
        print(json.dumps({
            "workload": name, "batch": inp.batch, "tree_rows": inp.total_nodes,
            "prefix": [int(inp.prefix_len.min()), int(inp.prefix_len.max())],
            "copies": n, "reps": reps, "us_per_launch": per_us,
            "nodes_per_s": inp.total_nodes / (per_us * 1e-6),
            "algorithmic_bytes": abytes, "hbm_GBs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
            "algorithmic_flops": flops, "tflops": tfl, "mfma_frac_bf16": tfl / 2500.0}),
            flush=True)
        del copies, calls, graph
        torch.cuda.empty_cache()


def commit_bench(layers, reps):
    """tree_kv_commit alone on the highload batch: keep-lists from the real
    sampling walk and path kernels over the same inputs, `layers` distinct
    K/V layer pools, a 1 GiB write before every timed call so the Infinity
    Cache holds none of the pages it touches. Algorithmic bytes: K and V of
    every entry that moves (kv_keep[j] != P + j), read once and written once,
    in every layer and kv head."""
    import torch
    import tree_verification_verify_amd as tv
    from workloads import make_config
    from workloads.device import attention_tensors, sampler_tensors
    cfg = make_config("highload")
    inp, s = cfg.attn, cfg.sampler
    a = attention_tensors(inp, "cuda")
    st = sampler_tensors(s, "cuda")
    md = max(8, inp.max_depth)
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
    tv.tree_accept_path(B, md, st["node_indptr"], st["parent"], st["tokens"], flag, nt,
                        a["prefix_len"], pn, ot, ol, kk, sws)
    del st
    torch.cuda.synchronize()
    keep = kk.cpu().numpy().reshape(B, md + 1)
    olen = ol.cpu().numpy()
    moved = sum(int((keep[r, :olen[r]] != inp.prefix_len[r] + np.arange(olen[r])).sum())
                for r in range(B) if olen[r] > 0)
    D, Hkv = inp.head_dim, inp.num_kv_heads
    abytes = moved * layers * Hkv * D * 2 * 2 * 2
    desc = tv.attn_desc(inp.batch, inp.num_q_heads, Hkv, D, inp.max_nodes, inp.max_depth,
                        inp.max_kv_len, inp.num_pages, inp.dtype)
    shape = (layers,) + tuple(a["k_pages"].shape)
    kp = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    vp = torch.empty((layers,) + tuple(a["v_pages"].shape), dtype=torch.bfloat16, device="cuda")
    ws = tv.alloc_workspace(4096)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    tv.tree_kv_commit(desc, kp, vp, a["page_indptr"], a["page_indices"], a["prefix_len"], kk,
                      ol, md, num_layers=layers, status_workspace=ws)  # checked call
    import ctypes
    from tree_verification_verify_amd import _lib
    lib = _lib.load()
    P_ = ctypes.c_void_p
    args = (ctypes.byref(desc), layers, kp[0].numel(), P_(kp.data_ptr()), P_(vp.data_ptr()),
            P_(a["page_indptr"].data_ptr()), P_(a["page_indices"].data_ptr()),
            P_(a["prefix_len"].data_ptr()), P_(kk.data_ptr()), P_(ol.data_ptr()), md,
            P_(ws.data_ptr()), P_(stream.cuda_stream))

    def call():  # the same call without the binding's Python-side checks
        lib.tree_kv_commit(*args)
    torch.cuda.synchronize()
    status, bits = tv.device_status(ws)
    if status != 0:
        raise SystemExit(f"device status {status} bits {bits}")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for e0, e1 in ev:
        flush.fill_(1)
        e0.record(stream)
        call()
        e1.record(stream)
    torch.cuda.synchronize()
    us = float(np.median([e0.elapsed_time(e1) for e0, e1 in ev])) * 1e3
    # the same calls back to back (keep-lists, page tables and the touched
    # pages warm in the caches and translation buffers): context only
    w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0.record(stream)
    for _ in range(reps):
        call()
    w1.record(stream)
    torch.cuda.synchronize()
    warm_us = w0.elapsed_time(w1) * 1e3 / reps
    gbs = abytes / (us * 1e-6) / 1e9
    print(json.dumps({
        "kernel": "tree_kv_commit (kv_commit_kernel<128, bf16>)",
        "workload": f"highload: {B} requests, keep-lists of the sampled paths "
                    f"(mean out_len {float(olen.mean()):.2f}, {moved} entries move), "
                    f"{layers} layers x {Hkv} kv heads x D {D} bf16",
        "us_per_call_median": us, "reps": reps, "algorithmic_bytes": abytes,
        "us_per_call_back_to_back": warm_us,
        "hbm_GBs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
        "bytes_per_moved_entry_per_layer": Hkv * D * 2 * 2 * 2}), flush=True)


def siblings_bench(reps):
    """tree_draw_siblings alone: every expanded node of the highload trees
    (k = its child count, its request's temperature), draft logits over
    V = 151936 resident in HBM. Algorithmic bytes: each expanded row's draft
    logits read once (the outputs are 64 bytes per row)."""
    import ctypes
    import torch
    import tree_verification_verify_amd as tv
    from tree_verification_verify_amd import _lib
    from workloads import make_config
    cfg = make_config("highload")
    s = cfg.sampler
    rows, counts, temps = [], [], []
    for r in range(s.batch):
        a, b = int(s.node_indptr[r]), int(s.node_indptr[r + 1])
        ch = np.bincount(s.parent[a + 1:b], minlength=b - a)
        for i in np.nonzero(ch)[0]:
            rows.append(a + int(i))
            counts.append(int(ch[i]))
            temps.append(float(s.temperature[r]))
    R, V = len(rows), s.vocab
    logits = torch.from_numpy(np.ascontiguousarray(s.draft_logits[rows])).to("cuda")
    c = torch.tensor(counts, dtype=torch.int32, device="cuda")
    t = torch.tensor(temps, dtype=torch.float32, device="cuda")
    out = torch.empty((R, _lib.MAX_CHILDREN), dtype=torch.int32, device="cuda")
    ws = tv.alloc_workspace(4096)
    tv.tree_draw_siblings(logits, c, t, out, stream_id=1, seed=42, status_workspace=ws)
    torch.cuda.synchronize()
    status, bits = tv.device_status(ws)
    if status != 0:
        raise SystemExit(f"device status {status} bits {bits}")
    lib = _lib.load()
    stream = torch.cuda.current_stream()
    P_ = ctypes.c_void_p
    args = (R, V, P_(logits.data_ptr()), P_(c.data_ptr()), P_(t.data_ptr()), 1, 42,
            P_(out.data_ptr()), P_(ws.data_ptr()), P_(stream.cuda_stream))
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for e0, e1 in ev:
        flush.fill_(1)  # the 256 MB Infinity Cache holds none of the rows
        e0.record(stream)
        lib.tree_draw_siblings(*args)
        e1.record(stream)
    torch.cuda.synchronize()
    us = float(np.median([e0.elapsed_time(e1) for e0, e1 in ev])) * 1e3
    abytes = R * V * 4
    gbs = abytes / (us * 1e-6) / 1e9
    nT = sum(1 for x in temps if x > 0)
    print(json.dumps({
        "kernel": "tree_draw_siblings (draw_siblings_kernel)",
        "workload": f"highload: {R} expanded nodes ({sum(counts)} children, k <= {max(counts)}; "
                    f"{nT} rows at T > 0), V {V} fp32 draft logits",
        "us_per_call_median": us, "reps": reps, "algorithmic_bytes": abytes,
        "hbm_GBs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
        "tokens_per_s": R * V / (us * 1e-6)}), flush=True)


def construct_bench(reps, batch=64, vocab=151936, k=10, rounds=6, m=60):
    """EAGLE-2 construction alone (top-k 10, depth 6, 60 kept nodes, the
    survey's EAGLE-2 setting) for a 64-request batch over V = 151936: the
    first expansion round expands each root row, expansion rounds 2..6 the 10
    frontier rows of every request (synthetic drafter rows resident in HBM),
    then the rerank. Algorithmic bytes of an expansion round: its draft rows
    read once (outputs are a few KB)."""
    import ctypes
    import torch
    import tree_verification_verify_amd as tv
    from tree_verification_verify_amd import _lib
    from workloads import make_construct_inputs
    rng = np.random.default_rng(2024)
    root_np, rows_np = make_construct_inputs(rng, batch, vocab, k, rounds)
    root = torch.from_numpy(root_np).to("cuda")
    rows = [torch.from_numpy(np.ascontiguousarray(rows_np[:, d])).to("cuda")
            for d in range(rounds - 1)]
    del root_np, rows_np
    cap = k + (rounds - 1) * k * k
    cv = torch.empty((batch, cap), dtype=torch.float32, device="cuda")
    ct = torch.empty((batch, cap), dtype=torch.int32, device="cuda")
    cp = torch.empty_like(ct)
    fr = [torch.empty((batch, k), dtype=torch.int32, device="cuda") for _ in range(rounds)]
    op = torch.empty((batch, m + 1), dtype=torch.int32, device="cuda")
    ot = torch.empty_like(op)
    oc = torch.empty(batch, dtype=torch.int32, device="cuda")
    ws = tv.alloc_workspace(tv.expand_workspace_size(batch, k, k))
    nws = ws.numel()
    lib = _lib.load()
    stream = torch.cuda.current_stream()
    P_ = ctypes.c_void_p
    ptr = lambda t: P_(t.data_ptr())
    outs = (ptr(cv), ptr(ct), ptr(cp))
    calls = [lambda: lib.tree_expand_step(batch, vocab, 1, k, ptr(root), None, cap, 0, *outs,
                                          ptr(fr[0]), ptr(ws), nws, P_(stream.cuda_stream))]
    for d in range(rounds - 1):
        calls.append(lambda d=d: lib.tree_expand_step(
            batch, vocab, k, k, ptr(rows[d]), ptr(fr[d]), cap, k + d * k * k, *outs,
            ptr(fr[d + 1]), ptr(ws), nws, P_(stream.cuda_stream)))
    calls.append(lambda: lib.tree_rerank(batch, cap, cap, m, *outs, ptr(op), ptr(ot), ptr(oc),
                                         ptr(ws), P_(stream.cuda_stream)))
    for c in calls:
        assert c() == 0
    torch.cuda.synchronize()
    status, bits = tv.device_status(ws)
    if status != 0:
        raise SystemExit(f"device status {status} bits {bits}")
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
          for _ in range(reps)]
    for e in ev:
        e[0].record(stream)
        for j, c in enumerate(calls):
            c()
            e[j + 1].record(stream)
    torch.cuda.synchronize()
    per = np.median([[e[j].elapsed_time(e[j + 1]) * 1e3 for j in range(len(calls))] for e in ev],
                    axis=0)
    total = float(np.median([e[0].elapsed_time(e[-1]) * 1e3 for e in ev]))
    row_bytes = vocab * 4
    b_root, b_round = batch * row_bytes, batch * k * row_bytes
    abytes = b_root + (rounds - 1) * b_round
    rest = float(np.mean(per[1:rounds]))
    print(json.dumps({
        "kernel": "tree_expand_step x rounds + tree_rerank (expand_kernel<12>, select_kernel, "
                  "rerank_kernel)",
        "workload": f"EAGLE-2 construction: {batch} requests, top-k {k}, depth {rounds}, "
                    f"keep {m}; V {vocab} fp32 synthetic draft rows",
        "us_total_median": total, "reps": reps,
        "us_round1": float(per[0]), "us_round_2_to_%d_mean" % rounds: rest,
        "us_rerank": float(per[-1]), "algorithmic_bytes": abytes,
        "hbm_GBs_total": abytes / (total * 1e-6) / 1e9,
        "hbm_GBs_round": b_round / (rest * 1e-6) / 1e9,
        "hbm_frac_round": b_round / (rest * 1e-6) / 1e9 / HBM_PEAK_GBS,
        "trees_per_s": batch / (total * 1e-6)}), flush=True)


def spark_bench(reps, batch=64, vocab=151936, rank=256, depths=7, N=64, K=8, theta=0.05,
                temps=("mixed",)):
    """TreeSpark's best-first construction alone (tree_spark_build): the pages'
    drafter shape (b = 7, r = 256, V = 151936, K = 8, node cap 64) for a
    64-request batch at theta, with synthetic backbone logits and Markov
    factors resident in HBM. Algorithmic bytes per call: w2 once per round
    (V r 2 B) plus, per expansion, its base-logit row (4 V B) and w1 row;
    the logits row each expansion writes and reads back is not counted."""
    import torch
    import tree_verification_verify_amd as tv
    from workloads import make_spark_inputs
    for tsel in temps:
        rng = np.random.default_rng(4242)
        t = [0.0, 0.5, 1.0] * (batch // 3 + 1) if tsel == "mixed" else [float(tsel)] * batch
        inp = make_spark_inputs(rng, batch, vocab=vocab, depths=depths, rank=rank,
                                temperatures=np.asarray(t[:batch], np.float32), thetas=theta)
        dev = "cuda"
        desc = tv.spark_desc(batch, vocab, rank, depths, N, K)
        ws = tv.alloc_workspace(tv.spark_workspace_size(desc))
        U = torch.from_numpy(inp.base_logits).to(dev)
        w1 = torch.from_numpy(inp.w1.view(np.int16)).to(dev).view(torch.bfloat16)
        w2 = torch.from_numpy(inp.w2.view(np.int16)).to(dev).view(torch.bfloat16)
        anchor = torch.from_numpy(inp.anchor).to(dev)
        temp = torch.from_numpy(inp.temperature).to(dev)
        th = torch.from_numpy(inp.theta).to(dev)
        par = torch.empty((batch, N + 1), dtype=torch.int32, device=dev)
        tok = torch.empty_like(par)
        cnt = torch.empty(batch, dtype=torch.int32, device=dev)
        call = lambda: tv.tree_spark_build(desc, U, w1, w2, anchor, temp, th, par, tok, cnt, ws,
                                           seed=7)
        call()
        torch.cuda.synchronize()
        status, bits = tv.device_status(ws)
        if status != 0:
            raise SystemExit(f"device status {status} bits {bits}")
        diag = ws[8:16].view(torch.int32).cpu().numpy()
        rounds, expanded = int(diag[0]), int(diag[1])
        stream = torch.cuda.current_stream()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for a, b in ev:
            a.record(stream)
            call()
            b.record(stream)
        torch.cuda.synchronize()
        us = float(np.median([a.elapsed_time(b) * 1e3 for a, b in ev]))
        nodes = int(cnt.sum().item()) - batch
        abytes = rounds * vocab * rank * 2 + expanded * (vocab * 4 + rank * 2)
        print(json.dumps({
            "kernel": "tree_spark_build (spark_kernel: select, bf16 MFMA logits, statistics)",
            "workload": f"TreeSpark construction: {batch} requests, T {tsel}, theta {theta}, "
                        f"b {depths}, r {rank}, V {vocab}, K {K}, cap {N}",
            "us_median": us, "reps": reps, "rounds": rounds, "expanded_rows": expanded,
            "drafted_nodes": nodes, "trees_per_s": batch / (us * 1e-6),
            "nodes_per_s": nodes / (us * 1e-6), "us_per_round": us / max(rounds, 1),
            "algorithmic_bytes": abytes, "hbm_GBs": abytes / (us * 1e-6) / 1e9,
            "hbm_frac": abytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="highload")
    ap.add_argument("--temperature", default="mixed")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="instead of the workload, time a plain device copy of this many "
                         "bytes (calibrates the HBM byte counters)")
    ap.add_argument("--attn-sweep", default="",
                    help="comma-separated workloads: time tree_verify_attn alone on each, "
                         "rotating >= --rotate-bytes of distinct copies (one JSON line each)")
    ap.add_argument("--rotate-bytes", type=int, default=1 << 30)
    ap.add_argument("--greedy", choices=("every", "path"), default="path",
                    help="greedy (T = 0) requests: argmax of the rows the walk visits (path, "
                         "the default) or of every row (every)")
    ap.add_argument("--replacement", action="store_true",
                    help="siblings drawn independently (with replacement) and verified by "
                         "the with-replacement rule")
    ap.add_argument("--construct-bench", action="store_true",
                    help="time the EAGLE-2 construction (expansion rounds + rerank) alone")
    ap.add_argument("--spark-bench", action="store_true",
                    help="time TreeSpark's best-first construction alone")
    ap.add_argument("--siblings-bench", action="store_true",
                    help="time tree_draw_siblings alone on the highload trees' expansions")
    ap.add_argument("--commit-bench", type=int, default=0, metavar="LAYERS",
                    help="time tree_kv_commit alone on the highload batch over this many "
                         "layers (one JSON line)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU; --gpus must be 1 "
                                   "(requests and kv heads would shard across GPUs with no "
                                   "exchange between them)"}))
        sys.exit(2)

    import torch
    if args.spark_bench:
        spark_bench(max(1, args.steps), temps=("0", "1", "mixed"))
        return
    if args.siblings_bench:
        siblings_bench(max(1, args.steps))
        return
    if args.construct_bench:
        construct_bench(max(1, args.steps))
        return
    if args.commit_bench:
        commit_bench(args.commit_bench, max(1, args.steps))
        return
    if args.attn_sweep:
        attn_sweep(args.attn_sweep.split(","), args.rotate_bytes, max(1, args.steps // 10))
        return
    if args.copy_bytes:
        src = torch.ones(args.copy_bytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.warmup):
            dst.copy_(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / args.steps
        print(json.dumps({"copy_bytes": src.numel() * 4, "ms": dt * 1e3,
                          "GBs_read_plus_write": 2 * src.numel() * 4 / dt / 1e9}))
        return
    import tree_verification_verify_amd as tv
    from workloads import make_config
    from workloads.device import attention_tensors, sampler_tensors

    temp = args.temperature if args.temperature == "mixed" else float(args.temperature)
    cfg = make_config(args.config, temperature=temp,
                      draws="with" if args.replacement else "without")
    inp, s = cfg.attn, cfg.sampler
    dev = "cuda"
    torch.cuda.set_device(0)
    a = attention_tensors(inp, dev)
    desc = tv.attn_desc(inp.batch, inp.num_q_heads, inp.num_kv_heads, inp.head_dim,
                        inp.max_nodes, inp.max_depth, inp.max_kv_len, inp.num_pages, inp.dtype)
    aws = tv.alloc_workspace(tv.attn_workspace_size(desc), dev)
    out = torch.empty_like(a["q"])
    have_sampler = s is not None
    if have_sampler:
        st = sampler_tensors(s, dev)
        md = max(8, inp.max_depth)
        sdesc = tv.sample_desc(s.batch, s.vocab, s.max_nodes, md, replacement=args.replacement,
                               greedy_path=args.greedy == "path")
        sws = tv.alloc_workspace(tv.sample_workspace_size(sdesc), dev)
        T = int(s.node_indptr[-1])
        flag = torch.empty(T, dtype=torch.int8, device=dev)
        nt = torch.empty(T, dtype=torch.int32, device=dev)
        B = s.batch
        pn = torch.empty(B * (md + 1), dtype=torch.int32, device=dev)
        ot, kk = torch.empty_like(pn), torch.empty_like(pn)
        ol = torch.empty(B, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]

    def step(e=None):
        if e:
            e[0].record(stream)
        tv.tree_verify_attn(desc, a["q"], a["k_pages"], a["v_pages"], a["page_indptr"],
                            a["page_indices"], a["prefix_len"], a["node_indptr"], a["parent"],
                            out, aws)
        if e:
            e[1].record(stream)
        if have_sampler:
            tv.tree_spec_sample(sdesc, st["target_logits"], st["draft_logits"], st["tokens"],
                                st["node_indptr"], st["parent"], st["temperature"],
                                st["uniforms"], flag, nt, sws)
            if e:
                e[2].record(stream)
            tv.tree_accept_path(B, md, st["node_indptr"], st["parent"], st["tokens"], flag, nt,
                                a["prefix_len"], pn, ot, ol, kk, sws)
        if e:
            e[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    for ws_ in (aws,) + ((sws,) if have_sampler else ()):
        status, bits = tv.device_status(ws_)
        if status != 0:
            raise SystemExit(f"device status {status} bits {bits}")
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for k in range(args.steps):
        step(ev[k])
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_step = total_ms / args.steps
    attn_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    samp_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev])) if have_sampler else 0.0
    path_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in ev])) if have_sampler else 0.0

    nodes = inp.total_nodes
    abytes = attn_algorithmic_bytes(inp)
    aflops = attn_algorithmic_flops(cfg)
    achieved = abytes / (attn_ms * 1e-3) / 1e9
    traffic = read_traffic()
    res = {
        "metric": METRIC,
        "value": nodes / (ms_step * 1e-3),
        "unit": "nodes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": inp.dtype,
        "data": "synthetic (seeded; shapes of the pages' workloads)",
        "config": {"workload": f"{args.config}: {inp.batch} requests, {nodes} tree rows, "
                               f"prefix {int(inp.prefix_len.min())}-{int(inp.prefix_len.max())}, "
                               f"Hq {inp.num_q_heads}/Hkv {inp.num_kv_heads}/D {inp.head_dim} "
                               f"{inp.dtype} paged KV"
                               + (f"; sampler V {s.vocab}, T {args.temperature}" if have_sampler else "")
                               + ("; siblings with replacement, rule (b)" if args.replacement else "")
                               + ("; greedy along the walk only" if args.greedy == "path" else ""),
                   "batch": inp.batch, "tree_rows": nodes, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic,
                     "kernel": "tree_verify_attn (attn_stream_kernel<128> + attn_merge_kernel<128>)",
                     "algorithmic_bytes": abytes, "algorithmic_flops": aflops,
                     "kernel_ms": attn_ms,
                     "tflops": aflops / (attn_ms * 1e-3) / 1e12},
        "breakdown_ms": {"tree_verify_attn": attn_ms, "tree_spec_sample": samp_ms,
                         "tree_accept_path": path_ms},
        "attn_nodes_per_s": nodes / (attn_ms * 1e-3),
    }
    if have_sampler:
        out_len = ol.cpu().numpy()
        sbytes = sampler_algorithmic_bytes(s, out_len, greedy_path=args.greedy == "path")
        res["sampler"] = {"algorithmic_bytes": sbytes,
                          "achieved_GBs": sbytes / (samp_ms * 1e-3) / 1e9 if samp_ms > 0 else None,
                          "mean_emitted": float(out_len.mean()), "dtype": "f64"}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, args.cpu_budget, args.replacement,
                                           greedy_path=args.greedy == "path")
    print(json.dumps(res))


if __name__ == "__main__":
    main()
