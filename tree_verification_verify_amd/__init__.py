"""Tree verification for tree-based speculative decoding on AMD MI355X.

A thin Python binding over libtreeverify (include/tree_verify.h). Every step
of the hot path runs in the library's HIP kernels; this module only checks
and marshals arguments (torch tensors are used for device memory and the
current stream) and raises TVError on a non-OK status. There is no CPU
fallback: if the library is missing, calls raise.

Entry points (same names as the C ABI):
  tree_verify_attn   tree-masked paged attention, one layer
  tree_spec_sample   greedy / rejection walk without or with replacement
  tree_accept_path   longest accepted path, emitted tokens, KV keep-list
  tv_tree_meta       depth, ancestor bitsets, children lists
"""
import ctypes

import numpy as np

from . import _lib
from ._lib import (AttnDesc, SampleDesc, TV_BF16, TV_FP32, STATUS_NAMES, DEV_BITS,
                   TV_RULE_WITHOUT_REPLACEMENT, TV_RULE_WITH_REPLACEMENT,
                   TV_GREEDY_EVERY_NODE, TV_GREEDY_PATH)

__all__ = [
    "TVError", "AttnDesc", "SampleDesc", "TV_BF16", "TV_FP32", "TV_RULE_WITHOUT_REPLACEMENT",
    "TV_RULE_WITH_REPLACEMENT", "TV_GREEDY_EVERY_NODE", "TV_GREEDY_PATH", "attn_desc",
    "sample_desc", "attn_workspace_size", "sample_workspace_size", "alloc_workspace",
    "workspace_init", "device_status", "tree_verify_attn", "tree_spec_sample",
    "tree_accept_path", "tree_kv_commit", "tree_draw_siblings", "tree_expand_step", "tree_rerank", "expand_workspace_size", "tv_tree_meta", "validate_tree", "validate_pages",
    "library",
]


class TVError(RuntimeError):
    def __init__(self, status, where=""):
        lib = _lib.load()
        msg = lib.tv_status_string(status).decode()
        if status == 7:
            msg += " (" + lib.tv_last_hip_error().decode() + ")"
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def library():
    return _lib.load()


def _check(status, where):
    if status != 0:
        raise TVError(status, where)


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, dtype=None, device=True):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if device and t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def attn_desc(batch, num_q_heads, num_kv_heads, head_dim, max_nodes, max_depth,
              max_kv_len, num_pages, dtype="bf16", sm_scale=0.0):
    return AttnDesc(batch, num_q_heads, num_kv_heads, head_dim, 16, max_nodes, max_depth,
                    max_kv_len, num_pages, TV_BF16 if dtype == "bf16" else TV_FP32,
                    float(sm_scale))


def sample_desc(batch, vocab, max_nodes, max_depth, replacement=False, greedy_path=False):
    """replacement selects the with-replacement walk (independent sibling
    draws) instead of the without-replacement one; greedy_path makes greedy
    (T == 0) requests read only the rows their walk visits."""
    return SampleDesc(batch, vocab, max_nodes, max_depth,
                      TV_RULE_WITH_REPLACEMENT if replacement else TV_RULE_WITHOUT_REPLACEMENT,
                      TV_GREEDY_PATH if greedy_path else TV_GREEDY_EVERY_NODE)


def attn_workspace_size(desc):
    n = _lib.load().tv_attn_workspace_size(ctypes.byref(desc))
    if n == 0:
        raise TVError(2, "tv_attn_workspace_size")
    return n


def sample_workspace_size(desc):
    n = _lib.load().tv_sample_workspace_size(ctypes.byref(desc))
    if n == 0:
        raise TVError(2, "tv_sample_workspace_size")
    return n


def alloc_workspace(nbytes, device="cuda"):
    """A 256-byte aligned uint8 device buffer of nbytes, zero-initialised by
    the library's fill kernel."""
    import torch
    raw = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-raw.data_ptr()) % 256
    ws = raw[off:off + nbytes]
    workspace_init(ws)
    return ws


def workspace_init(ws, stream=None):
    _need(ws, "workspace", None)
    _check(_lib.load().tv_workspace_init(_ptr(ws), ws.numel() * ws.element_size(),
                                         _stream(stream)), "tv_workspace_init")


def device_status(ws, stream=None):
    """(status, bits) of the workspace's device status word; synchronises."""
    bits = ctypes.c_uint32(0)
    st = _lib.load().tv_device_status(_ptr(ws), _stream(stream), ctypes.byref(bits))
    return st, bits.value


def tree_verify_attn(desc, q, k_pages, v_pages, page_indptr, page_indices, prefix_len,
                     node_indptr, parent, out, workspace, stream=None):
    import torch
    dt = torch.bfloat16 if desc.dtype == TV_BF16 else torch.float32
    for t, n in ((q, "q"), (k_pages, "k_pages"), (v_pages, "v_pages"), (out, "out")):
        _need(t, n, dt)
    for t, n in ((page_indptr, "page_indptr"), (page_indices, "page_indices"),
                 (prefix_len, "prefix_len"), (node_indptr, "node_indptr"), (parent, "parent")):
        _need(t, n, torch.int32)
    _need(workspace, "workspace", torch.uint8)
    if q.shape != out.shape:
        raise ValueError("q and out shapes differ")
    if tuple(k_pages.shape) != (desc.num_pages, desc.num_kv_heads, 16, desc.head_dim):
        raise ValueError("k_pages must be [num_pages][Hkv][16][D]")
    if tuple(v_pages.shape) != (desc.num_pages, desc.num_kv_heads, desc.head_dim, 16):
        raise ValueError("v_pages must be [num_pages][Hkv][D][16] (V transposed within a page)")
    if q.dim() != 3 or q.shape[1] != desc.num_q_heads or q.shape[2] != desc.head_dim:
        raise ValueError("q must be [T][Hq][D]")
    _check(_lib.load().tree_verify_attn(
        ctypes.byref(desc), _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(page_indptr),
        _ptr(page_indices), _ptr(prefix_len), _ptr(node_indptr), _ptr(parent), _ptr(out),
        _ptr(workspace), workspace.numel(), _stream(stream)), "tree_verify_attn")


def tree_spec_sample(desc, target_logits, draft_logits, tokens, node_indptr, parent,
                     temperature, uniforms, accept_flag, next_token, workspace, stream=None):
    import torch
    _need(target_logits, "target_logits", torch.float32)
    if draft_logits is not None:
        _need(draft_logits, "draft_logits", torch.float32)
    for t, n in ((tokens, "tokens"), (node_indptr, "node_indptr"), (parent, "parent"),
                 (next_token, "next_token")):
        _need(t, n, torch.int32)
    _need(temperature, "temperature", torch.float32)
    _need(uniforms, "uniforms", torch.float32)
    _need(accept_flag, "accept_flag", torch.int8)
    _need(workspace, "workspace", torch.uint8)
    if target_logits.dim() != 2 or target_logits.shape[1] != desc.vocab:
        raise ValueError("target_logits must be [T][V]")
    _check(_lib.load().tree_spec_sample(
        ctypes.byref(desc), _ptr(target_logits), _ptr(draft_logits), _ptr(tokens),
        _ptr(node_indptr), _ptr(parent), _ptr(temperature), _ptr(uniforms), _ptr(accept_flag),
        _ptr(next_token), _ptr(workspace), workspace.numel(), _stream(stream)),
        "tree_spec_sample")


def tree_spec_sample_noalloc(desc, target_logits, draft_logits, tokens, node_indptr, parent,
                             temperature, uniforms, accept_flag, next_token, status, stream=None):
    """tree_spec_sample with its synchronisation blocks in the library's own
    device array (no workspace); status is a caller-owned device int32/uint32
    word that receives the TV_DEV_* bits."""
    import torch
    _need(target_logits, "target_logits", torch.float32)
    if draft_logits is not None:
        _need(draft_logits, "draft_logits", torch.float32)
    for t, n in ((tokens, "tokens"), (node_indptr, "node_indptr"), (parent, "parent"),
                 (next_token, "next_token")):
        _need(t, n, torch.int32)
    _need(temperature, "temperature", torch.float32)
    _need(uniforms, "uniforms", torch.float32)
    _need(accept_flag, "accept_flag", torch.int8)
    _need(status, "status", None)
    if target_logits.dim() != 2 or target_logits.shape[1] != desc.vocab:
        raise ValueError("target_logits must be [T][V]")
    _check(_lib.load().tree_spec_sample_noalloc(
        ctypes.byref(desc), _ptr(target_logits), _ptr(draft_logits), _ptr(tokens),
        _ptr(node_indptr), _ptr(parent), _ptr(temperature), _ptr(uniforms), _ptr(accept_flag),
        _ptr(next_token), _ptr(status), _stream(stream)), "tree_spec_sample_noalloc")


def tree_accept_path(batch, max_depth, node_indptr, parent, tokens, accept_flag, next_token,
                     prefix_len, path_nodes, out_tokens, out_len, kv_keep,
                     status_workspace=None, stream=None):
    import torch
    for t, n in ((node_indptr, "node_indptr"), (parent, "parent"), (tokens, "tokens"),
                 (next_token, "next_token"), (prefix_len, "prefix_len"),
                 (path_nodes, "path_nodes"), (out_tokens, "out_tokens"), (out_len, "out_len"),
                 (kv_keep, "kv_keep")):
        _need(t, n, torch.int32)
    _need(accept_flag, "accept_flag", torch.int8)
    for t in (path_nodes, out_tokens, kv_keep):
        if t.numel() < batch * (max_depth + 1):
            raise ValueError("path outputs must hold [B][max_depth+1]")
    _check(_lib.load().tree_accept_path(
        batch, max_depth, _ptr(node_indptr), _ptr(parent), _ptr(tokens), _ptr(accept_flag),
        _ptr(next_token), _ptr(prefix_len), _ptr(path_nodes), _ptr(out_tokens), _ptr(out_len),
        _ptr(kv_keep), _ptr(status_workspace), _stream(stream)), "tree_accept_path")


def tree_kv_commit(desc, k_pages, v_pages, page_indptr, page_indices, prefix_len, kv_keep,
                   out_len, max_depth, num_layers=None, layer_stride=None,
                   status_workspace=None, stream=None):
    """k_pages / v_pages: [L][num_pages][Hkv][16][D] and [L][num_pages][Hkv][D][16]
    (or one layer without the leading L), modified in place."""
    import torch
    dt = torch.bfloat16 if desc.dtype == TV_BF16 else torch.float32
    for t, n in ((k_pages, "k_pages"), (v_pages, "v_pages")):
        _need(t, n, dt)
    for t, n in ((page_indptr, "page_indptr"), (page_indices, "page_indices"),
                 (prefix_len, "prefix_len"), (kv_keep, "kv_keep"), (out_len, "out_len")):
        _need(t, n, torch.int32)
    per_layer = desc.num_pages * desc.num_kv_heads * 16 * desc.head_dim
    if num_layers is None:
        num_layers = k_pages.numel() // per_layer
    if layer_stride is None:
        layer_stride = per_layer
    if k_pages.shape != v_pages.shape[:-2] + (16, desc.head_dim) and \
            k_pages.numel() != v_pages.numel():
        raise ValueError("k_pages and v_pages disagree")
    if k_pages.numel() < (num_layers - 1) * layer_stride + per_layer:
        raise ValueError("k_pages holds fewer layers than num_layers")
    if kv_keep.numel() < desc.batch * (max_depth + 1):
        raise ValueError("kv_keep must hold [B][max_depth+1]")
    _check(_lib.load().tree_kv_commit(
        ctypes.byref(desc), int(num_layers), int(layer_stride), _ptr(k_pages), _ptr(v_pages),
        _ptr(page_indptr), _ptr(page_indices), _ptr(prefix_len), _ptr(kv_keep), _ptr(out_len),
        int(max_depth), _ptr(status_workspace), _stream(stream)), "tree_kv_commit")


def tree_draw_siblings(draft_logits, counts, temperature, tokens, stream_id=0, seed=0,
                       status_workspace=None, stream=None):
    """draft_logits [rows][V] fp32, counts [rows] int32, temperature [rows] fp32;
    tokens [rows][MAX_CHILDREN] int32 (output)."""
    import torch
    _need(draft_logits, "draft_logits", torch.float32)
    _need(temperature, "temperature", torch.float32)
    _need(counts, "counts", torch.int32)
    _need(tokens, "tokens", torch.int32)
    if draft_logits.dim() != 2:
        raise ValueError("draft_logits must be [rows][V]")
    rows, V = draft_logits.shape
    if tokens.numel() < rows * _lib.MAX_CHILDREN or counts.numel() < rows or \
            temperature.numel() < rows:
        raise ValueError("counts / temperature must hold [rows], tokens [rows][16]")
    _check(_lib.load().tree_draw_siblings(
        rows, V, _ptr(draft_logits), _ptr(counts), _ptr(temperature), int(stream_id) & 0xFFFFFFFF,
        int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(tokens), _ptr(status_workspace), _stream(stream)),
        "tree_draw_siblings")


def expand_workspace_size(batch, k_in, k):
    return int(_lib.load().tv_expand_workspace_size(batch, k_in, k))


def tree_expand_step(draft_logits, frontier, cand_offset, cand_value, cand_token, cand_parent,
                     next_frontier, workspace=None, stream=None):
    """One expansion round. draft_logits [B][k_in][V] fp32; frontier [B][k_in]
    int32 candidate ids or None (every slot is the root); cand_* [B][C];
    next_frontier [B][k] int32 (k = children per node = its second size);
    workspace: None, or a uint8 workspace (status word; with
    expand_workspace_size bytes, rounds of few rows are split)."""
    import torch
    _need(draft_logits, "draft_logits", torch.float32)
    _need(cand_value, "cand_value", torch.float32)
    for t, n in ((cand_token, "cand_token"), (cand_parent, "cand_parent"),
                 (next_frontier, "next_frontier")):
        _need(t, n, torch.int32)
    if draft_logits.dim() != 3 or cand_value.dim() != 2 or next_frontier.dim() != 2:
        raise ValueError("draft_logits [B][k_in][V], cand_value [B][C], next_frontier [B][k]")
    B, k_in, V = draft_logits.shape
    k = next_frontier.shape[1]
    C = cand_value.shape[1]
    if frontier is not None:
        _need(frontier, "frontier", torch.int32)
        if tuple(frontier.shape) != (B, k_in):
            raise ValueError("frontier must be [B][k_in]")
    if cand_value.shape[0] != B or next_frontier.shape[0] != B or \
            tuple(cand_token.shape) != (B, C) or tuple(cand_parent.shape) != (B, C):
        raise ValueError("candidate arrays must be [B][C]")
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8)
    _check(_lib.load().tree_expand_step(
        B, V, k_in, k, _ptr(draft_logits), _ptr(frontier), C, int(cand_offset), _ptr(cand_value),
        _ptr(cand_token), _ptr(cand_parent), _ptr(next_frontier), _ptr(workspace),
        0 if workspace is None else workspace.numel(), _stream(stream)), "tree_expand_step")


def tree_rerank(num_cand, m, cand_value, cand_token, cand_parent, out_parent, out_token,
                out_count, status_workspace=None, stream=None):
    """Keep the m best of the first num_cand candidates per request; out_parent /
    out_token [B][m+1] int32, out_count [B] int32 (outputs)."""
    import torch
    _need(cand_value, "cand_value", torch.float32)
    for t, n in ((cand_token, "cand_token"), (cand_parent, "cand_parent"),
                 (out_parent, "out_parent"), (out_token, "out_token"), (out_count, "out_count")):
        _need(t, n, torch.int32)
    B, C = cand_value.shape
    if tuple(out_parent.shape) != (B, m + 1) or tuple(out_token.shape) != (B, m + 1) or \
            out_count.numel() != B or tuple(cand_token.shape) != (B, C) or \
            tuple(cand_parent.shape) != (B, C):
        raise ValueError("out_parent / out_token must be [B][m+1], out_count [B]")
    _check(_lib.load().tree_rerank(
        B, int(num_cand), C, int(m), _ptr(cand_value), _ptr(cand_token), _ptr(cand_parent),
        _ptr(out_parent), _ptr(out_token), _ptr(out_count), _ptr(status_workspace),
        _stream(stream)), "tree_rerank")


def spark_desc(batch, vocab, rank, depths, max_nodes, max_siblings, calib_a=0.67, calib_b=-0.46):
    return _lib.SparkDesc(batch, vocab, rank, depths, max_nodes, max_siblings, calib_a, calib_b)


def spark_workspace_size(desc):
    n = _lib.load().tv_spark_workspace_size(ctypes.byref(desc))
    if n == 0:
        raise TVError(2, "tv_spark_workspace_size")
    return n


def tree_spark_build(desc, base_logits, w1, w2, anchor, temperature, theta, out_parent, out_token,
                     out_count, workspace, out_logsurv=None, stream_id=0, seed=0, stream=None):
    """TreeSpark best-first construction; w1, w2 are bf16 [V][rank]."""
    import torch
    _need(base_logits, "base_logits", torch.float32)
    _need(w1, "w1", torch.bfloat16)
    _need(w2, "w2", torch.bfloat16)
    for t, n in ((anchor, "anchor"), (out_parent, "out_parent"), (out_token, "out_token"),
                 (out_count, "out_count")):
        _need(t, n, torch.int32)
    _need(temperature, "temperature", torch.float32)
    _need(theta, "theta", torch.float32)
    _need(workspace, "workspace", torch.uint8)
    if out_logsurv is not None:
        _need(out_logsurv, "out_logsurv", torch.float32)
    B, W = desc.batch, desc.max_nodes + 1
    if tuple(base_logits.shape) != (B, desc.depths, desc.vocab):
        raise ValueError("base_logits must be [B][depths][V]")
    if tuple(w1.shape) != (desc.vocab, desc.rank) or tuple(w2.shape) != (desc.vocab, desc.rank):
        raise ValueError("w1, w2 must be [V][rank]")
    for t in (out_parent, out_token) + ((out_logsurv,) if out_logsurv is not None else ()):
        if t.numel() != B * W:
            raise ValueError("tree outputs must be [B][max_nodes+1]")
    _check(_lib.load().tree_spark_build(
        ctypes.byref(desc), _ptr(base_logits), _ptr(w1), _ptr(w2), _ptr(anchor),
        _ptr(temperature), _ptr(theta), ctypes.c_uint32(stream_id), ctypes.c_uint64(seed),
        _ptr(out_parent), _ptr(out_token), _ptr(out_count), _ptr(out_logsurv),
        _ptr(workspace), workspace.numel(), _stream(stream)), "tree_spark_build")


def tv_tree_meta(batch, max_nodes, node_indptr, parent, depth=None, anc_bits=None,
                 first_child=None, next_sibling=None, status_workspace=None, stream=None):
    import torch
    _need(node_indptr, "node_indptr", torch.int32)
    _need(parent, "parent", torch.int32)
    _check(_lib.load().tv_tree_meta(
        batch, max_nodes, _ptr(node_indptr), _ptr(parent), _ptr(depth), _ptr(anc_bits),
        _ptr(first_child), _ptr(next_sibling), _ptr(status_workspace), _stream(stream)),
        "tv_tree_meta")


def _host_i32(a):
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def validate_tree(node_indptr, parent, max_nodes, max_depth):
    """Host-side check of the tree rules; returns the status code."""
    ni, pni = _host_i32(node_indptr)
    pa, ppa = _host_i32(parent)
    return _lib.load().tv_validate_tree(len(ni) - 1, pni, ppa, max_nodes, max_depth)


def validate_pages(page_indptr, page_indices, prefix_len, node_indptr, num_pages):
    a, pa = _host_i32(page_indptr)
    b, pb = _host_i32(page_indices if len(page_indices) else np.zeros(1, np.int32))
    c, pc = _host_i32(prefix_len)
    d, pd = _host_i32(node_indptr)
    return _lib.load().tv_validate_pages(len(a) - 1, pa, pb, pc, pd, num_pages, 16)
