"""Tree-masked attention over a paged prefix KV cache, in fp64.

Definition ([survey, Timeline]: SpecInfer's tree-based parallel decoding;
[TreeSpark §3.2 step 3]: one target pass with a tree attention mask):
for request r, query head h, tree row i,

  visible(i) = {0 .. P_r-1}  U  {P_r + j : j in anc(i)}      (anc includes i)
  o[i,h]     = sum_{t in visible(i)} softmax_t(scale * <q[i,h], K[t, h//G]>) V[t, h//G]

with K/V of logical position t read from physical page
pg = page_indices[page_indptr[r] + t // 16], slot s = t % 16, as
K[t, g, :] = k_pages[pg, g, s, :] and V[t, g, :] = v_pages[pg, g, :, s]
(V is stored transposed within each page), and scale = 1/sqrt(D) unless
given. The tree's own K/V sit at logical positions P_r .. P_r+N_r-1.
Inputs are widened exactly (bf16 bit patterns or fp32) to fp64.
"""
import numpy as np

from .tree import ancestors_or_self

PAGE = 16


def decode_values(a, dtype):
    """Exact fp64 value of stored inputs (bf16 = top half of an fp32)."""
    if dtype == "bf16":
        b = np.asarray(a, dtype=np.uint16)
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def _scale(inp):
    return inp.sm_scale if inp.sm_scale else 1.0 / np.sqrt(inp.head_dim)


def _visible_mask(inp, r, L):
    """[N][L] boolean: prefix always visible, tree key P+j iff j in anc(i)."""
    P = int(inp.prefix_len[r])
    a, b = int(inp.node_indptr[r]), int(inp.node_indptr[r + 1])
    anc = ancestors_or_self(inp.parent[a:b])
    vis = np.zeros((b - a, L), dtype=bool)
    vis[:, :P] = True
    for i, s in enumerate(anc):
        for j in s:
            vis[i, P + j] = True
    return vis


def _request_rows(inp, r, nodes, K, V, Q):
    """Outputs [len(nodes)][Hq][D] for the given request-local rows.

    Per KV head g: scores S = scale * Q_g K_g^T over all L logical keys,
    invisible keys set to -inf, softmax with the row max subtracted, then
    the weighted sum of V_g rows.
    """
    Hq, Hkv = inp.num_q_heads, inp.num_kv_heads
    G = Hq // Hkv
    a = int(inp.node_indptr[r])
    L = K.shape[0]
    vis = _visible_mask(inp, r, L)[nodes]
    scale = _scale(inp)
    nodes = np.asarray(nodes, dtype=np.int64)
    out = np.zeros((len(nodes), Hq, inp.head_dim))
    for g in range(Hkv):
        Kg = np.ascontiguousarray(K[:, g, :])
        Vg = np.ascontiguousarray(V[:, g, :])
        Qg = Q[a + nodes, g * G:(g + 1) * G, :]             # [n][G][D]
        S = scale * (Qg @ Kg.T)                               # [n][G][L]
        S = np.where(vis[:, None, :], S, -np.inf)
        W = np.exp(S - S.max(axis=2, keepdims=True))
        W /= W.sum(axis=2, keepdims=True)
        out[:, g * G:(g + 1) * G, :] = W @ Vg
    return out


def tree_attention(inp):
    """fp64 output [T][Hq][D] for every tree row of every request."""
    picks = [(r, i) for r in range(inp.batch)
             for i in range(int(inp.node_indptr[r + 1] - inp.node_indptr[r]))]
    return tree_attention_rows(inp, picks)


def tree_attention_rows(inp, picks):
    """fp64 outputs for sampled (request, local node) pairs -> [len][Hq][D]."""
    Q = decode_values(inp.q, inp.dtype)
    by_req = {}
    for n, (r, i) in enumerate(picks):
        by_req.setdefault(r, []).append((n, i))
    out = np.zeros((len(picks), inp.num_q_heads, inp.head_dim))
    for r, lst in by_req.items():
        # gather the request's listed pages, then read logical position t as
        # slot t % 16 of the (t // 16)-th listed page
        base = int(inp.page_indptr[r])
        L = int(inp.prefix_len[r]) + int(inp.node_indptr[r + 1] - inp.node_indptr[r])
        pages = inp.page_indices[base: base + (L + PAGE - 1) // PAGE]
        Ksub = decode_values(inp.k_pages[pages], inp.dtype)
        Vsub = decode_values(inp.v_pages[pages], inp.dtype)
        Hkv, D = inp.num_kv_heads, inp.head_dim
        K = Ksub.transpose(0, 2, 1, 3).reshape(-1, Hkv, D)[:L]   # [page][slot][g][d]
        V = Vsub.transpose(0, 3, 1, 2).reshape(-1, Hkv, D)[:L]   # [page][slot][g][d]
        rows = _request_rows(inp, r, [i for _, i in lst], K, V, Q)
        for (n, _), row in zip(lst, rows):
            out[n] = row
    return out
