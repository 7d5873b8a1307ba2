"""Committing the accepted path's K/V: in-place compaction by a gather.

[survey, Systems] (KV handling): the reference EAGLE implementation compacts
the accepted slots in place with gathers over the accepted positions
(retrieve_indices); slots past the accepted ones are left for reuse.
[survey, Timeline] (SpecInfer): tree tokens sit in the KV cache in topological
order, so node i of request r is at logical position P_r + i, and a root path
visits increasing node indices.

Definition, per request r with n = out_len[r] >= 1, per layer and kv head:

    new[P_r + j] = old[kv_keep[r][j]],      j = 0 .. n-1,

every other logical position unchanged; "old" is the cache before the call
(all sources are read before any destination is written). Logical position t
lives at slot t % 16 of page page_indices[page_indptr[r] + t // 16], with
K[t] = k_pages[pg, g, s, :] and V[t] = v_pages[pg, g, :, s] (V transposed
within each page). Requests with out_len < 1 are left untouched. A keep-list
is valid when kv_keep[r][0] = P_r, it increases strictly, kv_keep[r][j] >=
P_r + j, and every position lies in the request's listed pages.
"""
import numpy as np

PAGE = 16


class BadKeepList(ValueError):
    pass


def check_keep(kv_keep_row, n, prefix_len, num_listed_pages):
    """Raise BadKeepList unless the first n entries form a valid keep-list."""
    P = int(prefix_len)
    prev = None
    for j in range(n):
        s = int(kv_keep_row[j])
        if j == 0 and s != P:
            raise BadKeepList(f"kv_keep[0] = {s}, expected the root at {P}")
        if s < P + j or (prev is not None and s <= prev):
            raise BadKeepList(f"kv_keep[{j}] = {s} is not increasing from P + {j}")
        if s // PAGE >= num_listed_pages or (P + j) // PAGE >= num_listed_pages:
            raise BadKeepList(f"kv_keep[{j}] = {s} lies past the listed pages")
        prev = s


def kv_commit_layer(k_pages, v_pages, page_indptr, page_indices, prefix_len, kv_keep, out_len):
    """One layer: returns new (k_pages, v_pages) arrays; inputs are not modified.

    kv_keep: [B][W] (W >= max out_len), out_len: [B]."""
    k_new = k_pages.copy()
    v_new = v_pages.copy()
    for r in range(len(prefix_len)):
        n = int(out_len[r])
        if n < 1:
            continue
        base = int(page_indptr[r])
        listed = int(page_indptr[r + 1]) - base
        check_keep(kv_keep[r], n, prefix_len[r], listed)

        def loc(t):
            return int(page_indices[base + t // PAGE]), t % PAGE

        P = int(prefix_len[r])
        for j in range(n):
            ps, ss = loc(int(kv_keep[r][j]))
            pd, sd = loc(P + j)
            k_new[pd, :, sd, :] = k_pages[ps, :, ss, :]
            v_new[pd, :, :, sd] = v_pages[ps, :, :, ss]
    return k_new, v_new


def kv_commit(k_layers, v_layers, page_indptr, page_indices, prefix_len, kv_keep, out_len):
    """All layers ([L][num_pages][Hkv][16][D] and [L][num_pages][Hkv][D][16])."""
    k_out = np.empty_like(k_layers)
    v_out = np.empty_like(v_layers)
    for layer in range(k_layers.shape[0]):
        k_out[layer], v_out[layer] = kv_commit_layer(k_layers[layer], v_layers[layer],
                                                     page_indptr, page_indices, prefix_len,
                                                     kv_keep, out_len)
    return k_out, v_out
