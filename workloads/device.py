"""Upload generated inputs to the GPU as torch tensors (memory plumbing only)."""
import numpy as np


def _t(a, dtype, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=dtype)


def attention_tensors(inp, device="cuda"):
    """dict of device tensors for tree_verify_attn (bf16 stored as uint16 bits)."""
    import torch
    if inp.dtype == "bf16":
        def vals(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    else:
        def vals(a):
            return _t(a, torch.float32, device)
    return dict(
        q=vals(inp.q), k_pages=vals(inp.k_pages), v_pages=vals(inp.v_pages),
        page_indptr=_t(inp.page_indptr, torch.int32, device),
        page_indices=_t(inp.page_indices if len(inp.page_indices) else np.zeros(1, np.int32),
                        torch.int32, device),
        prefix_len=_t(inp.prefix_len, torch.int32, device),
        node_indptr=_t(inp.node_indptr, torch.int32, device),
        parent=_t(inp.parent, torch.int32, device))


def sampler_tensors(inp, device="cuda"):
    import torch
    return dict(
        target_logits=_t(inp.target_logits, torch.float32, device),
        draft_logits=None if inp.draft_logits is None else _t(inp.draft_logits, torch.float32, device),
        tokens=_t(inp.tokens, torch.int32, device),
        node_indptr=_t(inp.node_indptr, torch.int32, device),
        parent=_t(inp.parent, torch.int32, device),
        temperature=_t(inp.temperature, torch.float32, device),
        uniforms=_t(inp.uniforms, torch.float32, device))
