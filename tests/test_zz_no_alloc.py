"""tree_spec_sample_noalloc (its synchronisation blocks in the library's own
device array, no workspace) against tree_spec_sample with a workspace, through
the C ABI: flags and next tokens bit-identical, on calls in a row whose
batches shrink (so the second call runs over blocks the first one left
behind), and the status word usable by tree_accept_path."""
import numpy as np
import pytest

from workloads import make_config
from workloads.device import sampler_tensors

pytestmark = pytest.mark.gpu


def _outputs(inp):
    import torch
    T = int(inp.node_indptr[-1])
    return (torch.full((T,), -7, dtype=torch.int8, device="cuda"),
            torch.full((T,), -7, dtype=torch.int32, device="cuda"))


def _with_workspace(inp, desc, t):
    import tree_verification_verify_amd as tv
    ws = tv.alloc_workspace(tv.sample_workspace_size(desc))
    flag, nt = _outputs(inp)
    tv.tree_spec_sample(desc, t["target_logits"], t["draft_logits"], t["tokens"],
                        t["node_indptr"], t["parent"], t["temperature"], t["uniforms"],
                        flag, nt, ws)
    st, bits = tv.device_status(ws)
    assert st == 0, (st, bits)
    return flag.cpu().numpy(), nt.cpu().numpy()


def _noalloc(inp, desc, t, status):
    import tree_verification_verify_amd as tv
    flag, nt = _outputs(inp)
    tv.tree_spec_sample_noalloc(desc, t["target_logits"], t["draft_logits"], t["tokens"],
                                t["node_indptr"], t["parent"], t["temperature"],
                                t["uniforms"], flag, nt, status)
    return flag, nt


CASES = [  # (batch, vocab, temperature): each call smaller than the one before
    (64, None, "mixed"),
    (16, 4096, 1.0),
    (3, 1000, 0.0),
]


def test_noalloc_matches_workspace_entry_point():
    import torch
    import tree_verification_verify_amd as tv
    status = torch.full((64,), 0x7F, dtype=torch.int32, device="cuda")  # stale bits: cleared per call
    for batch, vocab, temp in CASES:
        cfg = make_config("highload", attention=False, batch=batch, vocab=vocab, temperature=temp)
        inp = cfg.sampler
        desc = tv.sample_desc(inp.batch, inp.vocab, inp.max_nodes, 8)
        t = sampler_tensors(inp)
        flag, nt = _noalloc(inp, desc, t, status)
        st, bits = tv.device_status(status)
        assert st == 0 and bits == 0, (batch, st, bits)
        ref_flag, ref_nt = _with_workspace(inp, desc, t)
        np.testing.assert_array_equal(flag.cpu().numpy(), ref_flag, err_msg=f"batch {batch}")
        np.testing.assert_array_equal(nt.cpu().numpy(), ref_nt, err_msg=f"batch {batch}")
        # the status word serves tree_accept_path as its status workspace
        B, W = inp.batch, 9
        pn = torch.empty(B * W, dtype=torch.int32, device="cuda")
        ot, kk = torch.empty_like(pn), torch.empty_like(pn)
        ol = torch.empty(B, dtype=torch.int32, device="cuda")
        prefix = torch.tensor(cfg.prefix_lens, dtype=torch.int32, device="cuda")
        tv.tree_accept_path(B, 8, t["node_indptr"], t["parent"], t["tokens"], flag, nt, prefix,
                            pn, ot, ol, kk, status)
        st, bits = tv.device_status(status)
        assert st == 0 and (ol.cpu().numpy() >= 1).all()


def test_noalloc_repeated_calls_are_identical():
    """Back-to-back calls on one stream over the same blocks give the same
    outputs (every call clears the blocks it uses)."""
    import torch
    import tree_verification_verify_amd as tv
    cfg = make_config("highload", attention=False, batch=32, vocab=8192, temperature="mixed")
    inp = cfg.sampler
    desc = tv.sample_desc(inp.batch, inp.vocab, inp.max_nodes, 8)
    t = sampler_tensors(inp)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    runs = [_noalloc(inp, desc, t, status) for _ in range(3)]
    st, bits = tv.device_status(status)
    assert st == 0, (st, bits)
    for f, n in runs[1:]:
        assert torch.equal(f, runs[0][0]) and torch.equal(n, runs[0][1])
