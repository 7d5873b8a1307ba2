"""The synthetic workloads have the shapes they are built for: the tiny
⟨1,1,3,1,1⟩ expansion-vector tree (TreeSpark §3.1's expansion vectors),
EAGLE-2's dynamic tree of 60 tokens to depth 6 and a Sequoia-sized tree of
768 nodes (both sizes from the survey page's Timeline section; depth 12 is
this workload's choice), a batch of 16 requests of 32-row trees, and the
high-load batch of 64 requests with 8-row chains, 16-row and 32-row trees
over prefixes of 512..8192 at T in {0, 0.5, 1}. The trees are topological
parent arrays and the page pools are shuffled."""
import numpy as np

import oracle
from workloads import make_config
from workloads.configs import VOCAB


def _check_trees(cfg):
    for parent in cfg.trees:
        p = np.asarray(parent)
        assert p[0] == -1
        assert np.all((p[1:] >= 0) & (p[1:] < np.arange(1, len(p))))


def _depth(parent):
    return int(np.max(oracle.depths(parent)))


def _shuffled(inp):
    idx = np.asarray(inp.page_indices)
    return not np.all(np.diff(idx) == 1)


def test_tiny():
    cfg = make_config("tiny")
    _check_trees(cfg)
    a = cfg.attn
    assert [len(t) for t in cfg.trees] == [12] and list(cfg.prefix_lens) == [128]
    assert (a.num_q_heads, a.num_kv_heads, a.head_dim, a.dtype) == (4, 1, 64, "fp32")
    assert cfg.sampler.vocab == 512 and list(cfg.sampler.temperature) == [1.0]
    # one root child, one grandchild, three children below it, then 1 and 1
    d = oracle.depths(cfg.trees[0])
    assert [int((d == k).sum()) for k in range(6)] == [1, 1, 1, 3, 3, 3]


def test_eagle2_and_sequoia():
    e = make_config("eagle2", sampler=False)
    s = make_config("sequoia", sampler=False)
    for cfg in (e, s):
        _check_trees(cfg)
        a = cfg.attn
        assert (a.num_q_heads, a.num_kv_heads, a.head_dim, a.dtype) == (32, 8, 128, "bf16")
    assert len(e.trees[0]) == 60 and _depth(e.trees[0]) == 6 and list(e.prefix_lens) == [2048]
    assert len(s.trees[0]) == 768 and _depth(s.trees[0]) == 12 and list(s.prefix_lens) == [8192]
    assert VOCAB == 151936
    t = make_config("sequoia", attention=False, vocab=16)
    assert list(t.sampler.temperature) == [1.0]


def test_batched():
    cfg = make_config("batched")
    _check_trees(cfg)
    assert len(cfg.trees) == 16 and all(len(t) == 32 and _depth(t) <= 8 for t in cfg.trees)
    assert all(1024 <= p <= 4096 for p in cfg.prefix_lens)
    assert _shuffled(cfg.attn)


def test_highload():
    cfg = make_config("highload", sampler=False)
    _check_trees(cfg)
    sizes = [len(t) for t in cfg.trees]
    assert len(sizes) == 64 and set(sizes) == {8, 16, 32} and sum(sizes) == 1216
    for t in cfg.trees:
        assert _depth(t) <= 8
        if len(t) == 8:
            assert _depth(t) == 7  # the chain budget
    assert all(512 <= p <= 8192 for p in cfg.prefix_lens)
    assert _shuffled(cfg.attn)
    t = make_config("highload", attention=False, vocab=16)
    assert set(np.asarray(t.sampler.temperature).tolist()) == {0.0, 0.5, 1.0}
