"""CPU-only checks of libtreeverify: it loads, exports every declared symbol,
and its host-side argument checks return the documented status before any
GPU work (no compute calls are made here)."""
import ctypes
import os
import re

import numpy as np
import pytest

import tree_verification_verify_amd as tv
from tree_verification_verify_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tree_verify.h")

OK, NULL, SHAPE, DTYPE, WORKSPACE, TREE, PAGES = 0, 1, 2, 3, 4, 5, 6
FAKE = ctypes.c_void_p(0x100000)   # never dereferenced: every case fails host checks first


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)
    skip = {"if", "while", "sizeof", "defined"}
    return sorted({n for n in names if n.startswith(("tv_", "tree_")) and n not in skip})


def test_library_exports_every_declared_symbol():
    lib = tv.library()
    declared = _declared_functions()
    assert len(declared) >= 13
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(_lib.EXPORTS)
    assert lib.tv_version() == 1


def _desc(**kw):
    base = dict(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, max_nodes=32,
                max_depth=8, max_kv_len=600, num_pages=100, dtype="bf16")
    base.update(kw)
    d = tv.attn_desc(**{k: v for k, v in base.items() if k != "page_size"})
    if "page_size" in kw:
        d.page_size = kw["page_size"]
    return d


def _attn_call(desc, ws_bytes=1 << 30, null=None):
    ptrs = [FAKE] * 9
    if null is not None:
        ptrs[null] = None
    return tv.library().tree_verify_attn(ctypes.byref(desc), *ptrs, FAKE, ws_bytes, None)


def test_attention_host_errors():
    lib = tv.library()
    assert lib.tv_attn_workspace_size(ctypes.byref(_desc())) > 0
    for bad in (dict(num_q_heads=7), dict(head_dim=96), dict(page_size=32),
                dict(max_nodes=0), dict(max_nodes=2000), dict(batch=0),
                dict(max_kv_len=10)):
        d = _desc(**bad)
        assert lib.tv_attn_workspace_size(ctypes.byref(d)) == 0, bad
        assert _attn_call(d) == SHAPE, bad
    d = _desc()
    d.dtype = 7
    assert _attn_call(d) == DTYPE
    for i in range(9):
        assert _attn_call(_desc(), null=i) == NULL
    need = lib.tv_attn_workspace_size(ctypes.byref(_desc()))
    assert _attn_call(_desc(), ws_bytes=need - 1) == WORKSPACE
    assert lib.tree_verify_attn(None, *([FAKE] * 10), 1 << 30, None) == NULL


def test_attention_workspace_grows_with_problem():
    lib = tv.library()
    a = lib.tv_attn_workspace_size(ctypes.byref(_desc(batch=1)))
    b = lib.tv_attn_workspace_size(ctypes.byref(_desc(batch=64)))
    c = lib.tv_attn_workspace_size(ctypes.byref(_desc(batch=64, max_kv_len=8224)))
    assert 0 < a < b <= c
    assert a % 256 == 0 and b % 256 == 0


def test_sampler_host_errors():
    lib = tv.library()
    d = tv.sample_desc(4, 151936, 32, 8)
    need = lib.tv_sample_workspace_size(ctypes.byref(d))
    assert need > 0
    call = lambda desc, ptrs, n=need: lib.tree_spec_sample(ctypes.byref(desc), *ptrs, FAKE, n, None)
    ok_ptrs = [FAKE] * 9
    for i in (0, 2, 3, 4, 5, 6, 7, 8):   # draft logits (1) may be NULL
        p = list(ok_ptrs)
        p[i] = None
        assert call(d, p) == NULL, i
    assert call(d, ok_ptrs, need - 1) == WORKSPACE
    for bad in (tv.sample_desc(0, 10, 4, 2), tv.sample_desc(1, 0, 4, 2),
                tv.sample_desc(1, 10, 70000, 2)):
        assert lib.tv_sample_workspace_size(ctypes.byref(bad)) == 0
        assert call(bad, ok_ptrs) == SHAPE
    for rule in (-1, 2):
        bad = tv.sample_desc(4, 151936, 32, 8)
        bad.rule = rule
        assert lib.tv_sample_workspace_size(ctypes.byref(bad)) == 0
        assert call(bad, ok_ptrs) == SHAPE
    rep = tv.sample_desc(4, 151936, 32, 8, replacement=True)
    assert rep.rule == tv.TV_RULE_WITH_REPLACEMENT
    assert lib.tv_sample_workspace_size(ctypes.byref(rep)) == need
    for greedy in (-1, 2):
        bad = tv.sample_desc(4, 151936, 32, 8)
        bad.greedy = greedy
        assert lib.tv_sample_workspace_size(ctypes.byref(bad)) == 0
        assert call(bad, ok_ptrs) == SHAPE
    gp = tv.sample_desc(4, 151936, 32, 8, greedy_path=True)
    assert gp.greedy == tv.TV_GREEDY_PATH
    assert lib.tv_sample_workspace_size(ctypes.byref(gp)) == need


def test_path_and_meta_host_errors():
    lib = tv.library()
    assert lib.tree_accept_path(0, 4, *([FAKE] * 10), None, None) == SHAPE
    assert lib.tree_accept_path(2, -1, *([FAKE] * 10), None, None) == SHAPE
    for i in range(10):
        p = [FAKE] * 10
        p[i] = None
        assert lib.tree_accept_path(2, 4, *p, None, None) == NULL
    assert lib.tv_tree_meta(0, 4, FAKE, FAKE, None, None, None, None, None, None) == SHAPE
    assert lib.tv_tree_meta(1, 4, None, FAKE, None, None, None, None, None, None) == NULL
    assert lib.tv_workspace_init(None, 1024, None) == NULL
    assert lib.tv_workspace_init(ctypes.c_void_p(0x100010), 1024, None) == WORKSPACE
    assert lib.tv_workspace_init(FAKE, 16, None) == WORKSPACE
    assert lib.tv_device_status(None, None, None) == NULL


def test_validate_tree():
    ni = np.array([0, 4, 7])
    good = np.array([-1, 0, 0, 1, -1, 0, 1])
    assert tv.validate_tree(ni, good, 4, 2) == OK
    assert tv.validate_tree(ni, good, 3, 2) == TREE          # N > max_nodes
    assert tv.validate_tree(ni, good, 4, 1) == TREE          # depth > max_depth
    for bad in ([-1, 0, 0, 3, -1, 0, 1],   # parent[i] >= i
                [0, 0, 0, 1, -1, 0, 1],    # root parent != -1
                [-1, 0, -1, 1, -1, 0, 1],  # second root
                [-1, 0, 0, 1, -1, 0, 5]):  # points past the request
        assert tv.validate_tree(ni, np.array(bad), 4, 3) == TREE, bad


def test_validate_pages():
    ni = np.array([0, 4, 6])
    prefix = np.array([20, 9])
    pi = np.array([0, 2, 3])          # request 0: 24 tokens in 2 pages, request 1: 11 in 1
    idx = np.array([5, 1, 0])
    assert tv.validate_pages(pi, idx, prefix, ni, 6) == OK
    assert tv.validate_pages(pi, np.array([5, 6, 0]), prefix, ni, 6) == PAGES   # id out of range
    assert tv.validate_pages(pi, np.array([5, -1, 0]), prefix, ni, 6) == PAGES
    assert tv.validate_pages(np.array([0, 1, 3]), idx, prefix, ni, 6) == PAGES  # too few pages
    assert tv.validate_pages(pi, idx, np.array([29, 9]), ni, 6) == PAGES        # 33 tokens > 32


def test_kv_commit_host_errors():
    lib = tv.library()
    d = _desc()
    per_layer = 100 * 2 * 16 * 128

    def call(desc=d, layers=2, stride=per_layer, max_depth=8, null=None, k=FAKE):
        ptrs = [k, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE]
        if null is not None:
            ptrs[null] = None
        return lib.tree_kv_commit(ctypes.byref(desc), layers, stride, *ptrs, max_depth, None, None)

    assert call(layers=0) == SHAPE
    assert call(stride=per_layer - 8) == SHAPE           # layers would overlap
    assert call(stride=per_layer + 3) == SHAPE           # layer starts not 16-byte aligned
    assert call(max_depth=-1) == SHAPE
    assert call(desc=_desc(head_dim=96)) == SHAPE
    assert call(desc=_desc(dtype="fp32"), stride=per_layer + 2) == SHAPE
    assert call(k=ctypes.c_void_p(0x100008)) == SHAPE    # misaligned pool
    for i in range(7):
        assert call(null=i) == NULL
    bad = _desc()
    bad.dtype = 7
    assert call(desc=bad) == DTYPE


def test_draw_siblings_host_errors():
    lib = tv.library()
    args = [4, 100, FAKE, FAKE, FAKE, 0, 0, FAKE, None, None]
    for i, bad in ((0, 0), (1, 0)):
        a = list(args)
        a[i] = bad
        assert lib.tree_draw_siblings(*a) == SHAPE
    for i in (2, 3, 4, 7):
        a = list(args)
        a[i] = None
        assert lib.tree_draw_siblings(*a) == NULL


def test_construct_host_errors():
    lib = tv.library()
    P = FAKE
    exp = lambda B, V, kin, k, logits, cap, off, *outs: lib.tree_expand_step(
        B, V, kin, k, logits, None, cap, off, *outs, None, 0, None)
    outs = [P, P, P, P]
    for bad in ((0, 100, 1, 4, 40, 0), (2, 3, 1, 4, 40, 0), (2, 100, 1, 17, 40, 0),
                (2, 100, 17, 4, 400, 0), (2, 100, 2, 4, 40, 33), (2, 100, 1, 0, 40, 0),
                (2, 100, 1, 4, 40, -1)):
        B, V, kin, k, cap, off = bad
        assert exp(B, V, kin, k, P, cap, off, *outs) == SHAPE, bad
    assert exp(2, 100, 1, 4, None, 40, 0, *outs) == NULL
    misaligned = lib.tree_expand_step(2, 100, 1, 4, P, None, 40, 0, *outs,
                                      ctypes.c_void_p(0x100010), 1 << 20, None)
    assert misaligned == WORKSPACE
    assert lib.tv_expand_workspace_size(64, 1, 10) > lib.tv_expand_workspace_size(2, 1, 10) > 256
    assert lib.tv_expand_workspace_size(0, 1, 10) == 0 and lib.tv_expand_workspace_size(2, 1, 17) == 0
    for i in range(4):
        o = list(outs)
        o[i] = None
        assert exp(2, 100, 1, 4, P, 40, 0, *o) == NULL, i
    rr = lambda B, n, cap, m, *ptrs: lib.tree_rerank(B, n, cap, m, *ptrs, None, None)
    ptrs = [P] * 6
    for bad in ((0, 10, 10, 5), (2, 0, 10, 5), (2, 11, 10, 5), (2, 5000, 5000, 5), (2, 10, 10, 0)):
        assert rr(*bad, *ptrs) == SHAPE, bad
    for i in range(6):
        p = list(ptrs)
        p[i] = None
        assert rr(2, 10, 10, 5, *p) == NULL, i


def test_noalloc_sampler_host_errors():
    """Rejected before any launch: a batch above the static array, NULL
    arguments, a misaligned status word."""
    lib = tv.library()
    ptrs = [FAKE] * 9
    big = tv.sample_desc(_lib.TV_SAMPLE_STATIC_MAX_BATCH + 1, 1000, 8, 4)
    assert lib.tree_spec_sample_noalloc(ctypes.byref(big), *ptrs, FAKE, None) == SHAPE
    d = tv.sample_desc(4, 1000, 8, 4)
    assert lib.tree_spec_sample_noalloc(ctypes.byref(d), *ptrs, None, None) == NULL
    bad = list(ptrs)
    bad[0] = None
    assert lib.tree_spec_sample_noalloc(ctypes.byref(d), *bad, FAKE, None) == NULL
    assert lib.tree_spec_sample_noalloc(ctypes.byref(d), *ptrs, ctypes.c_void_p(0x100002),
                                        None) == WORKSPACE
    assert lib.tree_spec_sample_noalloc(None, *ptrs, FAKE, None) == NULL
