"""Paged Q/K/V, logits, sibling tokens and uniforms for tree verification.

Layouts (the boundary's layouts; see include/tree_verify.h):
  q        [T][Hq][D]                 T = node_indptr[B]
  k_pages  [num_pages][Hkv][16][D]    one 16-token page per (page, kv head)
  v_pages  [num_pages][Hkv][D][16]    V transposed within each page: the 16
                                      values of one channel are contiguous
  page_indptr [B+1], page_indices [page_indptr[B]]   logical -> physical page
  prefix_len [B]; node i of request r sits at logical position P_r + i
  node_indptr [B+1]; parent [T] request-local, parent[0] = -1
bf16 tensors are stored as uint16 bit patterns; fp32 as float32.
"""
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

from .bf16 import f32_to_bf16_bits

PAGE = 16


@dataclass
class AttentionInputs:
    dtype: str                 # "fp32" or "bf16"
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    q: np.ndarray              # float32 or uint16 bits
    k_pages: np.ndarray
    v_pages: np.ndarray
    page_indptr: np.ndarray    # int32 [B+1]
    page_indices: np.ndarray   # int32
    prefix_len: np.ndarray     # int32 [B]
    node_indptr: np.ndarray    # int32 [B+1]
    parent: np.ndarray         # int32 [T]
    sm_scale: float = 0.0
    page_size: int = PAGE

    @property
    def batch(self):
        return len(self.prefix_len)

    @property
    def num_pages(self):
        return self.k_pages.shape[0]

    @property
    def total_nodes(self):
        return int(self.node_indptr[-1])

    def nodes(self, r):
        return int(self.node_indptr[r + 1] - self.node_indptr[r])

    def kv_len(self, r):
        return int(self.prefix_len[r]) + self.nodes(r)

    @property
    def max_nodes(self):
        return max(self.nodes(r) for r in range(self.batch))

    @property
    def max_kv_len(self):
        return max(self.kv_len(r) for r in range(self.batch))

    @property
    def max_depth(self):
        md = 0
        for r in range(self.batch):
            a, b = int(self.node_indptr[r]), int(self.node_indptr[r + 1])
            d = np.zeros(b - a, dtype=np.int64)
            p = self.parent[a:b]
            for i in range(1, b - a):
                d[i] = d[p[i]] + 1
            md = max(md, int(d.max()) if len(d) else 0)
        return md


@dataclass
class SamplerInputs:
    vocab: int
    target_logits: np.ndarray          # float32 [T][V]
    draft_logits: Optional[np.ndarray] # float32 [T][V] or None (all T == 0)
    tokens: np.ndarray                 # int32 [T]
    node_indptr: np.ndarray            # int32 [B+1]
    parent: np.ndarray                 # int32 [T]
    temperature: np.ndarray            # float32 [B]
    uniforms: np.ndarray               # float32 [T][2]
    extra: dict = field(default_factory=dict)

    @property
    def batch(self):
        return len(self.temperature)

    @property
    def max_nodes(self):
        return int(np.max(np.diff(self.node_indptr)))


def _normal_f32(rng, shape, scale=1.0, chunk=1 << 24):
    out = np.empty(int(np.prod(shape)), dtype=np.float32)
    for s in range(0, out.size, chunk):
        e = min(out.size, s + chunk)
        out[s:e] = rng.standard_normal(e - s, dtype=np.float32)
        if scale != 1.0:
            out[s:e] *= np.float32(scale)
    return out.reshape(shape)


def _normal_bf16(rng, shape, chunk=1 << 24):
    out = np.empty(int(np.prod(shape)), dtype=np.uint16)
    for s in range(0, out.size, chunk):
        e = min(out.size, s + chunk)
        out[s:e] = f32_to_bf16_bits(rng.standard_normal(e - s, dtype=np.float32))
    return out.reshape(shape)


def make_attention_inputs(rng_qkv, rng_pages, trees, prefix_lens, num_q_heads,
                          num_kv_heads, head_dim, dtype="bf16", shuffle=True,
                          spare_pages=0):
    """Q/K/V ~ N(0,1) in a shared page pool with a (shuffled) page table."""
    B = len(trees)
    assert len(prefix_lens) == B
    node_counts = [len(t) for t in trees]
    node_indptr = np.zeros(B + 1, dtype=np.int32)
    node_indptr[1:] = np.cumsum(node_counts)
    parent = np.concatenate([np.asarray(t, dtype=np.int32) for t in trees])
    kv_lens = [int(p) + n for p, n in zip(prefix_lens, node_counts)]
    npages = [(L + PAGE - 1) // PAGE for L in kv_lens]
    page_indptr = np.zeros(B + 1, dtype=np.int32)
    page_indptr[1:] = np.cumsum(npages)
    num_pages = int(page_indptr[-1]) + int(spare_pages)
    perm = rng_pages.permutation(num_pages) if shuffle else np.arange(num_pages)
    page_indices = perm[: page_indptr[-1]].astype(np.int32)
    T = int(node_indptr[-1])
    if dtype == "bf16":
        gen = _normal_bf16
    elif dtype == "fp32":
        gen = _normal_f32
    else:
        raise ValueError(dtype)
    q = gen(rng_qkv, (T, num_q_heads, head_dim))
    k = gen(rng_qkv, (num_pages, num_kv_heads, PAGE, head_dim))
    v = gen(rng_qkv, (num_pages, num_kv_heads, head_dim, PAGE))
    return AttentionInputs(
        dtype=dtype, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
        head_dim=head_dim, q=q, k_pages=k, v_pages=v, page_indptr=page_indptr,
        page_indices=page_indices,
        prefix_len=np.asarray(prefix_lens, dtype=np.int32),
        node_indptr=node_indptr, parent=parent,
        sm_scale=1.0 / float(np.sqrt(head_dim)))


def repage(inp, rng, spare_pages=0):
    """Same logical K/V sequence, moved to a fresh random page placement."""
    B = inp.batch
    n_used = int(inp.page_indptr[-1])
    num_pages = n_used + int(spare_pages)
    perm = rng.permutation(num_pages).astype(np.int32)
    k = np.zeros((num_pages,) + inp.k_pages.shape[1:], dtype=inp.k_pages.dtype)
    v = np.zeros((num_pages,) + inp.v_pages.shape[1:], dtype=inp.v_pages.dtype)
    new_idx = perm[:n_used]
    k[new_idx] = inp.k_pages[inp.page_indices]
    v[new_idx] = inp.v_pages[inp.page_indices]
    out = AttentionInputs(**{**inp.__dict__})
    out.k_pages, out.v_pages, out.page_indices = k, v, new_idx.astype(np.int32)
    return out


def gumbel_topk_tokens(rng, draft_row, k, temperature):
    """k distinct tokens in draw order. T > 0: Gumbel-top-k on d/T, which is
    sequential sampling without replacement (RSD, survey page Timeline);
    T == 0: the k largest draft logits, largest first."""
    if k <= 0:
        return np.zeros(0, dtype=np.int32)
    if temperature > 0:
        score = draft_row.astype(np.float64) / float(temperature) + rng.gumbel(size=draft_row.shape[0])
    else:
        score = draft_row.astype(np.float64)
    top = np.argpartition(-score, k - 1)[:k]
    top = top[np.argsort(-score[top], kind="stable")]
    return top.astype(np.int32)


def independent_draw_tokens(rng, draft_row, k, temperature):
    """k tokens drawn independently (repeats allowed) from softmax(d/T), one
    Gumbel-max draw each: the sibling draws of the with-replacement rule
    (SpecInfer's MSS, survey page Taxonomy rule (b)). T == 0 requests are
    verified by greedy exact match, which needs distinct siblings: the k
    largest draft logits, as for the without-replacement draws."""
    if k <= 0:
        return np.zeros(0, dtype=np.int32)
    d = draft_row.astype(np.float64)
    if temperature <= 0:
        return gumbel_topk_tokens(rng, draft_row, k, 0.0)
    g = rng.gumbel(size=(k, d.shape[0]))
    return np.argmax(d[None, :] / float(temperature) + g, axis=1).astype(np.int32)


def make_sampler_inputs(rng_logits, rng_draws, rng_uniforms, trees, vocab,
                        temperatures, mode="correlated", sigma=2.0,
                        noise=0.5, need_draft=None, draws="without"):
    """Per-node target/draft logits (row i = distribution of the token after
    node i), sibling tokens drawn from the parent's draft row, and uniforms.

    mode "correlated": t ~ N(0, sigma), d = t + N(0, noise).
    mode "independent": t, d i.i.d. N(0, sigma).
    draws "without": distinct siblings (Gumbel-top-k); "with": independent
    draws, repeats allowed.
    """
    B = len(trees)
    node_counts = [len(t) for t in trees]
    node_indptr = np.zeros(B + 1, dtype=np.int32)
    node_indptr[1:] = np.cumsum(node_counts)
    parent = np.concatenate([np.asarray(t, dtype=np.int32) for t in trees])
    T = int(node_indptr[-1])
    temps = np.asarray(temperatures, dtype=np.float32)
    assert temps.shape == (B,)
    t = _normal_f32(rng_logits, (T, vocab), scale=sigma)
    if mode == "correlated":
        d = t + _normal_f32(rng_logits, (T, vocab), scale=noise)
    elif mode == "independent":
        d = _normal_f32(rng_logits, (T, vocab), scale=sigma)
    else:
        raise ValueError(mode)
    tokens = np.zeros(T, dtype=np.int32)
    for r in range(B):
        a = int(node_indptr[r])
        p = parent[a:int(node_indptr[r + 1])]
        n = len(p)
        children = [[] for _ in range(n)]
        for i in range(1, n):
            children[p[i]].append(i)
        for v in range(n):
            if children[v]:
                draw = gumbel_topk_tokens if draws == "without" else independent_draw_tokens
                toks = draw(rng_draws, d[a + v], len(children[v]), float(temps[r]))
                for c, x in zip(children[v], toks):
                    tokens[a + c] = x
    uniforms = rng_uniforms.random((T, 2), dtype=np.float32)
    if need_draft is None:
        need_draft = bool((temps > 0).any())
    return SamplerInputs(vocab=vocab, target_logits=t,
                         draft_logits=d if need_draft else None,
                         tokens=tokens, node_indptr=node_indptr, parent=parent,
                         temperature=temps, uniforms=uniforms)


def make_construct_inputs(rng, batch, vocab, k, rounds, sigma=2.0, integer_levels=0):
    """Draft logit rows for tree construction by expansion rounds: root
    [B][V] and, for rounds 2..rounds, [B][rounds-1][k][V] (the drafter's rows
    for the k frontier slots of each round). N(0, sigma) logits; with
    integer_levels > 0, logits are integers in [0, integer_levels) (many
    exact ties)."""
    shape_rows = (batch, max(rounds - 1, 0), k, vocab)
    if integer_levels:
        root = rng.integers(0, integer_levels, size=(batch, vocab)).astype(np.float32)
        rows = rng.integers(0, integer_levels, size=shape_rows).astype(np.float32)
    else:
        root = _normal_f32(rng, (batch, vocab), scale=sigma)
        rows = _normal_f32(rng, shape_rows, scale=sigma)
    return root, rows


@dataclass
class SparkInputs:
    """Inputs of TreeSpark's best-first construction (one drafter backbone
    pass per request plus the shared Markov head)."""
    base_logits: np.ndarray   # float32 [B][depths][V]: U_1..U_b of each request
    w1: np.ndarray            # uint16 bf16 bits [V][r]
    w2: np.ndarray            # uint16 bf16 bits [V][r]
    anchor: np.ndarray        # int32 [B]: the root (last committed) token
    temperature: np.ndarray   # float32 [B]
    theta: np.ndarray         # float32 [B]

    @property
    def batch(self):
        return self.base_logits.shape[0]

    @property
    def depths(self):
        return self.base_logits.shape[1]

    @property
    def vocab(self):
        return self.base_logits.shape[2]

    @property
    def rank(self):
        return self.w1.shape[1]


def make_spark_inputs(rng, batch, vocab=151936, depths=7, rank=256, temperatures=0.0,
                      thetas=0.05, scale_range=(4.0, 8.0), w_sigma=0.3):
    """Synthetic drafter output of TreeSpark's shape (block of b = 7 depths,
    Markov head of rank r = 256 over V = 151936): base logits
    U ~ s_r N(0, 1) with a per-request scale s_r ~ U(scale_range) (confident
    and diffuse rounds side by side), Markov factors W1, W2 ~ N(0, w_sigma)
    stored as bf16. temperatures / thetas: a value for every request or a
    per-request sequence."""
    V, r = int(vocab), int(rank)
    scales = rng.uniform(scale_range[0], scale_range[1], size=batch).astype(np.float32)
    U = _normal_f32(rng, (batch, depths, V))
    U *= scales[:, None, None]
    w1 = _normal_bf16_scaled(rng, (V, r), w_sigma)
    w2 = _normal_bf16_scaled(rng, (V, r), w_sigma)
    anchor = rng.integers(0, V, size=batch).astype(np.int32)
    temps = np.broadcast_to(np.asarray(temperatures, np.float32), (batch,)).copy()
    ths = np.broadcast_to(np.asarray(thetas, np.float32), (batch,)).copy()
    return SparkInputs(base_logits=U, w1=w1, w2=w2, anchor=anchor, temperature=temps, theta=ths)


def _normal_bf16_scaled(rng, shape, sigma, chunk=1 << 24):
    out = np.empty(int(np.prod(shape)), dtype=np.uint16)
    for s in range(0, out.size, chunk):
        e = min(out.size, s + chunk)
        out[s:e] = f32_to_bf16_bits(rng.standard_normal(e - s, dtype=np.float32) * np.float32(sigma))
    return out.reshape(shape)
