"""The five synthetic workloads, restated as seeded recipes.

  tiny     1 request; 4 q / 1 kv heads, D 64, fp32; prefix 128; static tree
           from expansion vector <1,1,3,1,1> (12 rows incl. root); sampler on
           V = 512 with t, d i.i.d. N(0, 2), T = 1.
  eagle2   1 request; 32 q / 8 kv heads, D 128, bf16; prefix 2048; EAGLE-2
           shaped 60-row tree of depth 6 (top-k 8, N(0, 1.5) draft logits).
  sequoia  1 request; same layer; prefix 8192; random 768-row tree of depth
           12; sampler V = 151936, t ~ N(0,2), d = t + N(0,0.5), T = 1.
  batched  16 requests; prefixes U{1024..4096}; 32-row trees, depth <= 8;
           shuffled page pool.
  highload 64 requests; prefixes U{512..8192}; per-request budget from
           {8-row chain, 16-row tree, 32-row tree}; sampler V = 151936 with
           T in {0, 0.5, 1} (one value for all, or "mixed" per request).

Config i draws from np.random.SeedSequence(i) spawned into the streams
[tree, qkv, pages, logits, draws, uniforms].
"""
from dataclasses import dataclass
from typing import Optional

import numpy as np

from .trees import expansion_vector_tree, eagle2_tree, random_tree, chain_tree
from .inputs import make_attention_inputs, make_sampler_inputs

VOCAB = 151936


@dataclass
class Config:
    name: str
    seed_index: int
    attn: object = None
    sampler: object = None
    trees: list = None
    prefix_lens: list = None
    meta: dict = None


CONFIGS = ("tiny", "eagle2", "sequoia", "batched", "highload")


def _streams(index, seed_offset=0):
    ss = np.random.SeedSequence(index + seed_offset)
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(6)]


def make_config(name, attention=True, sampler=True, batch=None, vocab=None,
                temperature="mixed", seed_offset=0, mode=None, draws="without"):
    """Build a config's inputs.

    batch: keep only the first ``batch`` requests (trees and prefixes are
    drawn for the full batch first, so a sub-batch is a prefix of the full
    workload). vocab: override the sampler vocabulary (tests).
    temperature (highload only): "mixed" or a float applied to all requests.
    """
    index = CONFIGS.index(name)
    g_tree, g_qkv, g_pages, g_logits, g_draws, g_unif = _streams(index, seed_offset)
    meta = {}
    if name == "tiny":
        trees = [expansion_vector_tree([1, 1, 3, 1, 1])]
        prefix = [128]
        layer = dict(num_q_heads=4, num_kv_heads=1, head_dim=64, dtype="fp32")
        V = 512
        temps = [1.0]
        smode = "independent"
    elif name == "eagle2":
        t, hist = eagle2_tree(g_tree, return_stats=True)
        meta["depth_histogram"] = hist.tolist()
        trees = [t]
        prefix = [2048]
        layer = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16")
        V = None
        temps = None
        smode = None
    elif name == "sequoia":
        trees = [random_tree(g_tree, 768, depth_cap=12, spine_depth=12)]
        prefix = [8192]
        layer = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16")
        V = VOCAB
        temps = [1.0]
        smode = "correlated"
    elif name == "batched":
        B = 16
        prefix = [int(x) for x in g_tree.integers(1024, 4097, size=B)]
        trees = [random_tree(g_tree, 32, depth_cap=8) for _ in range(B)]
        layer = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16")
        V = None
        temps = None
        smode = None
    elif name == "highload":
        B = 64
        prefix = [int(x) for x in g_tree.integers(512, 8193, size=B)]
        kinds = g_tree.integers(0, 3, size=B)
        trees = []
        for k in kinds:
            if k == 0:
                trees.append(chain_tree(8))
            elif k == 1:
                trees.append(random_tree(g_tree, 16, depth_cap=8))
            else:
                trees.append(random_tree(g_tree, 32, depth_cap=8))
        meta["budget_kinds"] = kinds.tolist()
        layer = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16")
        V = VOCAB
        tchoice = g_tree.integers(0, 3, size=B)
        if temperature == "mixed":
            temps = [(0.0, 0.5, 1.0)[c] for c in tchoice]
        else:
            temps = [float(temperature)] * B
        smode = "correlated"
    else:
        raise ValueError(name)
    if mode is not None:
        smode = mode
    if batch is not None:
        trees, prefix = trees[:batch], prefix[:batch]
        if temps is not None:
            temps = temps[:batch]
    cfg = Config(name=name, seed_index=index, trees=trees, prefix_lens=prefix, meta=meta)
    if attention:
        cfg.attn = make_attention_inputs(g_qkv, g_pages, trees, prefix, **layer)
    if sampler and V is not None:
        cfg.sampler = make_sampler_inputs(g_logits, g_draws, g_unif, trees,
                                          vocab if vocab is not None else V,
                                          temps, mode=smode, draws=draws)
    return cfg
