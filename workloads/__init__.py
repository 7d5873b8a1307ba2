"""Seeded synthetic inputs for tree verification.

This package is shared by the CPU oracle, the tests and the benchmark. It
generates inputs only: tree shapes (parent arrays in topological order), paged
bf16/fp32 Q/K/V, target/draft logits, sibling tokens and uniforms. It contains
none of the verification arithmetic (no attention, no softmax-based acceptance,
no path selection): those live in the oracle and, independently, in the HIP
kernels.
"""
from .bf16 import f32_to_bf16_bits, bf16_bits_to_f32
from .trees import (expansion_vector_tree, random_tree, chain_tree, star_tree,
                    eagle2_tree, bfs_renumber, relabel_random_topological,
                    relabel_dfs, tree_depths)
from .inputs import (make_attention_inputs, make_sampler_inputs, make_construct_inputs,
                     gumbel_topk_tokens, independent_draw_tokens, AttentionInputs,
                     SamplerInputs, SparkInputs, make_spark_inputs)
from .configs import CONFIGS, make_config, Config

__all__ = [
    "f32_to_bf16_bits", "bf16_bits_to_f32",
    "expansion_vector_tree", "random_tree", "chain_tree", "star_tree",
    "eagle2_tree", "bfs_renumber", "relabel_random_topological", "relabel_dfs",
    "tree_depths", "make_attention_inputs", "make_sampler_inputs", "make_construct_inputs",
    "gumbel_topk_tokens", "independent_draw_tokens", "AttentionInputs", "SamplerInputs",
    "SparkInputs", "make_spark_inputs",
    "CONFIGS", "make_config", "Config",
]
