"""Seeded synthetic inputs for verification attention.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic.  Both the fp64 oracle (``oracle/``) and the HIP path
(``long_context_tree_verify_amd``) consume what it produces, so neither side
has to trust the other's input handling.

Workloads follow the shapes the LongSpec page (section 2.C, "Hybrid Tree
Attention") and the Dustin page (sections "Methodology 1" and "Verification
workflow") describe: a long cached prefix, a draft block or tree of N tokens
whose K/V sit at the cache tail, and (sparse case) a fixed-size per-KV-head
index set made of attention sinks, a recent window and a ranked fill.
"""

from .gen import (  # noqa: F401
    WORKLOADS,
    Workload,
    VerifyInputs,
    bf16_bits_to_f32,
    block_masks,
    random_masks,
    f32_to_bf16_bits,
    heavy_importance_maps,
    importance_maps,
    make_inputs,
    random_tree_parents,
    to_paged,
    chain_parents,
    uniform_parents,
    zipf_index_set,
    zipf_ranked_draw,
)
