"""Seeded synthetic inputs for MLA speculative-decoding verify attention.

This package only *generates* inputs (random numbers, permutations, draft
trees, draft and target tokens, bf16 encoding of the generated floats). It holds none of the attention
arithmetic: both the CPU oracle and the GPU path consume what it produces, and
neither shares any other code with the other.
"""

from .gen import (  # noqa: F401
    LATENT_DIM,
    VALUE_DIM,
    NAN_CANARY,
    DEFAULT_SCALE,
    Workload,
    CONFIGS,
    bf16_from_f32,
    chain_mask,
    tree_mask_from_parents,
    random_parents,
    make_config,
    make_workload,
    make_tree_accept_case,
)
