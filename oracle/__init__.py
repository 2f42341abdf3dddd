"""CPU oracle for MLA speculative-decoding verify attention and the steps next to
it, KV defragmentation and draft-tree acceptance (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this package; the product path never imports it. Every function is plain
fp64 numpy (or pure Python for the brute force) and shares no code with the
GPU implementation.

Parity status: every function here is pinned by the CPU test suite against
closed forms, invariants, a pure-Python brute force, independent rounding
routines (Python's own binary16 packing, torch's bfloat16 conversion) and
torch's scaled_dot_product_attention in fp64; none is "parity unpinned".
"""

from .attention import (  # noqa: F401
    LATENT,
    VALUE,
    decode_bf16,
    sequence_offsets,
    gather_latents,
    visibility,
    masked_softmax_rows,
    verify_attention,
    partial_attention,
    lse_merge,
    split_merge_attention,
    online_softmax_attention,
    chunked_attention_model,
    round_to,
    brute_force,
)
from .kvcache import defrag  # noqa: F401
from .tree import tree_accept, tree_accept_batch  # noqa: F401
