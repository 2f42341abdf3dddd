"""Plain CPU oracle for KV-cache defragmentation (test infrastructure only).

Nothing on the product path imports this module; only the test suite and the
benchmark's CPU-baseline leg use it. It shares no code with the GPU path.

What is computed. The pages name KV defragmentation as the step planned right
after the verify kernel (page "The Build That Unlocked 3-6x Decode Speedup",
sections "The Context: A Custom Kernel for an Unsupported Architecture" and
"The Broader Significance") and give nothing more; the plainest reading,
taken here: the latent rows a sequence's ``kv_indices`` point to, scattered
over the pool at page_size 1, are copied in position order into a contiguous
run of destination slots, and the index table is rewritten to point there.
For position j of the n given positions

    dst_pool[dst_base + j] = src_pool[kv_indices[j]]   (a zero row if the
                                                         slot is out of range)
    new_indices[j]         = dst_base + j

and every other destination row is left as it was. Attention over
(dst_pool, new_indices) then equals attention over (src_pool, kv_indices)
exactly, because it sees the same rows in the same order.
"""

from __future__ import annotations

from typing import Tuple

import numpy as np


def defrag(src_pool: np.ndarray, kv_indices: np.ndarray, dst_pool: np.ndarray,
           dst_base: int) -> Tuple[np.ndarray, np.ndarray]:
    """Return (new destination pool, new index table); inputs are not modified.

    src_pool, dst_pool: uint16 [slots, 576] (bf16 bit patterns); kv_indices:
    int32 [n]. The destination run [dst_base, dst_base + n) must lie inside
    dst_pool.
    """
    src_pool = np.asarray(src_pool)
    idx = np.asarray(kv_indices, dtype=np.int64)
    n = idx.shape[0]
    out = np.array(dst_pool, copy=True)
    if not (0 <= dst_base and dst_base + n <= out.shape[0]):
        raise ValueError("destination run outside the destination pool")
    slots = src_pool.shape[0]
    for j in range(n):
        s = idx[j]
        out[dst_base + j] = src_pool[s] if 0 <= s < slots else 0
    new_indices = np.arange(dst_base, dst_base + n, dtype=np.int32)
    return out, new_indices
