"""Seeded input generators for MLA verify attention.

The workload shapes follow the problem the pages describe (the paged bf16
verify kernel of page "The Build That Bridged Design and Deployment: Compiling
the Custom sm_120 Verify Kernel", section "What This Build Achieves: The
paged+bf16 Kernel"): several requests per launch, each with its own prefix
length, a page_size-1 KV pool addressed through ``kv_indices``, and a small
q x q visibility matrix for the speculative tail. Latent width 576 with the
first 512 dims as values, the 1/sqrt(192) scale, and the five concrete
configurations are the workload definition this package fixes; they are not
printed on the pages.

Every array is produced from ``numpy.random.default_rng([config, stream])``
with streams 0 = prefix lengths, 1 = draft tree, 2 = kv slot permutation,
3 = queries, 4 = latent rows. bf16 values are carried as their uint16 bit
patterns. Pool rows that no ``kv_indices`` entry references hold a bf16 NaN
(0x7FC0) so that any stray read poisons the result.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional, Sequence, Union

import numpy as np

LATENT_DIM = 576          # width of one compressed latent row (keys)
VALUE_DIM = 512           # leading dims of the same row that serve as values
NAN_CANARY = 0x7FC0       # bf16 quiet NaN written into unreferenced pool rows
DEFAULT_SCALE = np.float32(1.0 / np.sqrt(192.0))


def bf16_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even).

    Returns the uint16 bit patterns. Only used to encode generated normals, so
    NaN/inf inputs are not special-cased.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def chain_mask(q: int) -> np.ndarray:
    """Causal chain over the speculative tail: query i sees tail keys t <= i."""
    return np.tril(np.ones((q, q), dtype=np.uint8))


def random_parents(q: int, rng: np.random.Generator, max_depth: int = 8) -> np.ndarray:
    """Seeded draft tree in topological order.

    parent[0] = -1 (root, depth 1); for i >= 1 the parent is drawn uniformly
    from the earlier nodes whose depth is below ``max_depth``.
    """
    parent = np.full(q, -1, dtype=np.int64)
    depth = np.zeros(q, dtype=np.int64)
    if q == 0:
        return parent
    depth[0] = 1
    for i in range(1, q):
        cands = [j for j in range(i) if depth[j] < max_depth]
        parent[i] = cands[int(rng.integers(len(cands)))]
        depth[i] = depth[parent[i]] + 1
    return parent


def tree_mask_from_parents(parent: np.ndarray) -> np.ndarray:
    """mask[i][t] = 1 iff tail node t lies on the path root -> i (i included)."""
    q = len(parent)
    m = np.zeros((q, q), dtype=np.uint8)
    for i in range(q):
        j = i
        while j >= 0:
            m[i, j] = 1
            j = int(parent[j])
    return m


@dataclass
class Workload:
    """One verify-attention call's inputs (host numpy arrays)."""

    name: str
    q: np.ndarray            # uint16 bf16 bits [B, Q, H, 576]
    kv_pool: np.ndarray      # uint16 bf16 bits [num_slots, 576]
    kv_indices: np.ndarray   # int32 [total_kv]; per sequence: prefix slots, then the Q tail slots
    prefix_lens: np.ndarray  # int32 [B]
    tree_mask: np.ndarray    # uint8 [B, Q, Q]
    scale: np.float32
    meta: Dict[str, object] = field(default_factory=dict)

    @property
    def B(self) -> int:
        return int(self.q.shape[0])

    @property
    def Q(self) -> int:
        return int(self.q.shape[1])

    @property
    def H(self) -> int:
        return int(self.q.shape[2])

    @property
    def num_slots(self) -> int:
        return int(self.kv_pool.shape[0])

    @property
    def total_kv(self) -> int:
        return int(self.kv_indices.shape[0])


def make_workload(
    name: str,
    seed: Union[int, Sequence[int]],
    B: int,
    Q: int,
    H: int,
    prefix_lens: Union[Sequence[int], np.ndarray, None] = None,
    prefix_range: Optional[tuple] = None,
    mask: Union[str, np.ndarray] = "chain",
    num_slots: Optional[int] = None,
    contiguous: bool = False,
    q_scale: float = 1.0,
    scale: Optional[float] = None,
    q_zero: bool = False,
) -> Workload:
    """Build a workload from explicit sizes.

    ``mask`` is "chain", "tree" (seeded random tree per sequence, depth <= 8),
    "identity", "none" (tail invisible) or an explicit uint8 array [B, Q, Q].
    ``prefix_range`` = (lo, hi) draws prefix lengths uniformly (inclusive).
    """
    seed = [seed] if np.isscalar(seed) else list(seed)
    rng = lambda stream: np.random.default_rng(seed + [stream])  # noqa: E731
    if prefix_lens is None:
        lo, hi = prefix_range
        prefix_lens = rng(0).integers(lo, hi, size=B, endpoint=True)
    prefix_lens = np.asarray(prefix_lens, dtype=np.int32).reshape(B)
    seq_kv = prefix_lens.astype(np.int64) + Q
    total_kv = int(seq_kv.sum())

    if isinstance(mask, str):
        if mask == "chain":
            tm = np.broadcast_to(chain_mask(Q), (B, Q, Q)).copy()
        elif mask == "identity":
            tm = np.broadcast_to(np.eye(Q, dtype=np.uint8), (B, Q, Q)).copy()
        elif mask == "none":
            tm = np.zeros((B, Q, Q), dtype=np.uint8)
        elif mask == "tree":
            r = rng(1)
            tm = np.stack([tree_mask_from_parents(random_parents(Q, r)) for _ in range(B)])
        else:
            raise ValueError(mask)
    else:
        tm = np.ascontiguousarray(mask, dtype=np.uint8).reshape(B, Q, Q)

    if num_slots is None:
        num_slots = total_kv
    if num_slots < total_kv and not contiguous:
        raise ValueError("pool smaller than the number of referenced positions")
    if contiguous:
        kv_indices = np.arange(total_kv, dtype=np.int32)
        num_slots = max(num_slots, total_kv)
    else:
        kv_indices = rng(2).permutation(num_slots)[:total_kv].astype(np.int32)

    qf = rng(3).standard_normal((B, Q, H, LATENT_DIM), dtype=np.float32)
    if q_zero:
        qf[...] = 0.0
    elif q_scale != 1.0:
        qf *= np.float32(q_scale)
    q = bf16_from_f32(qf)

    rows = bf16_from_f32(rng(4).standard_normal((total_kv, LATENT_DIM), dtype=np.float32))
    pool = np.full((num_slots, LATENT_DIM), NAN_CANARY, dtype=np.uint16)
    pool[kv_indices] = rows

    return Workload(
        name=name,
        q=q,
        kv_pool=pool,
        kv_indices=kv_indices,
        prefix_lens=prefix_lens,
        tree_mask=tm,
        scale=np.float32(DEFAULT_SCALE if scale is None else scale),
        meta={"seed": seed, "mask": mask if isinstance(mask, str) else "explicit",
              "contiguous": contiguous, "q_scale": q_scale},
    )


# The five workloads (plus the per-rank shape of 8-way head sharding).
# Each entry: seed number, then make_workload keyword arguments.
CONFIGS: Dict[str, dict] = {
    "tiny": dict(seed=1, B=1, Q=4, H=8, prefix_lens=[256], mask="chain", num_slots=1024),
    "p4k": dict(seed=2, B=1, Q=16, H=64, prefix_lens=[4096], mask="chain", contiguous=True),
    "tree32k": dict(seed=3, B=1, Q=16, H=64, prefix_lens=[32768], mask="tree", num_slots=262144),
    "long185k": dict(seed=4, B=1, Q=16, H=64, prefix_lens=[185000], mask="chain",
                     num_slots=524288, q_scale=0.5),
    "batch8": dict(seed=5, B=8, Q=8, H=64, prefix_range=(1024, 131072), mask="tree",
                   num_slots=2097152),
    "long185k_h8": dict(seed=6, B=1, Q=16, H=8, prefix_lens=[185000], mask="chain",
                        num_slots=524288, q_scale=0.5),
    # The same two shapes over a defragmented cache (contiguous kv_indices).
    "long185k_contig": dict(seed=4, B=1, Q=16, H=64, prefix_lens=[185000], mask="chain",
                            contiguous=True, q_scale=0.5),
    "long185k_h8_contig": dict(seed=6, B=1, Q=16, H=8, prefix_lens=[185000], mask="chain",
                               contiguous=True, q_scale=0.5),
}

CONFIG_ORDER = ["tiny", "p4k", "tree32k", "long185k", "batch8", "long185k_h8"]


def make_config(name: str) -> Workload:
    """Generate one named configuration (see ``CONFIGS``)."""
    kw = dict(CONFIGS[name])
    seed = kw.pop("seed")
    return make_workload(name, seed, **kw)


def make_tree_accept_case(seed: int, B: int, Q: int, vocab: int = 32000, p_follow: float = 0.7,
                          max_depth: int = 8, chain: bool = False):
    """Seeded inputs for draft-tree acceptance: parents int32 [B, Q] (parents[b, 0] = -1,
    parents[b, i] < i), draft tokens and target tokens int32 [B, Q].

    Draft tokens are uniform over the vocabulary. The target token at node i
    copies the draft token of one of i's children (chosen uniformly) with
    probability p_follow, so that paths of several tokens occur; otherwise it
    is uniform too. Streams: 0 = tree shape, 1 = draft tokens, 2 = target tokens.
    """
    g_tree = np.random.default_rng([seed, 0])
    g_draft = np.random.default_rng([seed, 1])
    g_tgt = np.random.default_rng([seed, 2])
    parents = np.empty((B, Q), np.int32)
    draft = g_draft.integers(0, vocab, size=(B, Q), dtype=np.int64).astype(np.int32)
    target = np.empty((B, Q), np.int32)
    for b in range(B):
        par = np.arange(-1, Q - 1, dtype=np.int32) if chain else random_parents(Q, g_tree, max_depth)
        parents[b] = par
        for i in range(Q):
            kids = np.nonzero(par == i)[0]
            kids = kids[kids != 0]
            if kids.size and g_tgt.random() < p_follow:
                target[b, i] = draft[b, kids[g_tgt.integers(0, kids.size)]]
            else:
                target[b, i] = g_tgt.integers(0, vocab)
    return parents, draft, target
