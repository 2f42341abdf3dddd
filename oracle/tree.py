"""Plain CPU oracle for draft-tree acceptance (test infrastructure only).

Nothing on the product path imports this module; only the test suite and the
benchmark's CPU-baseline leg use it. It shares no code with the GPU path.

What is computed. The pages list a tree-acceptance kernel source beside the
verify kernels (page "The Build That Unlocked 3-6x Decode Speedup", section
"Why This Build Was Different"; page "The Build Script Edit: How a Single
Line of Infrastructure Unlocked Custom CUDA Kernels on sm_120", section
"Input Knowledge Required") and say nothing about what it does; the plainest
reading of greedy speculative decoding over a draft tree, taken here:

* node 0 is the root of the tree (the last token already accepted); every
  other node i has a parent parents[i] < i and carries a draft token;
* target[i] is the token the target model chooses after the path root -> i
  (from the verify pass over that path);
* starting at the root, step to a child c of the current node whose draft
  token equals the target's choice at the current node, as long as one
  exists; when several children match, the one with the smallest index;
* only a child with a larger index than the current node counts (every
  well-formed tree has parents[i] < i, so this changes nothing there; on a
  malformed parent array it keeps the walk finite, at most Q - 1 steps);
* the result is the accepted path (root first), its length in draft tokens
  (path nodes minus the root), and the bonus token: the target's choice at
  the last accepted node.
"""

from __future__ import annotations

from typing import List, Tuple

import numpy as np


def tree_accept(parents: np.ndarray, draft: np.ndarray, target: np.ndarray) -> Tuple[int, List[int], int]:
    """One sequence: (accepted draft tokens, accepted path of node indices, bonus token)."""
    parents = [int(p) for p in parents]
    draft = [int(t) for t in draft]
    target = [int(t) for t in target]
    q = len(parents)
    path = [0]
    cur = 0
    while True:
        nxt = None
        for c in range(q):                      # smallest matching child first
            if c > cur and parents[c] == cur and draft[c] == target[cur]:
                nxt = c
                break
        if nxt is None:
            break
        path.append(nxt)
        cur = nxt
    return len(path) - 1, path, target[cur]


def tree_accept_batch(parents: np.ndarray, draft: np.ndarray, target: np.ndarray):
    """Batch form [B, Q] -> (accept_len int32 [B], accepted int32 [B, Q] padded with -1,
    bonus int32 [B])."""
    parents = np.asarray(parents)
    B, Q = parents.shape
    accept_len = np.zeros(B, np.int32)
    accepted = np.full((B, Q), -1, np.int32)
    bonus = np.zeros(B, np.int32)
    for b in range(B):
        n, path, tok = tree_accept(parents[b], draft[b], target[b])
        accept_len[b] = n
        accepted[b, :len(path)] = path
        bonus[b] = tok
    return accept_len, accepted, bonus
