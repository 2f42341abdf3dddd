"""Pins for the oracles of the steps next to verify attention: KV defragmentation
and draft-tree acceptance. Each pin checks the oracle against something other
than itself: a hand-worked example, the attention oracle (an independent
function), a closed form for chains, or a brute-force search over root paths.
Planted mistakes in copies of the oracles must fail at least one pin."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from workloads import make_tree_accept_case, make_workload


# ---------------------------------------------------------------- KV defrag

def _defrag_pins(fn):
    # hand-worked: 4 source rows, positions [2, out of range, 0] into slots 1..3
    src = np.arange(4 * 576, dtype=np.uint16).reshape(4, 576)
    dst = np.full((5, 576), 7, np.uint16)
    new_pool, new_idx = fn(src, np.array([2, -1, 0], np.int32), dst, 1)
    want = dst.copy()
    want[1] = src[2]
    want[2] = 0
    want[3] = src[0]
    assert np.array_equal(new_pool, want)
    assert np.array_equal(new_idx, np.array([1, 2, 3], np.int32))
    # attention over the defragmented pool equals attention over the original
    w = make_workload("defrag_pin", [400], B=2, Q=4, H=4, prefix_lens=[90, 33], mask="tree", num_slots=512)
    dst = np.zeros((700, 576), np.uint16)
    new_pool, new_idx = fn(w.kv_pool, w.kv_indices, dst, 100)
    o1, l1 = oracle.verify_attention(w.q, w.kv_pool, w.kv_indices, w.prefix_lens, w.tree_mask, w.scale)
    o2, l2 = oracle.verify_attention(w.q, new_pool, new_idx, w.prefix_lens, w.tree_mask, w.scale)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # rows outside the destination run are untouched
    n = len(w.kv_indices)
    assert np.array_equal(new_pool[:100], dst[:100]) and np.array_equal(new_pool[100 + n:], dst[100 + n:])


def test_defrag_pins():
    _defrag_pins(oracle.defrag)


def test_defrag_rejects_run_outside_pool():
    with pytest.raises(ValueError):
        oracle.defrag(np.zeros((4, 576), np.uint16), np.zeros(3, np.int32), np.zeros((4, 576), np.uint16), 2)


def _defrag_off_by_one(src, idx, dst, base):
    out, new = oracle.defrag(src, idx, dst, base)
    return out, new + 1


def _defrag_reversed(src, idx, dst, base):
    return oracle.defrag(src, np.asarray(idx)[::-1].copy(), dst, base)


def _defrag_no_zero_rows(src, idx, dst, base):
    idx = np.clip(np.asarray(idx), 0, np.asarray(src).shape[0] - 1).astype(np.int32)
    return oracle.defrag(src, idx, dst, base)


@pytest.mark.parametrize("mutant", [_defrag_off_by_one, _defrag_reversed, _defrag_no_zero_rows])
def test_defrag_pins_catch_planted_mistakes(mutant):
    with pytest.raises(AssertionError):
        _defrag_pins(mutant)


# ------------------------------------------------------------ tree acceptance

def _root_paths(parents):
    """All root-to-node paths of a tree given by its parent array (brute force)."""
    q = len(parents)
    paths = []

    def walk(path):
        paths.append(list(path))
        for c in range(1, q):
            if parents[c] == path[-1]:
                walk(path + [c])

    walk([0])
    return paths


def _tree_pins(fn):
    # hand-worked example
    n, path, bonus = fn(np.array([-1, 0, 0, 1, 2]), np.array([9, 5, 7, 8, 4]), np.array([7, 1, 4, 3, 6]))
    assert (n, path, bonus) == (2, [0, 2, 4], 6)
    # all drafts wrong: only the root, bonus = the target's choice at the root
    assert fn(np.array([-1, 0, 1]), np.array([0, 1, 2]), np.array([5, 6, 7])) == (0, [0], 5)
    # two matching siblings: the smaller index wins
    assert fn(np.array([-1, 0, 0]), np.array([0, 3, 3]), np.array([3, 8, 9]))[1] == [0, 1]
    # malformed parent arrays: only a child with a larger index than the current
    # node counts (node 1 names the later node 2 as its parent and is skipped;
    # a node that is its own parent is never a child of anything else)
    assert fn(np.array([-1, 2, 0]), np.array([0, 5, 3]), np.array([3, 9, 5])) == (1, [0, 2], 5)
    assert fn(np.array([-1, 1, 0, 2]), np.array([0, 4, 4, 6]), np.array([4, 4, 6, 1])) == (2, [0, 2, 3], 1)
    # chains: the accepted length is the length of the leading run of matches
    par, dr, tg = make_tree_accept_case(41, 16, 12, vocab=4, p_follow=0.8, chain=True)
    for b in range(16):
        match = dr[b, 1:] == tg[b, :-1]
        k = int(np.argmin(match)) if not match.all() else len(match)
        n, path, bonus = fn(par[b], dr[b], tg[b])
        assert n == k and path == list(range(k + 1)) and bonus == tg[b, k]
    # trees with distinct sibling drafts: the accepted path is the unique
    # longest root path whose every step matches (brute force)
    par, dr, tg = make_tree_accept_case(42, 24, 16, vocab=50000, p_follow=0.85)
    for b in range(24):
        for i in range(16):
            kids = [c for c in range(1, 16) if par[b, c] == i]
            assert len({int(dr[b, c]) for c in kids}) == len(kids)
        best = max((p for p in _root_paths(par[b])
                    if all(dr[b, p[s + 1]] == tg[b, p[s]] for s in range(len(p) - 1))), key=len)
        n, path, bonus = fn(par[b], dr[b], tg[b])
        assert path == best and n == len(best) - 1 and bonus == tg[b, best[-1]]


def test_tree_accept_pins():
    _tree_pins(oracle.tree_accept)


def test_tree_accept_batch_matches_single():
    par, dr, tg = make_tree_accept_case(43, 5, 9)
    n, acc, bonus = oracle.tree_accept_batch(par, dr, tg)
    for b in range(5):
        nb, path, tok = oracle.tree_accept(par[b], dr[b], tg[b])
        assert n[b] == nb and bonus[b] == tok and list(acc[b, :nb + 1]) == path and np.all(acc[b, nb + 1:] == -1)


def _tree_any_index_child(parents, draft, target):
    """Steps to a matching child whatever its index (no cycle in the pins' trees)."""
    parents, draft, target = list(parents), list(draft), list(target)
    q, cur, path = len(parents), 0, [0]
    while True:
        m = [c for c in range(1, q) if parents[c] == cur and draft[c] == target[cur] and c not in path]
        if not m:
            return len(path) - 1, path, target[cur]
        cur = m[0]
        path.append(cur)


def _tree_largest_child(parents, draft, target):
    parents, draft, target = list(parents), list(draft), list(target)
    q, cur, path = len(parents), 0, [0]
    while True:
        m = [c for c in range(1, q) if parents[c] == cur and draft[c] == target[cur]]
        if not m:
            return len(path) - 1, path, target[cur]
        cur = m[-1]
        path.append(cur)


def _tree_bonus_from_parent(parents, draft, target):
    n, path, _ = oracle.tree_accept(parents, draft, target)
    return n, path, int(target[path[-2]]) if len(path) > 1 else int(target[0])


def _tree_counts_root(parents, draft, target):
    n, path, bonus = oracle.tree_accept(parents, draft, target)
    return n + 1, path, bonus


def _tree_matches_own_token(parents, draft, target):
    parents, draft, target = list(parents), list(draft), list(target)
    q, cur, path = len(parents), 0, [0]
    while True:
        m = [c for c in range(1, q) if parents[c] == cur and draft[c] == target[c]]
        if not m:
            return len(path) - 1, path, target[cur]
        cur = m[0]
        path.append(cur)


@pytest.mark.parametrize("mutant", [_tree_largest_child, _tree_bonus_from_parent, _tree_counts_root,
                                    _tree_matches_own_token, _tree_any_index_child])
def test_tree_pins_catch_planted_mistakes(mutant):
    with pytest.raises(AssertionError):
        _tree_pins(mutant)
