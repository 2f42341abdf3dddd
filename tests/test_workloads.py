"""CPU tests of the seeded input generators (shapes, structure, determinism)."""

import numpy as np
import pytest

from workloads import (CONFIGS, NAN_CANARY, bf16_from_f32, chain_mask, make_config,
                       make_workload, random_parents, tree_mask_from_parents)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -9], np.float32)
    b = bf16_from_f32(x)
    assert list(b) == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x3F80]


def test_random_tree_structure():
    rng = np.random.default_rng(0)
    for q in (1, 2, 8, 16, 40):
        par = random_parents(q, rng)
        m = tree_mask_from_parents(par)
        assert np.array_equal(np.diag(m), np.ones(q, np.uint8))      # ancestor-or-self
        assert np.all(m[:, 0] == 1)                                   # root is everyone's ancestor
        assert np.array_equal(m, np.tril(m))                          # topological order
        assert m.sum(axis=1).max() <= 8                               # depth <= 8
        for i in range(1, q):                                         # parent row is a prefix of own row
            assert np.all(m[i] >= m[par[i]])


def test_chain_is_special_tree():
    q = 9
    par = np.arange(q) - 1
    assert np.array_equal(tree_mask_from_parents(par), chain_mask(q))


@pytest.mark.parametrize("name", ["tiny", "p4k"])
def test_config_structure(name):
    w = make_config(name)
    kw = CONFIGS[name]
    assert w.q.shape == (kw["B"], kw["Q"], kw["H"], 576)
    assert w.total_kv == int((w.prefix_lens.astype(np.int64) + w.Q).sum())
    assert len(np.unique(w.kv_indices)) == w.total_kv
    assert w.kv_indices.min() >= 0 and w.kv_indices.max() < w.num_slots
    unused = np.setdiff1d(np.arange(w.num_slots), w.kv_indices)
    assert np.all(w.kv_pool[unused] == NAN_CANARY)
    assert w.scale == np.float32(1 / np.sqrt(192))


def test_contiguous_and_seeded():
    a = make_config("p4k")
    assert np.array_equal(a.kv_indices, np.arange(4112, dtype=np.int32))
    b = make_config("p4k")
    assert np.array_equal(a.q, b.q) and np.array_equal(a.kv_pool, b.kv_pool)


def test_batch_prefix_draws_within_range():
    w = make_workload("b", [5], B=8, Q=8, H=1, prefix_range=(1024, 131072), mask="tree", num_slots=2_000_000)
    assert np.all((w.prefix_lens >= 1024) & (w.prefix_lens <= 131072))
    assert w.tree_mask.shape == (8, 8, 8)
