"""CPU tests pinning the fp64 oracle (no GPU needed)."""

from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
import oracle.attention as oa
from workloads import make_workload, make_config, bf16_from_f32
from oracle_pins import ALL_PINS, torch_decode


# --------------------------------------------------------------------------
# The definition against every pin
# --------------------------------------------------------------------------

@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_verify_attention_pins(pin):
    pin(oracle.verify_attention)


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_online_softmax_pins(pin):
    """The tile-streaming restatement (ragged 7-key tiles) meets the same pins."""
    pin(lambda *a: oracle.online_softmax_attention(*a, tile=7))


def _random_bounds(prefix_lens, Q, rng):
    bounds = []
    for P in prefix_lens:
        N = int(P) + Q
        k = int(rng.integers(0, min(N, 6)))
        inner = sorted(set(int(x) for x in rng.integers(1, N, size=k))) if N > 1 else []
        bounds.append([0] + inner + [N])
    return bounds


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_split_merge_pins(pin):
    rng = np.random.default_rng(11)
    pin(lambda q, kv, idx, pl, tm, sc: oracle.split_merge_attention(
        q, kv, idx, pl, tm, sc, _random_bounds(pl, q.shape[1], rng)))


SMALL_PINS = [p for p in ALL_PINS if p.__name__ in (
    "pin_single_key", "pin_two_keys", "pin_brute_force", "pin_empty_visible_set", "pin_worked_example")]


@pytest.mark.parametrize("pin", SMALL_PINS, ids=lambda p: p.__name__)
def test_brute_force_pins(pin):
    pin(oracle.brute_force)


# --------------------------------------------------------------------------
# Invariants of the method
# --------------------------------------------------------------------------

def test_split_merge_invariant_with_empty_splits():
    """Any contiguous partition, including splits with no visible key for some
    rows (tail-only splits under a tree mask), merges to the unsplit result."""
    w = make_workload("inv", [201], B=2, Q=6, H=3, prefix_lens=[0, 37], mask="tree", num_slots=100)
    ref = oracle.verify_attention(w.q, w.kv_pool, w.kv_indices, w.prefix_lens, w.tree_mask, w.scale)
    for bounds in ([[0, 1, 2, 3, 4, 5, 6], [0, 43]],
                   [[0, 6], [0, 37, 38, 40, 43]],
                   [[0, 3, 6], [0, 1, 36, 37, 42, 43]]):
        out, lse = oracle.split_merge_attention(w.q, w.kv_pool, w.kv_indices, w.prefix_lens,
                                                w.tree_mask, w.scale, bounds)
        assert np.allclose(out, ref[0], rtol=0, atol=1e-12)
        assert np.allclose(lse, ref[1], rtol=0, atol=1e-12)


def test_lse_merge_handles_all_empty():
    o = [np.zeros((2, 3)), np.zeros((2, 3))]
    l = [np.array([-np.inf, 1.0]), np.array([-np.inf, -np.inf])]
    out, lse = oracle.lse_merge(o, l)
    assert lse[0] == -np.inf and np.all(out[0] == 0)
    assert lse[1] == 1.0


def test_relabel_invariance_bitwise():
    """Permuting pool rows together with kv_indices gives bitwise-identical fp64 results."""
    w = make_workload("relabel", [202], B=2, Q=4, H=2, prefix_lens=[20, 3], mask="tree", num_slots=64)
    out, lse = oracle.verify_attention(w.q, w.kv_pool, w.kv_indices, w.prefix_lens, w.tree_mask, w.scale)
    perm = np.random.default_rng(5).permutation(64)
    pool2 = np.empty_like(w.kv_pool)
    pool2[perm] = w.kv_pool
    o2, l2 = oracle.verify_attention(w.q, pool2, perm[w.kv_indices].astype(np.int32),
                                     w.prefix_lens, w.tree_mask, w.scale)
    assert np.array_equal(out, o2) and np.array_equal(lse, l2)


def test_decode_bf16_known_values():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0xFF80, 0x0001, 0x7F7F, 0x3E80], np.uint16)
    v = oracle.decode_bf16(bits)
    assert list(v[:6]) == [1.0, -2.0, 0.0, -0.0, np.inf, -np.inf]
    assert v[6] == 2.0 ** -133
    assert v[7] == (2 - 2 ** -7) * 2.0 ** 127
    assert v[8] == 0.25
    assert np.isnan(oracle.decode_bf16(np.array([0x7FC0], np.uint16)))[0]
    rnd = np.random.default_rng(0).integers(0, 1 << 16, 5000).astype(np.uint16)
    assert np.array_equal(oracle.decode_bf16(rnd), torch_decode(rnd), equal_nan=True)


def test_oracle_never_reads_unreferenced_rows():
    """Unreferenced pool rows hold NaN canaries; a finite result proves they are never gathered."""
    w = make_config("tiny")
    assert np.isnan(oracle.decode_bf16(w.kv_pool)).any()
    out, lse = oracle.verify_attention(w.q, w.kv_pool, w.kv_indices, w.prefix_lens, w.tree_mask, w.scale)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))


def test_heads_subset_matches_full():
    w = make_workload("heads", [203], B=1, Q=3, H=5, prefix_lens=[30], mask="chain", num_slots=40)
    out, lse = oracle.verify_attention(w.q, w.kv_pool, w.kv_indices, w.prefix_lens, w.tree_mask, w.scale)
    o2, l2 = oracle.verify_attention(w.q, w.kv_pool, w.kv_indices, w.prefix_lens, w.tree_mask, w.scale,
                                     heads=[1, 4])
    assert np.array_equal(out[:, :, [1, 4]], o2[:, :, [1, 4]])
    assert np.array_equal(lse[:, :, [1, 4]], l2[:, :, [1, 4]])


def test_head_grouping_does_not_change_result():
    """The bounded score block (head grouping) is an implementation detail only."""
    w = make_workload("grp", [204], B=2, Q=3, H=6, prefix_lens=[50, 9], mask="tree", num_slots=80)
    a = oracle.verify_attention(w.q, w.kv_pool, w.kv_indices, w.prefix_lens, w.tree_mask, w.scale)
    b = oracle.verify_attention(w.q, w.kv_pool, w.kv_indices, w.prefix_lens, w.tree_mask, w.scale,
                                max_score_bytes=1)
    assert np.allclose(a[0], b[0], rtol=0, atol=1e-14) and np.allclose(a[1], b[1], rtol=0, atol=1e-14)


# --------------------------------------------------------------------------
# Planted mistakes: every plausible slip in the oracle must trip some pin
# --------------------------------------------------------------------------

def _vis_no_diag(P, tm):
    v = _orig["visibility"](P, tm)
    Q = tm.shape[0]
    v[np.arange(Q), P + np.arange(Q)] = False
    return v


def _vis_transposed(P, tm):
    return _orig["visibility"](P, np.asarray(tm).T)


def _vis_prefix_short(P, tm):
    v = _orig["visibility"](P, tm)
    if P > 0:
        v[:, P - 1] = False
    return v


def _decode_shift15(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(15)
    return b.view(np.float32).astype(np.float64)


def _gather_skip_one(pool, idx, start, count):
    sl = np.asarray(idx[start + 1:start + 1 + count], dtype=np.int64)
    if len(sl) < count:
        sl = np.concatenate([sl, np.asarray(idx[start:start + count - len(sl)], dtype=np.int64)])
    return oa.decode_bf16(pool[sl])


def _offsets_without_tail(pl, Q):
    n = np.asarray(pl, dtype=np.int64)          # forgets the Q tail slots per sequence
    off = np.zeros(len(n) + 1, dtype=np.int64)
    off[1:] = np.cumsum(n)
    return off


def _softmax_log2(scores, vis, V):
    o, l = _orig["masked_softmax_rows"](scores, vis, V)
    return o, l / math.log(2.0)


def _softmax_unmasked(scores, vis, V):
    return _orig["masked_softmax_rows"](scores, np.ones_like(vis), V)


def _softmax_unnormalised(scores, vis, V):
    o, l = _orig["masked_softmax_rows"](scores, vis, V)
    return o * np.exp(np.where(np.isfinite(l), l, 0.0))[:, None], l


def _softmax_value_dims_shifted(scores, vis, V):
    return _orig["masked_softmax_rows"](scores, vis, np.roll(V, 1, axis=1))


def _softmax_lse_no_max(scores, vis, V):
    o, l = _orig["masked_softmax_rows"](scores, vis, V)
    m = np.where(vis, scores, -np.inf).max(axis=1)
    return o, np.where(np.isfinite(m), l - m, l)


_orig = {name: getattr(oa, name) for name in
         ("visibility", "decode_bf16", "gather_latents", "sequence_offsets", "masked_softmax_rows")}

MUTANTS = {
    "tail mask without diagonal": ("visibility", _vis_no_diag),
    "tail mask transposed": ("visibility", _vis_transposed),
    "prefix one short": ("visibility", _vis_prefix_short),
    "bf16 decoded with wrong shift": ("decode_bf16", _decode_shift15),
    "gather off by one position": ("gather_latents", _gather_skip_one),
    "sequence offsets without the tail": ("sequence_offsets", _offsets_without_tail),
    "lse in base 2": ("masked_softmax_rows", _softmax_log2),
    "hidden keys not masked": ("masked_softmax_rows", _softmax_unmasked),
    "output not normalised": ("masked_softmax_rows", _softmax_unnormalised),
    "value dims misaligned": ("masked_softmax_rows", _softmax_value_dims_shifted),
    "lse missing the max term": ("masked_softmax_rows", _softmax_lse_no_max),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(oa, attr, fn)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(oa.verify_attention)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake: {name}"


def test_planted_wrong_scale_is_caught():
    failed = []
    for pin in ALL_PINS:
        try:
            pin(lambda q, kv, idx, pl, tm, sc: oa.verify_attention(q, kv, idx, pl, tm, np.float32(sc) * 2))
        except AssertionError:
            failed.append(pin.__name__)
    assert failed


# --------------------------------------------------------------------------
# Golden regression values (written by tests/golden/make_golden.py from the oracle)
# --------------------------------------------------------------------------

def test_golden_tiny_config():
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_oracle.json")
    with open(path) as f:
        g = json.load(f)
    w = make_config("tiny")
    out, lse = oracle.verify_attention(w.q, w.kv_pool, w.kv_indices, w.prefix_lens, w.tree_mask, w.scale)
    assert np.allclose(lse.reshape(-1), np.array(g["lse"]), rtol=0, atol=1e-12)
    for (b, i, h, d), v in zip(g["out_index"], g["out_value"]):
        assert abs(out[b, i, h, d] - v) < 1e-12
    assert abs(float(np.linalg.norm(out)) - g["out_norm"]) < 1e-9
