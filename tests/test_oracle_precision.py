"""Pins of the oracle's precision model (``round_to``, the rounded branches of
``online_softmax_attention`` and ``chunked_attention_model``), on the CPU.

Each pin compares with something other than the model's own code: Python's
binary16 and binary32 packing (``struct``), torch's bfloat16 conversion, closed
forms written out element by element in plain Python, the exact oracle, and a
rounding-error bound derived from the arithmetic. Planted mistakes in copies of
the model must fail one of them.
"""

from __future__ import annotations

import json
import math
import os
import struct

import numpy as np
import pytest

import oracle
from oracle.attention import _online_rows, decode_bf16, gather_latents, lse_merge, sequence_offsets, visibility
from workloads import make_workload

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "precision_budget.json")


def half(x: float) -> float:
    """Python's own IEEE binary16 rounding (round half to even), independent of numpy."""
    return struct.unpack("<e", struct.pack("<e", x))[0]


def single(x: float) -> float:
    return struct.unpack("<f", struct.pack("<f", x))[0]


# ------------------------------------------------------------------ round_to

def _f16_cases():
    rng = np.random.default_rng(800)
    vals = list(rng.standard_normal(2000) * np.exp2(rng.integers(-26, 15, size=2000)))
    one = 1.0
    vals += [one + 2.0 ** -11, one + 3 * 2.0 ** -11, -(one + 2.0 ** -11), 2.0 ** -24, 2.0 ** -25,
             3 * 2.0 ** -25, 2.0 ** -26, 5 * 2.0 ** -26, 2.0 ** -14 - 2.0 ** -25, 65504.0, 65519.0,
             -65519.9, 0.0, -0.0, 1e-30]
    return vals


def test_round_to_f16_matches_python_half_packing():
    vals = _f16_cases()
    got = oracle.round_to(np.array(vals), "f16")
    want = np.array([half(v) for v in vals])
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))   # -0 stays -0
    # ties go to the even neighbour; the smallest subnormal's half rounds to 0
    assert half(1 + 2.0 ** -11) == 1.0 and half(1 + 3 * 2.0 ** -11) == 1 + 2.0 ** -9
    assert half(2.0 ** -25) == 0.0 and half(3 * 2.0 ** -25) == 2.0 ** -23


def test_round_to_f16_overflow_and_nan():
    got = oracle.round_to(np.array([65520.0, -1e6, np.inf, np.nan]), "f16")
    assert got[0] == np.inf and got[1] == -np.inf and got[2] == np.inf and np.isnan(got[3])
    with pytest.raises(OverflowError):   # Python refuses to pack it: beyond the largest binary16
        struct.pack("<e", 65520.0)


def test_round_to_bf16_matches_torch():
    import torch
    rng = np.random.default_rng(801)
    bits = list(rng.integers(0, 1 << 32, size=4000, dtype=np.uint64).astype(np.uint32))
    bits += [0x3F808000, 0x3F818000, 0xBF808000, 0x3F80FFFF, 0x00018000, 0x00008000, 0x7F7FFFFF,
             0x7F800001, 0xFF800001, 0x7FC00000, 0x7F800000, 0xFF800000, 0x80000000, 0x00000000]
    f = np.array(bits, dtype=np.uint32).view(np.float32)
    got = oracle.round_to(f.astype(np.float64), "bf16")
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).to(torch.float32).numpy().astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)                   # NaN stays NaN (0x7F800001 included)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))
    # ties to even: 1 + 2^-8 -> 1; 1 + 3 * 2^-8 -> 1 + 2^-6
    assert oracle.round_to(np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8]), "bf16").tolist() == [1.0, 1 + 2.0 ** -6]


def test_round_to_f32_matches_python_single_packing_and_identity_kinds():
    rng = np.random.default_rng(802)
    vals = list(rng.standard_normal(1000) * np.exp2(rng.integers(-140, 120, size=1000)))
    assert np.array_equal(oracle.round_to(np.array(vals), "f32"), np.array([single(v) for v in vals]))
    x = rng.standard_normal(10)
    assert np.array_equal(oracle.round_to(x, None), x) and np.array_equal(oracle.round_to(x, "f64"), x)
    with pytest.raises(ValueError):
        oracle.round_to(x, "f8")


# ------------------------------------------- online softmax with rounded operands

def _two_key_case():
    """One query row that sees exactly two keys (the chain's second query, no prefix)."""
    w = make_workload("two", [810], B=1, Q=2, H=1, prefix_lens=[0], mask="chain", num_slots=8)
    scale = float(np.float32(w.scale))
    qv = [float(x) for x in decode_bf16(w.q[0, 1, 0])]
    K = [[float(x) for x in decode_bf16(w.kv_pool[w.kv_indices[j]])] for j in range(2)]
    s = [scale * math.fsum(a * b for a, b in zip(qv, K[j])) for j in range(2)]
    return w, s, K


def _closed_two_key(s, K, tile_one: bool, p_round: bool, v_round: bool, l_rounded: bool = False):
    """out and lse of the two-key row, written out per element."""
    r = half if p_round else (lambda x: x)
    rv = half if v_round else (lambda x: x)
    mx = max(s)
    if tile_one:   # key 0 alone first (p = 1 against its own max), then key 1 with a rescale
        alpha = math.exp(s[0] - mx)
        p1 = math.exp(s[1] - mx)
        lsum = alpha + p1
        out = [(alpha * r(1.0) * rv(K[0][d]) + r(p1) * rv(K[1][d])) / lsum for d in range(512)]
    else:          # both keys in one tile, against the common max
        p = [math.exp(x - mx) for x in s]
        lsum = (r(p[0]) + r(p[1])) if l_rounded else (p[0] + p[1])
        out = [(r(p[0]) * rv(K[0][d]) + r(p[1]) * rv(K[1][d])) / lsum for d in range(512)]
    return np.array(out), mx + math.log(lsum)


@pytest.mark.parametrize("tile", [1, 2, 32])
@pytest.mark.parametrize("p_round,v_round", [("f16", None), ("f16", "f16"), (None, "f16")])
def test_online_softmax_rounding_matches_two_key_closed_form(tile, p_round, v_round):
    w, s, K = _two_key_case()
    out, lse = oracle.online_softmax_attention(w.q, w.kv_pool, w.kv_indices, w.prefix_lens, w.tree_mask,
                                               w.scale, tile=tile, p_round=p_round, v_round=v_round)
    want, wl = _closed_two_key(s, K, tile == 1, p_round == "f16", v_round == "f16")
    assert np.max(np.abs(out[0, 1, 0] - want)) < 1e-12 and abs(lse[0, 1, 0] - wl) < 1e-12
    exact, _ = _closed_two_key(s, K, tile == 1, False, False)
    if p_round:   # the pin is not vacuous: the rounding moved the result
        assert np.max(np.abs(want - exact)) > 1e-7


def _model_rounding_l_too(q, kv_pool, kv_indices, prefix_lens, tree_mask, scale, tile=32, p_round=None,
                          v_round=None, score_round=None):
    """Planted mistake: the normaliser sums the rounded probabilities."""
    B, Q, H, _ = q.shape
    out = np.zeros((B, Q, H, 512))
    lse = np.zeros((B, Q, H))
    off = sequence_offsets(prefix_lens, Q)
    scale = float(np.float32(scale))
    for b in range(B):
        N = int(prefix_lens[b]) + Q
        K = gather_latents(kv_pool, kv_indices, int(off[b]), N)
        vis = np.repeat(visibility(int(prefix_lens[b]), tree_mask[b]), H, axis=0)
        rows = decode_bf16(q[b]).reshape(Q * H, 576)
        s = np.where(vis, scale * rows @ K.T, -np.inf)
        m = s.max(axis=1)
        p = oracle.round_to(np.exp(s - m[:, None]), p_round)
        out[b] = ((p @ K[:, :512]) / p.sum(axis=1)[:, None]).reshape(Q, H, 512)
        lse[b] = (m + np.log(p.sum(axis=1))).reshape(Q, H)
    return out, lse


def test_two_key_pin_catches_rounded_normaliser():
    w, s, K = _two_key_case()
    out, _ = _model_rounding_l_too(w.q, w.kv_pool, w.kv_indices, w.prefix_lens, w.tree_mask, w.scale,
                                   p_round="f16")
    want, _ = _closed_two_key(s, K, False, True, False)
    assert np.max(np.abs(out[0, 1, 0] - want)) > 1e-8
    also, _ = _closed_two_key(s, K, False, True, False, l_rounded=True)
    assert np.max(np.abs(out[0, 1, 0] - also)) < 1e-12


def test_f16_probabilities_stay_within_the_rounding_bound():
    """|out(p rounded to fp16) - out| <= (2^-11 + N 2^-25) max|v| per element: each
    probability moves by at most 2^-11 of itself (normal range) or 2^-25 (subnormal),
    and the normaliser is the unrounded sum, at least 1. The coarser bf16 rounding
    (2^-8 of itself) moves the result further."""
    w = make_workload("bound", [811], B=2, Q=5, H=3, prefix_lens=[300, 77], mask="tree", num_slots=600)
    args = (w.q, w.kv_pool, w.kv_indices, w.prefix_lens, w.tree_mask, w.scale)
    exact, _ = oracle.verify_attention(*args)
    vmax = float(np.abs(decode_bf16(w.kv_pool[w.kv_indices])[:, :512]).max())
    n = int(w.prefix_lens.max()) + w.Q
    bound = (2.0 ** -11 + n * 2.0 ** -25) * vmax
    f16, _ = oracle.online_softmax_attention(*args, p_round="f16")
    err = np.abs(f16 - exact).max()
    assert 1e-7 < err <= bound
    bf16, _ = oracle.online_softmax_attention(*args, p_round="bf16")
    assert np.linalg.norm(bf16 - exact) > 4 * np.linalg.norm(f16 - exact)


def test_f16_values_beyond_the_fp16_range_overflow():
    """The precondition of the fp16 value product: a value of magnitude >= 65520
    becomes infinite in the model, and its rows lose their finite result."""
    w = make_workload("big", [812], B=1, Q=2, H=1, prefix_lens=[3], mask="chain", num_slots=16)
    pool = w.kv_pool.copy()
    row = w.kv_indices[1]
    pool[row, 7] = 0x4789          # bf16 70144
    out, _ = oracle.online_softmax_attention(w.q, pool, w.kv_indices, w.prefix_lens, w.tree_mask, w.scale,
                                             v_round="f16")
    assert not np.isfinite(out[0, :, 0, 7]).any()
    ok, _ = oracle.online_softmax_attention(w.q, pool, w.kv_indices, w.prefix_lens, w.tree_mask, w.scale)
    assert np.isfinite(ok).all()


# --------------------------------------------------- chunked model (kernel precision)

@pytest.mark.parametrize("chunk", [1, 32, 33, 100, 4096])
def test_chunked_model_without_rounding_is_the_definition(chunk):
    w = make_workload("chunked", [813], B=2, Q=6, H=3, prefix_lens=[250, 31], mask="tree", num_slots=600)
    args = (w.q, w.kv_pool, w.kv_indices, w.prefix_lens, w.tree_mask, w.scale)
    ro, rl = oracle.verify_attention(*args)
    o, l = oracle.chunked_attention_model(*args, chunk=chunk, p_round=None, v_round=None, partial_round=None)
    assert np.abs(o - ro).max() < 1e-12 and np.abs(l - rl).max() < 1e-12


def _zero_q_closed_form(w, chunk):
    """q = 0: every visible score is 0, so each chunk's partial is the mean of its
    visible values (rounded to fp16), and the merge weighs chunk s by n_s / n."""
    off = sequence_offsets(w.prefix_lens, w.Q)
    out = np.zeros((w.B, w.Q, w.H, 512))
    lse = np.zeros((w.B, w.Q, w.H))
    for b in range(w.B):
        P = int(w.prefix_lens[b])
        N = P + w.Q
        rows = [[half(float(x)) for x in decode_bf16(w.kv_pool[w.kv_indices[int(off[b]) + j]])[:512]]
                for j in range(N)]
        for i in range(w.Q):
            vis = [j for j in range(N) if j < P or w.tree_mask[b, i, j - P]]
            acc = [0.0] * 512
            for lo in range(0, N, chunk):
                js = [j for j in vis if lo <= j < lo + chunk]
                if not js:
                    continue
                for d in range(512):
                    acc[d] += len(js) / len(vis) * half(math.fsum(rows[j][d] for j in js) / len(js))
            out[b, i, :, :] = np.array(acc)[None, :]
            lse[b, i, :] = math.log(len(vis))
    return out, lse


def _model_rounding_merged(q, kv_pool, kv_indices, prefix_lens, tree_mask, scale, chunk, **kw):
    """Planted mistake: rounds the merged output instead of each chunk's partial."""
    o, l = oracle.chunked_attention_model(q, kv_pool, kv_indices, prefix_lens, tree_mask, scale, chunk,
                                          partial_round=None)
    return oracle.round_to(o, "f16"), l


def _model_chunk_off_by_one(q, kv_pool, kv_indices, prefix_lens, tree_mask, scale, chunk, **kw):
    """Planted mistake: chunks of chunk + 1 keys."""
    return oracle.chunked_attention_model(q, kv_pool, kv_indices, prefix_lens, tree_mask, scale, chunk + 1)


def _zero_q_pin(model):
    w = make_workload("zeroq", [814], B=2, Q=4, H=2, prefix_lens=[70, 5], mask="tree", num_slots=200)
    w.q = np.zeros_like(w.q)
    for chunk in (16, 48):
        o, l = model(w.q, w.kv_pool, w.kv_indices, w.prefix_lens, w.tree_mask, w.scale, chunk)
        ro, rl = _zero_q_closed_form(w, chunk)
        assert np.abs(o - ro).max() < 1e-12 and np.abs(l - rl).max() < 1e-12


def test_chunked_model_zero_query_closed_form():
    _zero_q_pin(oracle.chunked_attention_model)


@pytest.mark.parametrize("mutant", [_model_rounding_merged, _model_chunk_off_by_one])
def test_zero_query_pin_catches_planted_mistakes(mutant):
    with pytest.raises(AssertionError):
        _zero_q_pin(mutant)


def test_online_rows_empty_rows():
    rows = np.zeros((2, 576))
    K = np.ones((3, 576))
    vis = np.array([[False] * 3, [True, False, True]])
    o, l = _online_rows(rows, K, vis, 1.0, 2, "f16", "f16", None)
    assert np.all(o[0] == 0) and l[0] == -np.inf and abs(l[1] - math.log(2)) < 1e-15


def test_lse_merge_of_rounded_partials_keeps_weights():
    o, l = lse_merge([np.full((1, 512), 1.0), np.full((1, 512), 3.0)], [np.log([1.0]), np.log([3.0])])
    assert np.allclose(o, 2.5, atol=1e-15) and abs(l[0] - math.log(4.0)) < 1e-15


# --------------------------------------------------------- committed predictions

def test_committed_precision_budget_reproduces_on_tiny():
    """The committed predictions (tests/golden/make_precision_budget.py, which calls only
    the oracle) are what the model gives today, checked on the smallest workload."""
    from golden.make_precision_budget import predict
    with open(GOLDEN) as f:
        committed = json.load(f)
    now = predict("tiny", committed["tiny"]["chunk_keys"])
    for key in ("rel_l2", "max_abs", "lse_abs", "rel_l2_bf16_p", "rel_l2_f16_p_only"):
        assert abs(now[key] - committed["tiny"][key]) <= 1e-9 * max(1.0, abs(committed["tiny"][key])), key
