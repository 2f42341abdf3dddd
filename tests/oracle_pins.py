"""Pins for the CPU oracle: checks against facts that do not come from the oracle.

Each ``pin_*`` function takes an attention callable with the oracle's
signature ``attn(q, kv_pool, kv_indices, prefix_lens, tree_mask, scale) ->
(out, lse)`` and raises AssertionError when the callable disagrees with a
closed form, an invariant, a pure-Python brute force or torch's fp64
scaled_dot_product_attention. The same pins are run against deliberately
broken copies of the oracle to show that each plausible mistake is caught.

The decode of bf16 inputs inside the pins goes through torch's bfloat16 type,
not through the oracle's own decoder.
"""

from __future__ import annotations

import math

import numpy as np
import torch
import torch.nn.functional as F

from workloads import make_workload, tree_mask_from_parents, random_parents, bf16_from_f32

VALUE = 512


def torch_decode(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 via torch's bfloat16 dtype (independent decoder)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy()).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def _call(attn, w):
    return attn(w.q, w.kv_pool, w.kv_indices, w.prefix_lens, w.tree_mask, w.scale)


def pin_single_key(attn):
    """Only one visible key (no prefix, identity tail mask): out is that key's
    value row exactly and lse is its score."""
    w = make_workload("single", [101], B=2, Q=3, H=2, prefix_lens=[0, 0], mask="identity",
                      num_slots=16)
    out, lse = _call(attn, w)
    kv = torch_decode(w.kv_pool)
    qd = torch_decode(w.q)
    for b in range(2):
        for i in range(3):
            slot = int(w.kv_indices[b * 3 + i])
            for h in range(2):
                assert np.array_equal(out[b, i, h], kv[slot, :VALUE]), "single key: out != value row"
                s = float(np.float32(w.scale)) * math.fsum(qd[b, i, h] * kv[slot])
                assert abs(lse[b, i, h] - s) <= 1e-12 * max(1.0, abs(s)), "single key: lse != score"


def pin_zero_query_mean(attn):
    """q = 0 makes every score 0: out is the plain mean of the visible value
    rows and lse = ln(#visible). Exercises the gather and the tail mask."""
    Q = 5
    parents = random_parents(Q, np.random.default_rng(7))
    tm = np.stack([tree_mask_from_parents(parents), np.tril(np.ones((Q, Q), np.uint8)),
                   tree_mask_from_parents(random_parents(Q, np.random.default_rng(8)))])
    w = make_workload("zeroq", [102], B=3, Q=Q, H=2, prefix_lens=[9, 0, 33], mask=tm,
                      num_slots=200, q_zero=True)
    out, lse = _call(attn, w)
    kv = torch_decode(w.kv_pool)
    start = 0
    for b in range(3):
        P = int(w.prefix_lens[b])
        slots = [int(s) for s in w.kv_indices[start:start + P + Q]]
        for i in range(Q):
            vis = slots[:P] + [slots[P + t] for t in range(Q) if tm[b, i, t]]
            mean = np.array([math.fsum(kv[s, d] for s in vis) / len(vis) for d in range(VALUE)])
            for h in range(2):
                assert np.allclose(out[b, i, h], mean, rtol=0, atol=1e-13), "q=0: out != mean of visible rows"
                assert abs(lse[b, i, h] - math.log(len(vis))) < 1e-13, "q=0: lse != ln|visible|"
        start += P + Q


def pin_two_keys(attn):
    """Exactly two visible keys: out = sigmoid(s1 - s2) v1 + sigmoid(s2 - s1) v2,
    lse = log(e^s1 + e^s2)."""
    w = make_workload("twokeys", [103], B=1, Q=1, H=3, prefix_lens=[1], mask="identity",
                      num_slots=8)
    out, lse = _call(attn, w)
    kv = torch_decode(w.kv_pool)
    qd = torch_decode(w.q)
    sc = float(np.float32(w.scale))
    k1, k2 = kv[int(w.kv_indices[0])], kv[int(w.kv_indices[1])]
    for h in range(3):
        s1 = sc * math.fsum(qd[0, 0, h] * k1)
        s2 = sc * math.fsum(qd[0, 0, h] * k2)
        a = 1.0 / (1.0 + math.exp(s2 - s1))
        expect = a * k1[:VALUE] + (1.0 - a) * k2[:VALUE]
        assert np.allclose(out[0, 0, h], expect, rtol=0, atol=1e-12), "two keys: wrong weighting"
        mx = max(s1, s2)
        assert abs(lse[0, 0, h] - (mx + math.log1p(math.exp(-abs(s1 - s2))))) < 1e-12, "two keys: wrong lse"


def _brute(w):
    """Pure-Python loops with math.fsum; independent of numpy linear algebra."""
    B, Q, H, D = w.q.shape
    sc = float(np.float32(w.scale))
    kv = torch_decode(w.kv_pool).tolist()
    qd = torch_decode(w.q).tolist()
    out = np.zeros((B, Q, H, VALUE))
    lse = np.zeros((B, Q, H))
    start = 0
    for b in range(B):
        P = int(w.prefix_lens[b])
        rows = [kv[int(w.kv_indices[start + j])] for j in range(P + Q)]
        for i in range(Q):
            vis = [j for j in range(P + Q) if j < P or w.tree_mask[b, i, j - P]]
            for h in range(H):
                if not vis:
                    lse[b, i, h] = -math.inf
                    continue
                s = [sc * math.fsum(a * c for a, c in zip(qd[b][i][h], rows[j])) for j in vis]
                mx = max(s)
                e = [math.exp(x - mx) for x in s]
                tot = math.fsum(e)
                lse[b, i, h] = mx + math.log(tot)
                for d in range(VALUE):
                    out[b, i, h, d] = math.fsum(e[n] * rows[j][d] for n, j in enumerate(vis)) / tot
        start += P + Q
    return out, lse


def pin_brute_force(attn):
    """Agreement with explicit pure-Python loops on tiny shapes (two sequences,
    random tree, ragged prefixes including zero)."""
    w = make_workload("brute", [104], B=2, Q=3, H=2, prefix_lens=[6, 0], mask="tree", num_slots=40)
    out, lse = _call(attn, w)
    bo, bl = _brute(w)
    assert np.allclose(out, bo, rtol=0, atol=1e-12), "brute force: out differs"
    assert np.allclose(lse, bl, rtol=0, atol=1e-12), "brute force: lse differs"


def _sdpa_reference(w):
    """torch SDPA (math path, fp64, CPU) with an explicit boolean mask built here."""
    B, Q, H, D = w.q.shape
    sc = float(np.float32(w.scale))
    kv = torch.from_numpy(torch_decode(w.kv_pool))
    qd = torch.from_numpy(torch_decode(w.q))
    outs, lses = [], []
    start = 0
    for b in range(B):
        P = int(w.prefix_lens[b])
        idx = torch.from_numpy(w.kv_indices[start:start + P + Q].astype(np.int64))
        K = kv[idx]
        mask = torch.ones((Q, P + Q), dtype=torch.bool)
        mask[:, P:] = torch.from_numpy(w.tree_mask[b].astype(bool))
        qb = qd[b].permute(1, 0, 2)  # [H, Q, D]
        o = F.scaled_dot_product_attention(qb[None], K[None, None], K[None, None, :, :VALUE],
                                           attn_mask=mask, scale=sc)[0]
        s = sc * torch.matmul(qb, K.T)
        s = s.masked_fill(~mask, float("-inf"))
        outs.append(o.permute(1, 0, 2).numpy())
        lses.append(torch.logsumexp(s, dim=-1).permute(1, 0).numpy())
        start += P + Q
    return np.stack(outs), np.stack(lses)


def pin_sdpa(attn):
    """Agreement with torch's fp64 scaled_dot_product_attention under an explicit
    boolean mask (value width 512 != key width 576), three ragged sequences."""
    w = make_workload("sdpa", [105], B=3, Q=4, H=3, prefix_lens=[50, 1, 129], mask="tree",
                      num_slots=400)
    out, lse = _call(attn, w)
    so, sl = _sdpa_reference(w)
    assert np.allclose(out, so, rtol=0, atol=1e-11), "sdpa: out differs"
    assert np.allclose(lse, sl, rtol=0, atol=1e-11), "sdpa: lse differs"


def pin_causal_is_textbook(attn):
    """No prefix + chain mask is ordinary causal self-attention (is_causal=True)."""
    Q, H = 7, 2
    w = make_workload("causal", [106], B=1, Q=Q, H=H, prefix_lens=[0], mask="chain", num_slots=20)
    out, _ = _call(attn, w)
    kv = torch.from_numpy(torch_decode(w.kv_pool))
    K = kv[torch.from_numpy(w.kv_indices.astype(np.int64))]
    qb = torch.from_numpy(torch_decode(w.q))[0].permute(1, 0, 2)
    o = F.scaled_dot_product_attention(qb[None], K[None, None], K[None, None, :, :VALUE],
                                       is_causal=True, scale=float(np.float32(w.scale)))[0]
    assert np.allclose(out[0], o.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12), "causal special case differs"


def pin_prefix_permutation(attn):
    """Prefix positions form a set: permuting them (with kv_indices) leaves the result unchanged."""
    w = make_workload("perm", [107], B=2, Q=3, H=2, prefix_lens=[40, 17], mask="tree", num_slots=128)
    out, lse = _call(attn, w)
    rng = np.random.default_rng(3)
    idx = w.kv_indices.copy()
    start = 0
    for b in range(2):
        P = int(w.prefix_lens[b])
        idx[start:start + P] = idx[start:start + P][rng.permutation(P)]
        start += P + 3
    o2, l2 = attn(w.q, w.kv_pool, idx, w.prefix_lens, w.tree_mask, w.scale)
    assert np.allclose(out, o2, rtol=0, atol=1e-12) and np.allclose(lse, l2, rtol=0, atol=1e-12), \
        "prefix permutation changed the result"


def pin_tail_order(attn):
    """Tail slot t belongs to tail column t: swapping two tail slots changes the
    result exactly as swapping the matching mask columns back restores it."""
    Q = 4
    w = make_workload("tail", [108], B=1, Q=Q, H=2, prefix_lens=[10], mask="tree", num_slots=64)
    out, lse = _call(attn, w)
    idx = w.kv_indices.copy()
    P = 10
    idx[P + 1], idx[P + 3] = idx[P + 3], idx[P + 1]
    tm = w.tree_mask.copy()
    tm[:, :, [1, 3]] = tm[:, :, [3, 1]]
    o2, l2 = attn(w.q, w.kv_pool, idx, w.prefix_lens, tm, w.scale)
    assert np.allclose(out, o2, rtol=0, atol=1e-12) and np.allclose(lse, l2, rtol=0, atol=1e-12), \
        "tail slots and mask columns are not matched"


def pin_gaussian_tilting(attn):
    """Large-N statistics: for N(0,1) latents, the softmax-weighted mean of k
    estimates scale*q (exponential tilting of a Gaussian), and
    lse ~ ln N + |scale q|^2 / 2. Tolerance: 5 standard errors."""
    N, Q, H = 20000, 2, 2
    w = make_workload("tilt", [109], B=1, Q=Q, H=H, prefix_lens=[N - Q], mask="chain",
                      num_slots=N, q_scale=0.5)
    out, lse = _call(attn, w)
    qd = torch_decode(w.q)
    sc = float(np.float32(w.scale))
    for i in range(Q):
        for h in range(H):
            a = sc * qd[0, i, h]
            a2 = float(a @ a)
            n_vis = N - Q + (i + 1)
            se = math.sqrt(math.exp(a2) / n_vis)
            rms = float(np.sqrt(np.mean((out[0, i, h] - a[:VALUE]) ** 2)))
            assert rms < 5 * se, f"tilting: rms {rms} vs se {se}"
            se_l = math.sqrt((math.exp(a2) - 1.0) / n_vis)
            assert abs(lse[0, i, h] - (math.log(n_vis) + 0.5 * a2)) < 5 * se_l, "tilting: lse off"


def pin_empty_visible_set(attn):
    """A query with no prefix and a zero mask row sees nothing: out = 0, lse = -inf."""
    tm = np.array([[[1, 0], [0, 0]]], dtype=np.uint8)
    w = make_workload("empty", [110], B=1, Q=2, H=2, prefix_lens=[0], mask=tm, num_slots=4)
    out, lse = _call(attn, w)
    assert np.all(lse[0, 1] == -np.inf) and np.all(out[0, 1] == 0.0), "empty set not (0, -inf)"
    assert np.all(np.isfinite(lse[0, 0])), "non-empty row broken"


def pin_worked_example(attn):
    """Hand-worked example (values chosen to be exact in bf16).

    One head, prefix of two keys, one tail key visible to the single query.
    q = 2 e_0; k_a = e_0 (v_a[0] = 1), k_b = 0, k_c = -e_0 (v_c[0] = -1); scale
    s = 1/2 gives scores 1, 0, -1. Then lse = ln(e + 1 + 1/e) and
    out[0] = (e - 1/e) / (e + 1 + 1/e) = 2 sinh(1) / (1 + 2 cosh(1)).
    """
    q = np.zeros((1, 1, 1, 576), np.float32)
    q[0, 0, 0, 0] = 2.0
    rows = np.zeros((3, 576), np.float32)
    rows[0, 0] = 1.0
    rows[2, 0] = -1.0
    pool = bf16_from_f32(rows)
    out, lse = attn(bf16_from_f32(q), pool, np.array([0, 1, 2], np.int32), np.array([2], np.int32),
                    np.ones((1, 1, 1), np.uint8), np.float32(0.5))
    e = math.e
    assert abs(lse[0, 0, 0] - math.log(e + 1 + 1 / e)) < 1e-15
    assert abs(out[0, 0, 0, 0] - 2 * math.sinh(1) / (1 + 2 * math.cosh(1))) < 1e-15
    assert np.all(out[0, 0, 0, 1:] == 0.0)


ALL_PINS = [
    pin_single_key,
    pin_zero_query_mean,
    pin_two_keys,
    pin_brute_force,
    pin_sdpa,
    pin_causal_is_textbook,
    pin_prefix_permutation,
    pin_tail_order,
    pin_gaussian_tilting,
    pin_empty_visible_set,
    pin_worked_example,
]
