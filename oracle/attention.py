"""Plain fp64 CPU oracle for MLA speculative-decoding verify attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links
this module; only the test suite, the smoke check and the CPU-baseline leg of
the benchmark use it. It shares no code with the GPU path.

What is computed (page "The Build That Bridged Design and Deployment:
Compiling the Custom sm_120 Verify Kernel", section "What This Build Achieves:
The paged+bf16 Kernel"; page "The Build That Unlocked 3-6x Decode Speedup",
section "The Context: A Custom Kernel for an Unsupported Architecture"):

* KV rows are gathered through ``kv_indices`` with page_size 1: logical
  position j of sequence b is physical slot ``kv_indices[off_b + j]``.
* Each request has its own prefix length P_b; the first P_b positions are
  visible to every query. The last Q positions are the speculative tail; tail
  position t is visible to query i iff ``tree_mask[b, i, t]`` is set (the
  compact "prefix length plus q x q visibility matrix" mask).
* Attention is MLA over compressed latents: the key is the whole 576-d latent
  row and the value is its first 512 dims; scores are ``scale * q . k``.
* For every (b, i, h): lse = log sum_{visible j} exp(s_j) (natural log) and
  out = sum_{visible j} exp(s_j - lse) v_j. An empty visible set gives
  out = 0 and lse = -inf.

Readings where the pages are silent (all listed in the design notes): the tail
slots are the last Q entries of each sequence's ``kv_indices`` slice in query
order; the tree mask includes the diagonal (a query sees its own tail key);
the scale multiplies the fp64 dot product and is never folded into q.

Besides the plain definition (``verify_attention``) this module carries
restatements of the pages' flash-decode method, used only to pin the oracle
and to model the kernel's rounding: a KV split with a log-sum-exp merge
(``split_merge_attention``; the flash-decode KV split with its NSPLIT
parameter, page "The Build That Unlocked 3-6x Decode Speedup", section "The
Context: A Custom Kernel for an Unsupported Architecture", and page "The Build
Script Edit: How a Single Line of Infrastructure Unlocked Custom CUDA Kernels
on sm_120", section "Context: The Long Road to a Custom sm_120 Kernel"),
online softmax over KV tiles (``online_softmax_attention``; same sections),
and both together with a rounding model of where a kernel keeps which
precision (``chunked_attention_model``, with ``round_to``; the pages stress
the bf16 precision of their paged kernel, page "The Build That Bridged Design
and Deployment: Compiling the Custom sm_120 Verify Kernel", section "What
This Build Achieves: The paged+bf16 Kernel").
"""

from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

LATENT = 576
VALUE = 512


# ---------------------------------------------------------------------------
# Step helpers (kept separate so that each one can be checked on its own)
# ---------------------------------------------------------------------------

def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values.

    A bf16 number is the upper half of an IEEE float32, so widening the bits
    by 16 and reinterpreting is exact.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def sequence_offsets(prefix_lens: np.ndarray, Q: int) -> np.ndarray:
    """Start of each sequence's slice of ``kv_indices``: exclusive scan of P_b + Q."""
    n = np.asarray(prefix_lens, dtype=np.int64) + Q
    off = np.zeros(len(n) + 1, dtype=np.int64)
    off[1:] = np.cumsum(n)
    return off


def gather_latents(kv_pool: np.ndarray, kv_indices: np.ndarray, start: int, count: int) -> np.ndarray:
    """Rows of the page_size-1 pool for logical positions start..start+count-1, as fp64."""
    slots = np.asarray(kv_indices[start:start + count], dtype=np.int64)
    return decode_bf16(kv_pool[slots])


def visibility(prefix_len: int, tail_mask: np.ndarray) -> np.ndarray:
    """Boolean [Q, P+Q]: prefix columns all visible, tail columns per the q x q matrix."""
    Q = tail_mask.shape[0]
    vis = np.zeros((Q, prefix_len + Q), dtype=bool)
    vis[:, :prefix_len] = True
    vis[:, prefix_len:] = np.asarray(tail_mask, dtype=np.uint8) != 0
    return vis


def masked_softmax_rows(scores: np.ndarray, vis: np.ndarray, V: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Full softmax of each score row over its visible columns, weighted sum of V.

    scores: [R, N] fp64, vis: [R, N] bool, V: [N, Dv] fp64.
    Returns out [R, Dv] and natural-log lse [R]; empty rows give 0 and -inf.
    """
    s = np.where(vis, scores, -np.inf)
    m = s.max(axis=1)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(s - m_safe[:, None])          # exp(-inf) = 0 for hidden columns
    l = e.sum(axis=1)
    out = e @ V
    with np.errstate(divide="ignore", invalid="ignore"):
        out = out / l[:, None]
        lse = m_safe + np.log(l)
    out[empty] = 0.0
    lse[empty] = -np.inf
    return out, lse


# ---------------------------------------------------------------------------
# The definition
# ---------------------------------------------------------------------------

def verify_attention(q, kv_pool, kv_indices, prefix_lens, tree_mask, scale,
                     heads: Optional[Sequence[int]] = None,
                     max_score_bytes: int = 1 << 28) -> Tuple[np.ndarray, np.ndarray]:
    """Verify attention by its definition, in fp64.

    q: uint16 bf16 [B, Q, H, 576]; kv_pool: uint16 bf16 [S, 576];
    kv_indices: int32 [sum_b (P_b + Q)]; prefix_lens: int32 [B];
    tree_mask: uint8 [B, Q, Q]; scale: float (the fp32 value is used as is).
    ``heads`` restricts the computation to a subset of heads (others stay 0).
    Returns out fp64 [B, Q, H, 512] and lse fp64 [B, Q, H].
    """
    B, Q, H, D = q.shape
    assert D == LATENT
    scale = float(np.float32(scale))
    off = sequence_offsets(prefix_lens, Q)
    out = np.zeros((B, Q, H, VALUE), dtype=np.float64)
    lse = np.zeros((B, Q, H), dtype=np.float64)
    head_list = list(range(H)) if heads is None else list(heads)
    for b in range(B):
        P = int(prefix_lens[b])
        N = P + Q
        K = gather_latents(kv_pool, kv_indices, int(off[b]), N)   # [N, 576]
        V = K[:, :VALUE]                                          # values = leading 512 dims
        vis = visibility(P, tree_mask[b])                         # [Q, N]
        # Rows are (query i, head h); group heads so the score block stays bounded.
        group = max(1, int(max_score_bytes // (8 * Q * max(N, 1))))
        for g0 in range(0, len(head_list), group):
            hs = head_list[g0:g0 + group]
            qg = decode_bf16(q[b][:, hs, :])                      # [Q, G, 576]
            rows = qg.transpose(1, 0, 2).reshape(len(hs) * Q, LATENT)  # row = (h, i)
            scores = scale * (rows @ K.T)                         # [G*Q, N]
            o, l = masked_softmax_rows(scores, np.tile(vis, (len(hs), 1)), V)
            out[b][:, hs, :] = o.reshape(len(hs), Q, VALUE).transpose(1, 0, 2)
            lse[b][:, hs] = l.reshape(len(hs), Q).T
    return out, lse


# ---------------------------------------------------------------------------
# The method, restated: KV split + log-sum-exp merge; online softmax
# ---------------------------------------------------------------------------

def partial_attention(scores: np.ndarray, vis: np.ndarray, V: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """One KV split's normalised partial output and its lse (empty split: 0, -inf)."""
    return masked_softmax_rows(scores, vis, V)


def lse_merge(parts_out: List[np.ndarray], parts_lse: List[np.ndarray]) -> Tuple[np.ndarray, np.ndarray]:
    """Combine split partials: lse = log sum_s exp(lse_s), out = sum_s exp(lse_s - lse) out_s."""
    L = np.stack(parts_lse)                      # [S, R]
    O = np.stack(parts_out)                      # [S, R, Dv]
    m = L.max(axis=0)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.exp(L - m_safe[None, :])              # exp(-inf) = 0 for empty splits
    tot = w.sum(axis=0)
    with np.errstate(divide="ignore", invalid="ignore"):
        lse = m_safe + np.log(tot)
        out = (w[:, :, None] * O).sum(axis=0) / tot[:, None]
    out[empty] = 0.0
    lse[empty] = -np.inf
    return out, lse


def split_merge_attention(q, kv_pool, kv_indices, prefix_lens, tree_mask, scale,
                          bounds: Sequence[Sequence[int]]) -> Tuple[np.ndarray, np.ndarray]:
    """KV-split attention: sequence b's positions are cut at ``bounds[b]``
    (ascending, 0 and N_b included); each split is a partial, merged by lse."""
    B, Q, H, _ = q.shape
    scale = float(np.float32(scale))
    off = sequence_offsets(prefix_lens, Q)
    out = np.zeros((B, Q, H, VALUE))
    lse = np.zeros((B, Q, H))
    for b in range(B):
        P = int(prefix_lens[b])
        N = P + Q
        K = gather_latents(kv_pool, kv_indices, int(off[b]), N)
        vis = visibility(P, tree_mask[b])
        rows = decode_bf16(q[b]).reshape(Q * H, LATENT)           # row = (i, h)
        vis_rows = np.repeat(vis, H, axis=0)
        po, pl = [], []
        cuts = list(bounds[b])
        assert cuts[0] == 0 and cuts[-1] == N
        for lo, hi in zip(cuts[:-1], cuts[1:]):
            sc = scale * (rows @ K[lo:hi].T)
            o, l = partial_attention(sc, vis_rows[:, lo:hi], K[lo:hi, :VALUE])
            po.append(o)
            pl.append(l)
        o, l = lse_merge(po, pl)
        out[b] = o.reshape(Q, H, VALUE)
        lse[b] = l.reshape(Q, H)
    return out, lse


def round_to(x: np.ndarray, kind: Optional[str]) -> np.ndarray:
    """Round fp64 values to a storage type and back (the precision model only).

    * None / "f64": unchanged.
    * "f32": IEEE binary32, round to nearest, ties to even.
    * "f16": IEEE binary16, round to nearest, ties to even, directly from the
      fp64 value; gradual underflow to subnormals, overflow to +-inf.
    * "bf16": first rounded to binary32 (the precision of the values a kernel
      computes in fp32), then to bfloat16 (the upper half of a binary32),
      round to nearest, ties to even; NaN stays NaN.
    """
    if kind is None or kind == "f64":
        return x
    x = np.asarray(x, dtype=np.float64)
    if kind == "f32":
        return x.astype(np.float32).astype(np.float64)
    if kind == "f16":
        return x.astype(np.float16).astype(np.float64)
    if kind == "bf16":
        f = np.ascontiguousarray(x.astype(np.float32))
        u = f.view(np.uint32)
        bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
        r = ((u + bias) >> np.uint32(16)) << np.uint32(16)
        # a NaN whose payload sits in the low half would otherwise carry into
        # the exponent's all-ones pattern and read as infinity
        r = np.where(np.isnan(f), np.uint32(0x7FC00000), r).astype(np.uint32)
        return r.view(np.float32).astype(np.float64)
    raise ValueError(kind)


def _online_rows(rows: np.ndarray, K: np.ndarray, vis: np.ndarray, scale: float, tile: int,
                 p_round: Optional[str], v_round: Optional[str],
                 score_round: Optional[str]) -> Tuple[np.ndarray, np.ndarray]:
    """Online softmax of score rows over the keys K (the flash-decode inner loop).

    rows [R, 576] fp64 queries, K [N, 576] fp64 latents (values = K[:, :512]),
    vis [R, N] bool. Per row: a running max m, a running normaliser l and an
    unnormalised accumulator o. For each tile of keys: m' = max(m, max s),
    alpha = exp(m - m'), p = exp(s - m'), l = alpha l + sum p,
    o = alpha o + round(p) round(V). Returns out = o / l and lse = m + log l
    (a row that saw nothing: 0 and -inf). The p in l is not rounded: only the
    value product's operands are.
    """
    R, N = rows.shape[0], K.shape[0]
    V = round_to(K[:, :VALUE], v_round)
    m = np.full(R, -np.inf)
    l = np.zeros(R)
    o = np.zeros((R, VALUE))
    for lo in range(0, N, tile):
        hi = min(N, lo + tile)
        s = round_to(scale * (rows @ K[lo:hi].T), score_round)
        s = np.where(vis[:, lo:hi], s, -np.inf)
        m_new = np.maximum(m, s.max(axis=1))
        live = np.isfinite(m_new)
        ref = np.where(live, m_new, 0.0)
        alpha = np.where(live, np.exp(np.where(np.isfinite(m), m, -np.inf) - ref), 1.0)
        p = np.exp(s - ref[:, None])
        l = alpha * l + p.sum(axis=1)
        o = alpha[:, None] * o + round_to(p, p_round) @ V[lo:hi]
        m = m_new
    with np.errstate(divide="ignore", invalid="ignore"):
        ob = o / l[:, None]
        lb = m + np.log(l)
    empty = l == 0
    ob[empty] = 0.0
    lb[empty] = -np.inf
    return ob, lb


def online_softmax_attention(q, kv_pool, kv_indices, prefix_lens, tree_mask, scale,
                             tile: int = 32, p_round: Optional[str] = None,
                             v_round: Optional[str] = None,
                             score_round: Optional[str] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Online softmax over KV tiles of ``tile`` keys, one pass per sequence
    (see ``_online_rows``). ``p_round`` / ``v_round`` / ``score_round``
    optionally round p, V or the scores to a storage type (``round_to``)
    before use; that models where a kernel keeps which precision and is not
    part of the definition."""
    B, Q, H, _ = q.shape
    scale = float(np.float32(scale))
    off = sequence_offsets(prefix_lens, Q)
    out = np.zeros((B, Q, H, VALUE))
    lse = np.zeros((B, Q, H))
    for b in range(B):
        P = int(prefix_lens[b])
        N = P + Q
        K = gather_latents(kv_pool, kv_indices, int(off[b]), N)
        vis = np.repeat(visibility(P, tree_mask[b]), H, axis=0)
        rows = decode_bf16(q[b]).reshape(Q * H, LATENT)
        ob, lb = _online_rows(rows, K, vis, scale, tile, p_round, v_round, score_round)
        out[b] = ob.reshape(Q, H, VALUE)
        lse[b] = lb.reshape(Q, H)
    return out, lse


def chunked_attention_model(q, kv_pool, kv_indices, prefix_lens, tree_mask, scale, chunk: int,
                            tile: int = 32, p_round: Optional[str] = "f16",
                            v_round: Optional[str] = "f16",
                            partial_round: Optional[str] = "f16") -> Tuple[np.ndarray, np.ndarray]:
    """The pages' flash-decode method with a precision model: each sequence's
    positions are cut into chunks of ``chunk`` keys (the last one shorter);
    each chunk runs the online softmax over tiles of ``tile`` keys with p and V
    rounded as given, leaves its normalised partial output rounded to
    ``partial_round`` and its lse in fp64; the partials are merged by
    log-sum-exp (``lse_merge``) in fp64.

    With every rounding off this equals ``verify_attention`` up to fp64
    rounding (the split-merge invariant). With the defaults it models the
    precision the GPU kernel keeps (fp16 probabilities and values in the value
    product, fp16 chunk partials), so that the error it predicts against the
    exact result can be compared with the GPU's.
    """
    B, Q, H, _ = q.shape
    scale = float(np.float32(scale))
    off = sequence_offsets(prefix_lens, Q)
    out = np.zeros((B, Q, H, VALUE))
    lse = np.zeros((B, Q, H))
    for b in range(B):
        P = int(prefix_lens[b])
        N = P + Q
        K = gather_latents(kv_pool, kv_indices, int(off[b]), N)
        vis = np.repeat(visibility(P, tree_mask[b]), H, axis=0)
        rows = decode_bf16(q[b]).reshape(Q * H, LATENT)
        po, pl = [], []
        for lo in range(0, N, chunk):
            hi = min(N, lo + chunk)
            o, l = _online_rows(rows, K[lo:hi], vis[:, lo:hi], scale, tile, p_round, v_round, None)
            po.append(round_to(o, partial_round))
            pl.append(l)
        o, l = lse_merge(po, pl)
        out[b] = o.reshape(Q, H, VALUE)
        lse[b] = l.reshape(Q, H)
    return out, lse


# ---------------------------------------------------------------------------
# Pure-Python brute force for tiny inputs (no numpy arithmetic)
# ---------------------------------------------------------------------------

def _bf16_value(bits: int) -> float:
    """Decode one bf16 pattern with integer arithmetic only."""
    sign = -1.0 if bits & 0x8000 else 1.0
    exp = (bits >> 7) & 0xFF
    man = bits & 0x7F
    if exp == 0xFF:
        return float("nan") if man else sign * float("inf")
    if exp == 0:
        return sign * man * 2.0 ** (-133)
    return sign * (1.0 + man / 128.0) * 2.0 ** (exp - 127)


def brute_force(q, kv_pool, kv_indices, prefix_lens, tree_mask, scale):
    """Verify attention with explicit Python loops and math.fsum (tiny shapes only)."""
    B, Q, H, D = q.shape
    scale = float(np.float32(scale))
    out = [[[[0.0] * VALUE for _ in range(H)] for _ in range(Q)] for _ in range(B)]
    lse = [[[0.0] * H for _ in range(Q)] for _ in range(B)]
    start = 0
    for b in range(B):
        P = int(prefix_lens[b])
        N = P + Q
        rows = [[_bf16_value(int(x)) for x in kv_pool[int(kv_indices[start + j])]] for j in range(N)]
        for i in range(Q):
            visible = [j for j in range(N) if j < P or tree_mask[b][i][j - P]]
            for h in range(H):
                qv = [_bf16_value(int(x)) for x in q[b][i][h]]
                if not visible:
                    lse[b][i][h] = -math.inf
                    continue
                s = {j: scale * math.fsum(qv[d] * rows[j][d] for d in range(D)) for j in visible}
                mx = max(s.values())
                w = {j: math.exp(s[j] - mx) for j in visible}
                tot = math.fsum(w.values())
                lse[b][i][h] = mx + math.log(tot)
                for d in range(VALUE):
                    out[b][i][h][d] = math.fsum(w[j] * rows[j][d] for j in visible) / tot
        start += N
    return np.array(out), np.array(lse)
