"""GPU parity for the steps next to verify attention: KV defragmentation and
draft-tree acceptance, through the C ABI against the CPU oracle (bit-exact:
both are integer / byte work)."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_util import require_gpu, upload
from workloads import make_config, make_tree_accept_case, make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    torch, va = require_gpu()
    return torch, va


def _dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


# ---------------------------------------------------------------- KV defrag

@pytest.mark.parametrize("n,dst_base", [(1, 0), (37, 5), (1000, 123), (4113, 7)])
def test_defrag_bit_exact(env, n, dst_base):
    torch, va = env
    rng = np.random.default_rng(500 + n)
    src = rng.integers(0, 1 << 16, size=(6000, 576), dtype=np.uint16)
    idx = rng.permutation(6000)[:n].astype(np.int32)
    if n > 10:
        idx[3] = 6000 + 11       # out of range -> zero row
        idx[7] = -3
    dst = rng.integers(0, 1 << 16, size=(dst_base + n + 9, 576), dtype=np.uint16)
    want_pool, want_idx = oracle.defrag(src, idx, dst, dst_base)
    d_dst = _dev(torch, dst.view(np.int16))
    new_idx = va.kv_defrag(_dev(torch, src.view(np.int16)), _dev(torch, idx), d_dst, dst_base)
    torch.cuda.synchronize()
    assert np.array_equal(d_dst.cpu().numpy().view(np.uint16), want_pool)
    assert np.array_equal(new_idx.cpu().numpy(), want_idx)


def test_defrag_in_place_into_free_slots(env):
    """dst_pool may be the source pool when the run lies in slots nobody references
    (here a run appended past the slots the workload uses)."""
    torch, va = env
    w = make_workload("defrag_inplace", [501], B=2, Q=8, H=8, prefix_lens=[700, 300], mask="tree",
                      num_slots=4096)
    n = len(w.kv_indices)
    pool_np = np.concatenate([w.kv_pool, np.full((n, 576), 0x1234, np.uint16)])
    base = 4096
    want_pool, want_idx = oracle.defrag(pool_np, w.kv_indices, pool_np, base)
    pool = _dev(torch, pool_np.view(np.int16))
    new_idx = va.kv_defrag(pool, _dev(torch, w.kv_indices), pool, base)
    torch.cuda.synchronize()
    assert np.array_equal(pool.cpu().numpy().view(np.uint16), want_pool)
    assert np.array_equal(new_idx.cpu().numpy(), want_idx)


def test_verify_after_defrag_is_bitwise_unchanged(env):
    torch, va = env
    w = make_workload("defrag_verify", [502], B=3, Q=8, H=16, prefix_lens=[2500, 90, 1300], mask="tree",
                      num_slots=16384)
    d = upload(w)
    o1, l1 = va.verify_attn(d["q"], d["kv_pool"], d["kv_indices"], d["prefix_lens"], d["tree_mask"], float(w.scale))
    dst = torch.zeros((len(w.kv_indices) + 64, 576), dtype=torch.int16, device="cuda")
    new_idx = va.kv_defrag(d["kv_pool"], d["kv_indices"], dst, 64)
    o2, l2 = va.verify_attn(d["q"], dst, new_idx, d["prefix_lens"], d["tree_mask"], float(w.scale))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_defrag_full_size_bit_exact_and_timed(env):
    """The 185k-prefix workload's 185,016 positions: every copied row against the
    oracle's (bit-exact), every new index, and the achieved HBM rate."""
    torch, va = env
    w = make_config("long185k")
    src = _dev(torch, w.kv_pool.view(np.int16))
    idx = _dev(torch, w.kv_indices)
    n = len(w.kv_indices)
    dst = torch.empty((n, 576), dtype=torch.int16, device="cuda")
    new_idx = torch.empty(n, dtype=torch.int32, device="cuda")
    va.kv_defrag(src, idx, dst, 0, new_indices=new_idx)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 20
    e0.record()
    for _ in range(reps):
        va.kv_defrag(src, idx, dst, 0, new_indices=new_idx)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    gbps = n * (2 * 1152 + 8) / (us * 1e-6) / 1e9
    print(f"[defrag] {n} rows: {us:.1f} us/call, {gbps:.0f} GB/s algorithmic (warm)", flush=True)
    want_pool, want_idx = oracle.defrag(w.kv_pool, w.kv_indices, np.zeros((n, 576), np.uint16), 0)
    assert np.array_equal(new_idx.cpu().numpy(), want_idx)
    assert np.array_equal(dst.cpu().numpy().view(np.uint16), want_pool)


# ------------------------------------------------------------ tree acceptance

@pytest.mark.parametrize("Q,p_follow,chain", [(1, 0.9, False), (4, 0.9, True), (8, 0.0, False), (8, 0.9, False),
                                              (16, 0.7, False), (16, 0.95, True), (64, 0.9, False),
                                              (64, 1.0, True)])
def test_tree_accept_bit_exact(env, Q, p_follow, chain):
    torch, va = env
    B = 257
    par, dr, tg = make_tree_accept_case(600 + Q, B, Q, vocab=6 if Q > 4 else 40000, p_follow=p_follow,
                                        chain=chain)
    want = oracle.tree_accept_batch(par, dr, tg)
    got = va.tree_accept(_dev(torch, par), _dev(torch, dr), _dev(torch, tg))
    torch.cuda.synchronize()
    for g, w_ in zip(got, want):
        assert np.array_equal(g.cpu().numpy(), w_)
    print(f"[tree_accept] Q={Q} chain={chain}: mean accepted {want[0].mean():.2f}", flush=True)


def test_tree_accept_malformed_tree_matches_oracle(env):
    """Malformed parent arrays (self-parents, forward parents): the walk ends, and it
    equals the oracle's, which counts only children with a larger index."""
    torch, va = env
    B, Q = 6, 16
    par = np.tile(np.arange(Q, dtype=np.int32), (B, 1))      # every node its own parent
    par[:, 0] = -1
    par[1, 5] = 9                                            # a forward parent
    par[2] = [-1, 2, 0, 2, 0, 3, 3, 6, 9, 4, 1, 10, 10, 7, 13, 14]
    par[3] = [-1, 0, 0, 1, 0, 4, 4, 4, 2, 8, 8, 15, 3, 12, 3, 14]
    rng = np.random.default_rng(611)
    par[4] = rng.integers(-1, Q, size=Q)
    par[5] = rng.integers(0, Q, size=Q)
    dr = rng.integers(0, 3, size=(B, Q)).astype(np.int32)
    tg = rng.integers(0, 3, size=(B, Q)).astype(np.int32)
    dr[:3], tg[:3] = 0, 0
    want = oracle.tree_accept_batch(par, dr, tg)
    got = va.tree_accept(_dev(torch, par), _dev(torch, dr), _dev(torch, tg))
    torch.cuda.synchronize()
    for g, w_ in zip(got, want):
        assert np.array_equal(g.cpu().numpy(), w_)
    n, acc = want[0], want[1]
    for b in range(B):
        path = acc[b, :n[b] + 1]
        assert path[0] == 0 and np.all(np.diff(path) > 0) and np.all(acc[b, n[b] + 1:] == -1)


def test_tree_accept_timed(env):
    torch, va = env
    B, Q = 256, 64
    par, dr, tg = make_tree_accept_case(700, B, Q, vocab=8, p_follow=0.9)
    args = [_dev(torch, a) for a in (par, dr, tg)]
    out = va.tree_accept(*args)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(100):
        va.tree_accept(*args, out=out)
    e1.record()
    torch.cuda.synchronize()
    print(f"[tree_accept] B={B} Q={Q}: {e0.elapsed_time(e1) * 10:.1f} us/call", flush=True)
    want = oracle.tree_accept_batch(par, dr, tg)
    for g, w_ in zip(out, want):
        assert np.array_equal(g.cpu().numpy(), w_)
