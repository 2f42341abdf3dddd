"""HIP-graph capture and replay of verify_attn.

The call allocates nothing, never synchronises and plans its chunks on the
device from prefix_lens, so one capture serves every later set of inputs with
the same (B, Q, H, total_kv): each replay must equal an eager call on the
inputs the buffers hold at replay time, bit for bit.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_util import compare, require_gpu, upload
from workloads import make_workload

pytestmark = pytest.mark.gpu


def _bufs(torch, w):
    out = torch.empty((w.B, w.Q, w.H, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.B, w.Q, w.H), dtype=torch.float32, device="cuda")
    return out, lse


def _eager(torch, va, d, w, ws):
    out, lse = _bufs(torch, w)
    va.verify_attn(d["q"], d["kv_pool"], d["kv_indices"], d["prefix_lens"], d["tree_mask"],
                   float(w.scale), out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    return out.clone(), lse.clone()


def test_graph_replay_is_bitwise_eager_and_follows_new_lengths():
    torch, va = require_gpu()
    # two sequences; the second input set moves 700 positions from the first
    # sequence's prefix to the second's, keeping total_kv (the capture key)
    w1 = make_workload("graph1", [310], B=2, Q=8, H=16, prefix_lens=[3000, 1200], mask="tree",
                       num_slots=8192)
    w2 = make_workload("graph2", [311], B=2, Q=8, H=16, prefix_lens=[2300, 1900], mask="tree",
                       num_slots=8192)
    assert w1.total_kv == w2.total_kv
    d = upload(w1)
    ws = va.alloc_workspace(w1.B, w1.Q, w1.H, w1.total_kv, device="cuda")
    ref_out, ref_lse = _eager(torch, va, d, w1, ws)

    out_g, lse_g = _bufs(torch, w1)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up call outside the capture
        va.verify_attn(d["q"], d["kv_pool"], d["kv_indices"], d["prefix_lens"], d["tree_mask"],
                       float(w1.scale), out=out_g, lse=lse_g, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        va.verify_attn(d["q"], d["kv_pool"], d["kv_indices"], d["prefix_lens"], d["tree_mask"],
                       float(w1.scale), out=out_g, lse=lse_g, workspace=ws)
    torch.cuda.synchronize()

    for rep in range(3):
        out_g.fill_(float("nan"))   # eager work between replays
        lse_g.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, ref_out) and torch.equal(lse_g, ref_lse), f"replay {rep} differs"

    # new inputs in the same buffers, different prefix lengths
    for key in ("q", "kv_pool", "kv_indices", "prefix_lens", "tree_mask"):
        src = upload(w2)[key]
        d[key].copy_(src)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    ref2_out, ref2_lse = _eager(torch, va, d, w2, ws)
    assert torch.equal(out_g, ref2_out) and torch.equal(lse_g, ref2_lse)
    ro, rl = oracle.verify_attention(w2.q, w2.kv_pool, w2.kv_indices, w2.prefix_lens, w2.tree_mask, w2.scale)
    m = compare(out_g.cpu().numpy().astype(np.float64), lse_g.cpu().numpy().astype(np.float64), ro, rl,
                "graph replay, new lengths")
    print(f"[graph] replay on new lengths vs oracle: {m}", flush=True)


def test_graph_replay_time_small_call():
    """Launch overhead of a small call, eager against graph replay (reported), and the
    replayed result equals a later eager call bit for bit."""
    torch, va = require_gpu()
    w = make_workload("graph_small", [312], B=1, Q=4, H=8, prefix_lens=[256], mask="chain", num_slots=1024)
    d = upload(w)
    ws = va.alloc_workspace(w.B, w.Q, w.H, w.total_kv, device="cuda")
    out, lse = _bufs(torch, w)

    def call():
        va.verify_attn(d["q"], d["kv_pool"], d["kv_indices"], d["prefix_lens"], d["tree_mask"],
                       float(w.scale), out=out, lse=lse, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()

    def timed(fn, n=200):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    timed(call, 20)
    timed(graph.replay, 20)
    eager_us, graph_us = timed(call), timed(graph.replay)
    print(f"[graph] tiny call: eager {eager_us:.1f} us/call, graph replay {graph_us:.1f} us/call", flush=True)
    ref_out, ref_lse = out.clone(), lse.clone()
    call()
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
