"""The allocation-free entry point (verify_attn_noalloc, for callers that cannot
allocate): through the C ABI it gives verify_attn's results bit for bit, on two
calls in a row that share the fixed device scratch, the second with a smaller
input; and sizes beyond the scratch are rejected before anything runs."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_util import compare, require_gpu, upload
from workloads import make_config, make_workload

pytestmark = pytest.mark.gpu


def _bufs(torch, w):
    return (torch.full((w.B, w.Q, w.H, 512), float("nan"), dtype=torch.float32, device="cuda"),
            torch.full((w.B, w.Q, w.H), float("nan"), dtype=torch.float32, device="cuda"))


def _both(torch, va, w):
    d = upload(w)
    ref_out, ref_lse = va.verify_attn(d["q"], d["kv_pool"], d["kv_indices"], d["prefix_lens"], d["tree_mask"],
                                      float(w.scale))
    out, lse = _bufs(torch, w)
    va.verify_attn_noalloc(d["q"], d["kv_pool"], d["kv_indices"], d["prefix_lens"], d["tree_mask"],
                           float(w.scale), out, lse)
    torch.cuda.synchronize()
    return out, lse, ref_out, ref_lse


def test_noalloc_equals_verify_attn_on_two_calls_in_a_row():
    torch, va = require_gpu()
    big = make_config("tree32k")
    small = make_workload("noalloc_small", [320], B=3, Q=5, H=12, prefix_lens=[700, 0, 2100], mask="tree",
                          num_slots=4000)
    print(f"[noalloc] workspace bytes: tree32k {va.workspace_size(big.B, big.Q, big.H, big.total_kv)}, "
          f"small {va.workspace_size(small.B, small.Q, small.H, small.total_kv)}", flush=True)
    for label, w in (("tree32k", big), ("small", small)):
        print(f"[noalloc] start {label}", flush=True)
        out, lse, ref_out, ref_lse = _both(torch, va, w)
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), f"{label}: differs from verify_attn"
        ro, rl = oracle.verify_attention(w.q, w.kv_pool, w.kv_indices, w.prefix_lens, w.tree_mask, w.scale)
        m = compare(out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ro, rl, label)
        print(f"[noalloc] {label}: bitwise equal to verify_attn; vs oracle {m}", flush=True)


def test_noalloc_rejects_sizes_beyond_the_scratch():
    torch, va = require_gpu()
    B, Q, H, total = 64, 16, 64, 64 * 100_000
    assert va.workspace_size(B, Q, H, total) > (64 << 20)
    lib = va.load_library()
    x = torch.zeros(64, dtype=torch.float32, device="cuda")   # never read: rejected on the host
    p = x.data_ptr()
    rc = lib.verify_attn_noalloc(p, p, p, p, p, 0.1, p, p, B, Q, H, 1000, total, None)
    assert rc == va.VA_ENOSPC
    assert "scratch" in lib.verify_attn_last_error().decode()
