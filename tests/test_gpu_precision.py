"""GPU precision budget: the kernel's measured error against the exact fp64
oracle lies within a factor of two of what the oracle's precision model
predicts for it (fp16 probabilities and values in the value product, fp16
chunk partials; predictions committed in tests/golden/precision_budget.json by
tests/golden/make_precision_budget.py, which calls only the oracle). Kernel and
model cut the same chunks: the forced chunk length is passed to both."""

from __future__ import annotations

import json
import os

import pytest

import oracle
from gpu_util import compare, require_gpu, run_gpu, upload
from workloads import make_config

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "precision_budget.json")


@pytest.mark.parametrize("name", ["tiny", "p4k"])
def test_measured_error_within_twice_the_model(name):
    torch, va = require_gpu()
    with open(GOLDEN) as f:
        pred = json.load(f)[name]
    w = make_config(name)
    print(f"[precision] start {name} chunk_keys={pred['chunk_keys']}", flush=True)
    out, lse = run_gpu(va, upload(w), w.scale, chunk_keys=pred["chunk_keys"])
    ro, rl = oracle.verify_attention(w.q, w.kv_pool, w.kv_indices, w.prefix_lens, w.tree_mask, w.scale)
    m = compare(out, lse, ro, rl, name)
    r_rel = m["rel_l2"] / pred["rel_l2"]
    r_max = m["max_abs"] / pred["max_abs"]
    print(f"[precision] {name}: measured rel_l2 {m['rel_l2']:.3e} max_abs {m['max_abs']:.3e} lse_abs "
          f"{m['lse_abs']:.3e}; model rel_l2 {pred['rel_l2']:.3e} max_abs {pred['max_abs']:.3e}; "
          f"ratios {r_rel:.2f} / {r_max:.2f}", flush=True)
    assert 0.5 <= r_rel <= 2.0, f"{name}: measured rel-L2 {m['rel_l2']:.3e} vs model {pred['rel_l2']:.3e}"
    assert 0.5 <= r_max <= 2.0, f"{name}: measured max-abs {m['max_abs']:.3e} vs model {pred['max_abs']:.3e}"
