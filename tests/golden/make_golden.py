"""Write tests/golden/tiny_oracle.json from the fp64 oracle (no GPU code involved).

The pages print no numeric outputs for any worked example, so this file is a
regression fixture of the oracle itself on the seeded "tiny" workload
(1 sequence, 8 heads, 4 verify positions in a causal chain, prefix 256,
kv_indices from a permutation of a 1024-slot pool). Run from the repo root:

    python tests/golden/make_golden.py
"""

import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from workloads import make_config  # noqa: E402


def main():
    w = make_config("tiny")
    out, lse = oracle.verify_attention(w.q, w.kv_pool, w.kv_indices, w.prefix_lens, w.tree_mask, w.scale)
    rng = np.random.default_rng(0)
    idx = [[0, int(rng.integers(4)), int(rng.integers(8)), int(rng.integers(512))] for _ in range(24)]
    g = {
        "workload": "tiny (seeded, see workloads.gen.CONFIGS)",
        "lse": [float(x) for x in lse.reshape(-1)],
        "out_index": idx,
        "out_value": [float(out[b, i, h, d]) for b, i, h, d in idx],
        "out_norm": float(np.linalg.norm(out)),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle.json")
    with open(path, "w") as f:
        json.dump(g, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
