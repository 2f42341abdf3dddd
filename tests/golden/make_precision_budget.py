"""Write tests/golden/precision_budget.json: the error the oracle's precision
model predicts for the GPU kernel on the two smallest seeded workloads.

The model (``oracle.chunked_attention_model``) runs the flash-decode method
with the precision the kernel keeps: probabilities and values in fp16 in the
value product, and each chunk's normalised partial output in fp16, on the
same chunk boundaries (a forced chunk length, which the GPU test passes to the
kernel too). Its error against the exact fp64 oracle is the prediction; the
GPU test checks that the kernel's measured error lies within a factor of two
of it. The file also records the two alternatives the kernel's precision was
chosen from: bf16 probabilities, and fp16 probabilities without rounded
partials. Only ``oracle/`` and ``workloads/`` are used. Run from the repo root:

    python tests/golden/make_precision_budget.py
"""

import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from workloads import make_config  # noqa: E402

# Forced chunk lengths (keys) of the predictions: the ones the automatic plan
# picks for these workloads on a 256-CU device, passed explicitly so that the
# model and the kernel cut the same chunks anywhere.
CHUNK_KEYS = {"tiny": 128, "p4k": 160}


def _errors(o, l, ro, rl):
    return {"rel_l2": float(np.linalg.norm(o - ro) / np.linalg.norm(ro)),
            "max_abs": float(np.abs(o - ro).max()),
            "lse_abs": float(np.abs(l - rl).max())}


def predict(name: str, chunk_keys: int) -> dict:
    w = make_config(name)
    args = (w.q, w.kv_pool, w.kv_indices, w.prefix_lens, w.tree_mask, w.scale)
    ro, rl = oracle.verify_attention(*args)
    kernel = oracle.chunked_attention_model(*args, chunk=chunk_keys)
    res = {"chunk_keys": chunk_keys, **_errors(*kernel, ro, rl)}
    bf16_p = oracle.chunked_attention_model(*args, chunk=chunk_keys, p_round="bf16")
    res["rel_l2_bf16_p"] = _errors(*bf16_p, ro, rl)["rel_l2"]
    res["max_abs_bf16_p"] = _errors(*bf16_p, ro, rl)["max_abs"]
    f16_only = oracle.chunked_attention_model(*args, chunk=chunk_keys, partial_round=None)
    res["rel_l2_f16_p_only"] = _errors(*f16_only, ro, rl)["rel_l2"]
    res["max_abs_f16_p_only"] = _errors(*f16_only, ro, rl)["max_abs"]
    return res


def main():
    g = {"model": "oracle.chunked_attention_model: fp16 p and v in the value product, fp16 chunk partials, "
                  "32-key tiles, fp64 elsewhere; errors against oracle.verify_attention"}
    for name, ck in CHUNK_KEYS.items():
        g[name] = predict(name, ck)
        print(name, g[name], flush=True)
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "precision_budget.json")
    with open(path, "w") as f:
        json.dump(g, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
