"""Writes w8a8_layer_sensitivity.json: for the one-layer join workload at full
size with per-token E4M3 activations (16 anchors x 1024 tokens, 512 suffixes
x 64 tokens each, Qwen3-4B layer shapes, workloads.c2_case(seed=2), weights
workloads.model_weights(..., 0)), the oracle's logits of the sampled pairs
the GPU test checks, and how far they move when one-ulp bf16 disagreements
are planted in 1% of the oracle's bf16 values (make_w8a8_sensitivity.py
explains the model of disagreement). The GPU test's bar is twice the
largest such movement over the sampled pairs, never below 2e-2.

Calls only the seeded generators (``workloads``) and the CPU oracle. Run
from the repository root:

    python tests/golden/make_w8a8_layer_sensitivity.py      # about two minutes
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
sys.path.insert(0, HERE)

import make_w8a8_sensitivity as S  # noqa: E402
import workloads as W  # noqa: E402
from oracle import model as M  # noqa: E402

FRACTION = 0.01
OUT = os.path.join(HERE, "w8a8_layer_sensitivity.json")


def sample_pairs(n):
    """The pairs the GPU test checks: first and last pair of the first and
    last anchor, two more."""
    return [0, 511, 8192 - 512, 8191] + np.random.default_rng(2).integers(0, n, 2).tolist()


def main():
    shape = W.ModelShape(n_layers=1, hidden=2560, n_q_heads=32, n_kv_heads=8, head_dim=128,
                         intermediate=9728, vocab=W.QWEN3_4B.vocab, act_fp8=True)
    wts = W.model_weights(shape, 0)
    case = W.c2_case(seed=2)
    n = len(case["pair_anchor"])
    layers = [M.LayerWeights(wts["layers"][0], shape)]
    out = {"what": "oracle W8A8 logits of the sampled pairs of the one-layer full-size join, and their "
                   "movement under one-ulp bf16 disagreements planted in 1% of the oracle's bf16 values",
           "written_by": "tests/golden/make_w8a8_layer_sensitivity.py (workloads + oracle only)",
           "fraction": FRACTION, "pairs": {}}
    plain = M._bf
    for k, i in enumerate(sample_pairs(n)):
        a = int(case["pair_anchor"][i])
        at = case["a_tok"][case["a_off"][a]:case["a_off"][a + 1]]
        st = case["s_tok"][case["s_off"][i]:case["s_off"][i + 1]]
        ref = M.forward_pair(at, st, wts, shape, layers=layers)
        M._bf = S.disturbed_bf(FRACTION, 2000 + k)
        try:
            moved = M.forward_pair(at, st, wts, shape, layers=layers)
        finally:
            M._bf = plain
        rel = float(np.max(np.abs(moved["logits"] - ref["logits"])) / np.max(np.abs(ref["logits"])))
        out["pairs"][str(int(i))] = {"logits": [float(x) for x in ref["logits"]], "margin": float(ref["margin"]),
                                     "decision": int(ref["decision"]), "moved_rel": rel}
        print(f"pair {i}: planted-disagreement movement {rel:.4f}", flush=True)
    with open(OUT, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", OUT, flush=True)


if __name__ == "__main__":
    main()
