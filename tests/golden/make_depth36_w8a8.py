"""Writes depth36_qwen3_w8a8.json: the oracle's logits, margins and
decisions for the full-depth W8A8 parity case (36 Qwen3-4B-shaped layers,
random init, fp8 weights, per-token E4M3 activations on every projection):
the "bf16" join of make_depth36.py (three anchors of 17, 40 and 71 tokens,
22 suffixes each, 6 filter rows, bf16 anchor KV), after 1, 4, 12 and 36
layers.

Calls only the seeded generators (``workloads``) and the CPU oracle
(``oracle.model.forward_many`` with ``act_fp8``). Run from the repository
root:

    python tests/golden/make_depth36_w8a8.py        # a few minutes on 8 cores
"""
import dataclasses
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
sys.path.insert(0, HERE)

import make_depth36 as G  # noqa: E402
import workloads as W  # noqa: E402
from oracle import model as M  # noqa: E402

CASE = "bf16"
OUT = os.path.join(HERE, "depth36_qwen3_w8a8.json")


def main():
    t0 = time.time()
    shape = dataclasses.replace(W.QWEN3_4B, act_fp8=True)
    weights = W.model_weights(shape, G.WEIGHT_SEED)
    cases = G.build_cases()
    c = cases[CASE]
    seqs = []
    for i, a in enumerate(c["pair_anchor"]):
        at = c["a_tok"][c["a_off"][a]:c["a_off"][a + 1]] if a >= 0 else np.zeros(0, np.int32)
        st = c["s_tok"][c["s_off"][i]:c["s_off"][i + 1]]
        seqs.append(np.concatenate([at, st]).astype(np.int64))
    print(f"inputs ready ({time.time() - t0:.0f} s); {sum(map(len, seqs))} oracle tokens", flush=True)
    out = M.forward_many(seqs, weights, shape, mode="contract", dtype=np.float64, taps=G.TAPS)
    print(f"oracle done ({time.time() - t0:.0f} s)", flush=True)
    doc = {"what": "oracle logits of the full-depth W8A8 parity case (float64, bf16 contract, "
                   "per-token E4M3 projection inputs)",
           "written_by": "tests/golden/make_depth36_w8a8.py (workloads + oracle only)",
           "shape": "Qwen3-4B: 36 layers, hidden 2560, 32q/8kv x 128, intermediate 9728, vocab 151936; act_fp8",
           "weights": f"workloads.model_weights(QWEN3_4B, {G.WEIGHT_SEED})",
           "case": CASE, "true_mask": 15, "taps": list(G.TAPS) + [shape.n_layers],
           "inputs_sha256_16": G.input_digest(weights, cases), "results": {}}
    for d in list(G.TAPS) + [shape.n_layers]:
        r = out if d == shape.n_layers else out[d]
        doc["results"][str(d)] = {"logits": [[float(x) for x in row] for row in r["logits"]],
                                  "margin": [float(x) for x in r["margin"]],
                                  "decision": [int(x) for x in r["decision"]],
                                  "token": [int(x) for x in r["token"]]}
    with open(OUT, "w") as f:
        json.dump(doc, f, indent=0)
    print("wrote", OUT, flush=True)


if __name__ == "__main__":
    main()
