"""Writes depth36_qwen3_w8a8_sensitivity.json: how far the oracle's own W8A8
result moves when its bf16 roundings are disturbed the way two correct
implementations disagree, at depths 1, 4, 12 and 36 of the full-depth W8A8
case (tests/golden/make_depth36_w8a8.py).

An implementation that sums in another order (fp32 on the GPU, float64 here)
lands on the neighbouring bf16 value for a small fraction of its activations.
Without fp8 activations such one-ulp disagreements stay one-ulp sized. With
per-token E4M3 activations each one can flip an E4M3 code (a whole E4M3
step, 16 bf16 ulps) or, at a row's largest element, the row's scale. This
script plants exactly that disagreement in the oracle: at every bf16
rounding point of the contract, a seeded random fraction of the values
moves to a neighbouring bf16 value. It then measures the logits' infinity-norm
relative distance from the undisturbed oracle (the golden file). The GPU
parity test of the W8A8 stack takes its bar from these numbers.

Calls only the seeded generators (``workloads``) and the CPU oracle. Run
from the repository root (after make_depth36_w8a8.py):

    python tests/golden/make_w8a8_sensitivity.py      # ~12 minutes per fraction
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
import make_depth36_w8a8 as G8  # noqa: E402
import workloads as W  # noqa: E402
from oracle import model as M  # noqa: E402

FRACTIONS = (0.01, 0.05)
OUT = os.path.join(HERE, "depth36_qwen3_w8a8_sensitivity.json")


def disturbed_bf(frac, seed):
    rng = np.random.default_rng(seed)
    plain = M._bf

    def bf(x, mode):
        y = plain(x, mode)
        if mode != "contract":
            return y
        move = rng.random(y.shape) < frac
        _, e = np.frexp(y)
        ulp = np.ldexp(1.0, e - 8)          # the bf16 spacing at |y| (8 significant bits)
        return np.where(move, y + np.where(rng.random(y.shape) < 0.5, -ulp, ulp), y)
    return bf


def main():
    t0 = time.time()
    gold = json.load(open(G8.OUT))
    shape = dataclasses.replace(W.QWEN3_4B, act_fp8=True)
    weights = W.model_weights(shape, G.WEIGHT_SEED)
    cases = G.build_cases()
    assert G.input_digest(weights, cases) == gold["inputs_sha256_16"]
    c = cases[gold["case"]]
    seqs = []
    for i, a in enumerate(c["pair_anchor"]):
        at = c["a_tok"][c["a_off"][a]:c["a_off"][a + 1]] if a >= 0 else np.zeros(0, np.int32)
        seqs.append(np.concatenate([at, c["s_tok"][c["s_off"][i]:c["s_off"][i + 1]]]).astype(np.int64))
    doc = {"what": "infinity-norm relative distance of the oracle's W8A8 logits from the undisturbed oracle "
                   "when a fraction of its bf16 roundings land on the neighbouring bf16 value",
           "written_by": "tests/golden/make_w8a8_sensitivity.py (workloads + oracle only)",
           "case": gold["case"], "taps": gold["taps"], "inputs_sha256_16": gold["inputs_sha256_16"],
           "fractions": {}}
    plain = M._bf
    for k, frac in enumerate(FRACTIONS):
        M._bf = disturbed_bf(frac, 1000 + k)
        try:
            out = M.forward_many(seqs, weights, shape, mode="contract", dtype=np.float64, taps=G.TAPS)
        finally:
            M._bf = plain
        res = {}
        for d in gold["taps"]:
            r = out if d == shape.n_layers else out[d]
            ref = np.array(gold["results"][str(d)]["logits"])
            res[str(d)] = float(np.max(np.abs(r["logits"] - ref)) / np.max(np.abs(ref)))
        doc["fractions"][str(frac)] = res
        print(f"fraction {frac}: {res} ({time.time() - t0:.0f} s)", flush=True)
    with open(OUT, "w") as f:
        json.dump(doc, f, indent=1)
    print("wrote", OUT, flush=True)


if __name__ == "__main__":
    main()
