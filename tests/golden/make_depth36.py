"""Writes depth36_qwen3.json: the oracle's logits, margins and decisions for
the full-depth parity cases (36 Qwen3-4B-shaped layers, random init, fp8
weights): a join with bf16 anchor KV and one with E4M3 anchor KV (each with
filter rows), three joins over one anchor table with E4M3 anchor KV, and
suffix families sharing prefixes under anchors and among filter rows (bf16
KV), after 1, 4, 12 and 36 layers. Every pair's expected result is the
per-pair definition, whichever entry point the GPU runs it through.

Calls only the seeded generators (``workloads``) and the CPU oracle
(``oracle.model.forward_many``, the per-pair definition: a monolithic causal
forward over [anchor ‖ suffix], then the 8-column head at the last position).
The oracle runs in float64 with bf16 rounding at the contract points. Run from
the repository root:

    python tests/golden/make_depth36.py        # about 10 minutes on 8 cores
"""
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402
from oracle import model as M  # noqa: E402

WEIGHT_SEED = 40
TAPS = (1, 4, 12)
CASES = {
    # name: (seed, anchor lengths, suffixes per anchor, filter rows, fp8 anchor KV), run by
    # quail_join_run
    "bf16": (40, [17, 40, 71], 22, 6, False),
    "e4m3": (41, [33, 90], 14, 2, True),
}
# three joins over one anchor table (E4M3 KV), run by quail_multijoin_run
MULTIJOIN = dict(seed=42, a_len=[25, 60, 100, 44], n_joins=3, per_join=8, fp8_kv=True)
# suffix families sharing a prefix under two anchors and among filter rows
# (bf16 KV), run by quail_join_run_shared; (anchor, shared tokens, [own tokens])
SHARED = dict(seed=43, a_len=[30, 50], fp8_kv=False,
              families=[(0, 12, [3, 5, 7, 4]), (1, 10, [6, 2, 9]), (0, 6, [4, 4]), (-1, 14, [3, 5, 2])])
OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "depth36_qwen3.json")


def sha(a) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()[:16]


def input_digest(weights, cases) -> dict:
    """Hashes that let a consumer check it regenerated the same inputs."""
    l0, lz = weights["layers"][0], weights["layers"][-1]
    d = {"embed": sha(weights["embed"]), "head8": sha(weights["head8"]),
         "final_norm": sha(weights["final_norm"]),
         "layer0_w_qkv": sha(l0["w_qkv"]), "layer0_s_down": sha(l0["s_down"]),
         "layer35_w_gate_up": sha(lz["w_gate_up"]), "layer35_s_o": sha(lz["s_o"])}
    for name, c in cases.items():
        d[name + "_tokens"] = sha(np.concatenate([c["a_tok"], c["s_tok"], c["pair_anchor"], c["s_off"]]))
    return d


def build_cases() -> dict:
    out = {name: W.depth_case(seed, a_len, per, nf) for name, (seed, a_len, per, nf, _) in CASES.items()}
    m = MULTIJOIN
    out["multijoin_e4m3"] = W.depth_multijoin_case(m["seed"], m["a_len"], m["n_joins"], m["per_join"])
    sh = SHARED
    out["shared_bf16"] = W.shared_prefix_case(sh["seed"], W.QWEN3_4B.vocab, sh["a_len"], sh["families"],
                                              cfg_id=10)
    return out


def fp8_of(name) -> bool:
    if name in CASES:
        return CASES[name][4]
    return {"multijoin_e4m3": MULTIJOIN["fp8_kv"], "shared_bf16": SHARED["fp8_kv"]}[name]


def main():
    t0 = time.time()
    shape = W.QWEN3_4B
    weights = W.model_weights(shape, WEIGHT_SEED)
    cases = build_cases()
    seqs, upto, owner = [], [], []
    for name, c in cases.items():
        fp8 = fp8_of(name)
        for i, a in enumerate(c["pair_anchor"]):
            at = c["a_tok"][c["a_off"][a]:c["a_off"][a + 1]] if a >= 0 else np.zeros(0, np.int32)
            st = c["s_tok"][c["s_off"][i]:c["s_off"][i + 1]]
            seqs.append(np.concatenate([at, st]).astype(np.int64))
            upto.append(len(at) if fp8 else 0)
            owner.append(name)
    print(f"inputs ready ({time.time() - t0:.0f} s); {sum(map(len, seqs))} oracle tokens", flush=True)
    out = M.forward_many(seqs, weights, shape, mode="contract", dtype=np.float64,
                         fp8_kv_upto=upto, taps=TAPS)
    print(f"oracle done ({time.time() - t0:.0f} s)", flush=True)
    owner = np.array(owner)
    doc = {"what": "oracle logits of the full-depth parity cases (float64, bf16 contract)",
           "written_by": "tests/golden/make_depth36.py (workloads + oracle only)",
           "shape": "Qwen3-4B: 36 layers, hidden 2560, 32q/8kv x 128, intermediate 9728, vocab 151936",
           "weights": f"workloads.model_weights(QWEN3_4B, {WEIGHT_SEED})",
           "true_mask": 15, "taps": list(TAPS) + [shape.n_layers],
           "cases": {**{name: {"seed": v[0], "a_len": v[1], "per_anchor": v[2], "n_filter": v[3],
                               "fp8_kv": v[4], "run": "quail_join_run"} for name, v in CASES.items()},
                     "multijoin_e4m3": {**MULTIJOIN, "run": "quail_multijoin_run"},
                     "shared_bf16": {**{k: v for k, v in SHARED.items()}, "run": "quail_join_run_shared"}},
           "inputs_sha256_16": input_digest(weights, cases), "results": {}}
    for name in cases:
        sel = owner == name
        res = {}
        for d in list(TAPS) + [shape.n_layers]:
            r = out if d == shape.n_layers else out[d]
            res[str(d)] = {"logits": [[float(x) for x in row] for row in r["logits"][sel]],
                           "margin": [float(x) for x in r["margin"][sel]],
                           "decision": [int(x) for x in r["decision"][sel]],
                           "token": [int(x) for x in r["token"][sel]]}
        doc["results"][name] = res
    with open(OUT, "w") as f:
        json.dump(doc, f, indent=0)
    print("wrote", OUT, flush=True)


if __name__ == "__main__":
    main()
