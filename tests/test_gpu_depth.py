"""GPU parity at full depth: the 36-layer Qwen3-4B-shaped stack (random
init, fp8 weights) through quail_join_run, against the oracle's per-pair
forward (float64, bf16 contract) stored in tests/golden/depth36_qwen3.json by
tests/golden/make_depth36.py.

Two joins: three anchors of 17, 40 and 71 tokens with 22 suffixes of 2-12
tokens each plus 6 filter rows, with bf16 anchor KV; two anchors of 33 and 90
tokens with 14 suffixes each plus 2 filter rows, with E4M3 anchor KV. The
same weights run at depths 1, 4, 12 and 36 (the first d layers of the
36-layer model), so the error's growth with depth is printed as well as
checked. Bar at every depth: logits within 2e-2 (infinity-norm relative over
the case), and every decision equal to the oracle's wherever the oracle's
TRUE-vs-FALSE margin exceeds 2e-2 of the largest logit magnitude; at least 64
such decisions in the bf16 join."""
import dataclasses
import json
import os

import numpy as np
import pytest

import workloads as W
from tests.gpu_util import say

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "depth36_qwen3.json")


@pytest.fixture(scope="module")
def setup():
    import torch
    assert torch.cuda.is_available()
    import sys
    sys.path.insert(0, os.path.dirname(GOLDEN))
    import make_depth36 as G
    from query_aware_prefill_amd import binding as B
    from query_aware_prefill_amd.device import DeviceModel
    B.load()
    doc = json.load(open(GOLDEN))
    say("depth36: generating the 36-layer weights on the host (about a minute)")
    shape = W.QWEN3_4B
    weights = W.model_weights(shape, G.WEIGHT_SEED)
    cases = G.build_cases()
    digest = G.input_digest(weights, cases)
    assert digest == doc["inputs_sha256_16"], "regenerated inputs differ from the golden file's"
    say("depth36: uploading weights")
    dm = DeviceModel(shape, weights, max_anchor_len=128, max_suffix_len=64)
    del weights
    return B, dm, cases, doc, G


def _run(B, dm, case, depth, fp8):
    """quail_join_run on the first `depth` layers; returns logits, decisions."""
    import torch
    from query_aware_prefill_amd.device import model_config, to_device
    shape = dataclasses.replace(W.QWEN3_4B, n_layers=depth, kv_fp8=fp8)
    cfg = model_config(shape, 128, 64)
    pool_bytes = sum(B.quail_anchor_bytes(cfg, int(x)) for x in case["a_len"]) + 4096
    pool = torch.empty(pool_bytes, dtype=torch.uint8, device="cuda")
    ws = torch.empty(B.quail_workspace_bytes(cfg, 512), dtype=torch.uint8, device="cuda")
    ctx = B.Context(cfg, dm.weights, pool, ws, 512)
    n = len(case["pair_anchor"])
    logits = torch.empty((n, 8), dtype=torch.float32, device="cuda")
    dec = torch.empty(n, dtype=torch.uint8, device="cuda")
    B.quail_join_run(ctx, to_device(case["a_tok"]), case["a_off"], case["pair_anchor"],
                     to_device(case["s_tok"]), case["s_off"], 0x0F, logits, None, dec)
    torch.cuda.synchronize()
    st = B.quail_pool_stats(ctx)
    used = len({int(a) for a in case["pair_anchor"] if a >= 0})
    assert st["prefills"] == used and st["evictions"] == used and st["regret_tokens"] == 0
    assert B.quail_ctx_check(ctx) == {"guard_errors": 0, "bad_tokens": 0}
    return logits.cpu().numpy().astype(np.float64), dec.cpu().numpy()


@pytest.mark.parametrize("name", ["bf16", "e4m3"])
def test_full_depth_join_against_oracle(setup, name):
    B, dm, cases, doc, G = setup
    case = cases[name]
    fp8 = doc["cases"][name]["fp8_kv"]
    rows = []
    for depth in doc["taps"]:
        ref = doc["results"][name][str(depth)]
        ref_logits = np.array(ref["logits"])
        say(f"depth36 {name}: {depth} layers, {len(ref_logits)} pairs")
        lg, dec = _run(B, dm, case, depth, fp8)
        err = float(np.max(np.abs(lg - ref_logits)) / np.max(np.abs(ref_logits)))
        tau = 2e-2 * float(np.max(np.abs(ref_logits)))
        sure = np.abs(np.array(ref["margin"])) > tau
        agree = int(np.sum(dec[sure] == np.array(ref["decision"])[sure]))
        rows.append((depth, err, int(sure.sum()), agree, len(dec)))
        say(f"  depth {depth:2d}: logits rel err {err:.4f}; decisions beyond tau {agree}/{int(sure.sum())} "
            f"agree (of {len(dec)} pairs)")
    for depth, err, n_sure, agree, n in rows:
        assert err <= 2e-2, (name, depth, err)
        assert agree == n_sure, (name, depth, agree, n_sure)
    if name == "bf16":
        assert rows[-1][2] >= 64, rows[-1]
