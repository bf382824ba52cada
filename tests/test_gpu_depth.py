"""GPU parity at full depth: the 36-layer Qwen3-4B-shaped stack (random
init, fp8 weights) against the oracle's per-pair forward (float64, bf16
contract) stored in tests/golden/depth36_qwen3.json by
tests/golden/make_depth36.py.

Through quail_join_run, two joins: three anchors of 17, 40 and 71 tokens
with 22 suffixes of 2-12 tokens each plus 6 filter rows, with bf16 anchor KV;
two anchors of 33 and 90 tokens with 14 suffixes each plus 2 filter rows, with
E4M3 anchor KV. Through quail_multijoin_run, three joins of 8 pairs over four
anchors (E4M3 KV) in a pool for two anchors, so anchors are evicted and
prefilled again between joins (counters against the plan). Through
quail_join_run_shared, suffix families sharing 6-14 prefix tokens under two
anchors and among filter rows (bf16 KV; prefix nodes prefilled once). The
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


def _run(B, dm, case, depth, fp8, run, act_fp8=False):
    """The case through the first `depth` layers by entry point `run`
    (quail_join_run, quail_multijoin_run with a pool for the two largest
    anchors, or quail_join_run_shared); returns logits and decisions."""
    import torch
    from query_aware_prefill_amd.device import model_config, to_device
    shape = dataclasses.replace(W.QWEN3_4B, n_layers=depth, kv_fp8=fp8, act_fp8=act_fp8)
    cfg = model_config(shape, 128, 64)
    slabs = sorted(B.quail_anchor_bytes(cfg, int(x)) for x in case["a_len"])
    if run == "quail_multijoin_run":
        pool_bytes = slabs[-1] + slabs[-2] + B.GUARD_BYTES      # forces evictions between joins
    elif run == "quail_join_run_shared":
        pool_bytes = sum(slabs) + 6 * B.quail_anchor_bytes(cfg, int(np.max(case["s_len"]))) + 4096
    else:
        pool_bytes = sum(slabs) + 4096
    pool = torch.empty(pool_bytes, dtype=torch.uint8, device="cuda")
    ws = torch.empty(B.quail_workspace_bytes(cfg, 512), dtype=torch.uint8, device="cuda")
    ctx = B.Context(cfg, dm.weights, pool, ws, 512)
    n = len(case["pair_anchor"])
    logits = torch.empty((n, 8), dtype=torch.float32, device="cuda")
    dec = torch.empty(n, dtype=torch.uint8, device="cuda")
    a_tok, s_tok = to_device(case["a_tok"]), to_device(case["s_tok"])
    used = len({int(a) for a in case["pair_anchor"] if a >= 0})
    if run == "quail_multijoin_run":
        B.quail_multijoin_run(ctx, a_tok, case["a_off"], case["join_offsets"], case["pair_anchor"], s_tok,
                              case["s_off"], 0x0F, logits, None, dec)
    elif run == "quail_join_run_shared":
        B.quail_join_run_shared(ctx, a_tok, case["a_off"], case["pair_anchor"], s_tok, case["s_off"],
                                case["s_tok"], 4, 0x0F, logits, None, dec)
    else:
        B.quail_join_run(ctx, a_tok, case["a_off"], case["pair_anchor"], s_tok, case["s_off"], 0x0F, logits,
                         None, dec)
    torch.cuda.synchronize()
    st = B.quail_pool_stats(ctx)
    if run == "quail_multijoin_run":
        plan = B.quail_multiplan_build(cfg, pool_bytes - B.GUARD_BYTES, 512, case["a_len"], case["join_offsets"],
                                       case["pair_anchor"], case["s_len"])
        assert (st["prefills"], st["evictions"], st["regret_tokens"]) == \
            (plan["prefills"], plan["evictions"], plan["regret_tokens"]), (st, plan)
        assert plan["prefills"] > used          # the tight pool re-prefills some anchor
    elif run == "quail_join_run_shared":
        assert st["prefills"] > used and st["prefills"] == st["evictions"] and st["regret_tokens"] == 0
    else:
        assert st["prefills"] == used and st["evictions"] == used and st["regret_tokens"] == 0
    assert st["resident"] == 0
    assert B.quail_ctx_check(ctx) == {"guard_errors": 0, "bad_tokens": 0}
    return logits.cpu().numpy().astype(np.float64), dec.cpu().numpy()


@pytest.mark.parametrize("name", ["bf16", "e4m3", "multijoin_e4m3", "shared_bf16"])
def test_full_depth_join_against_oracle(setup, name):
    B, dm, cases, doc, G = setup
    case = cases[name]
    fp8 = doc["cases"][name]["fp8_kv"]
    run = doc["cases"][name]["run"]
    rows = []
    for depth in doc["taps"]:
        ref = doc["results"][name][str(depth)]
        ref_logits = np.array(ref["logits"])
        say(f"depth36 {name}: {depth} layers, {len(ref_logits)} pairs")
        lg, dec = _run(B, dm, case, depth, fp8, run)
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


GOLDEN_W8A8 = os.path.join(os.path.dirname(GOLDEN), "depth36_qwen3_w8a8.json")
SENSITIVITY_W8A8 = os.path.join(os.path.dirname(GOLDEN), "depth36_qwen3_w8a8_sensitivity.json")


def w8a8_bars():
    """Per depth: twice the distance by which the oracle's own W8A8 logits
    move when one-ulp bf16 disagreements are planted in 1% of its bf16 values
    (tests/golden/make_w8a8_sensitivity.py), and never below the 2e-2 bar.
    E4M3 codes are decided from bf16 values, so two correct implementations
    whose bf16 roundings differ in a few places differ by about that much; the
    GPU's first-layer K/V bf16 values differ from the oracle's in 0.1% (W8A16)
    and 1.1% (W8A8) of elements."""
    doc = json.load(open(SENSITIVITY_W8A8))
    return {int(d): max(2e-2, 2.0 * v) for d, v in doc["fractions"]["0.01"].items()}


def test_full_depth_w8a8_join_against_oracle(setup):
    """The bf16-KV join through the 36-layer stack with per-token E4M3
    activations (W8A8) against the oracle's W8A8 reading
    (tests/golden/depth36_qwen3_w8a8.json, tests/golden/make_depth36_w8a8.py)
    at depths 1, 4, 12 and 36: logits within the bar above, decisions equal
    wherever the oracle's margin exceeds the bar times the largest logit
    (bars from w8a8_bars)."""
    B, dm, cases, doc, G = setup
    d8 = json.load(open(GOLDEN_W8A8))
    assert d8["inputs_sha256_16"] == doc["inputs_sha256_16"]
    bars = w8a8_bars()
    case = cases[d8["case"]]
    rows = []
    for depth in d8["taps"]:
        ref = d8["results"][str(depth)]
        ref_logits = np.array(ref["logits"])
        say(f"depth36 w8a8: {depth} layers, {len(ref_logits)} pairs")
        lg, dec = _run(B, dm, case, depth, False, "quail_join_run", act_fp8=True)
        err = float(np.max(np.abs(lg - ref_logits)) / np.max(np.abs(ref_logits)))
        sure = np.abs(np.array(ref["margin"])) > bars[depth] * float(np.max(np.abs(ref_logits)))
        agree = int(np.sum(dec[sure] == np.array(ref["decision"])[sure]))
        all_agree = int(np.sum(dec == np.array(ref["decision"])))
        rows.append((depth, err, int(sure.sum()), agree))
        say(f"  depth {depth:2d}: logits rel err {err:.4f} (bar {bars[depth]:.4f}); decisions beyond the bar "
            f"{agree}/{int(sure.sum())} agree; all decisions {all_agree}/{len(dec)}")
    for depth, err, n_sure, agree in rows:
        assert err <= bars[depth], (depth, err, bars[depth])
        assert agree == n_sure, (depth, agree, n_sure)
