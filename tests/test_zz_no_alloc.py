"""The allocation-free cascade-attention entry point
(quail_cascade_attn_noalloc, per-call metadata in the library's static
scratch array) against the workspace entry point (quail_cascade_attn) on the
same inputs: identical outputs and LSE, bit for bit, on calls in a row whose
sizes shrink (the scratch keeps the previous call's contents), for bf16,
E4M3-anchor and fp32 inputs; and the packed (few tokens per anchor) tiling."""
import numpy as np
import pytest

import workloads as W
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    import torch
    assert torch.cuda.is_available()
    from query_aware_prefill_amd import binding
    binding.load()
    return binding


def _both(B, dtype, case, hq, hkv, d, out_dtype):
    import torch
    T = int(case["s_off"][-1])
    outs = []
    for which in ("workspace", "noalloc"):
        out = torch.full((T, hq, d), float("nan"), dtype=out_dtype, device="cuda")
        lse = torch.full((T, hq), float("nan"), dtype=torch.float32, device="cuda")
        if which == "workspace":
            ws = torch.empty(B.quail_cascade_workspace_bytes(case["a_off"], case["s_off"]), dtype=torch.uint8,
                             device="cuda")
            B.quail_cascade_attn(dtype, hq, hkv, d, case["sm_scale"], case["ak"], case["av"], case["a_off"],
                                 case["s_anchor"], case["q"], case["k"], case["v"], case["s_off"], out, lse, ws)
        else:
            B.quail_cascade_attn_noalloc(dtype, hq, hkv, d, case["sm_scale"], case["ak"], case["av"],
                                         case["a_off"], case["s_anchor"], case["q"], case["k"], case["v"],
                                         case["s_off"], out, lse)
        torch.cuda.synchronize()
        outs.append((out, lse))
    (o1, l1), (o2, l2) = outs
    assert torch.equal(o1.view(torch.uint8) if o1.dtype != torch.float32 else o1.view(torch.int32),
                       o2.view(torch.uint8) if o2.dtype != torch.float32 else o2.view(torch.int32))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    assert not torch.isnan(o2.float()).any() and not torch.isnan(l2).any()


@pytest.mark.parametrize("anchor_kv", ["bf16", "e4m3"])
def test_noalloc_equals_workspace_entry_bf16(B, anchor_kv):
    import torch
    dtype = B.DTYPE_BF16 if anchor_kv == "bf16" else B.DTYPE_FP8_E4M3
    r = np.random.default_rng(51)
    # call 1: 24 anchors of 100..700 tokens, 3 suffixes each, plus filter rows
    # call 2 (smaller): 5 anchors, 2 suffixes each
    # call 3 (smaller still, packed tiles): 4 anchors, one 3-token suffix each
    calls = []
    a_len = r.integers(100, 701, 24)
    s_anchor = np.concatenate([np.repeat(np.arange(24), 3), [-1, -1]])
    calls.append((a_len, s_anchor, r.integers(5, 91, len(s_anchor))))
    a_len = r.integers(40, 300, 5)
    s_anchor = np.repeat(np.arange(5), 2)
    calls.append((a_len, s_anchor, r.integers(1, 70, len(s_anchor))))
    calls.append((r.integers(60, 200, 4), np.arange(4), np.full(4, 3)))
    for i, (a_len, s_anchor, s_len) in enumerate(calls):
        say("noalloc", anchor_kv, "call", i, "tokens", int(np.sum(s_len)))
        case = W.cascade_device(60 + i, a_len, s_anchor, s_len, hq=32, hkv=8, d=128, anchor_kv=anchor_kv)
        _both(B, dtype, case, 32, 8, 128, torch.bfloat16)


def test_noalloc_equals_workspace_entry_f32(B):
    import torch
    from query_aware_prefill_amd.device import to_device
    for i, (a_len, s_anchor, s_len) in enumerate([([64, 90], [0, 0, 1, -1, 1], [32, 7, 20, 9, 31]),
                                                  ([17], [0, -1], [5, 3])]):
        say("noalloc f32 call", i)
        case = W.cascade_case(70 + i, a_len, s_anchor, s_len, hq=4, hkv=2, d=64, dtype="f32")
        dev = dict(case)
        for key in ("ak", "av", "q", "k", "v"):
            dev[key] = to_device(case[key])
        _both(B, B.DTYPE_F32, dev, 4, 2, 64, torch.float32)
