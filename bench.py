"""Benchmark: AI.IF join prefill on the 36-layer Qwen3-4B-shaped stack.

Headline workload: the 36-layer join -- 64 anchors of 1024 tokens, each
joined to 2048 suffixes of 64 tokens (131,072 pairs; random-init fp8
weights, bf16 activations and anchor KV). One step is a fixed 1/32 share of
that join: two consecutive anchors with all of their 4,096 pairs, run end to
end by quail_join_run (plan, anchor prefill + KV writer, join prefill through
all 36 layers with cascade attention, the 8-column head and the booleans).
Step k takes anchors 2k and 2k+1 (mod 64); every step is the same amount of
work, so 32 steps are the whole join.

Reported:
  value      logical prefill tokens per minute: sum over the step's pairs of
             La + Ls (1088 tokens per pair) -- the tokens a per-pair engine
             would prefill; the tokens actually computed (suffixes plus each
             anchor once) are reported beside it.
  roofline   the dominant kernel, the gate/up projection with the SwiGLU
             epilogue (W8A16 GEMM): algorithmic FLOP per launch (2 * M *
             19456 * 2560 for M batch tokens) / its average launch duration,
             both from HIP events recorded around every launch on the
             launch stream during the timed steps (quail_ctx_profile),
             against the bf16 dense MFMA peak (2.5 PFLOP/s). The other
             kernels' rates are listed beside it, and the headline
             cascade-attention configuration (256 anchors x 64 suffixes,
             one layer, bf16 Q/K/V) is timed as a field of its own.
  cpu_baseline  the CPU oracle's per-pair forward (36 layers over
             [anchor | suffix], float32 with the bf16 rounding points) on
             sampled pairs of the same join, scaled to logical tokens/min.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Secondary measurements (not the headline line; each prints its own JSON):
  --workload cascade the cascade-attention layer alone at the Qwen3-4B shape:
                     256 anchors of U{512..2048} tokens, each joined to 64
                     suffixes of U{32..128} tokens; bf16 Q/K/V ~ N(0, 1)
                     resident in HBM; TFLOP/s of the attention kernel
                     (4*Hq*d*La per suffix token for the cross part,
                     4*Hq*d*(j+1) at suffix position j for the self part).
  --workload gemm    the four W8A16 projection shapes of the Qwen3-4B layer
                     (QKV 6144x2560, O 2560x4096, gate/up 19456x2560, down
                     2560x9728) at M = 65536 tokens, TFLOP/s against the bf16
                     MFMA peak.
  --workload gemm8   the W8A8 path at the same four shapes and M = 65536:
                     per-token E4M3 activation quantisation (GB/s against
                     8 TB/s: 2 B read + 1 B written per element) and the
                     fp8 x fp8 GEMM (TFLOP/s against the fp8 MFMA peak),
                     beside the W8A16 kernel on the same shapes.
  --workload copy    a plain 4 GiB device-to-device copy (read 4 GiB, write
                     4 GiB): the calibration kernel for the HBM byte counters.
  --workload stream  anchor-KV streaming sweep: 1024 anchors of 768 tokens
                     (K/V of one layer: bf16, 3.2 GB, or E4M3 codes, 1.6 GB),
                     each read by one suffix of S tokens, S in {1, 4, 16, 32,
                     64, 256, 4096}; anchor KV bytes per launch / launch time against
                     8 TB/s, and TFLOP/s (4*S FLOP per bf16 KV byte, 8*S per
                     E4M3 byte); then the whole 36-layer E4M3 pool (57.98 GB,
                     one launch per layer) for S in {1, 4, 16, 32}.
  --workload join36 | filter36 | multijoin36
                     end to end on the 36-layer Qwen3-4B-shaped stack with
                     random-init fp8 weights (quail_join_run: plan, anchor
                     prefill + KV writer, join prefill, 8-column head):
                     join36 = 64 anchors x 1024 tokens, 2048 suffixes of 64
                     tokens each; filter36 = 10,000 rows of lognormal lengths
                     200..2000, no anchor; multijoin36 = 1024 anchors x 768
                     tokens with fp8 KV, rows of U{48..256} tokens each probing
                     51 anchors (--rows selects how many of the 5,000 rows).
                     Logical and computed tokens/min; the oracle leg runs the
                     per-pair definition on a few sampled pairs and compares
                     logits and decisions.
                     --act-fp8 runs them (and multijoin36full) with per-token E4M3 activations
                     (W8A8 projections on the fp8 MFMA) against the
                     oracle's W8A8 reading.
  --workload multiplan36
                     three joins over the join36 anchor table (64 anchors x
                     1024 tokens), 8,192 pairs of 64-token suffixes each, on
                     the 36-layer stack: plan-wide residency across the joins
                     (quail_multijoin_run: each anchor prefilled once) against
                     the joins run one by one (quail_join_run each: each anchor
                     prefilled once per join); times, prefills and whether the
                     logits are identical.
  --workload layer   one decoder layer of the Qwen3-4B shape, random-init fp8
                     weights: 16 anchors x 1024 tokens, 512 suffixes x 64
                     tokens per anchor: anchor prefill + KV writer, join
                     prefill of every suffix row (all hidden rows returned),
                     head.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0
# projection FLOP per token per layer (Qwen3-4B shapes): QKV 2*2560*6144, O
# 2*4096*2560, gate/up 2*2560*19456, down 2*9728*2560; and the QKV share
GEMM_FLOP_LAYER = 201_850_880.0
GEMM_FLOP_QKV = 31_457_280.0


def executed_gemm_flops(n_layers, suffix_tok, n_last, anchor_tok):
    """Projection FLOP a join prefill returning each pair's last row executes:
    suffix tokens run every layer but the last, and the last layer's QKV
    projection (their K/V feed the last rows' attention); the pairs' last rows
    also the last layer's O projection and MLP; anchors every layer but the
    last, and the last layer's QKV projection (their K/V is all the pairs
    read)."""
    per_tok = GEMM_FLOP_LAYER * (n_layers - 1) + GEMM_FLOP_QKV
    return per_tok * (suffix_tok + anchor_tok) + (GEMM_FLOP_LAYER - GEMM_FLOP_QKV) * n_last
HBM_PEAK_GBS = 8000.0
METRIC = "prefill tokens/min per GPU on join workload; cascade-attn TFLOP/s vs MFMA peak"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "cascade_attn_c1_hbm_traffic.txt")
KERNEL_SOURCES = ["query_aware_prefill_amd/csrc/attn.hip", "query_aware_prefill_amd/csrc/device_common.h",
                  "query_aware_prefill_amd/csrc/quail_internal.h"]
GEMM_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_gate_up_join36_hbm_traffic.txt")
GEMM_SOURCES = ["query_aware_prefill_amd/csrc/gemm.hip", "query_aware_prefill_amd/csrc/device_common.h",
                "query_aware_prefill_amd/csrc/quail_internal.h"]


def measured_traffic(path=TRAFFIC_FILE, sources=KERNEL_SOURCES):
    """HBM bytes per launch from a committed counter summary, or None when
    the kernel sources have changed since the counters were taken."""
    import hashlib
    try:
        kv = {}
        for line in open(path):
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
        h = hashlib.sha256()
        for f in sources:
            h.update(open(os.path.join(ROOT, f), "rb").read())
        if h.hexdigest() != kv.get("kernel_sources_sha256"):
            return None
        return float(kv["traffic_bytes"])
    except (OSError, KeyError, ValueError):
        return None


def algorithmic_flops(a_len, s_anchor, s_len, hq=32, d=128):
    la = np.where(s_anchor >= 0, a_len[np.maximum(s_anchor, 0)], 0).astype(np.float64)
    ls = s_len.astype(np.float64)
    cross = 4.0 * hq * d * np.sum(ls * la)
    self_ = 4.0 * hq * d * np.sum(ls * (ls + 1) / 2)
    return cross, self_


def algorithmic_bytes(a_len, s_len, hq=32, hkv=8, d=128):
    """Q read + O write + suffix K/V read + anchor K/V read once (bf16)."""
    ts, ta = float(np.sum(s_len)), float(np.sum(a_len))
    return 2.0 * (ts * hq * d * 2 + ts * hkv * d * 2 + ta * hkv * d * 2)


def cpu_baseline(case, budget_s=15.0):
    """Oracle on a time-bounded random sample of the workload's pairs, scaled
    to logical tokens/min. Only the oracle's compute is timed (not the
    device-to-host copies of its inputs)."""
    import torch
    from oracle import attention as OA
    threads = torch.get_num_threads()
    n_suf = len(case["s_len"])
    order = np.random.default_rng(0).permutation(n_suf)

    def host(t):
        return t.float().cpu().numpy().astype(np.float64)

    spent = 0.0
    done = logical = computed = 0
    for s in order:
        t_s0, t_s1 = int(case["s_off"][s]), int(case["s_off"][s + 1])
        a = int(case["s_anchor"][s])
        a0, a1 = int(case["a_off"][a]), int(case["a_off"][a + 1])
        q, k, v = host(case["q"][t_s0:t_s1]), host(case["k"][t_s0:t_s1]), host(case["v"][t_s0:t_s1])
        ka, va = host(case["ak"][a0:a1]), host(case["av"][a0:a1])
        c0 = time.perf_counter()
        OA.monolithic_pair_attention(q, ka, va, k, v, case["sm_scale"])
        spent += time.perf_counter() - c0
        done += 1
        logical += (a1 - a0) + (t_s1 - t_s0)
        computed += t_s1 - t_s0
        if spent >= budget_s:
            break
    return {"value": logical / spent * 60.0, "unit": "tokens/min", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {n_suf} (anchor, suffix) pairs drawn at random from the same workload, "
                      f"monolithic causal attention over [anchor | suffix] in float64 "
                      f"({logical} logical / {computed} suffix tokens in {spent:.1f} s of oracle compute)"}


def bench_gemm(args):
    import torch
    import workloads as W
    from query_aware_prefill_amd import binding as B
    from query_aware_prefill_amd.device import to_device
    B.load()
    M = 65536
    r = np.random.default_rng(0)
    out = {"metric": "W8A16 GEMM TFLOP/s", "unit": "TFLOP/s", "M": M, "shapes": {}}
    x_full = torch.randn((M, 9728), device="cuda", dtype=torch.float32).to(torch.bfloat16)
    for name, (N, K) in {"qkv": (6144, 2560), "o": (2560, 4096), "gate_up": (19456, 2560),
                         "down": (2560, 9728)}.items():
        x = x_full[:, :K].contiguous()
        w = to_device(W.draw_fp8_codes(r, (N, K)))
        sc = to_device(W.bf16_bits_from_f32((0.0002 * (1 + r.random(N))).astype(np.float32)))
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        for _ in range(args.warmup):
            B.quail_gemm_w8a16(x, w, sc, y)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        torch.cuda.synchronize()
        for a, b in ev:
            a.record()
            B.quail_gemm_w8a16(x, w, sc, y)
            b.record()
        torch.cuda.synchronize()
        ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
        tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
        # context only: the vendor library's plain bf16 GEMM of the same shape
        # (bf16 weights; not the W8A16 operation measured above)
        wb = torch.randn((N, K), device="cuda", dtype=torch.float32).to(torch.bfloat16)
        for _ in range(args.warmup):
            torch.matmul(x, wb.t())
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True); t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(args.steps):
            torch.matmul(x, wb.t())
        t1.record()
        torch.cuda.synchronize()
        ref_ms = t0.elapsed_time(t1) / args.steps
        del wb
        out["shapes"][name] = {"N": N, "K": K, "ms": ms, "tflops": tf, "frac": tf / PEAK_BF16_TFLOPS,
                               "torch_bf16_matmul_tflops": 2.0 * M * N * K / (ref_ms * 1e-3) / 1e12}
        log(f"gemm {name} {M}x{N}x{K}: {ms:.3f} ms, {tf:.1f} TFLOP/s "
            f"(torch bf16 matmul {out['shapes'][name]['torch_bf16_matmul_tflops']:.1f})")
    print(json.dumps(out), flush=True)


def _timed(fn, steps, warmup):
    """Mean ms of fn() over `steps` launches (events around each)."""
    import torch
    for _ in range(warmup):
        fn()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in ev]))


def bench_gemm8(args):
    import torch
    import workloads as W
    from query_aware_prefill_amd import binding as B
    from query_aware_prefill_amd.device import to_device
    B.load()
    M = 65536
    r = np.random.default_rng(0)
    out = {"metric": "W8A8 GEMM TFLOP/s", "unit": "TFLOP/s", "M": M, "peak_fp8_tflops": PEAK_FP8_TFLOPS,
           "shapes": {}}
    x_full = torch.randn((M, 9728), device="cuda", dtype=torch.float32).to(torch.bfloat16)
    for name, (N, K) in {"qkv": (6144, 2560), "o": (2560, 4096), "gate_up": (19456, 2560),
                         "down": (2560, 9728)}.items():
        x = x_full[:, :K].contiguous()
        xc = torch.empty((M, K), dtype=torch.uint8, device="cuda")
        xs = torch.empty(M, dtype=torch.float32, device="cuda")
        w = to_device(W.draw_fp8_codes(r, (N, K)))
        sc = to_device(W.bf16_bits_from_f32((0.0002 * (1 + r.random(N))).astype(np.float32)))
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        q_ms = _timed(lambda: B.quail_act_quant_e4m3(x, xc, xs), args.steps, args.warmup)
        g_ms = _timed(lambda: B.quail_gemm_w8a8(xc, xs, w, sc, y), args.steps, args.warmup)
        w16_ms = _timed(lambda: B.quail_gemm_w8a16(x, w, sc, y), args.steps, args.warmup)
        flop = 2.0 * M * N * K
        q_gbs = 3.0 * M * K / (q_ms * 1e-3) / 1e9
        tf = flop / (g_ms * 1e-3) / 1e12
        out["shapes"][name] = {
            "N": N, "K": K,
            "act_quant": {"ms": q_ms, "GB/s": q_gbs, "frac_hbm": q_gbs / HBM_PEAK_GBS},
            "gemm_w8a8": {"ms": g_ms, "tflops": tf, "frac": tf / PEAK_FP8_TFLOPS},
            "w8a8_total_ms": q_ms + g_ms,
            "gemm_w8a16": {"ms": w16_ms, "tflops": flop / (w16_ms * 1e-3) / 1e12}}
        log(f"w8a8 {name} {M}x{N}x{K}: quant {q_ms:.3f} ms ({q_gbs:.0f} GB/s), gemm {g_ms:.3f} ms "
            f"({tf:.1f} TFLOP/s, {tf / PEAK_FP8_TFLOPS:.3f} of fp8 peak); W8A16 {w16_ms:.3f} ms")
        del x, xc, xs, w, sc, y
    print(json.dumps(out), flush=True)


def bench_copy(args):
    import torch
    n = 4 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    print(json.dumps({"metric": "device copy", "bytes_read": n, "bytes_written": n, "ms": ms,
                      "GB/s": 2 * n / (ms * 1e-3) / 1e9}), flush=True)


def bench_stream(args):
    import torch
    import workloads as W
    from query_aware_prefill_amd import binding as B
    B.load()
    out = {"metric": "anchor-KV streaming (cascade attention)", "unit": "GB/s",
           "peak_GBs": HBM_PEAK_GBS, "anchors": 1024, "anchor_len": 768, "points": []}
    for kv, dtype, esz in (("bf16", B.DTYPE_BF16, 2), ("e4m3", B.DTYPE_FP8_E4M3, 1)):
        for S in (1, 4, 16, 32, 64, 256, 4096):
            a_len, s_anchor, s_len = W.stream_lengths(S)
            case = W.cascade_device(7, a_len, s_anchor, s_len, anchor_kv=kv)
            T = int(case["s_off"][-1])
            o = torch.empty((T, 32, 128), dtype=torch.bfloat16, device="cuda")
            ws = torch.empty(B.quail_cascade_workspace_bytes(case["a_off"], case["s_off"]),
                             dtype=torch.uint8, device="cuda")
            stream = torch.cuda.current_stream()

            def step():
                B.quail_cascade_attn(dtype, 32, 8, 128, case["sm_scale"], case["ak"], case["av"],
                                     case["a_off"], s_anchor, case["q"], case["k"], case["v"],
                                     case["s_off"], o, None, ws, stream=stream)

            for _ in range(max(args.warmup, 1)):
                step()
            torch.cuda.synchronize()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.steps)]
            for a, b in ev:
                a.record(stream)
                step()
                b.record(stream)
            torch.cuda.synchronize()
            ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
            kv_bytes = 2.0 * float(np.sum(a_len)) * 8 * 128 * esz
            cross, self_ = algorithmic_flops(a_len, s_anchor, s_len)
            pt = {"kv": kv, "S": S, "ms": ms, "anchor_kv_bytes": kv_bytes,
                  "GB/s": kv_bytes / (ms * 1e-3) / 1e9,
                  "frac_hbm": kv_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                  "tflops": (cross + self_) / (ms * 1e-3) / 1e12}
            out["points"].append(pt)
            log(f"stream {kv} S={S}: {ms:.3f} ms, {pt['GB/s']:.0f} GB/s ({pt['frac_hbm']:.2f} of HBM), "
                f"{pt['tflops']:.1f} TFLOP/s")
            del case, o, ws
            torch.cuda.empty_cache()
    # The whole E4M3 pool of the multi-join configuration: 36 layers of the
    # same 1024 anchors x 768 tokens (57.98 GB); one pass is 36 launches, each
    # reading its layer's anchor K/V once for S query tokens per anchor.
    n_layers = 36
    a_len, _, _ = W.stream_lengths(1)
    ta = int(np.sum(a_len))
    pool = torch.empty((n_layers, 2, ta, 8, 128), dtype=torch.float8_e4m3fn, device="cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(29)
    flat = pool.view(-1)
    for i in range(0, flat.numel(), 1 << 28):
        n = min(1 << 28, flat.numel() - i)
        flat[i:i + n] = torch.randn(n, generator=gen, device="cuda", dtype=torch.float32).to(torch.float8_e4m3fn)
    pool = pool.view(torch.uint8)
    pool_bytes = float(pool.numel())
    out["pool"] = {"layers": n_layers, "anchor_kv_bytes": pool_bytes, "points": []}
    for S in (1, 4, 16, 32):
        _, s_anchor, s_len = W.stream_lengths(S)
        case = W.cascade_device(7, a_len, s_anchor, s_len, anchor_kv="e4m3")
        del case["ak"], case["av"]
        T = int(case["s_off"][-1])
        o = torch.empty((T, 32, 128), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(B.quail_cascade_workspace_bytes(case["a_off"], case["s_off"]), dtype=torch.uint8,
                         device="cuda")
        stream = torch.cuda.current_stream()

        def one_pass():
            for layer in range(n_layers):
                B.quail_cascade_attn(B.DTYPE_FP8_E4M3, 32, 8, 128, case["sm_scale"], pool[layer, 0],
                                     pool[layer, 1], case["a_off"], s_anchor, case["q"], case["k"], case["v"],
                                     case["s_off"], o, None, ws, stream=stream)

        one_pass()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(max(args.steps // 2, 1))]
        for a, b in ev:
            a.record(stream)
            one_pass()
            b.record(stream)
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
        pt = {"kv": "e4m3", "S": S, "ms_per_pass": ms, "GB/s": pool_bytes / (ms * 1e-3) / 1e9,
              "frac_hbm": pool_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        out["pool"]["points"].append(pt)
        log(f"stream pool e4m3 S={S}: {ms:.2f} ms per pass of {pool_bytes / 1e9:.2f} GB, {pt['GB/s']:.0f} GB/s "
            f"({pt['frac_hbm']:.2f} of HBM)")
        del case, o, ws
    del pool
    torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


def cpu_baseline_e2e(wd, shape, pairs, gpu_logits, true_mask, budget_s):
    """Oracle leg of the end-to-end modes: the per-pair definition (monolithic
    causal forward over [anchor | suffix], head at the last position), fp32
    with the contract's bf16 rounding points, on pairs taken in the given
    (random) order until the time budget is spent; logits and decisions are
    compared with the GPU's. Dequantising the weights is setup, not timed."""
    import torch
    import workloads as W
    from oracle import model as OM
    t0 = time.perf_counter()
    wh = W.weights_to_host(wd)
    layers = [OM.LayerWeights(lw, shape, np.float32) for lw in wh["layers"]]
    setup = time.perf_counter() - t0
    spent, logical, done = 0.0, 0, 0
    worst, agree, decided = 0.0, 0, 0
    for i, a_tok, s_tok in pairs:
        c0 = time.perf_counter()
        r = OM.forward_pair(a_tok, s_tok, wh, shape, true_mask, mode="contract", dtype=np.float32,
                            layers=layers)
        spent += time.perf_counter() - c0
        done += 1
        logical += len(a_tok) + len(s_tok)
        g = gpu_logits[i]
        ref = np.asarray(r["logits"], np.float64)
        worst = max(worst, float(np.max(np.abs(g - ref)) / max(np.max(np.abs(ref)), 1e-30)))
        tau = 2e-2 * float(np.max(np.abs(ref)))
        if abs(r["margin"]) > tau:
            decided += 1
            gk = int(np.argmax(g))
            agree += int(((true_mask >> gk) & 1) == r["decision"])
        if spent >= budget_s:
            break
    return {"value": logical / spent * 60.0, "unit": "tokens/min", "cores": int(torch.get_num_threads()),
            "kind": "oracle",
            "sample": f"{done} pairs drawn at random from the workload, full 36-layer forward of "
                      f"[anchor | suffix] in float32 with the bf16 rounding points "
                      f"({logical} logical tokens in {spent:.1f} s; weight dequantisation "
                      f"{setup:.1f} s not timed)",
            "check": {"pairs": done, "max_rel_logit_err": worst, "decisions_beyond_tau": decided,
                      "decisions_agree": agree}}


def bench_e2e(args):
    import torch
    import workloads as W
    from query_aware_prefill_amd import binding as B
    from query_aware_prefill_amd.device import DeviceModel, to_device
    B.load()
    kind = args.workload
    shape = W.QWEN3_4B
    if kind == "multijoin36":
        shape = W.ModelShape(**{**shape.__dict__, "kv_fp8": True})
    if args.act_fp8:
        shape = W.ModelShape(**{**shape.__dict__, "act_fp8": True})
    log(f"{kind}: generating the workload")
    if kind == "join36":
        case = W.c3b_case()
        a_len, a_off, a_tok = case["a_len"], case["a_off"], case["a_tok"]
        pair_anchor, s_off, s_tok = case["pair_anchor"], case["s_off"], case["s_tok"]
        desc = "join: 64 anchors x 1024 tokens, 2048 suffixes of 64 tokens per anchor (131,072 pairs)"
    elif kind == "filter36":
        case = W.c3a_case()
        a_len, a_off = case["a_len"], case["a_off"]
        a_tok = case["a_tok"] if len(case["a_tok"]) else np.zeros(1, np.int32)
        pair_anchor, s_off, s_tok = case["pair_anchor"], case["s_off"], case["s_tok"]
        desc = "filter: 10,000 rows, lognormal lengths 200..2000, no anchor"
    else:
        case = W.c4_case()
        rows = min(args.rows, len(case["row_len"]))
        keep = case["pair_row"] < rows
        a_len, a_off, a_tok = case["a_len"], case["a_off"], case["a_tok"]
        pair_anchor = case["pair_anchor"][keep]
        prow = case["pair_row"][keep]
        plen = case["row_len"][prow]
        s_off = np.zeros(len(prow) + 1, np.int64)
        s_off[1:] = np.cumsum(plen)
        s_tok = np.concatenate([case["row_tok"][case["row_off"][r]:case["row_off"][r + 1]] for r in prow])
        s_off = s_off.astype(np.int32)
        desc = (f"multi-join: 1024 anchors x 768 tokens (fp8 KV), {rows} of the 5,000 rows of "
                f"U{{48..256}} tokens, 51 anchors per row ({len(prow)} pairs)")
    s_len = np.diff(s_off).astype(np.int64)
    log(f"{kind}: {len(pair_anchor)} pairs, {int(np.sum(s_len))} suffix tokens; weights on device")
    wd = W.model_weights_device(shape, 0)
    max_a = int(np.max(a_len)) if len(a_len) else 0
    dm = DeviceModel(shape, wd, max_anchor_len=max(max_a, 1), max_suffix_len=int(np.max(s_len)))
    T = 65536
    used = np.unique(pair_anchor[pair_anchor >= 0])
    pool = sum(B.quail_anchor_bytes(dm.cfg, int(a_len[a])) for a in used) + (1 << 20) if len(used) else 1 << 20
    pool = min(pool, 96 << 30)
    ctx = dm.context(pool, T)
    a_tok_d, s_tok_d = to_device(a_tok.astype(np.int32)), to_device(s_tok.astype(np.int32))
    n = len(pair_anchor)
    logits = torch.empty((n, 8), dtype=torch.float32, device="cuda")
    dec = torch.empty(n, dtype=torch.uint8, device="cuda")
    log(f"{kind}: pool {pool / 2**30:.2f} GiB; running")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    B.quail_join_run(ctx, a_tok_d, a_off, pair_anchor, s_tok_d, s_off, 0x0F, logits, None, dec)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1000.0
    la = np.where(pair_anchor >= 0, a_len[np.maximum(pair_anchor, 0)] if len(a_len) else 0, 0).astype(np.int64)
    suffix_tok = int(np.sum(s_len))
    anchor_tok = int(np.sum(a_len[used])) if len(used) else 0
    logical = int(np.sum(la) + suffix_tok)
    st = B.quail_pool_stats(ctx)
    gemm = executed_gemm_flops(shape.n_layers, suffix_tok, n, anchor_tok)
    attn = 16384.0 * shape.n_layers * float(np.sum(s_len * la) + np.sum(s_len * (s_len + 1) / 2))
    attn += 16384.0 * (shape.n_layers - 1) * float(sum(int(a_len[a]) * (int(a_len[a]) + 1) / 2 for a in used))
    if args.act_fp8:
        desc += "; W8A8 (per-token E4M3 activations on the fp8 MFMA)"
    res = {"metric": "end-to-end prefill tokens/min (36-layer stack)", "workload": desc, "unit": "tokens/min",
           "ms": ms, "pairs": int(n), "logical_tokens": logical, "computed_tokens": suffix_tok + anchor_tok,
           "logical_tokens_per_min": logical / (ms * 1e-3) * 60.0,
           "computed_tokens_per_min": (suffix_tok + anchor_tok) / (ms * 1e-3) * 60.0,
           "algorithmic_tflops": (gemm + attn) / (ms * 1e-3) / 1e12, "pool": st,
           "weights": "random init on device (W ~ N(0, 0.02), per-row bf16 scales, E4M3 codes)"}
    if kind == "join36":
        # the planner's speed-of-light time for this join: anchor table (64 rows
        # x 1024 tokens) against the suffix table (2048 rows x 64 tokens)
        sol = B.quail_join_search(dm.cfg, [(64, 1024), (2048, 64)], [(0, 1, 0, 0, 1.0, 1)],
                                  PEAK_BF16_TFLOPS * 1e12, HBM_PEAK_GBS * 1e9)
        res["speed_of_light_s"] = float(sol["metrics"][3])
        res["measured_over_speed_of_light"] = ms * 1e-3 / float(sol["metrics"][3])
    log(f"{kind}: {ms / 1000:.2f} s, {res['logical_tokens_per_min'] / 1e9:.3f} G logical tok/min, "
        f"{res['algorithmic_tflops']:.1f} TFLOP/s")
    if not args.no_cpu_baseline:
        lg = logits.cpu().numpy().astype(np.float64)
        order = np.random.default_rng(0).permutation(n)[:16]
        pairs = []
        for i in order:
            a = int(pair_anchor[i])
            at = a_tok[a_off[a]:a_off[a + 1]] if a >= 0 else np.zeros(0, np.int32)
            pairs.append((int(i), at, s_tok[s_off[i]:s_off[i + 1]]))
        log(f"{kind}: oracle leg")
        res["cpu_baseline"] = cpu_baseline_e2e(wd, shape, pairs, lg, 0x0F, args.cpu_budget)
    print(json.dumps(res), flush=True)


def bench_layer(args):
    import torch
    import workloads as W
    from query_aware_prefill_amd import binding as B
    from query_aware_prefill_amd.device import DeviceModel, to_device
    B.load()
    shape = W.ModelShape(n_layers=1, hidden=2560, n_q_heads=32, n_kv_heads=8, head_dim=128,
                         intermediate=9728, vocab=W.QWEN3_4B.vocab)
    log("generating one layer of random-init weights")
    wts = W.model_weights(shape, 0)
    case = W.c2_case(seed=2)
    n_pairs = len(case["pair_anchor"])
    dm = DeviceModel(shape, wts, max_anchor_len=1024, max_suffix_len=64)
    T = 65536
    pool = 16 * B.quail_anchor_bytes(dm.cfg, 1024) + (1 << 20)
    ctx = dm.context(pool, T)
    a_tok, s_tok = to_device(case["a_tok"]), to_device(case["s_tok"])
    logits = torch.empty((n_pairs, 8), dtype=torch.float32, device="cuda")
    dec = torch.empty(n_pairs, dtype=torch.uint8, device="cuda")
    n_anchors = len(case["a_off"]) - 1
    uses = np.bincount(case["pair_anchor"], minlength=n_anchors)
    h_last = torch.empty((n_pairs, shape.hidden), dtype=torch.int16, device="cuda")
    h_all = torch.empty((int(case["s_off"][-1]), shape.hidden), dtype=torch.int16, device="cuda")

    # the whole layer for every suffix row (h_all requested: a join prefill
    # that returns only the last rows would run the O projection and MLP of
    # its last layer, here the only one, on the last rows alone)
    def step():
        handles = B.quail_anchor_prefill(ctx, a_tok, case["a_off"], uses, anchor_ids=np.arange(n_anchors))
        B.quail_join_prefill(ctx, handles[case["pair_anchor"]], s_tok, case["s_off"], h_last, h_all)
        B.quail_head8(ctx, h_last, 0x0F, logits, None, dec)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1000.0 / args.steps
    anchor_tok = int(np.sum(case["a_len"]))
    suffix_tok = int(np.sum(case["s_len"]))
    logical = int(np.sum(case["a_len"][case["pair_anchor"]]) + suffix_tok)
    # executed algorithmic work: suffix tokens run the whole layer (201.85
    # MFLOP/token of projections); with one layer, the anchors' last layer only
    # needs its K/V, i.e. the QKV projection (31.46 MFLOP/token).
    gemm_flops = GEMM_FLOP_LAYER * suffix_tok + GEMM_FLOP_QKV * anchor_tok
    attn_flops = 16384.0 * (np.sum(case["s_len"] * case["a_len"][case["pair_anchor"]]) +
                            np.sum(case["s_len"] * (case["s_len"] + 1) / 2))
    st = B.quail_pool_stats(ctx)
    res = {"metric": "decoder-layer join prefill", "unit": "tokens/min", "ms_per_step": ms,
           "logical_tokens_per_min": logical / (ms * 1e-3) * 60, "computed_tokens_per_min":
           (anchor_tok + suffix_tok) / (ms * 1e-3) * 60, "pairs": n_pairs,
           "algorithmic_tflops": (gemm_flops + attn_flops) / (ms * 1e-3) / 1e12,
           "pool": st}
    log(f"layer: {ms:.2f} ms/step, {res['algorithmic_tflops']:.1f} TFLOP/s algorithmic")
    print(json.dumps(res), flush=True)


def bench_multiplan(args):
    """Three joins over one anchor table (64 anchors x 1024 tokens of the join
    workload; join k takes suffixes k*128 .. k*128+127 of every anchor, 64
    tokens each), 36-layer stack: plan-wide residency (quail_multijoin_run)
    against running the joins one by one (quail_join_run each)."""
    import torch
    import workloads as W
    from query_aware_prefill_amd import binding as B
    from query_aware_prefill_amd.device import DeviceModel, to_device
    B.load()
    shape = W.QWEN3_4B
    case = W.c3b_case()
    a_len, a_off, a_tok = case["a_len"], case["a_off"], case["a_tok"]
    pa_all, s_off_all, s_tok_all = case["pair_anchor"], case["s_off"], case["s_tok"]
    rank = np.zeros(len(pa_all), np.int64)
    seen = {}
    for i, a in enumerate(pa_all):
        rank[i] = seen.get(int(a), 0)
        seen[int(a)] = rank[i] + 1
    per = 128
    sel = [np.nonzero((rank >= k * per) & (rank < (k + 1) * per))[0] for k in range(3)]
    idx = np.concatenate(sel)
    jo = np.array([0, len(sel[0]), len(sel[0]) + len(sel[1]), len(idx)], np.int32)
    pair_anchor = pa_all[idx].astype(np.int32)
    s_len = np.diff(s_off_all)[idx].astype(np.int64)
    s_off = np.concatenate([[0], np.cumsum(s_len)]).astype(np.int32)
    s_tok = np.concatenate([s_tok_all[s_off_all[i]:s_off_all[i + 1]] for i in idx]).astype(np.int32)
    n = len(idx)
    log(f"multiplan36: 3 joins x {n // 3} pairs over {len(a_len)} anchors; weights on device")
    wd = W.model_weights_device(shape, 0)
    dm = DeviceModel(shape, wd, max_anchor_len=int(np.max(a_len)), max_suffix_len=int(np.max(s_len)))
    T = 65536
    pool = sum(B.quail_anchor_bytes(dm.cfg, int(x)) for x in a_len) + (1 << 20)
    a_tok_d, s_tok_d = to_device(a_tok.astype(np.int32)), to_device(s_tok)
    res = {"metric": "multi-join plan: plan-wide residency vs joins one by one (36-layer stack)",
           "workload": "3 joins over 64 anchors x 1024 tokens, 8,192 pairs of 64-token suffixes each",
           "pairs": int(n)}
    out = {}
    for mode in ("plan_wide", "one_by_one"):
        ctx = dm.context(pool, T)
        logits = torch.empty((n, 8), dtype=torch.float32, device="cuda")
        dec = torch.empty(n, dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        if mode == "plan_wide":
            B.quail_multijoin_run(ctx, a_tok_d, a_off, jo, pair_anchor, s_tok_d, s_off, 0x0F, logits, None, dec)
        else:
            for j in range(3):
                lo, hi = int(jo[j]), int(jo[j + 1])
                so = (s_off[lo:hi + 1] - s_off[lo]).astype(np.int32)
                B.quail_join_run(ctx, a_tok_d, a_off, pair_anchor[lo:hi], s_tok_d[int(s_off[lo]):int(s_off[hi])],
                                 so, 0x0F, logits[lo:hi], None, dec[lo:hi])
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1000.0
        st = B.quail_pool_stats(ctx)
        out[mode] = logits.cpu().numpy()
        res[mode] = {"ms": ms, "pool": st}
        log(f"multiplan36 {mode}: {ms / 1000:.2f} s, prefills {st['prefills']}, regret {st['regret_tokens']} tokens")
        del ctx
    res["logits_identical"] = bool(np.array_equal(out["plan_wide"], out["one_by_one"]))
    res["speedup"] = res["one_by_one"]["ms"] / res["plan_wide"]["ms"]
    print(json.dumps(res), flush=True)


def bench_shared(args):
    """Suffixes sharing prefixes, 36-layer stack. shared36: 16 anchors x 1024
    tokens, each probed by 16 families of 8 suffixes whose first 384 tokens
    are the family's, then U{16..64} tokens of their own. traces36 (agent-
    trace shaped filter, no anchor): 128 families of 16 documents that repeat
    a 768-token prefix, then U{32..128} tokens of their own. The run with
    shared-prefix nodes (quail_join_run_shared, min_shared 32) against the
    plain run (quail_join_run) on the same inputs; the second of two runs of
    each is timed."""
    import torch
    import workloads as W
    from query_aware_prefill_amd import binding as B
    from query_aware_prefill_amd.device import DeviceModel, to_device
    B.load()
    shape = W.QWEN3_4B
    r = np.random.default_rng([7, 0])
    traces = args.workload == "traces36"
    min_shared = 32
    if traces:
        n_anchors, n_fam, per_fam, shared = 0, 128, 16, 768
        fams = [(-1, shared, r.integers(32, 129, per_fam).tolist()) for _ in range(n_fam)]
    else:
        n_anchors, n_fam, per_fam, shared = 16, 16, 8, 384
        fams = [(a, shared, r.integers(16, 65, per_fam).tolist()) for a in range(n_anchors) for _ in range(n_fam)]
    case = W.shared_prefix_case(7, shape.vocab, [1024] * n_anchors, fams, cfg_id=7)
    pa, s_off, s_tok = case["pair_anchor"], case["s_off"], case["s_tok"]
    a_len, a_off = case["a_len"], case["a_off"]
    s_len = np.diff(s_off)
    n = len(pa)
    log(f"{args.workload}: {n} rows over {n_anchors} anchors, families of {per_fam} sharing {shared} tokens; "
        "weights on device")
    wd = W.model_weights_device(shape, 0)
    dm = DeviceModel(shape, wd, max_anchor_len=1024, max_suffix_len=int(np.max(s_len)))
    T = 65536
    pool = sum(B.quail_anchor_bytes(dm.cfg, int(x)) for x in a_len) + (8 << 30)
    # tokens the shared run computes: the library's plan steps and grouping
    g_all, _, nl_all = B.quail_prefix_groups(s_tok, s_off, np.where(pa >= 0, pa, n_anchors).astype(np.int32),
                                             min_shared)
    step_len = s_len.astype(np.int64).copy()
    for k in range(len(nl_all)):          # the shared run sizes its steps by computed tokens
        m = np.flatnonzero(g_all == k)
        step_len[m] = s_len[m] - nl_all[k] + (nl_all[k] + len(m) - 1) // len(m)
    reserve = B.quail_anchor_bytes(dm.cfg, int(np.max(s_len)))   # room kept for a prefix node
    order, bounds, _ = B.quail_plan_build(dm.cfg, pool - reserve, T, a_len, pa, step_len.astype(np.int32))
    node_tok = 0
    for b0, b1 in zip(bounds[:-1], bounds[1:]):
        idx = order[b0:b1]
        offs = np.concatenate([[0], np.cumsum(s_len[idx])]).astype(np.int32)
        toks = np.concatenate([s_tok[s_off[i]:s_off[i + 1]] for i in idx])
        g, _, nl = B.quail_prefix_groups(toks, offs, np.where(pa[idx] >= 0, pa[idx], n_anchors).astype(np.int32),
                                         min_shared)
        node_tok += int(np.sum(nl)) - int(np.sum(nl[g[g >= 0]]))
    a_tok_d = to_device(case["a_tok"].astype(np.int32) if n_anchors else np.zeros(1, np.int32))
    s_tok_d = to_device(s_tok.astype(np.int32))
    logical = float(np.sum(np.where(pa >= 0, a_len[np.maximum(pa, 0)] if n_anchors else 0, 0) + s_len))
    prefilled = float(np.sum(a_len))
    computed = {"plain": prefilled + float(np.sum(s_len)), "shared": prefilled + float(np.sum(s_len)) + node_tok}
    if traces:
        res = {"metric": "AI.IF filter over documents sharing prefixes: prefix prefilled once vs per row "
                         "(36-layer stack)",
               "workload": f"{n_fam} families x {per_fam} documents, {shared} shared tokens + U{{32..128}} own "
                           "tokens each, no anchor",
               "pairs": int(n), "logical_tokens": logical}
    else:
        res = {"metric": "AI.IF join with shared suffix prefixes: two-level cascade vs plain join (36-layer stack)",
               "workload": f"{n_anchors} anchors x 1024 tokens; {n_fam} families x {per_fam} suffixes per anchor, "
                           f"{shared} shared tokens + U{{16..64}} own tokens each",
               "pairs": int(n), "logical_tokens": logical}
    out = {}
    for mode in (("shared",) if args.shared_only else ("shared", "plain")):
        ctx = dm.context(pool, T)
        logits = torch.empty((n, 8), dtype=torch.float32, device="cuda")
        dec = torch.empty(n, dtype=torch.uint8, device="cuda")
        for _ in range(2):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            if mode == "shared":
                B.quail_join_run_shared(ctx, a_tok_d, a_off, pa, s_tok_d, s_off, s_tok, min_shared, 0x0F,
                                        logits, None, dec)
            else:
                B.quail_join_run(ctx, a_tok_d, a_off, pa, s_tok_d, s_off, 0x0F, logits, None, dec)
            torch.cuda.synchronize()
            ms = (time.perf_counter() - t0) * 1000.0
        st = B.quail_pool_stats(ctx)
        out[mode] = (logits.cpu().numpy(), dec.cpu().numpy())
        res[mode] = {"ms": ms, "logical_tokens_per_min": logical / ms * 60e3,
                     "computed_tokens": computed[mode], "computed_tokens_per_min": computed[mode] / ms * 60e3,
                     "pool_over_two_runs": st}
        log(f"{args.workload} {mode}: {ms / 1000:.2f} s, {computed[mode] / 1e6:.3f} M computed tokens, "
            f"{logical / ms * 60e3 / 1e6:.1f} M logical tokens/min")
        del ctx
    if args.shared_only:
        print(json.dumps(res), flush=True)
        return
    res["speedup"] = res["plain"]["ms"] / res["shared"]["ms"]
    if not args.no_cpu_baseline:
        # oracle leg on the shared run's outputs: the per-pair definition over
        # [anchor | whole suffix] (the shared prefix included)
        order = np.random.default_rng(1).permutation(n)[:8]
        pairs = [(int(i), case["a_tok"][a_off[pa[i]]:a_off[pa[i] + 1]] if pa[i] >= 0 else np.zeros(0, np.int32),
                  s_tok[s_off[i]:s_off[i + 1]]) for i in order]
        log(f"{args.workload}: oracle leg")
        res["cpu_baseline"] = cpu_baseline_e2e(wd, shape, pairs, out["shared"][0].astype(np.float64), 0x0F,
                                               args.cpu_budget)
    ls, lp = out["shared"][0].astype(np.float64), out["plain"][0].astype(np.float64)
    res["logits_rel_inf_shared_vs_plain"] = float(np.max(np.abs(ls - lp)) / np.max(np.abs(lp)))
    res["decisions_equal_frac"] = float(np.mean(out["shared"][1] == out["plain"][1]))
    # where the plain run's TRUE-vs-FALSE margin exceeds the tolerance
    # (2e-2 of the largest |logit| of the pair), the decision is fixed
    tmask = np.array([(0x0F >> j) & 1 for j in range(8)], bool)
    margin = np.max(np.where(tmask, lp, -np.inf), axis=1) - np.max(np.where(~tmask, lp, -np.inf), axis=1)
    sure = np.abs(margin) > 2e-2 * np.max(np.abs(lp), axis=1)
    res["decisions_beyond_tau"] = int(np.sum(sure))
    res["decisions_beyond_tau_equal"] = int(np.sum(out["shared"][1][sure] == out["plain"][1][sure]))
    print(json.dumps(res), flush=True)


def bench_nested(args):
    """Documents under two shared levels, 36-layer stack, no anchor: 2,048
    documents share a 512-token prompt, then each family of 16 shares a
    384-token document, then U{32..128} tokens of their own. Four runs on
    the same inputs: the plain filter (quail_join_run), one shared level
    (quail_join_run_shared, min_shared 32: the prompt), and the nested radix
    index (quail_prefix_tree) with its nodes prefilled parents first
    (quail_anchor_prefill for the prompt, quail_prefix_prefill for the
    family documents) and every document's own tokens joined after its node
    (quail_join_prefill, quail_head8), and the same nested grouping inside
    one call (quail_join_run_shared, nested). The second of two runs is
    timed."""
    import torch
    import workloads as W
    from query_aware_prefill_amd import binding as B
    from query_aware_prefill_amd.device import DeviceModel, to_device
    B.load()
    shape = W.QWEN3_4B
    r = np.random.default_rng([8, 0])
    n_fam, per_fam, min_shared = 128, 16, 32
    prompt = r.integers(0, shape.vocab, 512).astype(np.int32)
    fam_doc = [r.integers(0, shape.vocab, 384).astype(np.int32) for _ in range(n_fam)]
    seqs = [np.concatenate([prompt, fam_doc[i // per_fam], r.integers(0, shape.vocab, int(r.integers(32, 129)))
                            .astype(np.int32)]) for i in range(n_fam * per_fam)]
    n = len(seqs)
    s_off = np.zeros(n + 1, np.int32)
    s_off[1:] = np.cumsum([len(x) for x in seqs])
    s_tok = np.concatenate(seqs).astype(np.int32)
    s_len = np.diff(s_off)
    pa = -np.ones(n, np.int32)
    log(f"nested36: {n} documents, 512-token prompt, {n_fam} families x {per_fam} sharing 384 tokens; weights")
    wd = W.model_weights_device(shape, 0)
    dm = DeviceModel(shape, wd, max_anchor_len=1024, max_suffix_len=int(np.max(s_len)))
    T = 65536
    pool = 8 << 30
    s_tok_d, dummy = to_device(s_tok), to_device(np.zeros(1, np.int32))
    g, nodes = B.quail_prefix_tree(s_tok, s_off, np.zeros(n, np.int32), min_shared)
    assert nodes[0][0] < 0 and nodes[0][3] == 512 and len(nodes) == 1 + n_fam, nodes[:3]
    logical = float(np.sum(s_len))
    res = {"metric": "AI.IF filter over documents under two shared levels: nested prefix nodes vs one level vs "
                     "plain (36-layer stack)",
           "workload": f"{n} documents: 512 shared prompt tokens, {n_fam} families x {per_fam} sharing 384 "
                       "document tokens, U{32..128} own tokens each, no anchor",
           "rows": n, "logical_tokens": logical}
    out = {}
    for mode in ("nested", "nested_call", "shared", "plain"):
        ctx = dm.context(pool, T)
        logits = torch.empty((n, 8), dtype=torch.float32, device="cuda")
        dec = torch.empty(n, dtype=torch.uint8, device="cuda")
        for _ in range(2):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            if mode == "nested_call":
                B.quail_join_run_shared(ctx, dummy, [0], pa, s_tok_d, s_off, s_tok, min_shared, 0x0F, logits,
                                        None, dec, nested=True)
            elif mode == "plain":
                B.quail_join_run(ctx, dummy, [0], pa, s_tok_d, s_off, 0x0F, logits, None, dec)
            elif mode == "shared":
                B.quail_join_run_shared(ctx, dummy, [0], pa, s_tok_d, s_off, s_tok, min_shared, 0x0F, logits,
                                        None, dec)
            else:
                uses = [int(np.sum(g == k)) + sum(1 for q in nodes if q[0] == k) for k in range(len(nodes))]
                p0, f0, st0, en0 = nodes[0]
                root = B.quail_anchor_prefill(ctx, s_tok_d[int(s_off[f0]):int(s_off[f0]) + en0], [0, en0],
                                              [uses[0]])
                kids = list(range(1, len(nodes)))
                ktok = np.concatenate([s_tok[s_off[nodes[k][1]] + nodes[k][2]:s_off[nodes[k][1]] + nodes[k][3]]
                                       for k in kids])
                koff = np.concatenate([[0], np.cumsum([nodes[k][3] - nodes[k][2] for k in kids])]).astype(np.int32)
                kh = B.quail_prefix_prefill(ctx, [root[0]] * len(kids), to_device(ktok), koff,
                                            [uses[k] for k in kids])
                handle = [root[0]] + list(kh)
                tails = np.concatenate([s_tok[s_off[i] + nodes[g[i]][3]:s_off[i + 1]] for i in range(n)])
                toff = np.concatenate([[0], np.cumsum([s_len[i] - nodes[g[i]][3] for i in range(n)])]).astype(np.int32)
                h_last = torch.empty((n, shape.hidden), dtype=torch.int16, device="cuda")
                B.quail_join_prefill(ctx, [handle[g[i]] for i in range(n)], to_device(tails), toff, h_last)
                B.quail_head8(ctx, h_last, 0x0F, logits, None, dec)
            torch.cuda.synchronize()
            ms = (time.perf_counter() - t0) * 1000.0
        st = B.quail_pool_stats(ctx)
        out[mode] = (logits.cpu().numpy().astype(np.float64), dec.cpu().numpy())
        res[mode] = {"ms": ms, "logical_tokens_per_min": logical / ms * 60e3, "pool_over_two_runs": st}
        log(f"nested36 {mode}: {ms / 1000:.2f} s, {logical / ms * 60e3 / 1e6:.1f} M logical tokens/min")
        del ctx
    computed = {"plain": logical, "shared": 512.0 + float(np.sum(s_len - 512)),
                "nested": 512.0 + n_fam * 384.0 + float(np.sum(s_len - 896))}
    for mode in out:
        if mode in computed:       # the one-call nested run regroups per plan step
            res[mode]["computed_tokens"] = computed[mode]
            res[mode]["computed_tokens_per_min"] = computed[mode] / res[mode]["ms"] * 60e3
    lp = out["plain"][0]
    tmask = np.array([(0x0F >> j) & 1 for j in range(8)], bool)
    margin = np.max(np.where(tmask, lp, -np.inf), axis=1) - np.max(np.where(~tmask, lp, -np.inf), axis=1)
    sure = np.abs(margin) > 2e-2 * np.max(np.abs(lp), axis=1)
    for mode in ("nested", "nested_call", "shared"):
        res[mode]["speedup_over_plain"] = res["plain"]["ms"] / res[mode]["ms"]
        res[mode]["logits_rel_inf_vs_plain"] = float(np.max(np.abs(out[mode][0] - lp)) / np.max(np.abs(lp)))
        res[mode]["decisions_beyond_tau_equal"] = [int(np.sum(out[mode][1][sure] == out["plain"][1][sure])),
                                                   int(np.sum(sure))]
    print(json.dumps(res), flush=True)


def bench_multijoin_full(args):
    """The multi-join configuration at full size, 36-layer stack: 1024 anchors
    x 768 tokens with E4M3 KV (about 58 GB resident), 5,000 rows of
    U{48..256} tokens each probing 51 anchors (255,000 pairs). Every anchor is
    prefilled once (quail_anchor_prefill, use count = its pairs) into a pool
    that holds all of them; the rows then run in 8 chunks of 625 (one progress
    line each), each chunk's pairs through quail_join_prefill (grouped by
    anchor inside) and quail_head8; an anchor is evicted after its last pair."""
    import torch
    import workloads as W
    from query_aware_prefill_amd import binding as B
    from query_aware_prefill_amd.device import DeviceModel, to_device
    B.load()
    shape = W.ModelShape(**{**W.QWEN3_4B.__dict__, "kv_fp8": True, "act_fp8": bool(args.act_fp8)})
    log("multijoin36 full: generating the workload")
    case = W.c4_case()
    a_len, a_off, a_tok = case["a_len"], case["a_off"], case["a_tok"]
    pa, prow = case["pair_anchor"], case["pair_row"]
    plen = case["row_len"][prow].astype(np.int64)
    n = len(pa)
    s_off = np.zeros(n + 1, np.int64)
    s_off[1:] = np.cumsum(plen)
    s_tok = np.concatenate([case["row_tok"][case["row_off"][r]:case["row_off"][r + 1]] for r in prow]).astype(np.int32)
    log(f"multijoin36 full: {n} pairs, {int(s_off[-1])} suffix tokens; weights on device")
    wd = W.model_weights_device(shape, 0)
    dm = DeviceModel(shape, wd, max_anchor_len=768, max_suffix_len=int(np.max(plen)))
    T = 65536
    pool = len(a_len) * B.quail_anchor_bytes(dm.cfg, 768) + (1 << 20)
    ctx = dm.context(pool, T)
    a_tok_d, s_tok_d = to_device(a_tok), to_device(s_tok)
    uses = np.bincount(pa, minlength=len(a_len)).astype(np.int32)
    logits = torch.empty((n, 8), dtype=torch.float32, device="cuda")
    dec = torch.empty(n, dtype=torch.uint8, device="cuda")
    rows_per_chunk = 625
    chunk_pairs = int(np.max(np.bincount(prow // rows_per_chunk)))
    h_last = torch.empty((chunk_pairs, shape.hidden), dtype=torch.int16, device="cuda")
    log(f"multijoin36 full: pool {pool / 2**30:.1f} GiB; prefilling {len(a_len)} anchors")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    handles = B.quail_anchor_prefill(ctx, a_tok_d, a_off, uses, anchor_ids=np.arange(len(a_len)))
    torch.cuda.synchronize()
    t_pre = time.perf_counter() - t0
    log(f"multijoin36 full: anchors prefilled in {t_pre:.2f} s, resident {B.quail_pool_stats(ctx)['resident'] / 1e9:.1f} GB")
    for r0 in range(0, len(case["row_len"]), rows_per_chunk):
        p0 = int(np.searchsorted(prow, r0))
        p1 = int(np.searchsorted(prow, r0 + rows_per_chunk))
        off = (s_off[p0:p1 + 1] - s_off[p0]).astype(np.int32)
        B.quail_join_prefill(ctx, handles[pa[p0:p1]], s_tok_d[int(s_off[p0]):int(s_off[p1])], off, h_last[:p1 - p0])
        B.quail_head8(ctx, h_last[:p1 - p0], 0x0F, logits[p0:p1], None, dec[p0:p1])
        torch.cuda.synchronize()
        log(f"multijoin36 full: rows {r0}..{r0 + rows_per_chunk - 1} done at {time.perf_counter() - t0:.1f} s")
    ms = (time.perf_counter() - t0) * 1000.0
    st = B.quail_pool_stats(ctx)
    suffix_tok = float(np.sum(plen))
    anchor_tok = float(np.sum(a_len))
    logical = float(np.sum(a_len[pa]) + suffix_tok)
    L = shape.n_layers
    gemm = executed_gemm_flops(L, suffix_tok, n, anchor_tok)
    attn = 16384.0 * L * float(np.sum(plen * a_len[pa]) + np.sum(plen * (plen + 1) / 2))
    attn += 16384.0 * (L - 1) * float(np.sum(a_len.astype(np.float64) * (a_len + 1) / 2))
    res = {"metric": "end-to-end prefill tokens/min (36-layer stack)",
           "workload": "multi-join at full size: 1024 anchors x 768 tokens (E4M3 KV resident), 5,000 rows of "
                       "U{48..256} tokens x 51 anchors each (255,000 pairs)"
                       + ("; W8A8 (per-token E4M3 activations on the fp8 MFMA)" if args.act_fp8 else ""),
           "unit": "tokens/min", "ms": ms, "anchor_prefill_ms": t_pre * 1e3, "pairs": int(n),
           "logical_tokens": logical, "computed_tokens": suffix_tok + anchor_tok,
           "logical_tokens_per_min": logical / ms * 60e3,
           "computed_tokens_per_min": (suffix_tok + anchor_tok) / ms * 60e3,
           "algorithmic_tflops": (gemm + attn) / (ms * 1e-3) / 1e12, "pool": st}
    log(f"multijoin36 full: {ms / 1000:.1f} s, {res['logical_tokens_per_min'] / 1e6:.1f} M logical tokens/min, "
        f"{res['algorithmic_tflops']:.0f} TFLOP/s")
    print(json.dumps(res), flush=True)


def bench_search(args):
    """Planner latency (host only): quail_join_search on random tree queries of
    4 to 12 tables (Qwen3-4B cost constants, datasheet peaks)."""
    from query_aware_prefill_amd import binding as B
    import workloads as W
    B.load()
    shape = W.QWEN3_4B
    cfg = B.ModelConfig(n_layers=shape.n_layers, hidden=shape.hidden, n_q_heads=shape.n_q_heads,
                        n_kv_heads=shape.n_kv_heads, head_dim=shape.head_dim, intermediate=shape.intermediate,
                        vocab=shape.vocab, rope_theta=1e6, rms_eps=1e-6, kv_dtype=B.DTYPE_BF16, k_scale=1.0,
                        v_scale=1.0, max_anchor_len=2048, max_suffix_len=2048)
    out = {"metric": "join-order search latency (host)", "unit": "ms", "queries": {}}
    for n in (4, 8, 10, 12):
        r = np.random.default_rng([11, n])
        times, fronts = [], []
        for q in range(5):
            tables = [(int(r.integers(10, 100000)), float(r.integers(16, 2048))) for _ in range(n)]
            joins = []
            for t in range(1, n):
                u = int(r.integers(0, t))
                joins.append((u, t, float(r.integers(0, 64)), float(r.integers(0, 64)),
                              float(r.integers(1, 65)) / 1024.0, int(r.random() < 0.5)))
            t0 = time.perf_counter()
            res = B.quail_join_search(cfg, tables, joins, PEAK_BF16_TFLOPS * 1e12, HBM_PEAK_GBS * 1e9, cap=0)
            times.append((time.perf_counter() - t0) * 1e3)
            fronts.append(res["n_frontier"])
        out["queries"][str(n)] = {"tables": n, "median_ms": float(np.median(times)), "max_ms": float(np.max(times)),
                                  "frontier_sizes": fronts}
        log(f"search: {n} tables, median {np.median(times):.2f} ms, frontier sizes {fronts}")
    print(json.dumps(out), flush=True)


def host_cpu():
    """CPU model, logical CPUs and the BLAS thread count the oracle runs with."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"),
                      default=None)
    except Exception:
        threads = None
    if not threads:
        import torch
        threads = torch.get_num_threads()
    return {"cpu_model": model, "host_cpus": os.cpu_count(), "blas_threads": int(threads)}


JOIN_ANCHORS, JOIN_SUFFIXES, JOIN_LA, JOIN_LS = 64, 2048, 1024, 64
ANCHORS_PER_STEP = 2


def w8a8_join_field(args, B, shape, dm, inputs, step_inputs, logits, dec, per_step_pairs, logical, T):
    """The headline join steps again on a context whose projections read
    per-token E4M3 activations (act_dtype FP8_E4M3), same weights and inputs:
    ms per step, logical tokens/min, the gate/up launch against the fp8 MFMA
    peak, and how far its logits and decisions are from the W8A16 run of the
    last step (the precision this mode gives up)."""
    import dataclasses
    import torch
    from query_aware_prefill_amd.device import model_config
    shape8 = dataclasses.replace(shape, act_fp8=True)
    cfg8 = model_config(shape8, JOIN_LA, JOIN_LS)
    pool = torch.empty(ANCHORS_PER_STEP * B.quail_anchor_bytes(cfg8, JOIN_LA) + (1 << 20), dtype=torch.uint8,
                       device="cuda")
    ws = torch.empty(B.quail_workspace_bytes(cfg8, T), dtype=torch.uint8, device="cuda")
    ctx8 = B.Context(cfg8, dm.weights, pool, ws, T)
    stream = torch.cuda.current_stream()
    last = args.warmup + args.steps - 1
    ref_lg, ref_dec = logits.cpu().numpy().astype(np.float64), dec.cpu().numpy()   # W8A16, step `last`
    lg8 = torch.empty_like(logits)
    dec8 = torch.empty_like(dec)
    n_steps = min(args.steps, 10)
    ks = list(range(last - n_steps + 1, last + 1))

    def step(k):
        at, ao, pa, st, so, _, _ = inputs[k]
        B.quail_join_run(ctx8, at, ao, pa, st, so, 0x0F, lg8, None, dec8, stream=stream)

    for k in range(min(args.warmup, 2)):
        step(k)
    torch.cuda.synchronize()
    B.quail_ctx_profile(ctx8, True)
    t0 = time.perf_counter()
    for k in ks:
        step(k)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    prof = B.quail_ctx_profile_read(ctx8)
    B.quail_ctx_profile(ctx8, False)
    ms_step = el * 1000.0 / n_steps
    gu = prof["gate_up"]
    gu_ms = gu["ms"] / gu["launches"]
    gu_tf = gu["flop"] / gu["launches"] / (gu_ms * 1e-3) / 1e12
    gemm_ms = sum(prof[k]["ms"] for k in ("qkv", "o", "gate_up", "down"))
    gemm_flop = sum(prof[k]["flop"] for k in ("qkv", "o", "gate_up", "down"))
    g8 = lg8.cpu().numpy().astype(np.float64)
    out = {"steps": n_steps, "ms_per_step": ms_step, "logical_tokens_per_min": logical / (ms_step * 1e-3) * 60.0,
           "gate_up": {"kernel": "quail::gemm_a8_kernel<2>", "launch_ms": gu_ms, "tflops": gu_tf,
                       "frac_of_fp8_peak": gu_tf / PEAK_FP8_TFLOPS},
           "gemm_all_tflops": gemm_flop / (gemm_ms * 1e-3) / 1e12, "gemm_share_of_step": gemm_ms / (el * 1000.0),
           "norm_and_quant_share_of_step": prof["norm"]["ms"] / (el * 1000.0),
           "vs_w8a16_last_step": {"logits_rel_inf": float(np.max(np.abs(g8 - ref_lg)) / np.max(np.abs(ref_lg))),
                                  "decisions_equal": float(np.mean(dec8.cpu().numpy() == ref_dec))}}
    log(f"join w8a8: step {ms_step:.1f} ms, {out['logical_tokens_per_min'] / 1e6:.1f} M logical tok/min; gate/up "
        f"{gu_ms:.3f} ms, {gu_tf:.1f} TFLOP/s; logits {out['vs_w8a16_last_step']['logits_rel_inf']:.4f} from W8A16, "
        f"decisions {out['vs_w8a16_last_step']['decisions_equal']:.4f} equal")
    del ctx8
    return out


def bench_join(args):
    """Headline: the 36-layer join, one step = two anchors with all their pairs."""
    import torch
    import workloads as W
    from query_aware_prefill_amd import binding as B
    from query_aware_prefill_amd.device import DeviceModel, to_device
    B.load()
    shape = W.QWEN3_4B
    log("join: generating the workload (64 anchors x 1024 tokens, 2048 suffixes x 64 tokens each)")
    case = W.c3b_case(n_anchors=JOIN_ANCHORS, per_anchor=JOIN_SUFFIXES, la=JOIN_LA, ls=JOIN_LS)
    a_off, s_off, pair_anchor = case["a_off"], case["s_off"], case["pair_anchor"]
    assert np.all(np.diff(pair_anchor) >= 0)        # pairs grouped by anchor
    log("join: random-init weights on the device")
    wd = W.model_weights_device(shape, 0)
    dm = DeviceModel(shape, wd, max_anchor_len=JOIN_LA, max_suffix_len=JOIN_LS)
    T = 65536
    pool = ANCHORS_PER_STEP * B.quail_anchor_bytes(dm.cfg, JOIN_LA) + (1 << 20)
    ctx = dm.context(pool, T)
    a_tok_d = to_device(case["a_tok"])
    s_tok_d = to_device(case["s_tok"])
    per_step_pairs = ANCHORS_PER_STEP * JOIN_SUFFIXES
    logits = torch.empty((per_step_pairs, 8), dtype=torch.float32, device="cuda")
    dec = torch.empty(per_step_pairs, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    n_groups = JOIN_ANCHORS // ANCHORS_PER_STEP

    def step_inputs(k):
        g = k % n_groups
        a0, a1 = g * ANCHORS_PER_STEP, (g + 1) * ANCHORS_PER_STEP
        p0, p1 = a0 * JOIN_SUFFIXES, a1 * JOIN_SUFFIXES
        return (a_tok_d[int(a_off[a0]):int(a_off[a1])], (a_off[a0:a1 + 1] - a_off[a0]).astype(np.int32),
                (pair_anchor[p0:p1] - a0).astype(np.int32), s_tok_d[int(s_off[p0]):int(s_off[p1])],
                (s_off[p0:p1 + 1] - s_off[p0]).astype(np.int32), a0, p0)

    inputs = [step_inputs(k) for k in range(args.warmup + args.steps)]

    def step(k):
        at, ao, pa, st, so, _, _ = inputs[k]
        B.quail_join_run(ctx, at, ao, pa, st, so, 0x0F, logits, None, dec, stream=stream)

    log(f"join: warmup {args.warmup}")
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    B.quail_ctx_profile(ctx, True)
    log(f"join: timing {args.steps} steps")
    t0 = time.perf_counter()
    for k in range(args.warmup, args.warmup + args.steps):
        step(k)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    prof = B.quail_ctx_profile_read(ctx)
    B.quail_ctx_profile(ctx, False)
    chk = B.quail_ctx_check(ctx)
    st = B.quail_pool_stats(ctx)
    ms_step = el * 1000.0 / args.steps
    logical = per_step_pairs * (JOIN_LA + JOIN_LS)
    computed = per_step_pairs * JOIN_LS + ANCHORS_PER_STEP * JOIN_LA
    value = logical / (ms_step * 1e-3) * 60.0
    kern = {}
    for kname, v in prof.items():
        if v["launches"]:
            kern[kname] = {"launches": v["launches"], "ms": v["ms"], "avg_launch_ms": v["ms"] / v["launches"],
                           "share_of_step_time": v["ms"] / (el * 1000.0)}
            if v["flop"] > 0:
                kern[kname]["tflops"] = v["flop"] / (v["ms"] * 1e-3) / 1e12
                kern[kname]["frac"] = kern[kname]["tflops"] / PEAK_BF16_TFLOPS
    gu = prof["gate_up"]
    gu_ms = gu["ms"] / gu["launches"]
    gu_flop = gu["flop"] / gu["launches"]
    gu_tf = gu_flop / (gu_ms * 1e-3) / 1e12
    gemm_ms = sum(prof[k]["ms"] for k in ("qkv", "o", "gate_up", "down"))
    gemm_flop = sum(prof[k]["flop"] for k in ("qkv", "o", "gate_up", "down"))
    tokens_per_launch = gu_flop / (2.0 * 2 * shape.intermediate * shape.hidden)
    log(f"join: step {ms_step:.1f} ms, {value / 1e6:.1f} M logical tok/min; gate/up {gu_ms:.3f} ms per launch, "
        f"{gu_tf:.1f} TFLOP/s; all GEMMs {gemm_flop / (gemm_ms * 1e-3) / 1e12:.1f} TFLOP/s "
        f"({gemm_ms / (el * 1000.0):.1%} of the time)")
    res = {
        "metric": METRIC, "value": value, "unit": "tokens/min", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {
            "workload": "36-layer AI.IF join, Qwen3-4B shape with random-init fp8 weights: 64 anchors x 1024 "
                        "tokens, each joined to 2048 suffixes of 64 tokens (131,072 pairs, bf16 anchor KV); "
                        "one step = 2 anchors with their 4,096 pairs (1/32 of the join) through "
                        "quail_join_run: plan, anchor prefill + KV writer, 36-layer join prefill, 8-column head",
            "anchors_per_step": ANCHORS_PER_STEP, "pairs_per_step": per_step_pairs,
            "logical_tokens_per_step": logical, "computed_tokens_per_step": computed,
            "computed_tokens_per_min": computed / (ms_step * 1e-3) * 60.0,
            "whole_join_s_at_this_rate": ms_step * 1e-3 * n_groups,
            "max_batch_tokens": T, "parallelism": "single GPU",
            "kernels": kern,
            "gemm_all_tflops": gemm_flop / (gemm_ms * 1e-3) / 1e12,
            "pool": st, "debug_counters": chk,
        },
        "roofline": {
            "bound": "mfma", "achieved": gu_tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": gu_tf / PEAK_BF16_TFLOPS, "traffic": measured_traffic(GEMM_TRAFFIC_FILE, GEMM_SOURCES),
            "kernel": "quail::gemm_direct_kernel<2, 256, 256, 4, 2>",
            "what": "gate/up projection (W8A16 GEMM, 19456 x 2560) with the SwiGLU epilogue",
            "flops_per_launch": gu_flop, "launch_ms": gu_ms, "launches": gu["launches"],
            "tokens_per_launch": tokens_per_launch,
            "algorithmic_bytes_per_launch": 2 * shape.intermediate * shape.hidden
                + tokens_per_launch * (shape.hidden * 2 + shape.intermediate * 2),
        },
        "cpu_baseline": None,
    }
    # the cascade-attention headline configuration, timed on its own
    if not args.no_cascade:
        c1 = bench_cascade(args, steps=5, warmup=2, cpu=False)
        res["config"]["cascade_attention_layer"] = {
            "workload": c1["config"]["workload"], "tflops": c1["roofline"]["achieved"],
            "frac": c1["roofline"]["frac"], "launch_ms": c1["roofline"]["launch_ms"],
            "kernel": c1["roofline"]["kernel"], "traffic": c1["roofline"]["traffic"]}
    # the same steps with per-token E4M3 activations (W8A8 projections on the
    # fp8 MFMA): an opt-in mode outside the W8A16 contract, timed as a field
    if not args.no_w8a8:
        res["config"]["w8a8_same_steps"] = w8a8_join_field(args, B, shape, dm, inputs, step_inputs, logits, dec,
                                                           per_step_pairs, logical, T)
    if not args.no_cpu_baseline:
        lg = logits.cpu().numpy().astype(np.float64)
        at, ao, pa, st_, so, a0, p0 = inputs[args.warmup + args.steps - 1]
        order = np.random.default_rng(0).permutation(per_step_pairs)[:8]
        pairs = []
        for i in order:
            a = a0 + int(pa[i])
            pi = p0 + int(i)
            pairs.append((int(i), case["a_tok"][a_off[a]:a_off[a + 1]], case["s_tok"][s_off[pi]:s_off[pi + 1]]))
        log("join: oracle leg")
        cpu = cpu_baseline_e2e(wd, shape, pairs, lg, 0x0F, args.cpu_budget)
        cpu.update(host_cpu())
        cpu["cores"] = cpu["blas_threads"]
        res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


def bench_cascade(args, steps=None, warmup=None, cpu=True):
    """The cascade-attention layer alone (256 anchors of U{512..2048} tokens x
    64 suffixes of U{32..128} tokens, bf16 Q/K/V in HBM): its JSON line."""
    steps = args.steps if steps is None else steps
    warmup = args.warmup if warmup is None else warmup
    import torch
    import workloads as W
    from query_aware_prefill_amd import binding as B

    B.load()
    log("generating the workload in HBM")
    case = W.c1_device(seed=1)
    a_len, s_anchor, s_len = case["a_len"], case["s_anchor"], case["s_len"]
    T = int(case["s_off"][-1])
    out = torch.empty((T, 32, 128), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(B.quail_cascade_workspace_bytes(case["a_off"], case["s_off"]), dtype=torch.uint8,
                     device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        B.quail_cascade_attn(B.DTYPE_BF16, 32, 8, 128, case["sm_scale"], case["ak"], case["av"],
                             case["a_off"], s_anchor, case["q"], case["k"], case["v"], case["s_off"],
                             out, None, ws, stream=stream)

    log(f"cascade: warmup {warmup}")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    log(f"cascade: timing {steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    ms_step = el * 1000.0 / steps
    kernel_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))

    logical = float(np.sum(a_len[s_anchor] + s_len))
    computed = float(np.sum(s_len))
    cross, self_ = algorithmic_flops(a_len, s_anchor, s_len)
    flops = cross + self_
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    value = logical / (ms_step * 1e-3) * 60.0
    log(f"step {ms_step:.3f} ms, launch {kernel_ms:.3f} ms, {achieved:.1f} TFLOP/s")

    cpu = None
    if cpu and not args.no_cpu_baseline:
        log("oracle CPU baseline")
        cpu = cpu_baseline(case, args.cpu_budget)

    res = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/min",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "cascade-attention layer, Qwen3-4B shape: 256 anchors of U{512..2048} tokens x 64 "
                        "suffixes of U{32..128} tokens each, 32q/8kv heads x 128, bf16, N(0,1) Q/K/V",
            "anchors": 256, "suffixes": int(len(s_len)), "anchor_tokens": int(np.sum(a_len)),
            "suffix_tokens": int(computed), "logical_tokens_per_step": int(logical),
            "computed_tokens_per_min": computed / (ms_step * 1e-3) * 60.0,
            "cascade_tflops": achieved,
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS, "traffic": measured_traffic(),
            "kernel": "quail::attn_direct_kernel<4, false, false, 0, false>", "flops_per_launch": flops,
            "launch_ms": kernel_ms,
            "algorithmic_bytes_per_launch": algorithmic_bytes(a_len, s_len),
        },
        "cpu_baseline": cpu,
    }
    del case, out, ws
    torch.cuda.empty_cache()
    return res




def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cascade", action="store_true",
                    help="join: skip the separately timed cascade-attention layer (profiling runs)")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--workload", choices=["join", "cascade", "gemm", "gemm8", "layer", "copy", "stream", "join36",
                                           "filter36", "multijoin36", "multijoin36full", "multiplan36", "shared36",
                                           "traces36", "nested36", "search"],
                    default="join")
    ap.add_argument("--rows", type=int, default=625, help="multijoin36: rows of the 5,000 used")
    ap.add_argument("--no-w8a8", action="store_true",
                    help="headline: skip the W8A8 run of the same steps (a field of the line)")
    ap.add_argument("--act-fp8", action="store_true",
                    help="join36 / filter36 / multijoin36 / multijoin36full: per-token E4M3 activations "
                         "(W8A8 projections)")
    ap.add_argument("--shared-only", action="store_true", help="shared36: run only the join with prefix nodes")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(pairs grouped by anchor shard across GPUs with no communication but the "
              "1-byte decisions; see the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.workload == "gemm":
        return bench_gemm(args)
    if args.workload == "gemm8":
        return bench_gemm8(args)
    if args.workload == "layer":
        return bench_layer(args)
    if args.workload == "copy":
        return bench_copy(args)
    if args.workload == "stream":
        return bench_stream(args)
    if args.workload == "multiplan36":
        return bench_multiplan(args)
    if args.workload in ("shared36", "traces36"):
        return bench_shared(args)
    if args.workload == "search":
        return bench_search(args)
    if args.workload == "nested36":
        return bench_nested(args)
    if args.workload == "multijoin36full":
        return bench_multijoin_full(args)
    if args.workload in ("join36", "filter36", "multijoin36"):
        return bench_e2e(args)

    if args.workload == "cascade":
        res = bench_cascade(args)
        print(json.dumps(res), flush=True)
        return
    return bench_join(args)


if __name__ == "__main__":
    main()
