"""Plan order and anchor-KV residency: the reference semantics.

Test infrastructure (see the package header).

[pt] "Como funciona", bullet on the query-aware KV cache: because the engine
knows the whole plan in advance it can predict accesses and evict entries
with no regret. [it]/[de] quote the Modal blog: with a structured query in
hand one can order requests so that KV is cached (and evicted) better; [pl]
"Praca nad silnikiem, nie nad krzemem": Quail takes the query plan as input,
orders requests to reuse the cache and evicts it deliberately. [it] also names
"KV regret": tokens recomputed because KV needed later was discarded.

Readings taken (the pages give no algorithm):
  * order: pairs are stably sorted by anchor index; filter rows (no anchor)
    come last, in input order;
  * steps: consecutive runs of the ordered pairs, cut greedily; a step closes
    when adding the next pair would exceed the token budget of one batch or
    the pool bytes needed by the distinct anchors the step touches;
  * residency under that order: an anchor is prefilled just before the first
    step that uses it and evicted right after the last one, so the bytes
    resident during a step are the slabs of the distinct anchors it touches;
  * regret: an anchor prefilled a second time after an eviction counts its
    tokens as regret (never happens under the sorted order).

Pins (tests/test_oracle_plan.py): brute-force checks on small random cases --
every pair appears once; the order is sorted and stable; each step respects
both budgets and could not take the next pair; prefills = evictions = number
of anchors with at least one pair; regret 0; the peak equals the maximum over
steps, checked against an independent step-by-step replay.
"""
from __future__ import annotations

import numpy as np


def slab_bytes(anchor_len, n_layers, n_kv_heads, head_dim, kv_bytes, pad=64, align=256):
    """Pool bytes of one anchor's KV slab: layers x {K,V} x kv heads x padded
    tokens x head_dim x element size, rounded up to ``align``."""
    la_pad = -(-int(anchor_len) // pad) * pad
    b = n_layers * 2 * n_kv_heads * la_pad * head_dim * kv_bytes
    return -(-b // align) * align


def plan_reference(anchor_slab, pair_anchor, pair_len, pool_bytes, max_batch_tokens):
    """anchor_slab[a] = slab bytes of anchor a; pair_anchor[i] (-1 = filter row);
    pair_len[i] = suffix tokens. Returns dict(order, step_bounds, peak, uses)
    or raises ValueError naming the first impossible item."""
    pair_anchor = np.asarray(pair_anchor, np.int64)
    pair_len = np.asarray(pair_len, np.int64)
    n = len(pair_anchor)
    key = np.where(pair_anchor < 0, np.iinfo(np.int64).max, pair_anchor)
    order = np.argsort(key, kind="stable")
    uses = np.bincount(pair_anchor[pair_anchor >= 0], minlength=len(anchor_slab))
    bounds = [0]
    tokens = 0
    anchors = set()
    bytes_ = 0
    peak = 0
    for pos, i in enumerate(order):
        a = int(pair_anchor[i])
        L = int(pair_len[i])
        if L <= 0 or L > max_batch_tokens:
            raise ValueError(f"pair {i}: length {L} outside [1, {max_batch_tokens}]")
        add_b = int(anchor_slab[a]) if (a >= 0 and a not in anchors) else 0
        if a >= 0 and int(anchor_slab[a]) > pool_bytes:
            raise ValueError(f"anchor {a}: slab {anchor_slab[a]} B exceeds pool {pool_bytes} B")
        if pos > bounds[-1] and (tokens + L > max_batch_tokens or bytes_ + add_b > pool_bytes):
            peak = max(peak, bytes_)
            bounds.append(pos)
            tokens, anchors, bytes_ = 0, set(), 0
            add_b = int(anchor_slab[a]) if a >= 0 else 0
        tokens += L
        if a >= 0 and a not in anchors:
            anchors.add(a)
            bytes_ += add_b
    if n > 0:
        peak = max(peak, bytes_)
        bounds.append(n)
    return dict(order=order, step_bounds=np.asarray(bounds, np.int64), peak=peak,
                uses=uses)


def replay_residency(anchor_slab, anchor_len, pair_anchor, order, step_bounds):
    """Run steps in order with prefill-at-first-use and evict-at-last-use.
    Returns dict(prefills, evictions, regret_tokens, peak)."""
    pair_anchor = np.asarray(pair_anchor)
    remaining = np.bincount(pair_anchor[pair_anchor >= 0], minlength=len(anchor_slab)).astype(np.int64)
    resident = {}
    ever = set()
    prefills = evictions = regret = 0
    peak = 0
    for s in range(len(step_bounds) - 1):
        idx = order[step_bounds[s]:step_bounds[s + 1]]
        for i in idx:
            a = int(pair_anchor[i])
            if a >= 0 and a not in resident:
                if a in ever:
                    regret += int(anchor_len[a])
                resident[a] = int(anchor_slab[a])
                ever.add(a)
                prefills += 1
        peak = max(peak, sum(resident.values()))
        for i in idx:
            a = int(pair_anchor[i])
            if a >= 0:
                remaining[a] -= 1
        for a in [a for a in resident if remaining[a] == 0]:
            del resident[a]
            evictions += 1
    return dict(prefills=prefills, evictions=evictions, regret_tokens=regret, peak=peak)
