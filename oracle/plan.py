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


def multijoin_reference(anchor_slab, anchor_len, joins, pool_bytes, max_batch_tokens):
    """Several joins over one anchor table, run one after another (a later
    join may depend on an earlier one's results, so their pairs are not
    merged). [pt] query-aware KV cache bullet: with the whole plan known, KV
    is kept for its next use and evicted when nothing will use it again.

    Readings taken (the pages give no algorithm):
      * each join is ordered and cut into steps exactly as one join alone
        (plan_reference, full pool budget);
      * the steps of all joins form one sequence; an anchor's last use is its
        last step in that whole sequence (plan-wide), so an anchor used by
        several joins stays resident across the joins in between;
      * before a step, its anchors that are not resident are prefilled (a
        second prefill of an anchor counts its tokens as regret); when they
        do not fit beside the anchors kept for later steps, kept anchors are
        evicted farthest next use first (never used again first; ties: the
        larger slab, then the lower index) until they fit -- each step's own
        anchors always fit, the step cutting guarantees it;
      * after a step, the anchors whose last use it was are evicted.

    joins: list of (pair_anchor, pair_len). Returns dict with the per-join
    plans, and per global step: the join, its pair range, the anchors
    prefilled before it (in order of first use within the step), the anchors
    evicted to make room before it (in eviction order) and the anchors
    evicted after it (ascending); plus prefills, evictions, regret_tokens and
    peak (largest resident bytes, measured after each step's prefills)."""
    plans = [plan_reference(anchor_slab, pa, pl, pool_bytes, max_batch_tokens) for pa, pl in joins]
    steps = []   # (join, lo, hi, anchors in first-use order)
    for j, ((pa, _), p) in enumerate(zip(joins, plans)):
        pa = np.asarray(pa, np.int64)
        b = p["step_bounds"]
        for s in range(len(b) - 1):
            seen = []
            for i in p["order"][b[s]:b[s + 1]]:
                a = int(pa[i])
                if a >= 0 and a not in seen:
                    seen.append(a)
            steps.append((j, int(b[s]), int(b[s + 1]), seen))
    INF = len(steps)
    uses_at = {}
    for t, (_, _, _, an) in enumerate(steps):
        for a in an:
            uses_at.setdefault(a, []).append(t)

    def next_use(a, t):
        for u in uses_at[a]:
            if u > t:
                return u
        return INF

    resident = {}
    ever = set()
    prefills = evictions = regret = peak = 0
    out_steps = []
    for t, (j, lo, hi, an) in enumerate(steps):
        need = [a for a in an if a not in resident]
        need_b = sum(int(anchor_slab[a]) for a in need)
        room_evict = []
        while sum(resident.values()) + need_b > pool_bytes:
            cand = [a for a in resident if a not in an]
            a = max(cand, key=lambda x: (next_use(x, t), int(anchor_slab[x]), -x))
            del resident[a]
            evictions += 1
            room_evict.append(a)
        for a in need:
            if a in ever:
                regret += int(anchor_len[a])
            ever.add(a)
            resident[a] = int(anchor_slab[a])
            prefills += 1
        peak = max(peak, sum(resident.values()))
        after = sorted(a for a in an if next_use(a, t) == INF)
        for a in after:
            del resident[a]
            evictions += 1
        out_steps.append(dict(join=j, lo=lo, hi=hi, prefill=need, evict_before=room_evict, evict_after=after))
    return dict(plans=plans, steps=out_steps, prefills=prefills, evictions=evictions,
                regret_tokens=regret, peak=peak)


def multijoin_naive_regret(anchor_len, joins):
    """Regret of planning each join alone (every anchor evicted at its last use
    inside its join): an anchor used by k joins is prefilled k times."""
    k = {}
    for pa, _ in joins:
        for a in set(int(x) for x in pa if x >= 0):
            k[a] = k.get(a, 0) + 1
    return sum(int(anchor_len[a]) * (c - 1) for a, c in k.items())
