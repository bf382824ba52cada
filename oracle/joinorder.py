"""KV-aware join-order search and the speed-of-light cost model -- the
reference semantics, by brute-force enumeration. TEST INFRASTRUCTURE ONLY
(see the package header).

[pt] "Como funciona": the join-order search is aware of the KV cache; it keeps
several candidates and drops plans that are Pareto-dominated (more tokens,
more attention pairs and more cache), choosing among the rest with the cost
model; the "speed-of-light" cost model is a roofline model that overstates the
hardware's peak on purpose, as a guide for optimisation. [fa] body: the join
order is chosen with the KV cache in mind and a roofline-based speed-of-light
model estimates how fast each plan can at best run.

Readings taken (the pages give no formulas; the plainest ones that fit):
  * Query: tables t with R_t rows whose prompt field has l_t tokens; AI.IF
    predicates k between tables a_k and b_k, forming a tree over the tables,
    each with g^A_k template tokens that go with the anchor (shared prefix),
    g^S_k template tokens that go with the suffix, a selectivity s_k, and a
    flag saying whether either field may come first (symmetric). Otherwise the
    anchor is the template's first field, table a_k.
  * Plan: a left-deep order of the tables in which each table after the first
    joins the ones before it through exactly one predicate (true for a tree
    when every prefix is connected), plus the anchor side of every symmetric
    predicate.
  * Cardinality under independence: N(S) = prod R_t * prod s_k over the tables
    and predicates inside S. Distinct rows of table u in that result:
    D_u(S) = min(R_u, N(S)).
  * Step adding table t through predicate k, u = its other end (already in S):
    the predicate runs once per distinct (u row, t row): P = D_u(S) * R_t
    pairs. Anchor side x, suffix side y: A = distinct x rows (D_u(S) or R_t),
    La = l_x + g^A_k, Ls = l_y + g^S_k.
      computed tokens = A La + P Ls        (each anchor's KV computed once)
      attention pairs = P (La Ls + Ls (Ls+1)/2) + A La (La+1)/2
      cache bytes     = A La * (KV bytes per token over all layers)
  * A plan's metrics are the sums over its steps. Plan X is dominated when a
    plan Y is <= X in all three and differs; the frontier is the set of
    non-dominated metric vectors.
  * Speed-of-light time of a plan: the roofline of all its work,
    max(FLOP / peak FLOP/s, bytes / peak bytes/s), with
    FLOP = tokens * 2 * (weights per token over all layers)
         + attention pairs * 4 * Hq * d * L,  bytes = 2 * cache bytes (each
    anchor's KV written once and read once). The chosen plan is a frontier
    plan of least time. The peaks passed in are the datasheet's (optimistic).

Pins (tests/test_oracle_joinorder.py): two-table queries by hand (anchor side
choice, the formulas on a worked example), the single-join speed-of-light time
of the 64 x 2048 join workload against its independently derived FLOP count,
frontier invariants (no member dominated, every enumerated plan dominated by
or equal to a member), and order invariance of the cardinality.
"""
from __future__ import annotations

import itertools

import numpy as np


def model_constants(n_layers, hidden, n_q_heads, n_kv_heads, head_dim, intermediate, kv_bytes):
    """Per-token GEMM FLOP over all layers, attention FLOP per (query, key)
    pair over all layers, KV bytes per token over all layers."""
    qkv = hidden * (n_q_heads + 2 * n_kv_heads) * head_dim
    o = n_q_heads * head_dim * hidden
    mlp = 3 * hidden * intermediate
    gemm = 2.0 * (qkv + o + mlp) * n_layers
    attn = 4.0 * n_q_heads * head_dim * n_layers
    kv = 2.0 * n_kv_heads * head_dim * kv_bytes * n_layers
    return gemm, attn, kv


def _card(S, tables, preds):
    n = 1.0
    for t in S:
        n *= tables[t][0]
    for (a, b, _, _, s, _) in preds:
        if a in S and b in S:
            n *= s
    return n


def plan_metrics(order, anchor_right, tables, preds, consts):
    """Metrics (tokens, attention pairs, cache bytes) of one plan, or None if
    the order is not a valid left-deep tree order. tables[t] = (rows, tokens);
    preds[k] = (left, right, anchor glue, suffix glue, selectivity, symmetric);
    anchor_right[k] = the right table is the anchor (symmetric ones only)."""
    _, _, kv = consts
    tok = att = cache = 0.0
    S = {order[0]}
    for t in order[1:]:
        ks = [k for k, p in enumerate(preds) if (p[0] == t and p[1] in S) or (p[1] == t and p[0] in S)]
        if len(ks) != 1:
            return None
        k = ks[0]
        a, b, ga, gs, _, sym = preds[k]
        u = a if b == t else b
        N = _card(S, tables, preds)
        Du = min(tables[u][0], N)
        P = Du * tables[t][0]
        right_anchor = bool(anchor_right[k]) if sym else False
        x = b if right_anchor else a
        y = a if right_anchor else b
        A = Du if x == u else tables[t][0]
        La = tables[x][1] + ga
        Ls = tables[y][1] + gs
        tok += A * La + P * Ls
        att += P * (La * Ls + Ls * (Ls + 1) / 2.0) + A * La * (La + 1) / 2.0
        cache += A * La * kv
        S.add(t)
    return tok, att, cache


def sol_seconds(metrics, consts, peak_flops, peak_bytes):
    gemm, attn, _ = consts
    tok, att, cache = metrics
    return max((tok * gemm + att * attn) / peak_flops, 2.0 * cache / peak_bytes)


def search_reference(tables, preds, consts, peak_flops, peak_bytes):
    """Every valid plan enumerated. Returns dict(frontier = sorted list of
    (tokens, attention pairs, cache bytes, seconds), best_seconds, plans =
    list of (order, anchor_right, metrics))."""
    n = len(tables)
    sym = [k for k, p in enumerate(preds) if p[5]]
    plans = []
    for order in itertools.permutations(range(n)):
        for bits in itertools.product([0, 1], repeat=len(sym)):
            ar = [0] * len(preds)
            for k, bit in zip(sym, bits):
                ar[k] = bit
            m = plan_metrics(list(order), ar, tables, preds, consts)
            if m is not None:
                plans.append((list(order), ar, m))
    vecs = sorted({p[2] for p in plans})
    front = [v for v in vecs
             if not any(w != v and all(wi <= vi for wi, vi in zip(w, v)) for w in vecs)]
    front = [(*v, sol_seconds(v, consts, peak_flops, peak_bytes)) for v in front]
    best = min(f[3] for f in front) if front else 0.0
    return dict(frontier=front, best_seconds=best, plans=plans)
