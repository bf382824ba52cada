"""Pins for oracle/joinorder.py: a two-table case worked by hand, the
orientation choice of a symmetric join, the speed-of-light time of the
64 x 2048 join workload against FLOP and byte counts derived from the
Qwen3-4B shapes, and frontier invariants over random tree queries."""
import itertools

import numpy as np
import pytest

from oracle import joinorder as J

QWEN = J.model_constants(36, 2560, 32, 8, 128, 9728, 2)


def test_model_constants_from_shapes():
    gemm, attn, kv = QWEN
    # per token per layer: QKV 2560x6144, O 4096x2560, gate/up 2560x19456, down 9728x2560
    assert gemm == 2 * (2560 * 6144 + 4096 * 2560 + 2560 * 19456 + 9728 * 2560) * 36 == 201_850_880 * 36
    assert attn == 16_384 * 36                     # 4 * 32 heads * 128 dims per (query, key) pair
    assert kv == 2 * 8 * 128 * 2 * 36              # K and V, 8 kv heads x 128, bf16, 36 layers


def test_two_table_case_by_hand():
    consts = (1.0, 1.0, 1.0)
    tables = [(3, 10), (5, 4)]
    joins = [(0, 1, 2, 1, 0.5, 0)]
    # anchors: 3 rows of 10 + 2 tokens; 15 pairs of 4 + 1 suffix tokens
    assert J.plan_metrics([0, 1], [0], tables, joins, consts) == (3 * 12 + 15 * 5,
                                                                 15 * (12 * 5 + 15) + 3 * 78, 3 * 12)
    # the order does not change a single join; a symmetric join may flip
    assert J.plan_metrics([1, 0], [0], tables, joins, consts) == J.plan_metrics([0, 1], [0], tables, joins, consts)
    flipped = J.plan_metrics([0, 1], [1], tables, [(0, 1, 2, 1, 0.5, 1)], consts)
    assert flipped == (5 * 6 + 15 * 11, 15 * (6 * 11 + 66) + 5 * 21, 5 * 6)


def test_chain_order_changes_the_work():
    consts = (1.0, 0.0, 0.0)
    # A(10) - B(100) - C(1000), selectivities 1/100 and 1/1000, 1-token fields
    tables = [(10, 1), (100, 1), (1000, 1)]
    joins = [(0, 1, 0, 0, 0.01, 0), (1, 2, 0, 0, 0.001, 0)]
    abc = J.plan_metrics([0, 1, 2], [0, 0], tables, joins, consts)
    # A x B: 1000 pairs; N = 10 rows survive, so 10 distinct B rows x 1000 C rows
    assert abc[0] == (10 + 1000) + (10 + 10 * 1000)
    cba = J.plan_metrics([2, 1, 0], [0, 0], tables, joins, consts)
    # B x C: 100 anchors + 100,000 pairs; N = 100, so 100 distinct B rows x 10 A rows
    assert cba[0] == (100 + 100_000) + (10 + 100 * 10)
    assert J.plan_metrics([0, 2, 1], [0, 0], tables, joins, consts) is None   # C does not touch A


def test_symmetric_join_keeps_the_short_anchor_table():
    tables = [(64, 1024), (2048, 64)]
    r = J.search_reference(tables, [(0, 1, 0, 0, 1.0, 1)], QWEN, 2.5166e15, 8e12)
    assert len(r["frontier"]) == 1
    tok, att, cache, sec = r["frontier"][0]
    assert tok == 64 * 1024 + 64 * 2048 * 64
    assert cache == 64 * 1024 * 147_456                    # 9.66 GB of bf16 anchor KV
    flops = tok * 201_850_880 * 36 + att * 16_384 * 36
    assert abs(flops - 66.68e15) / 66.68e15 < 1e-3         # 66.7 PFLOP for the 64 x 2048 join
    assert abs(sec - flops / 2.5166e15) < 1e-9 and abs(sec - 26.50) < 0.01


def random_query(seed):
    r = np.random.default_rng(seed)
    n = int(r.integers(1, 6))
    tables = [(int(r.integers(1, 3000)), float(r.integers(0, 400))) for _ in range(n)]
    joins = []
    for t in range(1, n):                                   # random tree
        u = int(r.integers(0, t))
        a, b = (u, t) if r.random() < 0.5 else (t, u)
        joins.append((a, b, float(r.integers(0, 30)), float(r.integers(0, 30)),
                      float(r.integers(1, 65)) / 64.0, int(r.random() < 0.5)))
    return tables, joins


@pytest.mark.parametrize("seed", range(30))
def test_frontier_invariants(seed):
    tables, joins = random_query(seed)
    r = J.search_reference(tables, joins, QWEN, 2.5166e15, 8e12)
    vecs = [p[2] for p in r["plans"]]
    front = [f[:3] for f in r["frontier"]]
    assert len(vecs) >= 1 and len(front) >= 1
    for f in front:
        assert not any(v != f and all(a <= b for a, b in zip(v, f)) for v in vecs)
    for v in vecs:
        assert any(all(a <= b for a, b in zip(f, v)) for f in front)
    assert r["best_seconds"] == min(J.sol_seconds(v, QWEN, 2.5166e15, 8e12) for v in vecs)
