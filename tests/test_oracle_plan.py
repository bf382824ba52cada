"""Pins for oracle/plan.py by brute force over small random cases."""
import numpy as np
import pytest

from oracle import plan as P


def _case(seed):
    r = np.random.default_rng(seed)
    na = int(r.integers(1, 8))
    a_len = r.integers(1, 200, na)
    slab = np.array([P.slab_bytes(x, 2, 2, 64, 2) for x in a_len])
    n = int(r.integers(0, 40))
    pa = r.integers(-1, na, n)
    pl = r.integers(1, 50, n)
    pool = int(slab.max() * r.integers(1, 4))
    mbt = int(r.integers(50, 200))
    return a_len, slab, pa, pl, pool, mbt


@pytest.mark.parametrize("seed", range(60))
def test_plan_invariants(seed):
    a_len, slab, pa, pl, pool, mbt = _case(seed)
    p = P.plan_reference(slab, pa, pl, pool, mbt)
    order, b = p["order"], p["step_bounds"]
    n = len(pa)
    assert sorted(order.tolist()) == list(range(n))
    key = np.where(pa[order] < 0, 10 ** 9, pa[order])
    assert np.all(np.diff(key) >= 0)
    for i in range(n - 1):                   # stable inside equal keys
        if key[i] == key[i + 1]:
            assert order[i] < order[i + 1]
    if n == 0:
        assert len(b) == 1
        return
    assert b[0] == 0 and b[-1] == n and np.all(np.diff(b) > 0)
    peak = 0
    for s in range(len(b) - 1):
        idx = order[b[s]:b[s + 1]]
        toks = int(pl[idx].sum())
        anchors = {int(a) for a in pa[idx] if a >= 0}
        byts = sum(int(slab[a]) for a in anchors)
        assert toks <= mbt and byts <= pool
        peak = max(peak, byts)
        if b[s + 1] < n:                     # greedy: the next pair would not fit
            j = order[b[s + 1]]
            a = int(pa[j])
            nb = byts + (int(slab[a]) if a >= 0 and a not in anchors else 0)
            assert toks + int(pl[j]) > mbt or nb > pool
    assert peak == p["peak"]
    rep = P.replay_residency(slab, a_len, pa, order, b)
    used = len({int(a) for a in pa if a >= 0})
    assert rep["prefills"] == used and rep["evictions"] == used
    assert rep["regret_tokens"] == 0
    assert rep["peak"] == peak


def test_unsorted_order_can_cause_regret_in_replay():
    # anchor 0 used, evicted too early by a forced cut, used again: regret counted
    a_len = np.array([10, 20])
    slab = np.array([100, 100])
    pa = np.array([0, 1, 0])
    order = np.array([0, 1, 2])
    rep = P.replay_residency(slab, a_len, pa, order, np.array([0, 1, 2, 3]))
    assert rep["regret_tokens"] == 0        # use counts keep anchor 0 resident
    assert rep["peak"] == 200 and rep["prefills"] == 2


def test_plan_rejects_oversized_items():
    slab = np.array([1000])
    with pytest.raises(ValueError):
        P.plan_reference(slab, [0], [5], 999, 100)
    with pytest.raises(ValueError):
        P.plan_reference(slab, [0], [101], 1000, 100)


def test_slab_bytes_layout():
    # 36 layers x K/V x 8 kv heads x 768 tokens x 128 x 1 B (fp8) = 56.6 MB
    assert P.slab_bytes(768, 36, 8, 128, 1) == 36 * 2 * 8 * 768 * 128
    assert P.slab_bytes(1, 1, 1, 128, 2) == 2 * 64 * 128 * 2
