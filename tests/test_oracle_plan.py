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


# ---------------------------------------------------------------------------
# several joins over one anchor table (plan-wide residency)
# ---------------------------------------------------------------------------
def _multi_case(seed, equal_slabs=False, max_pool_slabs=4):
    r = np.random.default_rng(1000 + seed)
    na = int(r.integers(1, 7))
    a_len = r.integers(1, 200, na)
    if equal_slabs:
        a_len[:] = 100
    slab = np.array([P.slab_bytes(x, 2, 2, 64, 2) for x in a_len])
    joins = []
    for _ in range(int(r.integers(1, 4))):
        n = int(r.integers(0, 12))
        joins.append((r.integers(-1, na, n), r.integers(1, 50, n)))
    pool = int(slab.max() * r.integers(1, max_pool_slabs + 1))
    mbt = int(r.integers(50, 200))
    return a_len, slab, joins, pool, mbt


def _replay_multi(slab, a_len, joins, res, pool):
    """Independent replay of the event lists: checks residency at every step
    and recounts prefills, evictions, regret and peak."""
    resident, ever = {}, set()
    pre = ev = regret = peak = 0
    covered = [np.zeros(len(pa), bool) for pa, _ in joins]
    for st in res["steps"]:
        j = st["join"]
        pa = np.asarray(joins[j][0])
        plan = res["plans"][j]
        idx = plan["order"][st["lo"]:st["hi"]]
        covered[j][idx] = True
        for a in st["evict_before"]:
            assert a in resident
            del resident[a]
            ev += 1
        for a in st["prefill"]:
            assert a not in resident
            if a in ever:
                regret += int(a_len[a])
            ever.add(a)
            resident[a] = int(slab[a])
            pre += 1
        assert sum(resident.values()) <= pool
        peak = max(peak, sum(resident.values()))
        for i in idx:                       # every anchor of the step is resident
            if pa[i] >= 0:
                assert int(pa[i]) in resident
        for a in st["evict_after"]:
            del resident[a]
            ev += 1
    assert not resident                     # everything evicted at the end
    assert all(c.all() for c in covered)    # every pair ran exactly in its join's plan
    return pre, ev, regret, peak


@pytest.mark.parametrize("seed", range(60))
def test_multijoin_invariants(seed):
    a_len, slab, joins, pool, mbt = _multi_case(seed)
    res = P.multijoin_reference(slab, a_len, joins, pool, mbt)
    pre, ev, regret, peak = _replay_multi(slab, a_len, joins, res, pool)
    assert (pre, ev, regret, peak) == (res["prefills"], res["evictions"], res["regret_tokens"], res["peak"])
    # never worse than planning each join alone
    assert res["regret_tokens"] <= P.multijoin_naive_regret(a_len, joins)
    # the steps are the single-join plans, in join order
    k = 0
    for j, p in enumerate(res["plans"]):
        b = p["step_bounds"]
        for s in range(len(b) - 1):
            assert (res["steps"][k]["join"], res["steps"][k]["lo"], res["steps"][k]["hi"]) == (j, b[s], b[s + 1])
            k += 1
    assert k == len(res["steps"])


@pytest.mark.parametrize("seed", range(20))
def test_multijoin_ample_pool_has_no_regret(seed):
    """With a pool that holds every anchor, each anchor used anywhere is
    prefilled once and evicted once, whatever the number of joins."""
    a_len, slab, joins, _, mbt = _multi_case(seed)
    res = P.multijoin_reference(slab, a_len, joins, int(slab.sum()) + 1, mbt)
    used = set(int(a) for pa, _ in joins for a in pa if a >= 0)
    assert res["regret_tokens"] == 0
    assert res["prefills"] == res["evictions"] == len(used)


@pytest.mark.parametrize("seed", range(20))
def test_multijoin_single_join_is_the_single_join_plan(seed):
    a_len, slab, joins, pool, mbt = _multi_case(seed)
    pa, pl = joins[0]
    res = P.multijoin_reference(slab, a_len, [(pa, pl)], pool, mbt)
    p = P.plan_reference(slab, pa, pl, pool, mbt)
    ref = P.replay_residency(slab, a_len, pa, p["order"], p["step_bounds"])
    assert (res["prefills"], res["evictions"], res["regret_tokens"], res["peak"]) == \
        (ref["prefills"], ref["evictions"], ref["regret_tokens"], ref["peak"])


def _min_regret_brute(slab, a_len, steps_anchors, pool):
    """Smallest regret over every eviction choice (any set of resident anchors
    not used by the step may be evicted before it), by exhaustive search."""
    from functools import lru_cache
    from itertools import combinations
    T = len(steps_anchors)
    last = {}
    for t, an in enumerate(steps_anchors):
        for a in an:
            last[a] = t

    @lru_cache(maxsize=None)
    def go(t, resident, ever):
        if t == T:
            return 0
        an = steps_anchors[t]
        need = [a for a in an if a not in resident]
        cost = sum(int(a_len[a]) for a in need if a in ever)
        cand = [a for a in resident if a not in an]
        best = None
        for k in range(len(cand) + 1):
            for ev in combinations(sorted(cand), k):
                keep = set(resident) - set(ev)
                if sum(int(slab[a]) for a in keep) + sum(int(slab[a]) for a in need) > pool:
                    continue
                nr = frozenset(a for a in keep | set(need) if last[a] > t)
                v = go(t + 1, nr, frozenset(ever | set(need)))
                best = v if best is None else min(best, v)
        return cost + best

    return go(0, frozenset(), frozenset())


@pytest.mark.parametrize("seed", range(40))
def test_multijoin_farthest_next_use_is_optimal_for_equal_slabs(seed):
    """With equal slabs, evicting the farthest next use first is optimal
    (the classic paging result): the plan's regret equals the exhaustive
    minimum over all eviction choices."""
    a_len, slab, joins, pool, mbt = _multi_case(seed, equal_slabs=True, max_pool_slabs=3)
    res = P.multijoin_reference(slab, a_len, joins, pool, mbt)
    steps_anchors = []
    for st in res["steps"]:
        pa = np.asarray(joins[st["join"]][0])
        idx = res["plans"][st["join"]]["order"][st["lo"]:st["hi"]]
        steps_anchors.append(tuple(dict.fromkeys(int(a) for a in pa[idx] if a >= 0)))
    assert res["regret_tokens"] == _min_regret_brute(slab, a_len, steps_anchors, pool)
