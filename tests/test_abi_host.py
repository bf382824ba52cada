"""CPU tests of the C-ABI library: it loads, exports every function quail.h
declares, and its host logic (sizing, plan builder, validation and error
model) matches the oracle -- no GPU call is made here."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from oracle import plan as OP
from query_aware_prefill_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "quail.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|quail_status)\s+(quail_\w+)\s*\(", src, re.M)))


def test_library_exports_every_declared_symbol():
    lib = B.load()
    names = _declared()
    assert len(names) >= 20
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(B.EXPORTS) == names
    assert B.quail_version().startswith("quail-mi355x")


def _cfg(layers=36, fp8=False, **kw):
    d = dict(n_layers=layers, hidden=2560, n_q_heads=32, n_kv_heads=8, head_dim=128,
             intermediate=9728, vocab=151936, rope_theta=1e6, rms_eps=1e-6,
             kv_dtype=B.DTYPE_FP8_E4M3 if fp8 else B.DTYPE_BF16, k_scale=1.0, v_scale=1.0,
             max_anchor_len=2048, max_suffix_len=256)
    d.update(kw)
    return B.ModelConfig(**d)


# every slab the library carves ends with a guard region (quail.h)
G = B.GUARD_BYTES


def _slab(la, layers, kv_heads, d, esz):
    """Pool bytes of a slab: the oracle's KV layout plus the library's guard."""
    return OP.slab_bytes(la, layers, kv_heads, d, esz) + G


@pytest.mark.parametrize("fp8", [False, True])
def test_anchor_bytes_matches_oracle_slab(fp8):
    cfg = _cfg(fp8=fp8)
    for la in (1, 63, 64, 65, 768, 1024, 2048):
        assert B.quail_anchor_bytes(cfg, la) == _slab(la, 36, 8, 128, 1 if fp8 else 2)
    # 1024 anchors of 768 tokens: 57.98 GB in fp8 (twice that in bf16), plus the guards
    assert B.quail_anchor_bytes(cfg, 768) * 1024 == (36 * 2 * 8 * 768 * 128 * (1 if fp8 else 2) + G) * 1024


def test_workspace_bytes_grows_with_batch():
    cfg = _cfg()
    a = B.quail_workspace_bytes(cfg, 1024)
    b = B.quail_workspace_bytes(cfg, 2048)
    assert b > a > 1024 * 2560 * 2 * 8


@pytest.mark.parametrize("seed", range(40))
def test_plan_build_matches_oracle(seed):
    r = np.random.default_rng(100 + seed)
    cfg = _cfg(layers=2, n_kv_heads=2, n_q_heads=4, hidden=256, intermediate=384)
    na = int(r.integers(1, 9))
    a_len = r.integers(1, 300, na).astype(np.int32)
    slab = np.array([_slab(x, 2, 2, 128, 2) for x in a_len])
    n = int(r.integers(0, 60))
    pa = r.integers(-1, na, n).astype(np.int32)
    pl = r.integers(1, 64, n).astype(np.int32)
    pool = int(slab.max() * r.integers(1, 4))
    mbt = int(r.integers(64, 300))
    ref = OP.plan_reference(slab, pa, pl, pool, mbt)
    order, bounds, peak = B.quail_plan_build(cfg, pool, mbt, a_len, pa, pl)
    assert np.array_equal(order, ref["order"])
    assert np.array_equal(bounds, ref["step_bounds"])
    assert peak == ref["peak"]


@pytest.mark.parametrize("seed", range(40))
def test_multiplan_build_matches_oracle(seed):
    """Several joins over one anchor table: the library's plan (orders, steps,
    prefill / eviction events, totals) equals the oracle's, bit for bit."""
    r = np.random.default_rng(300 + seed)
    cfg = _cfg(layers=2, n_kv_heads=2, n_q_heads=4, hidden=256, intermediate=384)
    na = int(r.integers(1, 8))
    a_len = r.integers(1, 300, na).astype(np.int32)
    if seed % 3 == 0:
        a_len[:] = 128                       # equal slabs: eviction order decided by next use alone
    slab = np.array([_slab(x, 2, 2, 128, 2) for x in a_len])
    joins = []
    for _ in range(int(r.integers(1, 5))):
        n = int(r.integers(0, 25))
        joins.append((r.integers(-1, na, n).astype(np.int32), r.integers(1, 64, n).astype(np.int32)))
    pool = int(slab.max() * r.integers(1, 4))
    mbt = int(r.integers(64, 300))
    ref = OP.multijoin_reference(slab, a_len, joins, pool, mbt)
    jo = np.cumsum([0] + [len(pa) for pa, _ in joins]).astype(np.int32)
    pa_all = np.concatenate([pa for pa, _ in joins]) if jo[-1] else np.zeros(0, np.int32)
    pl_all = np.concatenate([pl for _, pl in joins]) if jo[-1] else np.zeros(0, np.int32)
    got = B.quail_multiplan_build(cfg, pool, mbt, a_len, jo, pa_all, pl_all)
    for j, p in enumerate(ref["plans"]):
        assert np.array_equal(got["pair_order"][jo[j]:jo[j + 1]], p["order"])
    assert len(got["steps"]) == len(ref["steps"])
    for g, e in zip(got["steps"], ref["steps"]):
        assert g == (e["join"], e["lo"], e["hi"], e["prefill"], e["evict_before"], e["evict_after"])
    assert (got["prefills"], got["evictions"], got["regret_tokens"], got["peak"]) == \
        (ref["prefills"], ref["evictions"], ref["regret_tokens"], ref["peak"])


def test_multiplan_build_errors():
    cfg = _cfg(layers=1)
    slab = B.quail_anchor_bytes(cfg, 100)
    with pytest.raises(B.QuailError) as e:      # an anchor larger than the pool
        B.quail_multiplan_build(cfg, slab - 1, 64, [100], [0, 1], [0], [5])
    assert e.value.status == B.E_NOMEM
    with pytest.raises(B.QuailError) as e:      # anchor index out of range in the second join
        B.quail_multiplan_build(cfg, slab, 64, [100], [0, 1, 2], [0, 1], [5, 5])
    assert e.value.status == B.E_INVAL
    with pytest.raises(B.QuailError) as e:      # decreasing join offsets
        B.quail_multiplan_build(cfg, slab, 64, [100], [0, 2, 1], [0, 0], [5, 5])
    assert e.value.status == B.E_INVAL
    got = B.quail_multiplan_build(cfg, slab, 64, [100], [0, 0, 0], [], [])   # two empty joins
    assert got["steps"] == [] and got["prefills"] == 0


def test_plan_build_errors():
    cfg = _cfg(layers=1)
    slab = B.quail_anchor_bytes(cfg, 100)
    with pytest.raises(B.QuailError) as e:
        B.quail_plan_build(cfg, slab - 1, 64, [100], [0], [5])
    assert e.value.status == B.E_NOMEM
    with pytest.raises(B.QuailError) as e:
        B.quail_plan_build(cfg, slab, 64, [100], [0], [65])
    assert e.value.status == B.E_INVAL
    with pytest.raises(B.QuailError) as e:
        B.quail_plan_build(cfg, slab, 64, [100], [1], [5])
    assert e.value.status == B.E_INVAL


def test_config_validation():
    lib = B.load()
    out = C.c_size_t()
    bad = _cfg(head_dim=64)
    assert lib.quail_workspace_bytes(C.byref(bad), 16, C.byref(out)) == B.E_UNSUPPORTED
    bad = _cfg(n_q_heads=24)     # group size 3
    assert lib.quail_workspace_bytes(C.byref(bad), 16, C.byref(out)) == B.E_UNSUPPORTED
    bad = _cfg(hidden=2500)
    assert lib.quail_workspace_bytes(C.byref(bad), 16, C.byref(out)) == B.E_UNSUPPORTED
    bad = _cfg(n_layers=0)
    assert lib.quail_workspace_bytes(C.byref(bad), 16, C.byref(out)) == B.E_INVAL
    assert b"positive" in lib.quail_last_error()


class _FakeCtx:
    """A context over fake (never dereferenced) device addresses: every call
    below must fail in host validation before touching the GPU."""

    def __init__(self, pool_bytes, layers=2, mbt=256):
        self.lib = B.load()
        self.cfg = _cfg(layers=layers, n_kv_heads=2, n_q_heads=4, hidden=256, intermediate=384,
                        max_anchor_len=512, max_suffix_len=128)
        fake = 0x7F0000000000
        self.lw = (B.LayerWeights * layers)()
        for i in range(layers):
            for f, _ in B.LayerWeights._fields_:
                setattr(self.lw[i], f, fake)
        self.w = B.Weights(embed=fake, layers=C.cast(self.lw, C.POINTER(B.LayerWeights)),
                           final_norm=fake, head8=fake)
        ws = B.quail_workspace_bytes(self.cfg, mbt)
        h = C.c_void_p()
        st = self.lib.quail_ctx_create(C.byref(self.cfg), C.byref(self.w), fake, pool_bytes, fake, ws,
                                       mbt, C.byref(h))
        assert st == 0, self.lib.quail_last_error()
        self.h = h

    def close(self):
        self.lib.quail_ctx_destroy(self.h)


def _i32(a):
    a = np.ascontiguousarray(a, np.int32)
    return a, a.ctypes.data_as(C.POINTER(C.c_int32))


def _i64(a):
    a = np.ascontiguousarray(a, np.int64)
    return a, a.ctypes.data_as(C.POINTER(C.c_int64))


def test_anchor_prefill_pool_too_small_is_nomem_and_keeps_nothing():
    cfg_slab = _slab(100, 2, 2, 128, 2)
    fc = _FakeCtx(pool_bytes=cfg_slab + cfg_slab // 2)
    off, offp = _i32([0, 100, 200])
    nu, nup = _i32([3, 4])
    out, outp = _i64([0, 0])
    st = fc.lib.quail_anchor_prefill(fc.h, 2, 0x7F0000000000, offp, nup, None, outp, None)
    assert st == B.E_NOMEM
    r, p = C.c_size_t(), C.c_size_t()
    pf, ev, rg = C.c_int64(), C.c_int64(), C.c_int64()
    fc.lib.quail_pool_stats(fc.h, C.byref(r), C.byref(p), C.byref(pf), C.byref(ev), C.byref(rg))
    assert r.value == 0 and pf.value == 0
    fc.close()


def test_anchor_prefill_rejects_bad_offsets():
    fc = _FakeCtx(pool_bytes=1 << 26)
    nu, nup = _i32([1, 1])
    out, outp = _i64([0, 0])
    for offs in ([0, 10, 5], [0, 0, 10], [0, 10, 10 + 513], [-1, 5, 10]):
        off, offp = _i32(offs)
        st = fc.lib.quail_anchor_prefill(fc.h, 2, 0x7F0000000000, offp, nup, None, outp, None)
        assert st == B.E_INVAL, offs
    fc.close()


def test_join_with_stale_handle_is_stale():
    fc = _FakeCtx(pool_bytes=1 << 26)
    for h in (5, (3 << 32) | 0, 0):
        ha, hap = _i64([h])
        off, offp = _i32([0, 4])
        st = fc.lib.quail_join_prefill(fc.h, 1, hap, 0x7F0000000000, offp, 0x7F0000000000, None, None)
        assert st == B.E_STALE
        assert fc.lib.quail_anchor_release(fc.h, h) == B.E_STALE
    fc.close()


def test_join_rejects_bad_suffix_lengths():
    fc = _FakeCtx(pool_bytes=1 << 26)
    ha, hap = _i64([B.NO_ANCHOR, B.NO_ANCHOR])
    for offs in ([0, 0, 4], [0, 129, 130], [0, 4, 2]):
        off, offp = _i32(offs)
        st = fc.lib.quail_join_prefill(fc.h, 2, hap, 0x7F0000000000, offp, 0x7F0000000000, None, None)
        assert st == B.E_INVAL, offs
    fc.close()


def test_multijoin_run_rejects_bad_arguments_before_any_gpu_work():
    fc = _FakeCtx(pool_bytes=1 << 26)
    fake = 0x7F0000000000
    ao, aop = _i32([0, 10])
    so, sop = _i32([0, 4, 8])
    cases = [
        ([0, 2, 1], [0, 0]),          # decreasing join offsets
        ([1, 2], [0, 0]),             # first offset not 0
        ([0, 1, 2], [0, 1]),          # anchor index out of range in the second join
        ([0, 1, 2], [0, -2]),         # anchor index below -1
    ]
    for jo_, pa_ in cases:
        jo, jop = _i32(jo_)
        pa, pap = _i32(pa_)
        st = fc.lib.quail_multijoin_run(fc.h, 1, fake, aop, len(jo_) - 1, jop, pap, fake, sop, 0x0F,
                                        None, None, fake, None)
        assert st == B.E_INVAL, (jo_, pa_)
    jo, jop = _i32([0, 2])
    pa, pap = _i32([0, 0])
    bad_so, bad_sop = _i32([0, 4, 4 + 129])        # a suffix longer than max_suffix_len
    st = fc.lib.quail_multijoin_run(fc.h, 1, fake, aop, 1, jop, pap, fake, bad_sop, 0x0F, None, None, fake,
                                    None)
    assert st == B.E_INVAL
    # nothing was prefilled
    r, p = C.c_size_t(), C.c_size_t()
    pf, ev, rg = C.c_int64(), C.c_int64(), C.c_int64()
    fc.lib.quail_pool_stats(fc.h, C.byref(r), C.byref(p), C.byref(pf), C.byref(ev), C.byref(rg))
    assert r.value == 0 and pf.value == 0
    fc.close()


def test_cascade_attn_argument_checks():
    lib = B.load()
    so, sop = _i32([0, 4])
    sa, sap = _i32([0])
    ao, aop = _i32([0, 8])
    ws = C.c_size_t()
    assert lib.quail_cascade_workspace_bytes(1, aop, 1, sop, C.byref(ws)) == 0
    fake = 0x7F0000000000
    # head_dim 64 is fp32-only
    assert lib.quail_cascade_attn(B.DTYPE_BF16, 4, 2, 64, 0.1, 1, fake, fake, aop, 1, sap, fake, fake,
                                  fake, sop, fake, None, fake, ws.value, None) == B.E_UNSUPPORTED
    # anchor index out of range
    sa2, sap2 = _i32([3])
    assert lib.quail_cascade_attn(B.DTYPE_BF16, 4, 2, 128, 0.1, 1, fake, fake, aop, 1, sap2, fake, fake,
                                  fake, sop, fake, None, fake, ws.value, None) == B.E_INVAL
    # workspace too small
    assert lib.quail_cascade_attn(B.DTYPE_BF16, 4, 2, 128, 0.1, 1, fake, fake, aop, 1, sap, fake, fake,
                                  fake, sop, fake, None, fake, 16, None) == B.E_NOMEM


def _prefix_cases():
    from tests.test_oracle_prefix import _cases
    return list(_cases())


@pytest.mark.parametrize("case", _prefix_cases())
def test_prefix_groups_match_oracle(case):
    """The library's radix grouping (sorted order + adjacent LCPs) equals the
    oracle's (hash of the first min_len tokens + token-by-token LCP)."""
    from oracle import prefix as OPX
    seqs, keys, m = case
    off = np.zeros(len(seqs) + 1, np.int32)
    off[1:] = np.cumsum([len(s) for s in seqs])
    toks = np.array([t for s in seqs for t in s], np.int32)
    g, f, ln = B.quail_prefix_groups(toks, off, keys, m)
    rg, rf, rl = OPX.prefix_groups_reference(seqs, keys, m)
    assert np.array_equal(g, rg) and np.array_equal(f, rf) and np.array_equal(ln, rl)


def test_prefix_groups_argument_checks():
    lib = B.load()
    toks, tp = _i32([1, 2, 3, 4])
    g, gp = _i32([0, 0])
    nn = C.c_int32(7)
    off, offp = _i32([0, 2, 4])
    assert lib.quail_prefix_groups(2, tp, offp, None, 0, gp, gp, gp, C.byref(nn)) == B.E_INVAL
    assert lib.quail_prefix_groups(2, tp, offp, None, 1, None, gp, gp, C.byref(nn)) == B.E_INVAL
    for offs in ([0, 3, 2], [0, 0, 4], [-1, 2, 4]):
        off, offp = _i32(offs)
        assert lib.quail_prefix_groups(2, tp, offp, None, 1, gp, gp, gp, C.byref(nn)) == B.E_INVAL, offs
    assert lib.quail_prefix_groups(0, None, None, None, 1, None, None, None, C.byref(nn)) == B.OK
    assert nn.value == 0


def test_prefix_prefill_and_shared_run_reject_bad_arguments():
    fc = _FakeCtx(pool_bytes=1 << 26)
    nu, nup = _i32([1])
    out, outp = _i64([0])
    off, offp = _i32([0, 4])
    for h in (5, (3 << 32) | 0, B.NO_ANCHOR):       # no live anchor behind these handles
        pa, pap = _i64([h])
        st = fc.lib.quail_prefix_prefill(fc.h, 1, pap, 0x7F0000000000, offp, nup, outp, None)
        assert st == B.E_STALE, h
    pa, pap = _i64([0])
    assert fc.lib.quail_prefix_prefill(fc.h, 1, None, 0x7F0000000000, offp, nup, outp, None) == B.E_INVAL
    off0, off0p = _i32([0, 0])
    assert fc.lib.quail_prefix_prefill(fc.h, 1, pap, 0x7F0000000000, off0p, nup, outp, None) == B.E_INVAL
    ao, aop = _i32([0, 8])
    pa1, pa1p = _i32([0])
    so, sop = _i32([0, 4])
    sh, shp = _i32([1, 2, 3, 4])
    dec = 0x7F0000000000
    st = fc.lib.quail_join_run_shared(fc.h, 1, dec, aop, 1, pa1p, dec, sop, shp, 0, 0, 0x0F, None, None, dec, None)
    assert st == B.E_INVAL
    st = fc.lib.quail_join_run_shared(fc.h, 1, dec, aop, 1, pa1p, dec, sop, None, 2, 1, 0x0F, None, None, dec, None)
    assert st == B.E_INVAL
    fc.close()


@pytest.mark.parametrize("seed", range(30))
def test_join_search_matches_brute_force(seed):
    """The library's subset DP with Pareto pruning returns the frontier and the
    least-time plan that enumerating every plan finds."""
    from oracle import joinorder as OJ
    from tests.test_oracle_joinorder import QWEN, random_query
    tables, joins = random_query(seed)
    res = B.quail_join_search(_cfg(max_anchor_len=512), tables, joins, 2.5166e15, 8e12)
    ref = OJ.search_reference(tables, joins, QWEN, 2.5166e15, 8e12)
    assert res["n_frontier"] == len(ref["frontier"])
    got = np.array(sorted(map(tuple, res["frontier"])))
    want = np.array(sorted(ref["frontier"]))
    assert np.allclose(got, want, rtol=1e-9, atol=0)
    assert abs(res["metrics"][3] - ref["best_seconds"]) <= 1e-9 * ref["best_seconds"]
    replay = OJ.plan_metrics(list(res["order"]), list(res["anchor_right"]), tables, joins, QWEN)
    assert replay is not None and np.allclose(replay, res["metrics"][:3], rtol=1e-9, atol=0)


def test_join_search_argument_checks():
    cfg = _cfg()
    good = [(10, 5.0), (20, 5.0), (30, 5.0)]
    with pytest.raises(B.QuailError):             # a cycle, and one join too many
        B.quail_join_search(cfg, good, [(0, 1, 0, 0, 0.5, 0), (1, 2, 0, 0, 0.5, 0), (2, 0, 0, 0, 0.5, 0)], 1e15, 8e12)
    for joins in ([(0, 1, 0, 0, 0.5, 0)],                               # too few joins
                  [(0, 1, 0, 0, 0.0, 0), (1, 2, 0, 0, 0.5, 0)],          # selectivity 0
                  [(0, 1, 0, 0, 1.5, 0), (1, 2, 0, 0, 0.5, 0)],          # selectivity > 1
                  [(0, 0, 0, 0, 0.5, 0), (1, 2, 0, 0, 0.5, 0)],          # self join
                  [(0, 3, 0, 0, 0.5, 0), (1, 2, 0, 0, 0.5, 0)],          # table out of range
                  [(0, 1, 0, 0, 0.5, 0), (0, 1, 0, 0, 0.5, 0)]):         # not spanning
        with pytest.raises(B.QuailError) as e:
            B.quail_join_search(cfg, good, joins, 1e15, 8e12)
        assert e.value.status == B.E_INVAL, joins
    with pytest.raises(B.QuailError):
        B.quail_join_search(cfg, good, [(0, 1, 0, 0, 0.5, 0), (1, 2, 0, 0, 0.5, 0)], 0.0, 8e12)
    with pytest.raises(B.QuailError):
        B.quail_join_search(cfg, [(0, 5.0)], [], 1e15, 8e12)
    with pytest.raises(B.QuailError):
        B.quail_join_search(cfg, [(1, 1.0)] * 13, [(i, i + 1, 0, 0, 0.5, 0) for i in range(12)], 1e15, 8e12)
    one = B.quail_join_search(cfg, [(7, 3.0)], [], 1e15, 8e12)
    assert list(one["order"]) == [0] and one["n_frontier"] == 1 and one["metrics"][0] == 0


@pytest.mark.parametrize("m", [1, 2, 3])
@pytest.mark.parametrize("case", _prefix_cases())
def test_prefix_tree_matches_oracle(case, m):
    """Nested radix grouping: library (recursive split of sorted members) equals
    the oracle's, nodes, numbering and deepest node of every sequence."""
    from oracle import prefix as OPX
    seqs, keys, _ = case
    off = np.zeros(len(seqs) + 1, np.int32)
    off[1:] = np.cumsum([len(s) for s in seqs])
    toks = np.array([t for s in seqs for t in s], np.int32)
    g, nodes = B.quail_prefix_tree(toks, off, keys, m)
    rg, rnodes = OPX.prefix_tree_reference(seqs, keys, m)
    assert np.array_equal(g, rg) and nodes == rnodes


def test_prefix_tree_argument_checks():
    lib = B.load()
    toks, tp = _i32([1, 2, 3, 4])
    a, ap = _i32([0, 0])
    nn = C.c_int32(7)
    off, offp = _i32([0, 2, 4])
    assert lib.quail_prefix_tree(2, tp, offp, None, 0, ap, ap, ap, ap, ap, C.byref(nn)) == B.E_INVAL
    assert lib.quail_prefix_tree(2, tp, offp, None, 1, ap, None, ap, ap, ap, C.byref(nn)) == B.E_INVAL
    assert lib.quail_prefix_tree(2, tp, offp, None, 1, ap, ap, ap, ap, ap, None) == B.E_INVAL
    for offs in ([0, 3, 2], [0, 0, 4]):
        off, offp = _i32(offs)
        assert lib.quail_prefix_tree(2, tp, offp, None, 1, ap, ap, ap, ap, ap, C.byref(nn)) == B.E_INVAL, offs
    assert lib.quail_prefix_tree(0, None, None, None, 1, None, None, None, None, None, C.byref(nn)) == B.OK
    assert nn.value == 0


def test_join_search_frontier_buffer():
    """The frontier output is optional with cap 0, truncated to cap, and
    rejected as NULL with cap > 0; n_frontier always gives the full size."""
    cfg = _cfg()
    tables = [(64, 1024.0), (2048, 64.0), (300, 200.0)]
    joins = [(0, 1, 4.0, 2.0, 0.25, 1), (1, 2, 3.0, 1.0, 0.5, 1)]
    full = B.quail_join_search(cfg, tables, joins, 2.5e15, 8e12)
    assert full["n_frontier"] >= 1
    one = B.quail_join_search(cfg, tables, joins, 2.5e15, 8e12, cap=1)
    assert one["n_frontier"] == full["n_frontier"] and len(one["frontier"]) == 1
    assert np.array_equal(one["frontier"][0], full["frontier"][0])
    lib = B.load()
    ta = (B.Table * 3)(*[B.Table(r, t) for r, t in tables])
    ja = (B.AIJoin * 2)(*[B.AIJoin(*j) for j in joins])
    order, op = _i32([0, 0, 0])
    ar, arp = _i32([0, 0])
    met = np.zeros(4)
    nf = C.c_int32()
    f64p = C.POINTER(C.c_double)
    st = lib.quail_join_search(C.byref(cfg), 3, ta, 2, ja, 2.5e15, 8e12, op, arp, met.ctypes.data_as(f64p),
                               None, 4, C.byref(nf))
    assert st == B.E_INVAL
    st = lib.quail_join_search(C.byref(cfg), 3, ta, 2, ja, 2.5e15, 8e12, op, arp, met.ctypes.data_as(f64p),
                               None, 0, C.byref(nf))
    assert st == B.OK and nf.value == full["n_frontier"]


def test_noalloc_cascade_rejects_metadata_beyond_its_scratch():
    """The allocation-free cascade entry point refuses, before any GPU work, a
    call whose metadata exceeds its 16 MiB scratch array (here 5 M query
    tokens: 20 MB of per-token segments alone)."""
    lib = B.load()
    fake = 0x7F0000000000
    so, sop = _i32([0, 5_000_000])
    sa, sap = _i32([-1])
    st = lib.quail_cascade_attn_noalloc(B.DTYPE_BF16, 32, 8, 128, 0.088, 0, None, None, None, 1, sap, fake,
                                        fake, fake, sop, fake, None, None)
    assert st == B.E_NOMEM
    assert b"16777216" in lib.quail_last_error()


def test_w8a8_argument_checks():
    """Shape, alignment and NULL checks of the W8A8 calls return before any
    GPU work (no device is touched)."""
    lib = B.load()
    fake = 0x7F0000000000
    assert lib.quail_act_quant_e4m3(4, 12, fake, fake, fake, None) == B.E_UNSUPPORTED      # K % 8
    assert lib.quail_act_quant_e4m3(-1, 8, fake, fake, fake, None) == B.E_INVAL
    assert lib.quail_act_quant_e4m3(4, 8, None, fake, fake, None) == B.E_INVAL
    assert lib.quail_act_quant_e4m3(4, 8, fake + 8, fake, fake, None) == B.E_UNSUPPORTED   # x alignment
    assert lib.quail_act_quant_e4m3(0, 8, None, None, None, None) == B.OK
    assert lib.quail_gemm_w8a8(4, 256, 192, fake, fake, fake, fake, fake, None) == B.E_UNSUPPORTED  # K % 128
    assert lib.quail_gemm_w8a8(4, 128, 128, fake, fake, fake, fake, fake, None) == B.E_UNSUPPORTED  # N % 256
    assert lib.quail_gemm_w8a8(4, 256, 128, fake, fake, None, fake, fake, None) == B.E_INVAL
    assert lib.quail_gemm_w8a8(4, 256, 128, fake, fake, fake, fake + 4, fake, None) == B.E_UNSUPPORTED
    assert lib.quail_gemm_w8a8(0, 256, 128, None, None, None, None, None, None) == B.OK


def test_act_dtype_validation_and_workspace():
    """act_dtype: 0 and BF16 are W8A16, FP8_E4M3 is W8A8 (needs hidden % 256,
    intermediate % 128 and even n_q_heads); W8A8 workspaces add the codes of
    the widest projection input and one scale per token."""
    lib = B.load()
    out = C.c_size_t()
    base = {}
    for a in (0, B.DTYPE_BF16):
        cfg = _cfg(act_dtype=a)
        assert lib.quail_workspace_bytes(C.byref(cfg), 64, C.byref(out)) == B.OK
        base[a] = out.value
    assert base[0] == base[B.DTYPE_BF16]
    cfg = _cfg(act_dtype=B.DTYPE_FP8_E4M3)
    assert lib.quail_workspace_bytes(C.byref(cfg), 64, C.byref(out)) == B.OK
    assert out.value >= base[0] + 64 * 9728 + 64 * 4
    for bad in (_cfg(act_dtype=3), _cfg(act_dtype=B.DTYPE_FP8_E4M3, hidden=2560 + 128),
                _cfg(act_dtype=B.DTYPE_FP8_E4M3, intermediate=9728 + 64),
                _cfg(act_dtype=B.DTYPE_FP8_E4M3, n_q_heads=1, n_kv_heads=1)):
        assert lib.quail_workspace_bytes(C.byref(bad), 64, C.byref(out)) == B.E_UNSUPPORTED
