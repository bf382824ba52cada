"""GPU parity of the two-level cascade (anchor -> shared suffix prefix ->
suffix) against the oracle's per-pair monolithic forward: prefix-node
prefill (slab contents), joins through node handles (packed and unpacked
attention tiles, bf16 and E4M3 stores, unit and non-unit scales), residency
of nodes and their anchors, handle errors, and the whole-join entry point
with sharing against the one without."""
import numpy as np
import pytest

import workloads as W
from oracle import model as OM, prefix as OPX
from tests.gpu_util import bf16_f64, decisions_agree, rel_inf, say, u16
from tests.test_gpu_model import _fp8_codes_valid, _slab

pytestmark = pytest.mark.gpu

FAMILIES = [(1, 40, [5, 1, 33]), (2, 64, [17, 2]), (0, 3, [1, 4, 2]), (1, 2, [6]), (-1, 5, [3, 4]),
            (2, 9, [3, 2])]


@pytest.fixture(scope="module")
def B():
    import torch
    assert torch.cuda.is_available()
    from query_aware_prefill_amd import binding
    binding.load()
    return binding


def _pack(tok, ranges):
    off = np.zeros(len(ranges) + 1, np.int32)
    off[1:] = np.cumsum([b - a for a, b in ranges])
    return np.concatenate([tok[a:b] for a, b in ranges]).astype(np.int32), off


def shared_keys(case):
    """Grouping keys of the shared run: the anchor, or one key of their own
    for filter rows (their shared prefix becomes a plain anchor)."""
    pa = np.asarray(case["pair_anchor"])
    return np.where(pa >= 0, pa, len(case["a_len"])).astype(np.int32)


def shared_step_lengths(B, case, min_shared):
    """Tokens each pair computes with sharing, as the shared run sizes its
    plan steps: own tokens after the shared prefix + its share of the prefix."""
    g, _, nl = B.quail_prefix_groups(case["s_tok"], case["s_off"], shared_keys(case), min_shared)
    s_len = np.diff(case["s_off"]).astype(np.int64)
    out = s_len.copy()
    for k in range(len(nl)):
        m = np.flatnonzero(g == k)
        out[m] = s_len[m] - nl[k] + (nl[k] + len(m) - 1) // len(m)
    return out.astype(np.int32)


@pytest.mark.parametrize("kv_fp8,k_scale,v_scale", [(False, 1.0, 1.0), (True, 1.0, 1.0), (True, 0.5, 2.0)])
def test_two_level_cascade_model(B, kv_fp8, k_scale, v_scale):
    import torch
    from query_aware_prefill_amd.device import DeviceModel, to_device
    shape = W.tiny_shape(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=128,
                         intermediate=384, vocab=512, kv_fp8=kv_fp8, k_scale=k_scale, v_scale=v_scale)
    wts = W.model_weights(shape, 7)
    a_len = [1, 70, 130]
    case = W.shared_prefix_case(7, shape.vocab, a_len, FAMILIES)
    s_tok, s_off, pa = case["s_tok"], case["s_off"], case["pair_anchor"]
    n = len(pa)
    g, nfirst, nlen = B.quail_prefix_groups(s_tok, s_off, pa, 2)
    seqs = [s_tok[s_off[i]:s_off[i + 1]] for i in range(n)]
    rg, rf, rl = OPX.prefix_groups_reference(seqs, pa, 2)
    assert np.array_equal(g, rg) and np.array_equal(nfirst, rf) and np.array_equal(nlen, rl)
    nn = len(nfirst)
    assert nn == 4      # families 0, 1, 2, 5; the lone pair and the filter rows stay ungrouped
    node_anchor = pa[nfirst]
    uses = np.zeros(3, np.int32)
    for i in range(n):
        if pa[i] >= 0 and g[i] < 0:
            uses[pa[i]] += 1
    for a in node_anchor:
        uses[a] += 1
    dm = DeviceModel(shape, wts, max_anchor_len=1024, max_suffix_len=256)
    pool_bytes = sum(B.quail_anchor_bytes(dm.cfg, x) for x in a_len) + \
        sum(B.quail_anchor_bytes(dm.cfg, int(x)) for x in nlen) + 4096
    ctx = dm.context(pool_bytes, 512)
    say("two-level: anchor prefill", "fp8" if kv_fp8 else "bf16", k_scale, v_scale)
    handles = B.quail_anchor_prefill(ctx, to_device(case["a_tok"]), case["a_off"], uses)
    # nodes: the short ones (packed tiles) and the rest, in two calls
    node_tok, node_off = _pack(s_tok, [(s_off[f], s_off[f] + L) for f, L in zip(nfirst, nlen)])
    members = np.array([np.sum(g == k) for k in range(nn)], np.int32)
    nh = np.zeros(nn, np.int64)
    for sel in (nlen <= 16, nlen > 16):
        idx = np.flatnonzero(sel)
        if len(idx) == 0:
            continue
        tk, of = _pack(node_tok, [(node_off[k], node_off[k + 1]) for k in idx])
        say("two-level: prefix prefill", idx.tolist())
        nh[idx] = B.quail_prefix_prefill(ctx, handles[node_anchor[idx]], to_device(tk), of, members[idx])
    torch.cuda.synchronize()
    # node slabs hold the K/V of positions La.. of the monolithic run
    for k in range(nn):
        a = int(node_anchor[k])
        at = case["a_tok"][case["a_off"][a]:case["a_off"][a + 1]]
        toks = np.concatenate([at, node_tok[node_off[k]:node_off[k + 1]]])
        _, kv = OM.forward_tokens(toks, wts, shape, return_kv=True, fp8_kv_upto=len(toks) if kv_fp8 else 0)
        for l in range(shape.n_layers):
            kk, vv = _slab(ctx, nh[k], l, B, shape)
            la = len(at)
            if not kv_fp8:
                assert rel_inf(kk, kv[l][0][la:]) <= 2e-2, (k, l, "K")
                assert rel_inf(vv, kv[l][1][la:]) <= 2e-2, (k, l, "V")
            else:
                for got, stored, pre in ((kk, kv[l][0][la:], kv[l][2][la:]), (vv, kv[l][1][la:], kv[l][3][la:])):
                    _fp8_codes_valid(got, stored, pre)
    # an anchor with live nodes cannot be released; an anchor whose declared
    # uses are all held cannot take another node
    with pytest.raises(B.QuailError) as e:
        B.quail_anchor_release(ctx, handles[1])
    assert e.value.status == B.E_INVAL
    with pytest.raises(B.QuailError) as e:
        B.quail_prefix_prefill(ctx, [handles[0]], to_device(node_tok[:4]), [0, 4], [1])
    assert e.value.status == B.E_STALE
    # joins: the members of the short nodes (few tokens per node: packed
    # tiles), then everything else (node members and ungrouped pairs)
    order_a = [i for i in range(n) if g[i] >= 0 and nlen[g[i]] <= 16 and
               sum(s_off[j + 1] - s_off[j] - nlen[g[j]] for j in range(n) if g[j] == g[i]) <= 16]
    order_b = [i for i in range(n) if i not in order_a]
    h_last = torch.empty((n, shape.hidden), dtype=torch.int16, device="cuda")
    for part in (order_a, order_b):
        if not part:
            continue
        rng = [(s_off[i] + (nlen[g[i]] if g[i] >= 0 else 0), s_off[i + 1]) for i in part]
        tk, of = _pack(s_tok, rng)
        hp = [nh[g[i]] if g[i] >= 0 else (handles[pa[i]] if pa[i] >= 0 else B.NO_ANCHOR) for i in part]
        hl = torch.empty((len(part), shape.hidden), dtype=torch.int16, device="cuda")
        say("two-level: join", len(part), "pairs")
        B.quail_join_prefill(ctx, hp, to_device(tk), of, hl)
        h_last[torch.tensor(part, device="cuda")] = hl
    assert len(order_a) >= 2
    logits = torch.empty((n, 8), dtype=torch.float32, device="cuda")
    tok = torch.empty(n, dtype=torch.uint8, device="cuda")
    dec = torch.empty(n, dtype=torch.uint8, device="cuda")
    B.quail_head8(ctx, h_last, 0x0F, logits, tok, dec)
    torch.cuda.synchronize()
    hl = bf16_f64(u16(h_last))
    ref_logits, ref_dec, ref_margin = [], [], []
    for i in range(n):
        a = int(pa[i])
        at = case["a_tok"][case["a_off"][a]:case["a_off"][a + 1]] if a >= 0 else []
        ref = OM.forward_pair(at, seqs[i], wts, shape, true_mask=0x0F,
                              shared_len=int(nlen[g[i]]) if g[i] >= 0 else 0)
        assert rel_inf(hl[i], ref["h_last"]) <= 2e-2, (i, rel_inf(hl[i], ref["h_last"]))
        ref_logits.append(ref["logits"]); ref_dec.append(ref["decision"]); ref_margin.append(ref["margin"])
    ref_logits = np.array(ref_logits)
    assert rel_inf(logits.cpu().numpy(), ref_logits) <= 2e-2
    ok, _ = decisions_agree(dec.cpu().numpy(), ref_dec, ref_margin, 2e-2 * np.max(np.abs(ref_logits)))
    assert ok
    st = B.quail_pool_stats(ctx)
    assert st["prefills"] == 3 + nn and st["evictions"] == 3 + nn and st["resident"] == 0
    with pytest.raises(B.QuailError) as e:
        B.quail_join_prefill(ctx, [nh[0]], to_device(node_tok[:2]), [0, 2], h_last[:1])
    assert e.value.status == B.E_STALE


def test_join_run_shared_matches_join_run(B):
    """Whole join with and without sharing on the same inputs: the same
    logits up to rounding, the oracle's decisions, node prefills counted, no
    regret, nothing left resident."""
    import torch
    from query_aware_prefill_amd.device import DeviceModel, to_device
    shape = W.tiny_shape(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=128,
                         intermediate=384, vocab=512)
    wts = W.model_weights(shape, 9)
    r = np.random.default_rng(9)
    a_len = r.integers(20, 120, 4).tolist()
    fam = []
    for f in range(10):
        fam.append((int(r.integers(0, 4)), int(r.integers(1, 50)),
                    r.integers(1, 20, int(r.integers(1, 5))).tolist()))
    fam.append((-1, 6, [5, 7]))
    case = W.shared_prefix_case(9, shape.vocab, a_len, fam)
    n = len(case["pair_anchor"])
    dm = DeviceModel(shape, wts, max_anchor_len=1024, max_suffix_len=256)
    ctx = dm.context(64 << 20, 128)           # small batches: several plan steps
    a_tok, s_tok = to_device(case["a_tok"]), to_device(case["s_tok"])
    outs = []
    for shared in (False, True):
        logits = torch.empty((n, 8), dtype=torch.float32, device="cuda")
        dec = torch.empty(n, dtype=torch.uint8, device="cuda")
        say("join_run", "shared" if shared else "plain", n, "pairs")
        if shared:
            B.quail_join_run_shared(ctx, a_tok, case["a_off"], case["pair_anchor"], s_tok, case["s_off"],
                                    case["s_tok"], 4, 0x0F, logits, None, dec)
        else:
            B.quail_join_run(ctx, a_tok, case["a_off"], case["pair_anchor"], s_tok, case["s_off"], 0x0F,
                             logits, None, dec)
        torch.cuda.synchronize()
        outs.append((logits.cpu().numpy(), dec.cpu().numpy(), B.quail_pool_stats(ctx)))
    (l0, d0, s0), (l1, d1, s1) = outs
    assert rel_inf(l1, l0) <= 2e-2
    used = len({a for a in case["pair_anchor"] if a >= 0})
    assert s0["prefills"] == used and s0["regret_tokens"] == 0
    # nodes: the oracle's grouping of each plan step's pairs (plan from the
    # library's builder, pool fully free as at the shared run's start)
    # the shared run plans against the pool less the slab of its longest possible prefix node
    reserve = B.quail_anchor_bytes(dm.cfg, int(np.max(case["s_len"])))
    order, bounds, _ = B.quail_plan_build(dm.cfg, (64 << 20) - reserve, 128, a_len, case["pair_anchor"],
                                          shared_step_lengths(B, case, 4))
    expect = 0
    for b0, b1 in zip(bounds[:-1], bounds[1:]):
        idx = order[b0:b1]
        seqs = [case["s_tok"][case["s_off"][i]:case["s_off"][i + 1]] for i in idx]
        expect += len(OPX.prefix_groups_reference(seqs, shared_keys(case)[idx], 4)[1])
    nodes = s1["prefills"] - s0["prefills"] - used
    assert nodes == expect and nodes >= 4, (nodes, expect)
    assert s1["evictions"] == s1["prefills"] and s1["resident"] == 0 and s1["regret_tokens"] == 0
    ref_logits, ref_dec, ref_margin = [], [], []
    for i in range(n):
        a = int(case["pair_anchor"][i])
        at = case["a_tok"][case["a_off"][a]:case["a_off"][a + 1]] if a >= 0 else []
        ref = OM.forward_pair(at, case["s_tok"][case["s_off"][i]:case["s_off"][i + 1]], wts, shape)
        ref_logits.append(ref["logits"]); ref_dec.append(ref["decision"]); ref_margin.append(ref["margin"])
    ref_logits = np.array(ref_logits)
    assert rel_inf(l1, ref_logits) <= 2e-2
    ok, _ = decisions_agree(d1, ref_dec, ref_margin, 2e-2 * np.max(np.abs(ref_logits)))
    assert ok


def test_join_run_shared_under_a_tight_pool(B):
    """A pool that holds the anchors and one prefix node at a time: nodes are
    prefilled one per chunk and evicted after their members; the results
    equal the plain run's and the oracle's."""
    import torch
    from query_aware_prefill_amd.device import DeviceModel, to_device
    shape = W.tiny_shape(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=128,
                         intermediate=384, vocab=512)
    wts = W.model_weights(shape, 12)
    a_len = [60, 90]
    fam = [(0, 40, [3, 4, 5]), (0, 30, [2, 6]), (1, 50, [4, 4, 4, 4]), (1, 20, [7, 9])]
    case = W.shared_prefix_case(12, shape.vocab, a_len, fam)
    n = len(case["pair_anchor"])
    dm = DeviceModel(shape, wts, max_anchor_len=1024, max_suffix_len=256)
    slab64 = B.quail_anchor_bytes(dm.cfg, 64)
    tight = B.quail_anchor_bytes(dm.cfg, 60) + B.quail_anchor_bytes(dm.cfg, 90) + 2 * slab64 + 4096
    a_tok, s_tok = to_device(case["a_tok"]), to_device(case["s_tok"])
    res = []
    for shared, pool in ((True, tight), (False, 64 << 20)):
        ctx = dm.context(pool, 512)
        logits = torch.empty((n, 8), dtype=torch.float32, device="cuda")
        dec = torch.empty(n, dtype=torch.uint8, device="cuda")
        say("join_run tight pool", "shared" if shared else "plain")
        if shared:
            B.quail_join_run_shared(ctx, a_tok, case["a_off"], case["pair_anchor"], s_tok, case["s_off"],
                                    case["s_tok"], 8, 0x0F, logits, None, dec)
        else:
            B.quail_join_run(ctx, a_tok, case["a_off"], case["pair_anchor"], s_tok, case["s_off"], 0x0F,
                             logits, None, dec)
        torch.cuda.synchronize()
        res.append((logits.cpu().numpy(), dec.cpu().numpy(), B.quail_pool_stats(ctx)))
    (l1, d1, st1), (l0, d0, _) = res
    assert st1["prefills"] == 2 + 4 and st1["evictions"] == 6 and st1["resident"] == 0
    assert st1["peak"] <= tight
    assert rel_inf(l1, l0) <= 2e-2
    ref = [OM.forward_pair(case["a_tok"][case["a_off"][a]:case["a_off"][a + 1]],
                           case["s_tok"][case["s_off"][i]:case["s_off"][i + 1]], wts, shape)
           for i, a in enumerate(case["pair_anchor"])]
    ref_logits = np.array([r["logits"] for r in ref])
    assert rel_inf(l1, ref_logits) <= 2e-2
    ok, _ = decisions_agree(d1, [r["decision"] for r in ref], [r["margin"] for r in ref],
                            2e-2 * np.max(np.abs(ref_logits)))
    assert ok


def test_qwen3_shaped_layer_through_prefix_nodes(B):
    """One decoder layer with the Qwen3-4B shapes (hidden 2560, 32q/8kv x 128,
    SwiGLU 9728, fp8 weights): 2 anchors x 1000 tokens, a 300-token prefix
    node under each, and members of 64 and 33 tokens after it; all positions
    of one member per anchor and the first node's slab against the oracle's
    monolithic layer over [anchor | node | member]."""
    import torch
    from query_aware_prefill_amd.device import DeviceModel, to_device
    shape = W.ModelShape(n_layers=1, hidden=2560, n_q_heads=32, n_kv_heads=8, head_dim=128,
                         intermediate=9728, vocab=4096)
    wts = W.model_weights(shape, 13)
    a_len = [1000, 1000]
    case = W.shared_prefix_case(13, shape.vocab, a_len, [(0, 300, [64, 33]), (1, 300, [33, 64])])
    s_tok, s_off = case["s_tok"], case["s_off"]
    g, nfirst, nlen = B.quail_prefix_groups(s_tok, s_off, case["pair_anchor"], 16)
    assert list(nlen) == [300, 300] and list(g) == [0, 0, 1, 1]
    dm = DeviceModel(shape, wts, max_anchor_len=1024, max_suffix_len=512)
    pool = 2 * B.quail_anchor_bytes(dm.cfg, 1000) + 2 * B.quail_anchor_bytes(dm.cfg, 300) + 4096
    ctx = dm.context(pool, 2048)
    say("qwen3 layer through prefix nodes: anchors")
    handles = B.quail_anchor_prefill(ctx, to_device(case["a_tok"]), case["a_off"], [1, 1])
    node_tok, node_off = _pack(s_tok, [(s_off[f], s_off[f] + L) for f, L in zip(nfirst, nlen)])
    say("qwen3 layer through prefix nodes: nodes")
    nh = B.quail_prefix_prefill(ctx, handles, to_device(node_tok), node_off, [2, 2])
    tails, toff = _pack(s_tok, [(s_off[i] + 300, s_off[i + 1]) for i in range(4)])
    T = int(toff[-1])
    h_last = torch.empty((4, shape.hidden), dtype=torch.int16, device="cuda")
    h_all = torch.empty((T, shape.hidden), dtype=torch.int16, device="cuda")
    k0, v0, la, lap = B.quail_anchor_kv(ctx, int(nh[0]), 0)
    node0 = _slab(ctx, nh[0], 0, B, shape)
    say("qwen3 layer through prefix nodes: join")
    B.quail_join_prefill(ctx, [nh[g[i]] for i in range(4)], to_device(tails), toff, h_last, h_all)
    torch.cuda.synchronize()
    ha = bf16_f64(u16(h_all))
    for i in (0, 3):                       # one member per anchor (the oracle layer is slow)
        a = int(case["pair_anchor"][i])
        at = case["a_tok"][case["a_off"][a]:case["a_off"][a + 1]]
        st = s_tok[s_off[i]:s_off[i + 1]]
        if i == 0:
            h, kv = OM.forward_tokens(np.concatenate([at, st]), wts, shape, return_kv=True)
            assert la == 300
            assert rel_inf(node0[0], kv[0][0][1000:1300]) <= 2e-2
            assert rel_inf(node0[1], kv[0][1][1000:1300]) <= 2e-2
        else:
            h = OM.forward_tokens(np.concatenate([at, st]), wts, shape)
        err = rel_inf(ha[toff[i]:toff[i + 1]], h[1300:])
        say("  member", i, "rel", err)
        assert err <= 2e-2
    st = B.quail_pool_stats(ctx)
    assert st["prefills"] == 4 and st["evictions"] == 4 and st["resident"] == 0


@pytest.mark.parametrize("kv_fp8", [False, True])
def test_filter_rows_sharing_a_prefix(B, kv_fp8):
    """Filter rows (no anchor) whose leading tokens repeat: each group's prefix
    is prefilled once as a plain anchor and the rows run their own tokens after
    it. Logits and decisions against the oracle's per-row forward (the shared
    positions stored like anchor KV: E4M3 with an fp8 store)."""
    import torch
    from query_aware_prefill_amd.device import DeviceModel, to_device
    shape = W.tiny_shape(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=128,
                         intermediate=384, vocab=512, kv_fp8=kv_fp8)
    wts = W.model_weights(shape, 14)
    fam = [(-1, 70, [3, 9, 1]), (-1, 12, [20, 2]), (-1, 5, [6]), (-1, 40, [1, 1, 30, 4])]
    case = W.shared_prefix_case(14, shape.vocab, [], fam)
    n = len(case["pair_anchor"])
    g, _, nl = B.quail_prefix_groups(case["s_tok"], case["s_off"], shared_keys(case), 8)
    assert len(nl) == 3
    dm = DeviceModel(shape, wts, max_anchor_len=1024, max_suffix_len=256)
    ctx = dm.context(16 << 20, 256)
    logits = torch.empty((n, 8), dtype=torch.float32, device="cuda")
    dec = torch.empty(n, dtype=torch.uint8, device="cuda")
    say("filter rows sharing prefixes", "fp8" if kv_fp8 else "bf16")
    B.quail_join_run_shared(ctx, to_device(np.zeros(1, np.int32)), case["a_off"], case["pair_anchor"],
                            to_device(case["s_tok"]), case["s_off"], case["s_tok"], 8, 0x0F, logits, None, dec)
    torch.cuda.synchronize()
    st = B.quail_pool_stats(ctx)
    assert st["prefills"] == 3 and st["evictions"] == 3 and st["resident"] == 0
    lg = logits.cpu().numpy()
    ref = [OM.forward_pair([], case["s_tok"][case["s_off"][i]:case["s_off"][i + 1]], wts, shape,
                           shared_len=int(nl[g[i]]) if g[i] >= 0 else 0) for i in range(n)]
    ref_logits = np.array([r["logits"] for r in ref])
    assert rel_inf(lg, ref_logits) <= 2e-2, rel_inf(lg, ref_logits)
    ok, _ = decisions_agree(dec.cpu().numpy(), [r["decision"] for r in ref], [r["margin"] for r in ref],
                            2e-2 * np.max(np.abs(ref_logits)))
    assert ok


def test_join_run_shared_rejects_a_pool_without_room_for_a_node(B):
    """A pool that holds the anchors but not one more slab: E_NOMEM before
    anything is enqueued, and nothing stays resident."""
    from query_aware_prefill_amd.device import DeviceModel, to_device
    shape = W.tiny_shape(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=128,
                         intermediate=384, vocab=512)
    wts = W.model_weights(shape, 16)
    case = W.shared_prefix_case(16, shape.vocab, [60], [(0, 40, [3, 4])])
    dm = DeviceModel(shape, wts, max_anchor_len=1024, max_suffix_len=256)
    ctx = dm.context(B.quail_anchor_bytes(dm.cfg, 60) + 4096, 512)
    import torch
    dec = torch.empty(2, dtype=torch.uint8, device="cuda")
    with pytest.raises(B.QuailError) as e:
        B.quail_join_run_shared(ctx, to_device(case["a_tok"]), case["a_off"], case["pair_anchor"],
                                to_device(case["s_tok"]), case["s_off"], case["s_tok"], 8, 0x0F, None, None, dec)
    assert e.value.status == B.E_NOMEM
    st = B.quail_pool_stats(ctx)
    assert st["prefills"] == 0 and st["resident"] == 0


@pytest.mark.parametrize("kv_fp8", [False, True])
def test_nested_prefix_nodes(B, kv_fp8):
    """anchor (70 tokens) -> node P (30 shared tokens) -> node N (20 more):
    N's slab starts with P's rows (copied) and continues at positions 100..;
    one join mixes a direct anchor pair, a member of P and two members of N.
    Logits against the oracle's per-pair forward, N's own rows against the
    oracle's K/V, residency through the chain."""
    import torch
    from query_aware_prefill_amd.device import DeviceModel, to_device
    shape = W.tiny_shape(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=128,
                         intermediate=384, vocab=512, kv_fp8=kv_fp8)
    wts = W.model_weights(shape, 17)
    r = np.random.default_rng(17)
    a_tok = r.integers(0, 512, 70).astype(np.int32)
    lvl1, lvl2 = r.integers(0, 512, 30).astype(np.int32), r.integers(0, 512, 20).astype(np.int32)
    own = [r.integers(0, 512, k).astype(np.int32) for k in (9, 5, 7, 1)]
    suffixes = [own[0], np.concatenate([lvl1, own[1]]), np.concatenate([lvl1, lvl2, own[2]]),
                np.concatenate([lvl1, lvl2, own[3]])]
    shared = [0, 30, 50, 50]
    dm = DeviceModel(shape, wts, max_anchor_len=1024, max_suffix_len=256)
    ctx = dm.context(8 << 20, 256)
    say("nested nodes: anchor, P, N", "fp8" if kv_fp8 else "bf16")
    ha = B.quail_anchor_prefill(ctx, to_device(a_tok), [0, 70], [3])       # direct pair, P, N
    hp = B.quail_prefix_prefill(ctx, ha, to_device(lvl1), [0, 30], [2])     # member of P, N
    hn = B.quail_prefix_prefill(ctx, hp, to_device(lvl2), [0, 20], [2])     # two members
    torch.cuda.synchronize()
    kp, vp = _slab(ctx, hp[0], 1, B, shape)
    kn, vn = _slab(ctx, hn[0], 1, B, shape)
    assert kn.shape[0] == 50 and np.array_equal(kn[:30], kp) and np.array_equal(vn[:30], vp)
    _, kv = OM.forward_tokens(np.concatenate([a_tok, lvl1, lvl2]), wts, shape, return_kv=True,
                              fp8_kv_upto=120 if kv_fp8 else 0)
    if not kv_fp8:
        assert rel_inf(kn[30:], kv[1][0][100:120]) <= 2e-2 and rel_inf(vn[30:], kv[1][1][100:120]) <= 2e-2
    else:
        _fp8_codes_valid(kn[30:], kv[1][0][100:120], kv[1][2][100:120])
        _fp8_codes_valid(vn[30:], kv[1][1][100:120], kv[1][3][100:120])
    tails, toff = _pack(np.concatenate(own), [(0, 9), (9, 14), (14, 21), (21, 22)])
    h_last = torch.empty((4, shape.hidden), dtype=torch.int16, device="cuda")
    say("nested nodes: join")
    B.quail_join_prefill(ctx, [ha[0], hp[0], hn[0], hn[0]], to_device(tails), toff, h_last)
    logits = torch.empty((4, 8), dtype=torch.float32, device="cuda")
    tok = torch.empty(4, dtype=torch.uint8, device="cuda")
    dec = torch.empty(4, dtype=torch.uint8, device="cuda")
    B.quail_head8(ctx, h_last, 0x0F, logits, tok, dec)
    torch.cuda.synchronize()
    ref = [OM.forward_pair(a_tok, suffixes[i], wts, shape, shared_len=shared[i]) for i in range(4)]
    ref_logits = np.array([x["logits"] for x in ref])
    lg = logits.cpu().numpy()
    assert rel_inf(lg, ref_logits) <= 2e-2, rel_inf(lg, ref_logits)
    ok, _ = decisions_agree(dec.cpu().numpy(), [x["decision"] for x in ref], [x["margin"] for x in ref],
                            2e-2 * np.max(np.abs(ref_logits)))
    assert ok
    st = B.quail_pool_stats(ctx)
    assert st["prefills"] == 3 and st["evictions"] == 3 and st["resident"] == 0


@pytest.mark.parametrize("kv_fp8", [False, True])
def test_prefix_tree_composed_with_nested_nodes(B, kv_fp8):
    """Suffixes of one anchor that share a 24-token prompt, then one of two
    documents (20 and 16 tokens) in families of three, or nothing more: the
    nested grouping finds the prompt node and the two document nodes under it;
    they are prefilled parents first, every suffix runs its own tokens after
    its deepest node, and the logits match the oracle's per-pair forward."""
    import torch
    from query_aware_prefill_amd.device import DeviceModel, to_device
    shape = W.tiny_shape(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=128,
                         intermediate=384, vocab=512, kv_fp8=kv_fp8)
    wts = W.model_weights(shape, 18)
    r = np.random.default_rng(18)
    a_tok = r.integers(0, 512, 70).astype(np.int32)
    prompt = r.integers(0, 512, 24).astype(np.int32)
    docs = [r.integers(0, 512, 20).astype(np.int32), r.integers(0, 512, 16).astype(np.int32)]
    seqs = [np.concatenate([prompt, docs[i // 3], r.integers(0, 512, 3 + i).astype(np.int32)]) for i in range(6)]
    seqs.append(np.concatenate([prompt, r.integers(0, 512, 5).astype(np.int32)]))
    off = np.zeros(len(seqs) + 1, np.int32)
    off[1:] = np.cumsum([len(x) for x in seqs])
    s_tok = np.concatenate(seqs).astype(np.int32)
    keys = np.zeros(len(seqs), np.int32)
    g, nodes = B.quail_prefix_tree(s_tok, off, keys, 8)
    assert [(p, st, en) for p, _, st, en in nodes] == [(-1, 0, 24), (0, 24, 44), (0, 24, 40)]
    n = len(seqs)
    uses = [int(np.sum(g == k)) + sum(1 for q in nodes if q[0] == k) for k in range(len(nodes))]
    dm = DeviceModel(shape, wts, max_anchor_len=1024, max_suffix_len=256)
    ctx = dm.context(8 << 20, 256)
    say("prefix tree: anchor and nodes, parents first", "fp8" if kv_fp8 else "bf16")
    ha = B.quail_anchor_prefill(ctx, to_device(a_tok), [0, 70], [len(nodes)])   # each node holds one use
    handles = []
    for k, (par, first, start, end) in enumerate(nodes):
        tk = s_tok[off[first] + start:off[first] + end]
        parent = ha[0] if par < 0 else handles[par]
        handles.append(B.quail_prefix_prefill(ctx, [parent], to_device(tk), [0, end - start], [uses[k]])[0])
    tails, toff = _pack(s_tok, [(off[i] + nodes[g[i]][3], off[i + 1]) for i in range(n)])
    h_last = torch.empty((n, shape.hidden), dtype=torch.int16, device="cuda")
    say("prefix tree: join")
    B.quail_join_prefill(ctx, [handles[g[i]] for i in range(n)], to_device(tails), toff, h_last)
    logits = torch.empty((n, 8), dtype=torch.float32, device="cuda")
    tok = torch.empty(n, dtype=torch.uint8, device="cuda")
    dec = torch.empty(n, dtype=torch.uint8, device="cuda")
    B.quail_head8(ctx, h_last, 0x0F, logits, tok, dec)
    torch.cuda.synchronize()
    ref = [OM.forward_pair(a_tok, seqs[i], wts, shape, shared_len=nodes[g[i]][3]) for i in range(n)]
    ref_logits = np.array([x["logits"] for x in ref])
    lg = logits.cpu().numpy()
    assert rel_inf(lg, ref_logits) <= 2e-2, rel_inf(lg, ref_logits)
    ok, _ = decisions_agree(dec.cpu().numpy(), [x["decision"] for x in ref], [x["margin"] for x in ref],
                            2e-2 * np.max(np.abs(ref_logits)))
    assert ok
    st = B.quail_pool_stats(ctx)
    assert st["prefills"] == 1 + len(nodes) and st["evictions"] == 1 + len(nodes) and st["resident"] == 0


def test_join_run_shared_nested(B):
    """The one-call join with nested grouping: under two anchors and among
    filter rows, suffixes share a prompt and then, in families, a document.
    Logits equal the plain run's and the oracle's; the nested run prefills
    more nodes than one level does (a prompt node and document nodes under
    it), evicts everything and has no regret."""
    import torch
    from query_aware_prefill_amd.device import DeviceModel, to_device
    shape = W.tiny_shape(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=128,
                         intermediate=384, vocab=512)
    wts = W.model_weights(shape, 19)
    r = np.random.default_rng(19)
    a_len = [40, 90]
    a_tok = r.integers(0, 512, sum(a_len)).astype(np.int32)
    a_off = np.array([0, 40, 130], np.int32)
    pairs, seqs = [], []
    for a in (0, 1, -1):
        prompt = r.integers(0, 512, 20).astype(np.int32)
        for f in range(2):
            doc = r.integers(0, 512, 12 + 4 * f).astype(np.int32)
            for m in range(3):
                seqs.append(np.concatenate([prompt, doc, r.integers(0, 512, 2 + m).astype(np.int32)]))
                pairs.append(a)
        seqs.append(np.concatenate([prompt, r.integers(0, 512, 6).astype(np.int32)]))
        pairs.append(a)
    n = len(seqs)
    pa = np.array(pairs, np.int32)
    s_off = np.zeros(n + 1, np.int32)
    s_off[1:] = np.cumsum([len(x) for x in seqs])
    s_tok = np.concatenate(seqs).astype(np.int32)
    dm = DeviceModel(shape, wts, max_anchor_len=1024, max_suffix_len=256)
    outs = {}
    for mode in ("plain", "one", "nested"):
        ctx = dm.context(16 << 20, 1024)           # one plan step: every tree whole
        logits = torch.empty((n, 8), dtype=torch.float32, device="cuda")
        dec = torch.empty(n, dtype=torch.uint8, device="cuda")
        say("join_run", mode)
        if mode == "plain":
            B.quail_join_run(ctx, to_device(a_tok), a_off, pa, to_device(s_tok), s_off, 0x0F, logits, None, dec)
        else:
            B.quail_join_run_shared(ctx, to_device(a_tok), a_off, pa, to_device(s_tok), s_off, s_tok, 8, 0x0F,
                                    logits, None, dec, nested=(mode == "nested"))
        torch.cuda.synchronize()
        outs[mode] = (logits.cpu().numpy(), dec.cpu().numpy(), B.quail_pool_stats(ctx))
    l0 = outs["plain"][0]
    for mode in ("one", "nested"):
        lg, _, st = outs[mode]
        assert rel_inf(lg, l0) <= 2e-2, (mode, rel_inf(lg, l0))
        assert st["evictions"] == st["prefills"] and st["resident"] == 0 and st["regret_tokens"] == 0
    assert outs["one"][2]["prefills"] == 2 + 3          # anchors + one prompt node per tree
    assert outs["nested"][2]["prefills"] == 2 + 3 * 3   # anchors + prompt and two document nodes per tree
    ref = [OM.forward_pair(a_tok[a_off[a]:a_off[a + 1]] if a >= 0 else [], seqs[i], wts, shape)
           for i, a in enumerate(pairs)]
    ref_logits = np.array([x["logits"] for x in ref])
    assert rel_inf(outs["nested"][0], ref_logits) <= 2e-2
    ok, _ = decisions_agree(outs["nested"][1], [x["decision"] for x in ref], [x["margin"] for x in ref],
                            2e-2 * np.max(np.abs(ref_logits)))
    assert ok


def _full_size_case(kind, vocab):
    """Token layouts of the 36-layer benchmark workloads at their full sizes:
    the plain join (64 anchors x 1024, 2048 suffixes of 64 per anchor), the
    join with shared suffix prefixes (16 anchors x 1024, 16 families x 8 per
    anchor sharing 384 tokens), documents sharing a prefix per family (128 x
    16 sharing 768, no anchor) and documents under two shared levels (a
    512-token prompt, families of 16 sharing 384 more, no anchor)."""
    if kind == "join":
        c = W.c3b_case()
        return c["a_tok"], c["a_off"], c["pair_anchor"], c["s_tok"], c["s_off"]
    r = np.random.default_rng([7, 0])
    if kind == "nested":
        r = np.random.default_rng([8, 0])
        prompt = r.integers(0, vocab, 512).astype(np.int32)
        docs = [r.integers(0, vocab, 384).astype(np.int32) for _ in range(128)]
        seqs = [np.concatenate([prompt, docs[i // 16], r.integers(0, vocab, int(r.integers(32, 129)))
                                .astype(np.int32)]) for i in range(128 * 16)]
        s_off = np.zeros(len(seqs) + 1, np.int32)
        s_off[1:] = np.cumsum([len(x) for x in seqs])
        return (np.zeros(1, np.int32), np.zeros(1, np.int32), -np.ones(len(seqs), np.int32),
                np.concatenate(seqs).astype(np.int32), s_off)
    if kind == "traces":
        n_anchors = 0
        fams = [(-1, 768, r.integers(32, 129, 16).tolist()) for _ in range(128)]
    else:
        n_anchors = 16
        fams = [(a, 384, r.integers(16, 65, 8).tolist()) for a in range(16) for _ in range(16)]
    c = W.shared_prefix_case(7, vocab, [1024] * n_anchors, fams, cfg_id=7)
    a_tok = c["a_tok"] if len(c["a_tok"]) else np.zeros(1, np.int32)
    return a_tok, c["a_off"], c["pair_anchor"], c["s_tok"], c["s_off"]


@pytest.mark.parametrize("kind", ["join", "shared", "traces", "nested"])
def test_full_size_workloads_one_layer_sampled(B, kind):
    """The 36-layer benchmark workloads at full size through one
    Qwen3-4B-shaped layer, in the calls the benchmark makes (quail_join_run
    for the plain join; quail_join_run_shared with min_shared 32, one level or
    nested, for the others): four sampled pairs (first, last, two more)
    against the oracle's per-pair forward over [anchor | whole suffix], every
    pair by properties (finite logits, decision = the mask bit of its logits'
    first argmax), and every slab evicted after its last use with no regret."""
    import torch
    from query_aware_prefill_amd.device import DeviceModel, to_device
    shape = W.ModelShape(n_layers=1, hidden=2560, n_q_heads=32, n_kv_heads=8, head_dim=128,
                         intermediate=9728, vocab=W.QWEN3_4B.vocab)
    say("full size", kind, ": weights and workload")
    wts = W.model_weights(shape, 0)
    a_tok, a_off, pa, s_tok, s_off = _full_size_case(kind, shape.vocab)
    n = len(pa)
    s_len = np.diff(s_off)
    a_len = np.diff(a_off)
    dm = DeviceModel(shape, wts, max_anchor_len=1024, max_suffix_len=int(s_len.max()))
    pool = sum(B.quail_anchor_bytes(dm.cfg, int(x)) for x in a_len) + (2 << 30)
    ctx = dm.context(pool, 65536)
    logits = torch.empty((n, 8), dtype=torch.float32, device="cuda")
    dec = torch.empty(n, dtype=torch.uint8, device="cuda")
    a_d, s_d = to_device(a_tok), to_device(s_tok)
    say("full size", kind, ":", n, "pairs,", int(s_off[-1]), "suffix tokens")
    if kind == "join":
        B.quail_join_run(ctx, a_d, a_off, pa, s_d, s_off, 0x0F, logits, None, dec)
    else:
        B.quail_join_run_shared(ctx, a_d, a_off, pa, s_d, s_off, s_tok, 32, 0x0F, logits, None, dec,
                                nested=(kind == "nested"))
    torch.cuda.synchronize()
    lg, dg = logits.cpu().numpy(), dec.cpu().numpy()
    st = B.quail_pool_stats(ctx)
    say("  pool", st)
    assert st["resident"] == 0 and st["evictions"] == st["prefills"] and st["regret_tokens"] == 0
    if kind != "join":
        assert st["prefills"] > len(a_len)              # prefix nodes were prefilled
    assert np.isfinite(lg).all()
    assert np.array_equal(dg, ((0x0F >> np.argmax(lg, axis=1)) & 1).astype(np.uint8))
    sample = [0, n - 1] + np.random.default_rng(6).integers(0, n, 2).tolist()
    layers = [OM.LayerWeights(wts["layers"][0], shape)]
    for i in sample:
        a = int(pa[i])
        at = a_tok[a_off[a]:a_off[a + 1]] if a >= 0 else np.zeros(0, np.int32)
        ref = OM.forward_pair(at, s_tok[s_off[i]:s_off[i + 1]], wts, shape, layers=layers)
        err = rel_inf(lg[i], ref["logits"])
        say("  pair", i, "rel", err)
        assert err <= 2e-2, (kind, i, err)
        if abs(ref["margin"]) > 2e-2 * np.max(np.abs(ref["logits"])):
            assert dg[i] == ref["decision"], (kind, i)
