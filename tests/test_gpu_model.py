"""GPU parity of the model path against the oracle's per-pair monolithic
forward: anchor prefill + KV writer (slab contents), join prefill (last and
all hidden rows), the 8-column head and its booleans, residency counters and
handle errors, the whole-join entry point, the fp8 KV store, and one
Qwen3-4B-shaped decoder layer."""
import numpy as np
import pytest

import workloads as W
from oracle import codecs, model as OM
from tests.gpu_util import bf16_f64, decisions_agree, rel_inf, say, u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    import torch
    assert torch.cuda.is_available()
    from query_aware_prefill_amd import binding
    binding.load()
    return binding


def _slab(ctx, handle, layer, B, shape):
    """Read one layer's K and V of an anchor back from the pool tensor."""
    kp, vp, la, lap = B.quail_anchor_kv(ctx, handle, layer)
    pool = ctx._pool
    esz = 1 if shape.kv_fp8 else 2
    n = shape.n_kv_heads * lap * shape.head_dim * esz
    out = []
    for p in (kp, vp):
        off = p - pool.data_ptr()
        raw = pool[off:off + n].cpu().numpy()
        if esz == 2:
            vals = bf16_f64(raw.view(np.uint16))
        else:
            vals = codecs.e4m3_decode(raw) * (shape.k_scale if p == kp else shape.v_scale)
        out.append(vals.reshape(shape.n_kv_heads, lap, shape.head_dim)[:, :la].transpose(1, 0, 2))
    return out


def _fp8_codes_valid(got, stored, pre):
    """An fp8 store decides a code from a float. The GPU's pre-quantisation
    values differ from the oracle's within the tensor tolerance (2e-2 of the
    largest magnitude), and a midpoint between them flips the code; such a
    flip also feeds later layers. So every stored value must be a valid E4M3
    rounding of some value within that tolerance of the oracle's
    pre-quantisation value, and nearly all codes must be the oracle's."""
    grid = codecs.e4m3_decode(np.arange(127, dtype=np.uint8))   # non-negative values
    tol = 2e-2 * np.max(np.abs(pre))
    a = np.minimum(np.abs(pre), 448.0)
    i = np.clip(np.searchsorted(grid, a), 1, 126)
    half_step = 0.5 * (grid[i] - grid[i - 1])
    excess = np.abs(got - pre) - half_step
    assert np.max(excess) <= tol, (np.max(excess), tol)
    # a value within the tolerance of a midpoint flips: at a few 1e-3 relative
    # difference and E4M3 steps of 6-12%, a few percent of codes may differ
    assert np.mean(got == stored) >= 0.95, np.mean(got == stored)


def _setup(shape, seed, a_len, pairs, B, pool_bytes=None, mbt=512):
    import torch
    from query_aware_prefill_amd.device import DeviceModel, to_device
    wts = W.model_weights(shape, seed)
    pa = [p[0] for p in pairs]
    sl = [p[1] for p in pairs]
    case = W.join_case(seed, shape.vocab, a_len, pa, sl, cfg_id=20)
    dm = DeviceModel(shape, wts, max_anchor_len=1024, max_suffix_len=256)
    if pool_bytes is None:
        pool_bytes = sum(B.quail_anchor_bytes(dm.cfg, x) for x in a_len) + 4096
    ctx = dm.context(pool_bytes, mbt)
    return wts, case, dm, ctx, to_device(case["a_tok"]), to_device(case["s_tok"])


@pytest.mark.parametrize("kv_fp8,k_scale,v_scale", [(False, 1.0, 1.0), (True, 1.0, 1.0), (True, 0.5, 2.0)])
def test_tiny_model_anchor_join_head(B, kv_fp8, k_scale, v_scale):
    """bf16 slabs; E4M3 slabs with unit scales (read directly by the attention
    kernel); E4M3 slabs with non-unit scales (the register-staged kernel)."""
    import torch
    shape = W.tiny_shape(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=128,
                         intermediate=384, vocab=512, kv_fp8=kv_fp8, k_scale=k_scale, v_scale=v_scale)
    a_len = [1, 70, 130]
    pairs = [(1, 5), (0, 3), (1, 33), (-1, 7), (2, 17), (1, 64), (0, 1), (-1, 2)]
    wts, case, dm, ctx, a_tok, s_tok = _setup(shape, 3, a_len, pairs, B)
    uses = np.bincount([p[0] for p in pairs if p[0] >= 0], minlength=3)
    say("tiny model: anchor prefill", "fp8" if kv_fp8 else "bf16")
    handles = B.quail_anchor_prefill(ctx, a_tok, case["a_off"], uses, anchor_ids=np.arange(3))
    torch.cuda.synchronize()
    # KV writer: the slab holds the oracle's per-layer post-RoPE K and V
    for a in range(3):
        toks = case["a_tok"][case["a_off"][a]:case["a_off"][a + 1]]
        _, kv = OM.forward_tokens(toks, wts, shape, return_kv=True,
                                  fp8_kv_upto=len(toks) if kv_fp8 else 0)
        for l in range(shape.n_layers):
            k, v = _slab(ctx, handles[a], l, B, shape)
            if not kv_fp8:
                assert rel_inf(k, kv[l][0]) <= 2e-2, (a, l, "K")
                assert rel_inf(v, kv[l][1]) <= 2e-2, (a, l, "V")
            else:
                for got, stored, pre in ((k, kv[l][0], kv[l][2]), (v, kv[l][1], kv[l][3])):
                    _fp8_codes_valid(got, stored, pre)
    say("tiny model: join prefill")
    n = len(pairs)
    T = int(case["s_off"][-1])
    h_last = torch.empty((n, shape.hidden), dtype=torch.int16, device="cuda")
    h_all = torch.empty((T, shape.hidden), dtype=torch.int16, device="cuda")
    pair_handles = [handles[a] if a >= 0 else B.NO_ANCHOR for a, _ in pairs]
    B.quail_join_prefill(ctx, pair_handles, s_tok, case["s_off"], h_last, h_all)
    logits = torch.empty((n, 8), dtype=torch.float32, device="cuda")
    tok = torch.empty(n, dtype=torch.uint8, device="cuda")
    dec = torch.empty(n, dtype=torch.uint8, device="cuda")
    B.quail_head8(ctx, h_last, 0x0F, logits, tok, dec)
    torch.cuda.synchronize()
    hl, ha = bf16_f64(u16(h_last)), bf16_f64(u16(h_all))
    ref_logits, ref_dec, ref_margin = [], [], []
    for i, (a, L) in enumerate(pairs):
        at = case["a_tok"][case["a_off"][a]:case["a_off"][a + 1]] if a >= 0 else []
        st = case["s_tok"][case["s_off"][i]:case["s_off"][i + 1]]
        ref = OM.forward_pair(at, st, wts, shape, true_mask=0x0F)
        assert rel_inf(hl[i], ref["h_last"]) <= 2e-2, (i, rel_inf(hl[i], ref["h_last"]))
        assert rel_inf(ha[case["s_off"][i]:case["s_off"][i + 1]], ref["h"][len(at):]) <= 2e-2
        ref_logits.append(ref["logits"]); ref_dec.append(ref["decision"]); ref_margin.append(ref["margin"])
    ref_logits = np.array(ref_logits)
    assert rel_inf(logits.cpu().numpy(), ref_logits) <= 2e-2
    tau = 2e-2 * np.max(np.abs(ref_logits))
    ok, n_sure = decisions_agree(dec.cpu().numpy(), ref_dec, ref_margin, tau)
    assert ok
    st = B.quail_pool_stats(ctx)
    assert st["prefills"] == 3 and st["evictions"] == 3 and st["regret_tokens"] == 0
    assert st["resident"] == 0 and st["peak"] > 0
    with pytest.raises(B.QuailError) as e:
        B.quail_join_prefill(ctx, [handles[1]], s_tok, case["s_off"][:2], h_last)
    assert e.value.status == B.E_STALE


def test_release_and_regret_counting(B):
    import torch
    shape = W.tiny_shape(n_layers=1, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=128,
                         intermediate=384, vocab=512)
    wts, case, dm, ctx, a_tok, s_tok = _setup(shape, 4, [50], [(0, 4)], B)
    say("release + regret")
    h = B.quail_anchor_prefill(ctx, a_tok, case["a_off"], [2], anchor_ids=[77])
    B.quail_anchor_release(ctx, h[0])
    with pytest.raises(B.QuailError) as e:
        B.quail_anchor_release(ctx, h[0])
    assert e.value.status == B.E_STALE
    h2 = B.quail_anchor_prefill(ctx, a_tok, case["a_off"], [1], anchor_ids=[77])
    h_last = torch.empty((1, shape.hidden), dtype=torch.int16, device="cuda")
    B.quail_join_prefill(ctx, [h2[0]], s_tok, case["s_off"], h_last)
    torch.cuda.synchronize()
    st = B.quail_pool_stats(ctx)
    assert st["prefills"] == 2 and st["evictions"] == 2 and st["regret_tokens"] == 50


def test_join_run_end_to_end(B):
    """Multi-join shaped: 6 anchors, 5 rows probing 3 anchors each (in row
    order, unsorted), 2 filter rows; plan + prefill + join + head in one call."""
    import torch
    from query_aware_prefill_amd.device import to_device
    shape = W.tiny_shape(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=128,
                         intermediate=384, vocab=512)
    r = np.random.default_rng(8)
    a_len = r.integers(20, 120, 6).tolist()
    pairs = []
    for row in range(5):
        L = int(r.integers(2, 40))
        for a in r.choice(6, 3, replace=False):
            pairs.append((int(a), L))
    pairs += [(-1, 9), (-1, 3)]
    # small batch budget so the plan has several steps
    wts, case, dm, ctx, a_tok, s_tok = _setup(shape, 5, a_len, pairs, B, mbt=128)
    n = len(pairs)
    logits = torch.empty((n, 8), dtype=torch.float32, device="cuda")
    tok = torch.empty(n, dtype=torch.uint8, device="cuda")
    dec = torch.empty(n, dtype=torch.uint8, device="cuda")
    say("join_run", n, "pairs")
    B.quail_join_run(ctx, a_tok, case["a_off"], case["pair_anchor"], s_tok, case["s_off"], 0x0F,
                     logits, tok, dec)
    torch.cuda.synchronize()
    ref_logits, ref_dec, ref_margin = [], [], []
    for i, (a, L) in enumerate(pairs):
        at = case["a_tok"][case["a_off"][a]:case["a_off"][a + 1]] if a >= 0 else []
        st = case["s_tok"][case["s_off"][i]:case["s_off"][i + 1]]
        ref = OM.forward_pair(at, st, wts, shape, true_mask=0x0F)
        ref_logits.append(ref["logits"]); ref_dec.append(ref["decision"]); ref_margin.append(ref["margin"])
    ref_logits = np.array(ref_logits)
    assert rel_inf(logits.cpu().numpy(), ref_logits) <= 2e-2
    ok, _ = decisions_agree(dec.cpu().numpy(), ref_dec, ref_margin, 2e-2 * np.max(np.abs(ref_logits)))
    assert ok
    st = B.quail_pool_stats(ctx)
    used = len({a for a, _ in pairs if a >= 0})
    assert st["prefills"] == used and st["evictions"] == used and st["regret_tokens"] == 0
    # a second, identical query on the same context is a new plan: no regret
    dec2 = torch.empty(n, dtype=torch.uint8, device="cuda")
    B.quail_join_run(ctx, a_tok, case["a_off"], case["pair_anchor"], s_tok, case["s_off"], 0x0F,
                     None, None, dec2)
    torch.cuda.synchronize()
    assert np.array_equal(dec2.cpu().numpy(), dec.cpu().numpy())
    st = B.quail_pool_stats(ctx)
    assert st["prefills"] == 2 * used and st["regret_tokens"] == 0 and st["resident"] == 0


@pytest.mark.parametrize("kv_fp8", [False, True])
def test_last_layer_runs_only_the_last_rows(B, kv_fp8):
    """A join prefill that returns only each pair's last row runs the last
    layer's O projection and MLP on the last rows alone (gathered through row
    maps in the GEMMs and the norm). Its last rows must be bit-identical to
    those of the same prefill returning every row (which runs every row), and
    match the oracle. More than 256 pairs, so the gathered rows span several
    GEMM row tiles; lengths from 1 (the last row is the only row) to 64."""
    import torch
    shape = W.tiny_shape(n_layers=3, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=128,
                         intermediate=384, vocab=512, kv_fp8=kv_fp8)
    r = np.random.default_rng(31)
    a_len = [40, 97, 150]
    pairs = [(int(r.integers(-1, 3)), int(r.integers(1, 13))) for _ in range(300)]
    pairs += [(0, 64), (1, 1), (2, 64), (-1, 1), (-1, 64)]
    wts, case, dm, ctx, a_tok, s_tok = _setup(shape, 11, a_len, pairs, B, mbt=2048)
    uses = 2 * np.bincount([p[0] for p in pairs if p[0] >= 0], minlength=3)
    say("last-layer rows: anchor prefill", "fp8" if kv_fp8 else "bf16")
    handles = B.quail_anchor_prefill(ctx, a_tok, case["a_off"], uses, anchor_ids=np.arange(3))
    n = len(pairs)
    T = int(case["s_off"][-1])
    ph = [handles[a] if a >= 0 else B.NO_ANCHOR for a, _ in pairs]
    h_full = torch.empty((n, shape.hidden), dtype=torch.int16, device="cuda")
    h_all = torch.empty((T, shape.hidden), dtype=torch.int16, device="cuda")
    say("last-layer rows: every row", n, "pairs,", T, "rows")
    B.quail_join_prefill(ctx, ph, s_tok, case["s_off"], h_full, h_all)
    h_tail = torch.empty((n, shape.hidden), dtype=torch.int16, device="cuda")
    say("last-layer rows: last rows only")
    B.quail_join_prefill(ctx, ph, s_tok, case["s_off"], h_tail, None)
    torch.cuda.synchronize()
    full, tail = u16(h_full), u16(h_tail)
    assert np.array_equal(full, tail), int(np.sum(full != tail))
    assert np.array_equal(u16(h_all)[case["s_off"][1:] - 1], full)
    st = B.quail_pool_stats(ctx)
    assert st["evictions"] == 3 and st["regret_tokens"] == 0 and st["resident"] == 0
    for i in list(range(0, n, 37)) + [n - 5, n - 4, n - 1]:
        a = pairs[i][0]
        at = case["a_tok"][case["a_off"][a]:case["a_off"][a + 1]] if a >= 0 else []
        st_ = case["s_tok"][case["s_off"][i]:case["s_off"][i + 1]]
        ref = OM.forward_pair(at, st_, wts, shape)
        assert rel_inf(bf16_f64(tail[i]), ref["h_last"]) <= 2e-2, i


def test_qwen3_shaped_layer(B):
    """One decoder layer with the Qwen3-4B shapes (hidden 2560, 32q/8kv x 128,
    SwiGLU 9728, RoPE theta 1e6, fp8 weights): 2 anchors x 1024 tokens, two
    64-token suffixes each, against the oracle on every suffix position."""
    import torch
    shape = W.ModelShape(n_layers=1, hidden=2560, n_q_heads=32, n_kv_heads=8, head_dim=128,
                         intermediate=9728, vocab=4096)
    pairs = [(0, 64), (1, 64), (0, 64), (1, 64)]
    wts, case, dm, ctx, a_tok, s_tok = _setup(shape, 6, [1024, 1024], pairs, B, mbt=2048)
    say("qwen3 layer: prefill + join")
    handles = B.quail_anchor_prefill(ctx, a_tok, case["a_off"], [2, 2])
    T = int(case["s_off"][-1])
    h_last = torch.empty((4, shape.hidden), dtype=torch.int16, device="cuda")
    h_all = torch.empty((T, shape.hidden), dtype=torch.int16, device="cuda")
    B.quail_join_prefill(ctx, [handles[a] for a, _ in pairs], s_tok, case["s_off"], h_last, h_all)
    torch.cuda.synchronize()
    ha = bf16_f64(u16(h_all))
    for i in (0, 1):
        a = pairs[i][0]
        at = case["a_tok"][case["a_off"][a]:case["a_off"][a + 1]]
        st = case["s_tok"][case["s_off"][i]:case["s_off"][i + 1]]
        h = OM.forward_tokens(np.concatenate([at, st]), wts, shape)
        err = rel_inf(ha[case["s_off"][i]:case["s_off"][i + 1]], h[len(at):])
        say("  pair", i, "rel", err)
        assert err <= 2e-2


def test_multijoin_run_keeps_anchors_across_joins(B):
    """Three joins over one anchor table run one after another: with a pool
    for every anchor, each anchor is prefilled once for all joins (regret 0,
    where planning the joins one by one prefills an anchor once per join);
    with a pool for two anchors, the prefills and regret are the plan's. Every
    pair's logits equal those of running its join alone (same kernels on the
    same rows), and the decisions agree with the oracle on a sample."""
    import torch
    shape = W.tiny_shape(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=128,
                         intermediate=384, vocab=512)
    r = np.random.default_rng(21)
    a_len = [64] * 5                        # equal slabs: the pool never fragments
    joins = [[(0, 9), (2, 14), (0, 3), (3, 30)],
             [(2, 5), (4, 17), (1, 8), (-1, 6)],
             [(0, 11), (3, 2), (2, 25), (4, 4), (1, 19)]]
    pairs = [p for j in joins for p in j]
    jo = np.cumsum([0] + [len(j) for j in joins]).astype(np.int32)
    n = len(pairs)
    slab = None
    results = {}
    for label, n_slabs in (("ample", 5), ("tight", 2)):
        wts, case, dm, ctx, a_tok, s_tok = _setup(shape, 9, a_len, pairs, B, mbt=96)
        slab = B.quail_anchor_bytes(dm.cfg, 64)
        if n_slabs != 5:
            ctx = dm.context(n_slabs * slab + B.GUARD_BYTES, 96)   # + the pool's tail guard
        logits = torch.empty((n, 8), dtype=torch.float32, device="cuda")
        dec = torch.empty(n, dtype=torch.uint8, device="cuda")
        say("multijoin_run", label, n, "pairs in", len(joins), "joins")
        B.quail_multijoin_run(ctx, a_tok, case["a_off"], jo, case["pair_anchor"], s_tok, case["s_off"], 0x0F,
                              logits, None, dec)
        torch.cuda.synchronize()
        st = B.quail_pool_stats(ctx)
        plan = B.quail_multiplan_build(dm.cfg, n_slabs * slab if n_slabs != 5 else
                                       sum(B.quail_anchor_bytes(dm.cfg, x) for x in a_len) + 4096, 96,
                                       a_len, jo, case["pair_anchor"], np.diff(case["s_off"]))
        assert (st["prefills"], st["evictions"], st["regret_tokens"]) == \
            (plan["prefills"], plan["evictions"], plan["regret_tokens"]), (label, st, plan)
        assert st["resident"] == 0 and st["peak"] <= plan["peak"]
        results[label] = (logits.cpu().numpy(), dec.cpu().numpy(), st)
    used = {a for a, _ in pairs if a >= 0}
    assert results["ample"][2]["prefills"] == len(used) and results["ample"][2]["regret_tokens"] == 0
    assert results["tight"][2]["regret_tokens"] > 0
    # a tighter pool cuts smaller steps, so batches (and with them the
    # attention tile shapes) differ: same results within the bf16 contract
    la, lt = results["ample"][0], results["tight"][0]
    assert rel_inf(lt, la) <= 2e-2
    tau = 2e-2 * np.max(np.abs(la))
    gap = np.sort(la, axis=1)[:, -1] - np.sort(la, axis=1)[:, -2]
    sure = gap > tau
    assert np.array_equal(results["ample"][1][sure], results["tight"][1][sure])
    # each join alone on a fresh context
    wts, case, dm, ctx, a_tok, s_tok = _setup(shape, 9, a_len, pairs, B, mbt=96)
    alone = np.zeros((n, 8), np.float32)
    naive_prefills = 0
    for j in range(len(joins)):
        idx = np.arange(jo[j], jo[j + 1])
        s_off = np.concatenate([[0], np.cumsum(np.diff(case["s_off"])[idx])]).astype(np.int32)
        toks = np.concatenate([case["s_tok"][case["s_off"][i]:case["s_off"][i + 1]] for i in idx]).astype(np.int32)
        lg = torch.empty((len(idx), 8), dtype=torch.float32, device="cuda")
        dj = torch.empty(len(idx), dtype=torch.uint8, device="cuda")
        from query_aware_prefill_amd.device import to_device
        B.quail_join_run(ctx, a_tok, case["a_off"], case["pair_anchor"][idx], to_device(toks), s_off, 0x0F,
                         lg, None, dj)
        torch.cuda.synchronize()
        alone[idx] = lg.cpu().numpy()
        naive_prefills += len({a for a in case["pair_anchor"][idx] if a >= 0})
    # same pool, so the same steps: the same batches through the same kernels
    assert np.array_equal(alone, results["ample"][0])
    assert B.quail_pool_stats(ctx)["prefills"] == naive_prefills > len(used)
    # oracle on a sample of pairs
    for i in (0, 5, 7, 12):
        a = pairs[i][0]
        at = case["a_tok"][case["a_off"][a]:case["a_off"][a + 1]] if a >= 0 else []
        stoks = case["s_tok"][case["s_off"][i]:case["s_off"][i + 1]]
        ref = OM.forward_pair(at, stoks, wts, shape, true_mask=0x0F)
        assert rel_inf(results["ample"][0][i], ref["logits"]) <= 2e-2
        if abs(ref["margin"]) > 2e-2 * np.max(np.abs(ref["logits"])):
            assert results["ample"][1][i] == ref["decision"]


def test_many_anchors_per_batch_split_by_source_table(B):
    """60 anchors with one 1-token suffix each, 6 layers, a 64-token batch:
    one batch would read 61 KV sources, whose per-layer tables exceed the
    batch metadata region; batches are cut so they fit (anchor prefill and
    join alike), and every pair matches the oracle."""
    import torch
    shape = W.tiny_shape(n_layers=6, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=128,
                         intermediate=384, vocab=512)
    a_len = [3] * 60
    pairs = [(a, 1) for a in range(60)]
    wts, case, dm, ctx, a_tok, s_tok = _setup(shape, 15, a_len, pairs, B, mbt=64)
    n = len(pairs)
    logits = torch.empty((n, 8), dtype=torch.float32, device="cuda")
    dec = torch.empty(n, dtype=torch.uint8, device="cuda")
    say("many anchors per batch: join_run")
    B.quail_join_run(ctx, a_tok, case["a_off"], case["pair_anchor"], s_tok, case["s_off"], 0x0F, logits, None, dec)
    torch.cuda.synchronize()
    ref = [OM.forward_pair(case["a_tok"][case["a_off"][a]:case["a_off"][a + 1]],
                           case["s_tok"][case["s_off"][i]:case["s_off"][i + 1]], wts, shape)
           for i, (a, _) in enumerate(pairs)]
    ref_logits = np.array([r["logits"] for r in ref])
    assert rel_inf(logits.cpu().numpy(), ref_logits) <= 2e-2
    ok, _ = decisions_agree(dec.cpu().numpy(), [r["decision"] for r in ref], [r["margin"] for r in ref],
                            2e-2 * np.max(np.abs(ref_logits)))
    assert ok
    st = B.quail_pool_stats(ctx)
    assert st["prefills"] == 60 and st["evictions"] == 60 and st["resident"] == 0


def test_c2_full_size_layer_sampled(B):
    """The one-layer workload at full size in the launch configuration the
    bench times (16 anchors x 1024 tokens, 512 suffixes x 64 tokens each,
    8,192 pairs, 65,536-token batches, Qwen3-4B layer shapes): logits of
    sampled pairs (first and last pair of the first and last anchor, two
    more) against the oracle's per-pair forward, decisions where the margin
    exceeds the tolerance; every pair by properties (finite logits, decision
    = the mask bit of its logits' first argmax, identical bits on a second
    run)."""
    import torch
    from query_aware_prefill_amd.device import DeviceModel, to_device
    shape = W.ModelShape(n_layers=1, hidden=2560, n_q_heads=32, n_kv_heads=8, head_dim=128,
                         intermediate=9728, vocab=W.QWEN3_4B.vocab)
    say("C2 full size: weights and workload")
    wts = W.model_weights(shape, 0)
    case = W.c2_case(seed=2)
    n = len(case["pair_anchor"])
    dm = DeviceModel(shape, wts, max_anchor_len=1024, max_suffix_len=64)
    ctx = dm.context(16 * B.quail_anchor_bytes(dm.cfg, 1024) + (1 << 20), 65536)
    logits = torch.empty((n, 8), dtype=torch.float32, device="cuda")
    dec = torch.empty(n, dtype=torch.uint8, device="cuda")
    say("C2 full size: join_run over", n, "pairs")
    B.quail_join_run(ctx, to_device(case["a_tok"]), case["a_off"], case["pair_anchor"], to_device(case["s_tok"]),
                     case["s_off"], 0x0F, logits, None, dec)
    torch.cuda.synchronize()
    lg, dg = logits.cpu().numpy(), dec.cpu().numpy()
    st = B.quail_pool_stats(ctx)
    assert st["prefills"] == 16 and st["evictions"] == 16 and st["regret_tokens"] == 0
    sample = [0, 511, 8192 - 512, 8191] + np.random.default_rng(2).integers(0, n, 2).tolist()
    say("C2 full size: oracle on pairs", sample)
    for i in sample:
        a = int(case["pair_anchor"][i])
        ref = OM.forward_pair(case["a_tok"][case["a_off"][a]:case["a_off"][a + 1]],
                              case["s_tok"][case["s_off"][i]:case["s_off"][i + 1]], wts, shape)
        err = rel_inf(lg[i], ref["logits"])
        say("  pair", i, "rel", err)
        assert err <= 2e-2, (i, err)
        if abs(ref["margin"]) > 2e-2 * np.max(np.abs(ref["logits"])):
            assert dg[i] == ref["decision"], i
    # every pair: finite logits, each decision is its own logits' first
    # argmax mapped through the TRUE mask, and a second run (anchors
    # prefilled again after their eviction) gives the same bits
    say("C2 full size: properties of every pair and a second run")
    assert np.isfinite(lg).all()
    tok = np.argmax(lg, axis=1)
    assert np.array_equal(dg, ((0x0F >> tok) & 1).astype(np.uint8))
    logits2 = torch.empty_like(logits)
    dec2 = torch.empty_like(dec)
    B.quail_join_run(ctx, to_device(case["a_tok"]), case["a_off"], case["pair_anchor"], to_device(case["s_tok"]),
                     case["s_off"], 0x0F, logits2, None, dec2)
    torch.cuda.synchronize()
    assert np.array_equal(logits2.cpu().numpy().view(np.uint32), lg.view(np.uint32))
    assert np.array_equal(dec2.cpu().numpy(), dg)


def test_filter_full_size_one_layer_sampled(B):
    """The filter workload at full size (10,000 rows, lognormal lengths
    200..2000, 7.2 M tokens, no anchor) through one Qwen3-4B-shaped layer in
    the launch configuration the benchmark uses (one quail_join_run call,
    65,536-token batches): the shortest, the longest and two more rows
    against the oracle's per-row forward, and every row by properties
    (finite logits, decision = the mask bit of its logits' first argmax)."""
    import torch
    from query_aware_prefill_amd.device import DeviceModel, to_device
    shape = W.ModelShape(n_layers=1, hidden=2560, n_q_heads=32, n_kv_heads=8, head_dim=128,
                         intermediate=9728, vocab=W.QWEN3_4B.vocab)
    say("filter full size: weights and workload")
    wts = W.model_weights(shape, 0)
    case = W.c3a_case()
    s_off, s_tok = case["s_off"], case["s_tok"]
    s_len = np.diff(s_off)
    n = len(s_len)
    assert n == 10000 and 200 <= s_len.min() and s_len.max() <= 2000
    pa = -np.ones(n, np.int32)
    dm = DeviceModel(shape, wts, max_anchor_len=1, max_suffix_len=int(s_len.max()))
    ctx = dm.context(1 << 20, 65536)
    logits = torch.empty((n, 8), dtype=torch.float32, device="cuda")
    dec = torch.empty(n, dtype=torch.uint8, device="cuda")
    say("filter full size: join_run over", n, "rows,", int(s_off[-1]), "tokens")
    B.quail_join_run(ctx, to_device(np.zeros(1, np.int32)), [0], pa, to_device(s_tok), s_off, 0x0F,
                     logits, None, dec)
    torch.cuda.synchronize()
    lg, dg = logits.cpu().numpy(), dec.cpu().numpy()
    assert np.isfinite(lg).all()
    assert np.array_equal(dg, ((0x0F >> np.argmax(lg, axis=1)) & 1).astype(np.uint8))
    sample = [int(np.argmin(s_len)), int(np.argmax(s_len))] + np.random.default_rng(3).integers(0, n, 2).tolist()
    say("filter full size: oracle on rows", sample, "of lengths", [int(s_len[i]) for i in sample])
    layers = [OM.LayerWeights(wts["layers"][0], shape)]
    for i in sample:
        ref = OM.forward_pair(np.zeros(0, np.int32), s_tok[s_off[i]:s_off[i + 1]], wts, shape, layers=layers)
        err = rel_inf(lg[i], ref["logits"])
        say("  row", i, "rel", err)
        assert err <= 2e-2, (i, err)
        if abs(ref["margin"]) > 2e-2 * np.max(np.abs(ref["logits"])):
            assert dg[i] == ref["decision"], i


def test_multijoin_full_size_one_layer_sampled(B):
    """The multi-join workload at full size (1024 anchors x 768 tokens with
    E4M3 K/V slabs; 5,000 rows of U{48..256} tokens, each against 51 random
    anchors: 255,000 pairs, 38.9 M suffix tokens) through one Qwen3-4B-shaped
    layer in one quail_join_run call: every anchor prefilled once and evicted
    after its last pair, sampled pairs (first, last, two more) against the
    oracle's per-pair forward with the anchor's K/V stored in E4M3, and every
    pair by properties (finite logits, decision = the mask bit of its logits'
    first argmax)."""
    import torch
    from query_aware_prefill_amd.device import DeviceModel, to_device
    shape = W.ModelShape(n_layers=1, hidden=2560, n_q_heads=32, n_kv_heads=8, head_dim=128,
                         intermediate=9728, vocab=W.QWEN3_4B.vocab, kv_fp8=True)
    say("multi-join full size: weights and workload")
    wts = W.model_weights(shape, 0)
    case = W.c4_case()
    pa, prow = case["pair_anchor"], case["pair_row"]
    plen = case["row_len"][prow]
    n = len(pa)
    assert n == 255000
    s_off = np.zeros(n + 1, np.int64)
    s_off[1:] = np.cumsum(plen)
    assert s_off[-1] < 2 ** 31
    s_off = s_off.astype(np.int32)
    ro = case["row_off"]
    s_tok = np.concatenate([case["row_tok"][ro[r]:ro[r + 1]] for r in prow])
    dm = DeviceModel(shape, wts, max_anchor_len=768, max_suffix_len=int(plen.max()))
    pool = 1024 * B.quail_anchor_bytes(dm.cfg, 768) + (1 << 20)
    ctx = dm.context(pool, 65536)
    logits = torch.empty((n, 8), dtype=torch.float32, device="cuda")
    dec = torch.empty(n, dtype=torch.uint8, device="cuda")
    say("multi-join full size: join_run over", n, "pairs,", int(s_off[-1]), "suffix tokens")
    B.quail_join_run(ctx, to_device(case["a_tok"]), case["a_off"], pa, to_device(s_tok), s_off, 0x0F,
                     logits, None, dec)
    torch.cuda.synchronize()
    lg, dg = logits.cpu().numpy(), dec.cpu().numpy()
    st = B.quail_pool_stats(ctx)
    assert st["prefills"] == 1024 and st["evictions"] == 1024 and st["resident"] == 0
    assert st["regret_tokens"] == 0
    assert np.isfinite(lg).all()
    assert np.array_equal(dg, ((0x0F >> np.argmax(lg, axis=1)) & 1).astype(np.uint8))
    sample = [0, n - 1] + np.random.default_rng(4).integers(0, n, 2).tolist()
    say("multi-join full size: oracle on pairs", sample)
    layers = [OM.LayerWeights(wts["layers"][0], shape)]
    for i in sample:
        a = int(pa[i])
        ref = OM.forward_pair(case["a_tok"][case["a_off"][a]:case["a_off"][a + 1]], s_tok[s_off[i]:s_off[i + 1]],
                              wts, shape, layers=layers)
        err = rel_inf(lg[i], ref["logits"])
        say("  pair", i, "rel", err)
        assert err <= 2e-2, (i, err)
        if abs(ref["margin"]) > 2e-2 * np.max(np.abs(ref["logits"])):
            assert dg[i] == ref["decision"], i


def test_fragmented_pool_is_replanned_before_enqueueing(B):
    """A plan that fits the pool by its byte total but not by placement: slabs
    of 1, 2 and 3 units (64-token steps), a pool of 5 units, pairs [A, C | C,
    D] in two 400-token steps. First-fit puts A at [0, 1) and C at [1, 3);
    once A is evicted, D (3 units) finds only [0, 1) and [3, 5). The join
    replays its placements on the host first and, finding that, re-plans with
    a smaller budget (C's second pair, then D's pair, in steps of their own)
    before anything is enqueued; results match the oracle, no regret."""
    import torch
    shape = W.tiny_shape(n_layers=1, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=128,
                         intermediate=384, vocab=512)
    a_len = [64, 128, 192]
    pairs = [(0, 200), (1, 200), (1, 200), (2, 200)]
    wts, case, dm, ctx, a_tok, s_tok = _setup(shape, 23, a_len, pairs, B)
    pool = B.quail_anchor_bytes(dm.cfg, 128) + B.quail_anchor_bytes(dm.cfg, 192) + B.GUARD_BYTES
    ctx = dm.context(pool, 400)
    # the plan alone (byte totals) puts C and D in one step
    order, bounds, peak = B.quail_plan_build(dm.cfg, pool - B.GUARD_BYTES, 400, a_len, case["pair_anchor"],
                                             case["s_len"])
    assert len(bounds) - 1 == 2 and peak == pool - B.GUARD_BYTES
    n = len(pairs)
    logits = torch.empty((n, 8), dtype=torch.float32, device="cuda")
    dec = torch.empty(n, dtype=torch.uint8, device="cuda")
    say("fragmented pool: join_run", n, "pairs")
    B.quail_join_run(ctx, a_tok, case["a_off"], case["pair_anchor"], s_tok, case["s_off"], 0x0F,
                     logits, None, dec)
    torch.cuda.synchronize()
    ref = [OM.forward_pair(case["a_tok"][case["a_off"][a]:case["a_off"][a + 1]],
                           case["s_tok"][case["s_off"][i]:case["s_off"][i + 1]], wts, shape)
           for i, (a, _) in enumerate(pairs)]
    ref_logits = np.array([r["logits"] for r in ref])
    assert rel_inf(logits.cpu().numpy(), ref_logits) <= 2e-2
    ok, _ = decisions_agree(dec.cpu().numpy(), [r["decision"] for r in ref], [r["margin"] for r in ref],
                            2e-2 * np.max(np.abs(ref_logits)))
    assert ok
    st = B.quail_pool_stats(ctx)
    assert st["prefills"] == 3 and st["evictions"] == 3 and st["regret_tokens"] == 0 and st["resident"] == 0


def test_out_of_range_token_ids_are_counted_not_read(B):
    """Token ids outside [0, vocab) are a caller error: the embedding counts
    each one in the context's debug counter and reads row 0 instead (never
    outside the table); every in-range pair is unaffected."""
    import torch
    from query_aware_prefill_amd.device import to_device
    shape = W.tiny_shape(n_layers=1, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=128,
                         intermediate=384, vocab=512)
    pairs = [(0, 5), (-1, 6), (0, 7)]
    wts, case, dm, ctx, a_tok, s_tok = _setup(shape, 24, [40], pairs, B)
    bad = case["s_tok"].copy()
    o = case["s_off"]
    bad[o[1] + 2] = shape.vocab + 5          # filter row: one id past the table
    bad[o[1] + 4] = -3                       # and a negative one
    n = len(pairs)
    logits = torch.empty((n, 8), dtype=torch.float32, device="cuda")
    dec = torch.empty(n, dtype=torch.uint8, device="cuda")
    say("out-of-range token ids")
    B.quail_join_run(ctx, a_tok, case["a_off"], case["pair_anchor"], to_device(bad), o, 0x0F, logits, None, dec)
    torch.cuda.synchronize()
    chk = B.quail_ctx_check(ctx)
    assert chk == {"guard_errors": 0, "bad_tokens": 2}, chk
    ctx.expect_counts = chk
    lg = logits.cpu().numpy()
    assert np.all(np.isfinite(lg))
    for i in (0, 2):
        ref = OM.forward_pair(case["a_tok"], case["s_tok"][o[i]:o[i + 1]], wts, shape)
        assert rel_inf(lg[i], ref["logits"]) <= 2e-2


def test_overwritten_guard_is_detected(B):
    """The guard region after a live slab, overwritten from the host, is
    reported by quail_ctx_check; an intact pool reports nothing."""
    import torch
    shape = W.tiny_shape(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=128,
                         intermediate=384, vocab=512)
    wts, case, dm, ctx, a_tok, s_tok = _setup(shape, 25, [30, 100], [(0, 3), (1, 4)], B)
    h = B.quail_anchor_prefill(ctx, a_tok, case["a_off"], [1, 1])
    torch.cuda.synchronize()
    assert B.quail_ctx_check(ctx) == {"guard_errors": 0, "bad_tokens": 0}
    # the guard follows the last layer's V block of the slab
    kp, vp, la, lap = B.quail_anchor_kv(ctx, h[1], shape.n_layers - 1)
    guard = vp + shape.n_kv_heads * lap * shape.head_dim * 2 - ctx._pool.data_ptr()
    ctx._pool[guard + 8] ^= 0xFF
    torch.cuda.synchronize()
    chk = B.quail_ctx_check(ctx)
    assert chk == {"guard_errors": 1, "bad_tokens": 0}, chk
    ctx.expect_counts = {"guard_errors": 2, "bad_tokens": 0}   # checked again at teardown


@pytest.mark.parametrize("kv_fp8", [False, True])
def test_join_with_packed_multiwave_tiles(B, kv_fp8):
    """Pairs so short that every anchor's run of query tokens in a batch fits
    two waves of packed rows (G = 2: 16 tokens per wave; runs of 17-32 tokens),
    so the join's attention runs packed tiles of two waves, with several
    16-key self tiles per tile when the slabs are E4M3: logits and decisions
    against the oracle."""
    import torch
    shape = W.tiny_shape(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=128,
                         intermediate=384, vocab=512, kv_fp8=kv_fp8)
    a_len = [40, 97, 3]
    pairs = [(0, 20), (0, 12), (1, 9), (1, 8), (1, 11), (2, 30), (-1, 7)]
    wts, case, dm, ctx, a_tok, s_tok = _setup(shape, 26, a_len, pairs, B)
    n = len(pairs)
    logits = torch.empty((n, 8), dtype=torch.float32, device="cuda")
    dec = torch.empty(n, dtype=torch.uint8, device="cuda")
    say("packed multi-wave join", "fp8" if kv_fp8 else "bf16")
    B.quail_join_run(ctx, a_tok, case["a_off"], case["pair_anchor"], s_tok, case["s_off"], 0x0F,
                     logits, None, dec)
    torch.cuda.synchronize()
    ref = []
    for i, (a, _) in enumerate(pairs):
        at = case["a_tok"][case["a_off"][a]:case["a_off"][a + 1]] if a >= 0 else []
        ref.append(OM.forward_pair(at, case["s_tok"][case["s_off"][i]:case["s_off"][i + 1]], wts, shape))
    ref_logits = np.array([r["logits"] for r in ref])
    lg = logits.cpu().numpy()
    for i in range(n):
        assert rel_inf(lg[i], ref_logits[i]) <= 2e-2 * np.max(np.abs(ref_logits)) / np.max(np.abs(ref_logits[i])), i
    assert rel_inf(lg, ref_logits) <= 2e-2
    ok, _ = decisions_agree(dec.cpu().numpy(), [r["decision"] for r in ref], [r["margin"] for r in ref],
                            2e-2 * np.max(np.abs(ref_logits)))
    assert ok
