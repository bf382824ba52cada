"""Pins for oracle/attention.py: library SDPA, closed forms, and the cascade
identity (cross + self partials merged by LSE == monolithic causal attention
over [anchor ‖ suffix])."""
import itertools
import math

import numpy as np
import pytest
import torch

from oracle import attention as A


def _rand(r, *shape):
    return r.standard_normal(shape)


def _sdpa_reference(q, k, v, visible, scale):
    """torch SDPA in float64 with an explicit boolean mask; GQA expanded by
    repeating each KV head over its contiguous group of query heads."""
    hq, hkv = q.shape[1], k.shape[1]
    G = hq // hkv
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]                       # [1, Hq, Nq, d]
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(G, 0)[None]
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(G, 0)[None]
    m = torch.from_numpy(visible)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    return o[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("hq,hkv,nq,nk", [(4, 2, 9, 13), (4, 4, 1, 5), (8, 2, 17, 17), (4, 1, 3, 30)])
def test_partial_matches_torch_sdpa_with_mask(hq, hkv, nq, nk):
    r = np.random.default_rng(hq * 100 + nk)
    d = 16
    q, k, v = _rand(r, nq, hq, d), _rand(r, nk, hkv, d), _rand(r, nk, hkv, d)
    vis = r.random((nq, nk)) < 0.6
    vis[:, 0] = True
    o, lse = A.attention_partial(q, k, v, vis, 0.25)
    ref = _sdpa_reference(q, k, v, vis, 0.25)
    assert np.max(np.abs(o - ref)) < 1e-12
    # LSE against a direct log-sum-exp for one head
    G = hq // hkv
    for h in range(hq):
        s = (q[:, h] @ k[:, h // G].T) * 0.25
        s = np.where(vis, s, -np.inf)
        ref_l = np.log(np.sum(np.exp(s), axis=1))
        assert np.max(np.abs(lse[:, h] - ref_l)) < 1e-12


def test_causal_la0_matches_sdpa_is_causal():
    r = np.random.default_rng(5)
    q, k, v = _rand(r, 11, 4, 8), _rand(r, 11, 2, 8), _rand(r, 11, 2, 8)
    o, _ = A.attention_causal(q, k, v, 1 / math.sqrt(8))
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(k).permute(1, 0, 2)[None]
    vt = torch.from_numpy(v).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True,
                                                           enable_gqa=True)
    assert np.max(np.abs(o - ref[0].permute(1, 0, 2).numpy())) < 1e-12


def test_closed_form_constant_values():
    r = np.random.default_rng(1)
    q, k = _rand(r, 6, 2, 4), _rand(r, 9, 1, 4)
    v = np.broadcast_to(np.array([1.5, -2.0, 0.25, 7.0]), (9, 1, 4)).copy()
    o, _ = A.attention_causal(q, k, v, 0.5)
    assert np.allclose(o, v[0, 0], atol=1e-14, rtol=0)


def test_closed_form_identical_keys_average_visible_values():
    r = np.random.default_rng(2)
    q = _rand(r, 5, 1, 4)
    k = np.broadcast_to(_rand(r, 1, 1, 4), (5, 1, 4)).copy()
    v = _rand(r, 5, 1, 4)
    o, lse = A.attention_causal(q, k, v, 1.0)
    for i in range(5):
        assert np.allclose(o[i, 0], v[: i + 1, 0].mean(axis=0), atol=1e-14)
        s = float(q[i, 0] @ k[0, 0])
        assert abs(lse[i, 0] - (s + math.log(i + 1))) < 1e-12


def test_closed_form_two_keys_is_logistic():
    # one anchor key and one suffix token: weight of the anchor value = sigma(s1 - s2)
    r = np.random.default_rng(3)
    q = _rand(r, 1, 1, 4)
    ka, va = _rand(r, 1, 1, 4), _rand(r, 1, 1, 4)
    ks, vs = _rand(r, 1, 1, 4), _rand(r, 1, 1, 4)
    o, _ = A.cascade_attention(q, ka, va, ks, vs, 0.5)
    s1, s2 = 0.5 * float(q[0, 0] @ ka[0, 0]), 0.5 * float(q[0, 0] @ ks[0, 0])
    w = 1.0 / (1.0 + math.exp(-(s1 - s2)))
    assert np.allclose(o[0, 0], w * va[0, 0] + (1 - w) * vs[0, 0], atol=1e-14)


@pytest.mark.parametrize("la,ls,G", list(itertools.product([0, 1, 7, 64], [1, 2, 33], [1, 2, 4])))
def test_cascade_equals_monolithic(la, ls, G):
    r = np.random.default_rng(la * 1000 + ls * 10 + G)
    hkv, d = 2, 8
    hq = hkv * G
    q = _rand(r, ls, hq, d)
    ka, va = _rand(r, la, hkv, d), _rand(r, la, hkv, d)
    ks, vs = _rand(r, ls, hkv, d), _rand(r, ls, hkv, d)
    oc, lc = A.cascade_attention(q, ka, va, ks, vs, 1 / math.sqrt(d))
    om, lm = A.monolithic_pair_attention(q, ka, va, ks, vs, 1 / math.sqrt(d))
    assert np.max(np.abs(oc - om)) < 1e-12
    assert np.max(np.abs(lc - lm)) < 1e-12


def test_merge_commutative_and_associative_over_random_splits():
    r = np.random.default_rng(11)
    nq, nk, hq, hkv, d = 7, 40, 4, 2, 8
    q, k, v = _rand(r, nq, hq, d), _rand(r, nk, hkv, d), _rand(r, nk, hkv, d)
    full = A.attention_partial(q, k, v, np.ones((nq, nk), bool), 0.3)
    for trial in range(20):
        cuts = np.sort(r.choice(np.arange(1, nk), size=r.integers(1, 5), replace=False))
        bounds = [0, *cuts.tolist(), nk]
        parts = []
        for a, b in zip(bounds[:-1], bounds[1:]):
            vis = np.zeros((nq, nk), bool)
            vis[:, a:b] = True
            parts.append(A.attention_partial(q, k, v, vis, 0.3))
        o1, l1 = A.lse_merge(parts)
        perm = r.permutation(len(parts))
        o2, l2 = A.lse_merge([parts[i] for i in perm])
        # nested: merge the first two, then the rest
        if len(parts) >= 3:
            o3, l3 = A.lse_merge([A.lse_merge(parts[:2]), *parts[2:]])
            assert np.max(np.abs(o3 - full[0])) < 1e-12
        for o, l in ((o1, l1), (o2, l2)):
            assert np.max(np.abs(o - full[0])) < 1e-12
            assert np.max(np.abs(l - full[1])) < 1e-12


def test_empty_partial_has_zero_weight():
    r = np.random.default_rng(4)
    q, k, v = _rand(r, 3, 2, 4), _rand(r, 5, 1, 4), _rand(r, 5, 1, 4)
    empty = A.attention_partial(q, k[:0], v[:0], np.zeros((3, 0), bool), 1.0)
    assert np.all(np.isneginf(empty[1])) and np.all(empty[0] == 0)
    full = A.attention_partial(q, k, v, np.ones((3, 5), bool), 1.0)
    o, l = A.lse_merge([empty, full])
    assert np.array_equal(o, full[0]) and np.array_equal(l, full[1])


def test_planted_gqa_mistake_is_caught():
    """A GQA map h % Hkv (instead of h // G) must disagree with the SDPA pin."""
    r = np.random.default_rng(9)
    q, k, v = _rand(r, 4, 4, 8), _rand(r, 6, 2, 8), _rand(r, 6, 2, 8)
    vis = np.ones((4, 6), bool)
    ref = _sdpa_reference(q, k, v, vis, 0.3)
    wrong = np.stack([A.attention_partial(q[:, h:h + 1], k[:, h % 2:h % 2 + 1],
                                          v[:, h % 2:h % 2 + 1], vis, 0.3)[0][:, 0]
                      for h in range(4)], axis=1)
    assert np.max(np.abs(wrong - ref)) > 1e-3


@pytest.mark.parametrize("la,lp,ls,G", [(1, 1, 1, 1), (7, 64, 2, 2), (64, 7, 33, 4), (65, 1, 2, 2),
                                        (1, 33, 33, 1)])
def test_two_level_cascade_equals_monolithic(la, lp, ls, G):
    """anchor -> shared prefix -> suffix: two fully visible levels and the
    causal suffix, merged by LSE, equal causal attention over the concatenation
    (and the two-level cascade with anchor and prefix as one level)."""
    r = np.random.default_rng(la * 1000 + lp * 10 + ls)
    hkv, d = 2, 16
    hq = hkv * G
    ka, va = _rand(r, la, hkv, d), _rand(r, la, hkv, d)
    kp, vp = _rand(r, lp, hkv, d), _rand(r, lp, hkv, d)
    q, ks, vs = _rand(r, ls, hq, d), _rand(r, ls, hkv, d), _rand(r, ls, hkv, d)
    o, lse = A.cascade_attention_levels(q, [(ka, va), (kp, vp)], ks, vs, 0.3)
    n = la + lp + ls
    k = np.concatenate([ka, kp, ks]); v = np.concatenate([va, vp, vs])
    om, lm = A.attention_causal(q, k, v, 0.3, q_pos=np.arange(la + lp, n), k_pos=np.arange(n))
    assert np.max(np.abs(o - om)) < 1e-12 and np.max(np.abs(lse - lm)) < 1e-12
    o1, l1 = A.cascade_attention(q, np.concatenate([ka, kp]), np.concatenate([va, vp]), ks, vs, 0.3)
    assert np.max(np.abs(o - o1)) < 1e-12 and np.max(np.abs(lse - l1)) < 1e-12
    # the SDPA pin on the same visibility
    vis = np.arange(n)[None, :] <= np.arange(la + lp, n)[:, None]
    assert np.max(np.abs(o - _sdpa_reference(q, k, v, vis, 0.3))) < 1e-12
