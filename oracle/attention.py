"""Attention: the monolithic definition, and the cascade form the method uses.

Test infrastructure (see the package header).

[pt] "Como funciona", bullet on simplified cascade attention: for joins the
suffixes attend to the anchor (cross-attention), then to themselves, and the
two results are combined by LSE rescaling. Readings taken where the page is
silent:
  * masks: a suffix token sees every anchor token and the suffix tokens up to
    and including itself; an anchor token sees the anchor causally and never a
    suffix (so its K/V do not depend on the suffix);
  * softmax scale 1/sqrt(d); LSE in natural log;
  * GQA groups are contiguous: query head h reads KV head h // (Hq / Hkv);
  * merge of partials (O_i, L_i): L = log(sum_i exp(L_i)),
    O = sum_i exp(L_i - L) O_i; an empty key set has L = -inf and weight 0.

Everything is float64 unless a caller passes float32 arrays for a large case.

Pins (tests/test_oracle_attention.py): the monolithic form against
torch.nn.functional.scaled_dot_product_attention with an explicit mask;
closed forms (constant V, identical keys, two-key softmax); cascade + merge
equal to the monolithic form on brute-force sweeps; merge commutative and
associative over random key splits.
"""
from __future__ import annotations

import numpy as np


def attention_partial(q, k, v, visible, scale):
    """Softmax attention of q over the visible keys.

    q [Nq, Hq, d]; k, v [Nk, Hkv, d]; visible bool [Nq, Nk] (shared by heads).
    Returns O [Nq, Hq, d] and LSE [Nq, Hq]; a row with no visible key has
    O = 0 and LSE = -inf.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    nq, hq, d = q.shape
    hkv = k.shape[1]
    G = hq // hkv
    dt = np.result_type(q.dtype, k.dtype, np.float32)
    O = np.zeros((nq, hq, v.shape[2]), dt)
    L = np.full((nq, hq), -np.inf, dt)
    if nq == 0 or k.shape[0] == 0:
        return O, L
    any_vis = visible.any(axis=1)
    for h in range(hq):
        g = h // G
        s = (q[:, h, :] @ k[:, g, :].T) * scale
        s = np.where(visible, s, -np.inf)
        mx = np.max(s, axis=1, initial=-np.inf)
        mx_safe = np.where(any_vis, mx, 0.0)
        p = np.exp(s - mx_safe[:, None])
        p = np.where(visible, p, 0.0)
        den = p.sum(axis=1)
        den_safe = np.where(any_vis, den, 1.0)
        O[:, h, :] = (p @ v[:, g, :]) / den_safe[:, None]
        L[:, h] = np.where(any_vis, mx_safe + np.log(den_safe), -np.inf)
    return O, L


def causal_visible(q_pos, k_pos):
    """Key j is visible to query i iff k_pos[j] <= q_pos[i]."""
    return np.asarray(k_pos)[None, :] <= np.asarray(q_pos)[:, None]


def attention_causal(q, k, v, scale, q_pos=None, k_pos=None):
    """Causal attention over one sequence (positions 0..N-1 by default)."""
    nq, nk = q.shape[0], k.shape[0]
    q_pos = np.arange(nk - nq, nk) if q_pos is None else q_pos
    k_pos = np.arange(nk) if k_pos is None else k_pos
    return attention_partial(q, k, v, causal_visible(q_pos, k_pos), scale)


def lse_merge(parts):
    """Merge partials [(O_i, L_i), ...] by LSE rescaling."""
    Ls = np.stack([p[1] for p in parts])            # [n, Nq, Hq]
    finite = np.isfinite(Ls)
    mx = np.max(np.where(finite, Ls, -np.inf), axis=0)
    mx_safe = np.where(np.isfinite(mx), mx, 0.0)
    w = np.where(finite, np.exp(Ls - mx_safe[None]), 0.0)
    tot = w.sum(axis=0)
    L = np.where(tot > 0, mx_safe + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
    tot_safe = np.where(tot > 0, tot, 1.0)
    O = sum(w[i][..., None] * parts[i][0] for i in range(len(parts))) / tot_safe[..., None]
    return O, L


def cascade_attention(q, k_anchor, v_anchor, k_suffix, v_suffix, scale):
    """One suffix against its anchor, in the cascade form.

    q [Ls, Hq, d] (suffix queries); anchor keys [La, Hkv, d]; suffix keys
    [Ls, Hkv, d]. Cross partial: every anchor key visible. Self partial:
    causal inside the suffix. Then the LSE merge. Returns (O, LSE).
    """
    ls = q.shape[0]
    la = k_anchor.shape[0]
    cross = attention_partial(q, k_anchor, v_anchor, np.ones((ls, la), bool), scale)
    self_ = attention_partial(q, k_suffix, v_suffix,
                              causal_visible(np.arange(ls), np.arange(ls)), scale)
    return lse_merge([cross, self_])


def cascade_attention_levels(q, levels, k_suffix, v_suffix, scale):
    """Suffix queries against several fully visible key sets, then causally
    against themselves, merged by LSE rescaling.

    ``levels`` = [(K, V), ...] in position order, e.g. the anchor and then a
    prefix shared by several suffixes (a multi-level cascade: every key of an
    earlier level precedes every suffix token, so no mask applies to it).
    q [Ls, Hq, d]; each K, V [n_i, Hkv, d]; suffix keys [Ls, Hkv, d].
    Returns (O, LSE).
    """
    ls = q.shape[0]
    parts = [attention_partial(q, k, v, np.ones((ls, k.shape[0]), bool), scale) for k, v in levels]
    parts.append(attention_partial(q, k_suffix, v_suffix,
                                   causal_visible(np.arange(ls), np.arange(ls)), scale))
    return lse_merge(parts)


def monolithic_pair_attention(q_suffix, k_anchor, v_anchor, k_suffix, v_suffix,
                              scale, q_anchor=None):
    """The definition: causal attention over the concatenation [anchor ‖ suffix],
    output rows of the suffix (and of the anchor if q_anchor is given)."""
    k = np.concatenate([k_anchor, k_suffix], axis=0)
    v = np.concatenate([v_anchor, v_suffix], axis=0)
    la, ls = k_anchor.shape[0], k_suffix.shape[0]
    if q_anchor is None:
        return attention_causal(q_suffix, k, v, scale,
                                q_pos=np.arange(la, la + ls), k_pos=np.arange(la + ls))
    q = np.concatenate([q_anchor, q_suffix], axis=0)
    return attention_causal(q, k, v, scale)


def cascade_case_reference(case, mode="monolithic", suffixes=None):
    """Oracle output for a packed cascade case (see workloads.cascade_case).

    Returns O [sum Ls, Hq, d] and LSE [sum Ls, Hq] (float64) for the listed
    suffixes (all by default; rows of unlisted suffixes are left at 0 / -inf).
    ``mode`` = "monolithic" (the definition) or "cascade".
    """
    f32 = case["dtype"] == "f32"

    def val(x):
        x = np.asarray(x)
        if f32:
            return x.astype(np.float64)
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)

    s_off, a_off, s_anchor = case["s_off"], case["a_off"], case["s_anchor"]
    n_tok = int(s_off[-1])
    hq, d = case["hq"], case["d"]
    O = np.zeros((n_tok, hq, d))
    L = np.full((n_tok, hq), -np.inf)
    idx = range(len(case["s_len"])) if suffixes is None else suffixes
    for s in idx:
        sl = slice(int(s_off[s]), int(s_off[s + 1]))
        q, k, v = val(case["q"][sl]), val(case["k"][sl]), val(case["v"][sl])
        a = int(s_anchor[s])
        if a >= 0:
            al = slice(int(a_off[a]), int(a_off[a + 1]))
            ka, va = val(case["ak"][al]), val(case["av"][al])
        else:
            ka = np.zeros((0,) + k.shape[1:])
            va = np.zeros((0,) + v.shape[1:])
        if mode == "cascade":
            o, l = cascade_attention(q, ka, va, k, v, case["sm_scale"])
        else:
            o, l = monolithic_pair_attention(q, ka, va, k, v, case["sm_scale"])
        O[sl] = o
        L[sl] = l
    return O, L
