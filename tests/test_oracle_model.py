"""Pins for oracle/model.py: library RMSNorm/SiLU, RoPE properties, one decoder
layer against the transformers library's Llama decoder layer (float64), the
8-column head against the same columns of a full head, argmax tie-break,
anchor-KV independence from the suffix, and the whole stack against the
transformers library's Llama causal LM (float64)."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import codecs, model as M


def test_rmsnorm_matches_torch():
    r = np.random.default_rng(0)
    x = r.standard_normal((7, 96))
    g = 1 + 0.1 * r.standard_normal(96)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (96,), torch.from_numpy(g), eps=1e-6)
    assert np.max(np.abs(M.rmsnorm(x, g, 1e-6) - ref.numpy())) < 1e-13
    u = M.rmsnorm(x, np.ones(96), 0.0)
    assert np.allclose(np.sqrt(np.mean(u * u, axis=1)), 1.0, atol=1e-13)


def test_silu_matches_torch():
    t = np.linspace(-30, 30, 1001)
    ref = torch.nn.functional.silu(torch.from_numpy(t)).numpy()
    assert np.max(np.abs(M.silu(t) - ref)) < 1e-13


def test_rope_properties():
    r = np.random.default_rng(1)
    d = 128
    x = r.standard_normal((5, 3, d))
    # position 0 is the identity
    assert np.array_equal(M.rope(x, np.zeros(5, int), 1e6), x)
    # each rotated pair (i, i + d/2) keeps its norm
    y = M.rope(x, np.arange(5) * 977, 1e6)
    n0 = x[..., :64] ** 2 + x[..., 64:] ** 2
    n1 = y[..., :64] ** 2 + y[..., 64:] ** 2
    assert np.max(np.abs(n0 - n1)) < 1e-12
    # relative: <R_p q, R_p' k> = <R_(p-p') q, k>
    q = r.standard_normal((1, 1, d))
    k = r.standard_normal((1, 1, d))
    for p, pp in [(5, 2), (1500, 3), (3000, 2999)]:
        lhs = float(np.sum(M.rope(q, [p], 1e6) * M.rope(k, [pp], 1e6)))
        rhs = float(np.sum(M.rope(q, [p - pp], 1e6) * k))
        assert abs(lhs - rhs) < 1e-10
    # inverse frequency of pair i is theta^(-2i/d): at p = 1, the first pair
    # rotates by exactly 1 radian
    e = np.zeros((1, 1, d)); e[0, 0, 0] = 1.0
    y = M.rope(e, [1], 1e6)
    assert abs(y[0, 0, 0] - math.cos(1.0)) < 1e-15 and abs(y[0, 0, 64] - math.sin(1.0)) < 1e-15


def _tiny_layer_case(seed=0, n=12):
    shape = W.tiny_shape(n_layers=1, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                         intermediate=384, vocab=64)
    wts = W.model_weights(shape, seed)
    return shape, wts


def test_decoder_layer_exact_matches_transformers_llama_layer():
    from transformers import LlamaConfig
    from transformers.models.llama import modeling_llama as ml
    shape, wts = _tiny_layer_case()
    lw = M.LayerWeights(wts["layers"][0], shape)
    cfg = LlamaConfig(hidden_size=shape.hidden, intermediate_size=shape.intermediate,
                      num_attention_heads=shape.n_q_heads, num_key_value_heads=shape.n_kv_heads,
                      head_dim=shape.head_dim, rms_norm_eps=shape.rms_eps, rope_theta=shape.rope_theta,
                      max_position_embeddings=8192, attention_bias=False, mlp_bias=False,
                      vocab_size=shape.vocab, num_hidden_layers=1)
    cfg._attn_implementation = "sdpa"
    layer = ml.LlamaDecoderLayer(cfg, layer_idx=0).double()
    rot = ml.LlamaRotaryEmbedding(cfg).double()
    qd, kd = shape.q_dim, shape.kv_dim
    with torch.no_grad():
        layer.self_attn.q_proj.weight.copy_(torch.from_numpy(lw.w_qkv[:qd]))
        layer.self_attn.k_proj.weight.copy_(torch.from_numpy(lw.w_qkv[qd:qd + kd]))
        layer.self_attn.v_proj.weight.copy_(torch.from_numpy(lw.w_qkv[qd + kd:]))
        layer.self_attn.o_proj.weight.copy_(torch.from_numpy(lw.w_o))
        layer.mlp.gate_proj.weight.copy_(torch.from_numpy(lw.w_gate))
        layer.mlp.up_proj.weight.copy_(torch.from_numpy(lw.w_up))
        layer.mlp.down_proj.weight.copy_(torch.from_numpy(lw.w_down))
        layer.input_layernorm.weight.copy_(torch.from_numpy(lw.attn_norm))
        layer.post_attention_layernorm.weight.copy_(torch.from_numpy(lw.mlp_norm))
    r = np.random.default_rng(3)
    n = 40
    h = r.standard_normal((n, shape.hidden))
    base = 700  # non-zero start position exercises RoPE angles
    pos = np.arange(base, base + n)
    ours = M.decoder_layer(h, pos, lw, shape, mode="exact")
    with torch.no_grad():
        x = torch.from_numpy(h)[None]
        pid = torch.from_numpy(pos)[None]
        ref = layer(x, attention_mask=None, position_ids=pid, position_embeddings=rot(x, pid))[0].numpy()
        # the library layer must be causal here: changing the last row leaves earlier rows
        x2 = x.clone(); x2[0, -1] += 1.0
        ref2 = layer(x2, attention_mask=None, position_ids=pid, position_embeddings=rot(x2, pid))[0].numpy()
    assert np.array_equal(ref[:-1], ref2[:-1])
    rel = np.max(np.abs(ours - ref)) / np.max(np.abs(ref))
    # transformers computes its inverse frequencies in float32 (relative 6e-8
    # per angle, times positions up to ~740)
    assert rel < 1e-5, rel


def test_contract_mode_rounds_and_stays_close_to_exact():
    shape, wts = _tiny_layer_case(seed=1)
    toks = np.random.default_rng(2).integers(0, shape.vocab, 20)
    he = M.forward_tokens(toks, wts, shape, mode="exact")
    hc, kv = M.forward_tokens(toks, wts, shape, mode="contract", return_kv=True)
    k, v = kv[0][0], kv[0][1]
    assert np.array_equal(codecs.bf16_round(k), k) and np.array_equal(codecs.bf16_round(v), v)  # bf16 K/V
    assert not np.array_equal(codecs.bf16_round(hc), hc)   # the residual stream is not rounded
    assert np.max(np.abs(he - hc)) / np.max(np.abs(he)) < 2e-2
    assert not np.array_equal(he, hc)


def test_head8_equals_columns_of_full_head():
    shape = W.tiny_shape(hidden=256, vocab=64)
    r = np.random.default_rng(4)
    full = W.full_head(shape, seed=3, vocab=64)             # [H, 64] bf16 bits
    cols = np.array([3, 17, 0, 63, 22, 41, 8, 50])
    gamma = W.draw_bf16(r, (256,), std=0.1, mean=1.0)
    h = r.standard_normal((9, 256)) * 3
    logits, tok, dec, margin = M.head8(h, gamma, full[:, cols], 0x0F, shape, mode="exact")
    # full head with the library: rms_norm then matmul, then take the 8 columns
    ht = torch.from_numpy(h)
    z = torch.nn.functional.rms_norm(ht, (256,), torch.from_numpy(codecs.bf16_value(gamma)), eps=1e-6)
    full_logits = (z @ torch.from_numpy(codecs.bf16_value(full))).numpy()
    assert np.max(np.abs(logits - full_logits[:, cols])) < 1e-12


def test_decide_first_max_tie_break_and_margin():
    logits = np.array([[1.0, 3.0, 3.0, 0.0, 0, 0, 0, 0],     # tie 1/2 -> 1 (TRUE col)
                       [0.0, 0, 0, 0, 5.0, 5.0, 0, 0],        # tie 4/5 -> 4 (FALSE col)
                       [2.0, 0, 0, 0, 0, 0, 0, 2.5]])         # 7 (FALSE)
    tok, dec, margin = M.decide(logits, 0x0F)
    assert tok.tolist() == [1, 4, 7]
    assert dec.tolist() == [1, 0, 0]
    assert np.allclose(margin, [3.0, -5.0, -0.5])
    tok, dec, _ = M.decide(logits, 0x10)
    assert dec.tolist() == [0, 1, 0]


def test_anchor_kv_independent_of_suffix():
    shape = W.tiny_shape(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                         intermediate=384, vocab=64)
    wts = W.model_weights(shape, 5)
    r = np.random.default_rng(6)
    a = r.integers(0, 64, 13)
    s1, s2 = r.integers(0, 64, 5), r.integers(0, 64, 9)
    for mode in ("exact", "contract"):
        _, kv0 = M.forward_tokens(a, wts, shape, mode=mode, return_kv=True)
        _, kv1 = M.forward_tokens(np.concatenate([a, s1]), wts, shape, mode=mode, return_kv=True)
        _, kv2 = M.forward_tokens(np.concatenate([a, s2]), wts, shape, mode=mode, return_kv=True)
        # equal up to the BLAS summation order of different-height products
        # (exact mode), or up to rare one-ulp bf16 flips that order causes
        tol = 1e-12 if mode == "exact" else 1e-2
        for l in range(2):
            for t in range(2):
                for other in (kv1, kv2):
                    diff = np.max(np.abs(kv0[l][t] - other[l][t][:13]))
                    assert diff <= tol * np.max(np.abs(kv0[l][t])), (mode, l, t, diff)


def test_fp8_kv_applies_to_anchor_positions_only():
    shape = W.tiny_shape(n_layers=1, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                         intermediate=384, vocab=64, kv_fp8=True)
    wts = W.model_weights(shape, 7)
    lw = M.LayerWeights(wts["layers"][0], shape)
    h = M.embed(np.arange(10), wts)
    _, (k, v, kp, vp) = M.decoder_layer(h, np.arange(10), lw, shape, "contract", fp8_kv_upto=6,
                                        return_kv=True)
    _, (k0, v0, _, _) = M.decoder_layer(h, np.arange(10), lw, shape, "contract", fp8_kv_upto=0,
                                        return_kv=True)
    assert np.array_equal(kp, k0) and np.array_equal(vp, v0)
    assert np.array_equal(k[6:], k0[6:]) and np.array_equal(v[6:], v0[6:])
    assert np.array_equal(k[:6], codecs.e4m3_roundtrip(k0[:6]))
    assert not np.array_equal(k[:6], k0[:6])


def test_forward_pair_filter_row_and_decision_consistency():
    shape = W.tiny_shape(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                         intermediate=384, vocab=64)
    wts = W.model_weights(shape, 8)
    r = np.random.default_rng(9)
    out = M.forward_pair([], r.integers(0, 64, 7), wts, shape, true_mask=0x0F)
    assert out["token"] == int(np.argmax(out["logits"]))
    assert out["decision"] == (0x0F >> out["token"]) & 1
    a, s = r.integers(0, 64, 11), r.integers(0, 64, 4)
    o1 = M.forward_pair(a, s, wts, shape)
    h = M.forward_tokens(np.concatenate([a, s]), wts, shape)
    assert np.array_equal(o1["h_last"], codecs.bf16_round(h[-1]))   # handed to the head as bf16


def test_stack_exact_matches_transformers_llama_model():
    """The composition: embedding lookup, several decoder layers over
    [anchor | suffix] at positions 0..N-1, the final RMSNorm and the head at
    the last position, against the transformers library's Llama causal LM in
    float64 whose first 8 vocabulary rows are the 8-column head (the other
    rows zero) -- so a mistake in the stacking (a layer skipped or repeated,
    the positions, the final norm, the row the head reads) fails here."""
    from transformers import LlamaConfig, LlamaForCausalLM
    shape = W.tiny_shape(n_layers=3, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                         intermediate=384, vocab=64)
    wts = W.model_weights(shape, 5)
    cfg = LlamaConfig(hidden_size=shape.hidden, intermediate_size=shape.intermediate,
                      num_attention_heads=shape.n_q_heads, num_key_value_heads=shape.n_kv_heads,
                      head_dim=shape.head_dim, rms_norm_eps=shape.rms_eps, rope_theta=shape.rope_theta,
                      max_position_embeddings=8192, attention_bias=False, mlp_bias=False,
                      vocab_size=shape.vocab, num_hidden_layers=shape.n_layers, tie_word_embeddings=False)
    cfg._attn_implementation = "sdpa"
    lm = LlamaForCausalLM(cfg).double().eval()
    qd, kd = shape.q_dim, shape.kv_dim
    with torch.no_grad():
        lm.model.embed_tokens.weight.copy_(torch.from_numpy(codecs.bf16_value(wts["embed"])))
        for l, layer in enumerate(lm.model.layers):
            lw = M.LayerWeights(wts["layers"][l], shape)
            layer.self_attn.q_proj.weight.copy_(torch.from_numpy(lw.w_qkv[:qd]))
            layer.self_attn.k_proj.weight.copy_(torch.from_numpy(lw.w_qkv[qd:qd + kd]))
            layer.self_attn.v_proj.weight.copy_(torch.from_numpy(lw.w_qkv[qd + kd:]))
            layer.self_attn.o_proj.weight.copy_(torch.from_numpy(lw.w_o))
            layer.mlp.gate_proj.weight.copy_(torch.from_numpy(lw.w_gate))
            layer.mlp.up_proj.weight.copy_(torch.from_numpy(lw.w_up))
            layer.mlp.down_proj.weight.copy_(torch.from_numpy(lw.w_down))
            layer.input_layernorm.weight.copy_(torch.from_numpy(lw.attn_norm))
            layer.post_attention_layernorm.weight.copy_(torch.from_numpy(lw.mlp_norm))
        lm.model.norm.weight.copy_(torch.from_numpy(codecs.bf16_value(wts["final_norm"])))
        head = np.zeros((shape.vocab, shape.hidden))
        head[:8] = codecs.bf16_value(wts["head8"]).T
        lm.lm_head.weight.copy_(torch.from_numpy(head))
    r = np.random.default_rng(11)
    for a_len, s_len in [(23, 9), (0, 17), (40, 1)]:
        a = r.integers(0, shape.vocab, a_len)
        s = r.integers(0, shape.vocab, s_len)
        ours = M.forward_pair(a, s, wts, shape, true_mask=0x0F, mode="exact")
        with torch.no_grad():
            ids = torch.from_numpy(np.concatenate([a, s]).astype(np.int64))[None]
            ref = lm(input_ids=ids).logits[0, -1, :8].numpy()
        rel = np.max(np.abs(ours["logits"] - ref)) / np.max(np.abs(ref))
        assert rel < 1e-5, (a_len, s_len, rel)
        tok, dec, _ = M.decide(ref[None], 0x0F)
        assert ours["token"] == int(tok[0]) and ours["decision"] == int(dec[0])


def test_forward_many_equals_forward_pair():
    """The batched form is the per-pair definition applied to each sequence:
    the same logits, tokens and decisions as forward_pair for every sequence
    (joins, a filter row, fp8 anchor K/V on some sequences), and each tapped
    depth d equals forward_pair truncated to d layers. A position that ran on
    across sequences, a row mixed into another sequence's attention, or an
    fp8 store applied to the wrong rows fails here."""
    shape = W.tiny_shape(n_layers=3, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                         intermediate=384, vocab=64, kv_fp8=True)
    wts = W.model_weights(shape, 21)
    r = np.random.default_rng(22)
    pairs = [(r.integers(0, 64, 19), r.integers(0, 64, 5)), ([], r.integers(0, 64, 11)),
             (r.integers(0, 64, 7), r.integers(0, 64, 1)), (r.integers(0, 64, 30), r.integers(0, 64, 12))]
    seqs = [np.concatenate([np.asarray(a, np.int64), s]) for a, s in pairs]
    upto = [len(a) for a, _ in pairs]
    for mode in ("exact", "contract"):
        got = M.forward_many(seqs, wts, shape, mode=mode, fp8_kv_upto=upto, taps=(1, 2))
        for depth in (1, 2, 3):
            g = got if depth == 3 else got[depth]
            for i, (a, s) in enumerate(pairs):
                ref = M.forward_pair(a, s, wts, shape, mode=mode, n_layers=depth)
                rel = np.max(np.abs(g["logits"][i] - ref["logits"])) / np.max(np.abs(ref["logits"]))
                # exact: equal up to BLAS summation order; contract: also up to
                # the rare one-ulp bf16 flip that order causes
                assert rel <= (1e-12 if mode == "exact" else 2e-2), (mode, depth, i, rel)
                if mode == "exact":
                    assert g["token"][i] == ref["token"] and g["decision"][i] == ref["decision"]
    # without fp8 rows it is the bf16-KV definition again
    plain = W.tiny_shape(n_layers=3, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                         intermediate=384, vocab=64)
    got = M.forward_many(seqs, wts, plain, mode="exact")
    for i, (a, s) in enumerate(pairs):
        ref = M.forward_pair(a, s, wts, plain, mode="exact")
        assert np.max(np.abs(got["logits"][i] - ref["logits"])) <= 1e-12 * np.max(np.abs(ref["logits"]))


def test_depth_scaled_residual_projections():
    """The random-init reading: QKV and gate/up weights have std 0.02, the
    residual-writing O and down projections 0.02 / sqrt(2 * n_layers)."""
    shape = W.tiny_shape(n_layers=8, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                         intermediate=384, vocab=64)
    lw = M.LayerWeights(W.layer_weights(shape, 3, 0), shape)
    for w, std in ((lw.w_qkv, 0.02), (lw.w_gate, 0.02), (lw.w_up, 0.02),
                   (lw.w_o, 0.02 / 4.0), (lw.w_down, 0.02 / 4.0)):
        assert abs(np.std(w) / std - 1.0) < 0.15, (np.std(w), std)


def _w8a8_case():
    shape = W.tiny_shape(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                         intermediate=384, vocab=64, act_fp8=True)
    wts = W.model_weights(shape, 31)
    r = np.random.default_rng(32)
    pairs = [(r.integers(0, 64, 17), r.integers(0, 64, 6)), ([], r.integers(0, 64, 9)),
             (r.integers(0, 64, 25), r.integers(0, 64, 3))]
    return shape, wts, pairs


def test_w8a8_batched_and_per_pair_forms_agree():
    """With act_fp8 the stacked forward and the per-pair forward give the same
    logits: each token's scale is its own row's, so stacking sequences into
    one matrix changes nothing. A scale taken over the wrong axis (per column
    or per matrix) fails here."""
    shape, wts, pairs = _w8a8_case()
    seqs = [np.concatenate([np.asarray(a, np.int64), s]) for a, s in pairs]
    got = M.forward_many(seqs, wts, shape, mode="exact")
    for i, (a, s) in enumerate(pairs):
        ref = M.forward_pair(a, s, wts, shape, mode="exact")
        assert np.max(np.abs(got["logits"][i] - ref["logits"])) <= 1e-12 * np.max(np.abs(ref["logits"]))


def test_w8a8_every_quantisation_point_is_applied(monkeypatch):
    """Dropping any one of the four quantised projection inputs changes the
    hidden states; all four together move them from the W8A16 result by
    about what E4M3 rounding (3 mantissa bits, per-token scale) allows: more
    than 0.1% and less than 5% after two layers."""
    shape, wts, pairs = _w8a8_case()
    a, s = pairs[0]
    full = M.forward_pair(a, s, wts, shape)["h"]
    import dataclasses
    w16 = M.forward_pair(a, s, wts, dataclasses.replace(shape, act_fp8=False))["h"]
    rel = np.max(np.abs(full - w16)) / np.max(np.abs(w16))
    assert 1e-3 < rel < 5e-2, rel
    for point in sorted(M.ACT_POINTS):
        monkeypatch.setattr(M, "ACT_POINTS", M.ACT_POINTS - {point})
        part = M.forward_pair(a, s, wts, shape)["h"]
        monkeypatch.undo()
        assert np.max(np.abs(part - full)) > 1e-6 * np.max(np.abs(full)), point
