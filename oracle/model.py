"""The decoder forward pass, the 8-column head and the AI.IF boolean.

Test infrastructure (see the package header).

What the pages fix: the engine runs prefill only and the final prefill
position emits one token ([pt] "Como funciona", zero-decode bullet; [fa]
"no decode stage, the last prefill pass predicts one token"); the output head
keeps 8 vocabulary columns ([pt] same section, last bullet; [fa] key points);
the model is Qwen3 4B with FP8 weights on one GPU ([it] second paragraph; [fa]
key points). The per-pair definition evaluated here is the monolithic causal
forward over [anchor ‖ suffix].

Readings where the pages are silent (all standard for this model family):
  * RMSNorm: x / sqrt(mean(x^2) + eps) * gamma, eps = 1e-6, over the hidden dim;
  * RoPE: rotate-half pairing (i, i + d/2), inverse frequency theta^(-2i/d),
    theta = 1e6, angles in float64; a suffix token j of a pair sits at
    position La + j;
  * GQA with contiguous groups; no QK-norm;
  * SwiGLU: silu(x W_gate^T) * (x W_up^T); the fused weight stacks the gate
    rows first, then the up rows;
  * FP8 weights with one bf16 scale per output row: W_eff = decode(code) *
    scale (exact in float64);
  * a final RMSNorm precedes the head; logits are not rounded;
  * the boolean: ``true_mask`` bit j marks column j as a TRUE answer; the token
    is the first maximum of the 8 logits; decision = (true_mask >> token) & 1;
    the margin is the best TRUE logit minus the best FALSE logit;
  * fp8 anchor KV (multi-join configuration): the anchor's post-RoPE K and its
    V are stored as E4M3 codes of k / k_scale and v / v_scale, and every
    reader (the anchor itself and all suffixes) sees the decoded values.
  * W8A8 (shape.act_fp8, off by default): the four projections read their
    activations (u before QKV and before gate/up, o, m) as per-token E4M3
    codes times the token's scale (oracle/w8a8.py), quantised from the values
    the W8A16 pipeline hands them; nothing else changes.

Precision modes:
  * "contract": round to bf16 exactly where a bf16 tensor exists in the
    pipeline: the activations every projection reads (the normed input u,
    the attention output o, the MLP product m), the post-RoPE q/k/v, the last
    position's hidden state handed to the head (h_last) and the normed head
    input z. The residual stream itself -- the running sum the O and down
    projections add into -- is not an activation any projection reads and
    is kept unrounded (the GPU keeps it in fp32). Everything between those
    points is float64 (or float32 for large cases when the caller asks).
  * "exact": no bf16 rounding at all (inputs are still bf16/fp8 values).

Pins (tests/test_oracle_model.py): RMSNorm and SiLU against torch; RoPE at
position 0 is the identity, preserves pair norms and is relative
(<R_p q, R_p' k> = <R_(p-p') q, k>); one decoder layer in "exact" mode against
the transformers library's Llama decoder layer (rotate-half RoPE, RMSNorm,
SwiGLU, GQA) in float64; the 8-column head equals the same columns of a full
head; argmax tie-break; anchor K/V independent of the suffix; the whole
stack (embedding, three decoder layers over [anchor | suffix], final norm, the
head at the last position) in "exact" mode against the transformers library's
Llama causal LM in float64 whose first 8 vocabulary rows are the 8-column
head. The 36-layer stack is the same loop at a larger count. W8A8: the
batched and per-pair forms agree with act_fp8 on; dropping any one of the
four quantisation points changes the result; the whole effect stays within
the few-percent size that E4M3's 3 mantissa bits allow.
"""
from __future__ import annotations

import numpy as np

from . import codecs, w8a8
from .attention import attention_causal

# projection inputs that the W8A8 reading quantises (all four; the pins drop
# one at a time to show each is applied)
ACT_POINTS = frozenset({"qkv", "o", "gate_up", "down"})


def _aq(x, shape, point):
    """What a projection reads: with per-token E4M3 activations
    (shape.act_fp8) the dequantised per-token codes of x, else x itself."""
    if not getattr(shape, "act_fp8", False) or point not in ACT_POINTS:
        return x
    codes, scale = w8a8.act_quant_e4m3(np.asarray(x, np.float32))
    return w8a8.act_dequant(codes, scale).astype(x.dtype)


def _bf(x, mode):
    return codecs.bf16_round(x) if mode == "contract" else x


def weight_eff(codes, scale_bits, dtype=np.float64):
    """W_eff[o, i] = decode(codes[o, i]) * scale[o]. The decode is looked up
    in the 256-entry table of e4m3_decode over every code (same values)."""
    table = codecs.e4m3_decode(np.arange(256, dtype=np.uint8))
    w = table[np.asarray(codes, np.uint8)] * codecs.bf16_value(scale_bits)[:, None]
    return w.astype(dtype)


def rmsnorm(x, gamma, eps):
    x = np.asarray(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * gamma


def silu(t):
    return t / (1.0 + np.exp(-t))


def rope(x, pos, theta):
    """Rotate-half RoPE on x [N, heads, d] at integer positions pos [N]."""
    d = x.shape[-1]
    half = d // 2
    inv = theta ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    ang = np.asarray(pos, np.float64)[:, None] * inv[None, :]      # [N, half]
    c = np.cos(ang)[:, None, :].astype(x.dtype)
    s = np.sin(ang)[:, None, :].astype(x.dtype)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


class LayerWeights:
    """Dequantised views of one layer's weights (float64 or float32)."""

    def __init__(self, lw, shape, dtype=np.float64):
        I = shape.intermediate
        self.attn_norm = codecs.bf16_value(lw["attn_norm"]).astype(dtype)
        self.mlp_norm = codecs.bf16_value(lw["mlp_norm"]).astype(dtype)
        self.w_qkv = weight_eff(lw["w_qkv"], lw["s_qkv"], dtype)
        self.w_o = weight_eff(lw["w_o"], lw["s_o"], dtype)
        gu = weight_eff(lw["w_gate_up"], lw["s_gate_up"], dtype)
        self.w_gate, self.w_up = gu[:I], gu[I:]
        self.w_down = weight_eff(lw["w_down"], lw["s_down"], dtype)


def decoder_layer(h, pos, W: LayerWeights, shape, mode="contract", fp8_kv_upto=0,
                  return_kv=False):
    """One decoder layer over a whole sequence h [N, H] at positions pos [N].

    ``fp8_kv_upto`` = number of leading positions whose K/V are held as fp8
    (the anchor, in the multi-join configuration).
    """
    N = h.shape[0]
    Hq, Hkv, d = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    u = _bf(rmsnorm(h, W.attn_norm, shape.rms_eps), mode)
    qkv = _aq(u, shape, "qkv") @ W.w_qkv.T
    q = qkv[:, :Hq * d].reshape(N, Hq, d)
    k = qkv[:, Hq * d:(Hq + Hkv) * d].reshape(N, Hkv, d)
    v = qkv[:, (Hq + Hkv) * d:].reshape(N, Hkv, d)
    q = _bf(rope(q, pos, shape.rope_theta), mode)
    k = _bf(rope(k, pos, shape.rope_theta), mode)
    v = _bf(v, mode)
    k_pre, v_pre = k, v          # the values an fp8 store quantises
    if fp8_kv_upto > 0:
        n = fp8_kv_upto
        k = k.copy()
        v = v.copy()
        k[:n] = codecs.e4m3_roundtrip(k[:n], shape.k_scale)
        v[:n] = codecs.e4m3_roundtrip(v[:n], shape.v_scale)
    o, _ = attention_causal(q, k, v, 1.0 / np.sqrt(d), q_pos=pos, k_pos=pos)
    o = _bf(o.reshape(N, Hq * d), mode)
    h = h + _aq(o, shape, "o") @ W.w_o.T
    u = _aq(_bf(rmsnorm(h, W.mlp_norm, shape.rms_eps), mode), shape, "gate_up")
    m = _bf(silu(u @ W.w_gate.T) * (u @ W.w_up.T), mode)
    h = h + _aq(m, shape, "down") @ W.w_down.T
    if return_kv:
        return h, (k, v, k_pre, v_pre)
    return h


def embed(tokens, weights, dtype=np.float64):
    return codecs.bf16_value(weights["embed"][np.asarray(tokens)]).astype(dtype)


def forward_tokens(tokens, weights, shape, mode="contract", fp8_kv_upto=0,
                   dtype=np.float64, layers=None, return_kv=False, n_layers=None):
    """Hidden states after ``n_layers`` decoder layers for one token sequence
    (positions 0..N-1). ``layers`` may hold pre-built LayerWeights."""
    L = shape.n_layers if n_layers is None else n_layers
    h = embed(tokens, weights, dtype)
    pos = np.arange(len(tokens))
    kvs = []
    for l in range(L):
        W = layers[l] if layers is not None else LayerWeights(weights["layers"][l], shape, dtype)
        out = decoder_layer(h, pos, W, shape, mode, fp8_kv_upto, return_kv=return_kv)
        if return_kv:
            h, kv = out
            kvs.append(kv)          # (k, v, k before fp8 storage, v before fp8 storage)
        else:
            h = out
    return (h, kvs) if return_kv else h


def head8(h_last, final_norm_bits, w8_bits, true_mask, shape, mode="contract"):
    """8-column head on last-position hidden states h_last [P, H].

    Returns logits [P, 8], token [P] (first maximum), decision [P] (0/1) and
    margin [P] (best TRUE logit minus best FALSE logit)."""
    h_last = np.atleast_2d(h_last)
    gamma = codecs.bf16_value(final_norm_bits) if final_norm_bits is not None else None
    z = h_last if gamma is None else rmsnorm(h_last, gamma, shape.rms_eps)
    z = _bf(z, mode)
    W8 = codecs.bf16_value(w8_bits) if np.asarray(w8_bits).dtype == np.uint16 else np.asarray(w8_bits, np.float64)
    logits = z.astype(np.float64) @ W8
    return logits, *decide(logits, true_mask)


def decide(logits, true_mask):
    """First-maximum token, its boolean, and the TRUE-vs-FALSE logit margin."""
    logits = np.atleast_2d(logits)
    tok = np.argmax(logits, axis=1)           # numpy returns the first maximum
    dec = (int(true_mask) >> tok) & 1
    bits = np.array([(int(true_mask) >> j) & 1 for j in range(logits.shape[1])], bool)
    best_t = np.max(np.where(bits[None, :], logits, -np.inf), axis=1)
    best_f = np.max(np.where(~bits[None, :], logits, -np.inf), axis=1)
    return tok.astype(np.uint8), dec.astype(np.uint8), best_t - best_f


def forward_pair(anchor_tokens, suffix_tokens, weights, shape, true_mask=0x0F,
                 mode="contract", dtype=np.float64, layers=None, n_layers=None, shared_len=0):
    """The per-pair definition: causal forward over [anchor ‖ suffix], then the
    head at the last position. An empty anchor is a filter row.

    ``shared_len``: the suffix's first tokens are a prefix shared with other
    suffixes of the anchor, whose K/V is stored once like the anchor's; with an
    fp8 KV store those positions are stored (and read) in E4M3 too."""
    a = np.asarray(anchor_tokens, np.int64)
    s = np.asarray(suffix_tokens, np.int64)
    tokens = np.concatenate([a, s])
    fp8_upto = len(a) + int(shared_len) if shape.kv_fp8 else 0
    h = forward_tokens(tokens, weights, shape, mode, fp8_upto, dtype, layers,
                       n_layers=n_layers)
    h_last = _bf(h[-1:], mode)          # the hidden state handed to the head
    logits, tok, dec, margin = head8(h_last, weights.get("final_norm"), weights["head8"],
                                     true_mask, shape, mode)
    return dict(h=h, h_last=h_last[0], logits=logits[0], token=int(tok[0]),
                decision=int(dec[0]), margin=float(margin[0]))


def forward_many(seqs, weights, shape, true_mask=0x0F, mode="contract", dtype=np.float64,
                 fp8_kv_upto=None, n_layers=None, taps=()):
    """The per-pair definition applied to many sequences at once.

    seqs: list of token sequences (each [anchor ‖ suffix], or a filter row);
    each is its own causal sequence at positions 0..N-1, exactly as in
    forward_pair. The per-token maps (norms, projections, RoPE, SwiGLU,
    residual adds) are applied to the rows of all sequences stacked into one
    matrix, which changes nothing for any row; attention runs per sequence.
    fp8_kv_upto: per sequence, the leading positions whose K/V are held as
    fp8 (None = none). Each layer's weights are dequantised once.

    Returns a dict with logits [S, 8], token, decision, margin [S] after
    n_layers layers and, for every depth d in ``taps``, the same four arrays
    for the head applied after layer d (key d).
    """
    L = shape.n_layers if n_layers is None else n_layers
    lens = [len(x) for x in seqs]
    starts = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    tokens = np.concatenate([np.asarray(x, np.int64) for x in seqs])
    pos = np.concatenate([np.arange(n) for n in lens])
    last = starts[1:] - 1
    upto = [0] * len(seqs) if fp8_kv_upto is None else list(fp8_kv_upto)
    Hq, Hkv, d = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    h = embed(tokens, weights, dtype)
    out = {}

    def head(hl):
        lg, tk, dc, mg = head8(_bf(hl, mode), weights.get("final_norm"), weights["head8"], true_mask,
                               shape, mode)
        return dict(logits=lg, token=tk, decision=dc, margin=mg)

    for l in range(L):
        W = LayerWeights(weights["layers"][l], shape, dtype)
        N = h.shape[0]
        u = _bf(rmsnorm(h, W.attn_norm, shape.rms_eps), mode)
        qkv = _aq(u, shape, "qkv") @ W.w_qkv.T
        q = qkv[:, :Hq * d].reshape(N, Hq, d)
        k = qkv[:, Hq * d:(Hq + Hkv) * d].reshape(N, Hkv, d)
        v = qkv[:, (Hq + Hkv) * d:].reshape(N, Hkv, d)
        q = _bf(rope(q, pos, shape.rope_theta), mode)
        k = _bf(rope(k, pos, shape.rope_theta), mode)
        v = _bf(v, mode)
        o = np.empty((N, Hq, d), q.dtype)
        for i in range(len(seqs)):
            a, b = starts[i], starts[i + 1]
            ks, vs = k[a:b], v[a:b]
            if upto[i] > 0:
                ks = ks.copy()
                vs = vs.copy()
                ks[:upto[i]] = codecs.e4m3_roundtrip(ks[:upto[i]], shape.k_scale)
                vs[:upto[i]] = codecs.e4m3_roundtrip(vs[:upto[i]], shape.v_scale)
            o[a:b], _ = attention_causal(q[a:b], ks, vs, 1.0 / np.sqrt(d))
        o = _bf(o.reshape(N, Hq * d), mode)
        h = h + _aq(o, shape, "o") @ W.w_o.T
        u = _aq(_bf(rmsnorm(h, W.mlp_norm, shape.rms_eps), mode), shape, "gate_up")
        m = _bf(silu(u @ W.w_gate.T) * (u @ W.w_up.T), mode)
        h = h + _aq(m, shape, "down") @ W.w_down.T
        del W
        if (l + 1) in taps:
            out[l + 1] = head(h[last])
    out.update(head(h[last]))
    out["h_last"] = _bf(h[last], mode)
    return out
