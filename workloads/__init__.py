"""Seeded synthetic inputs for AI.IF join prefill.

This module draws random numbers and lays them out in the byte formats the
prefill path consumes. It computes nothing that the prefill computes: no
normalisation, projection, attention, rounding rule or fp8 codec lives here.
Both the CPU oracle (through the tests) and the HIP path (tests and the
benchmark) take their inputs from these functions, so neither side can bias
the other through its inputs.

Byte formats
  * bf16 tensors are numpy ``uint16`` bit patterns. They are produced by
    keeping the top 16 bits of a float32 draw (truncation). That choice only
    shapes the input distribution; it is not the round-to-nearest-even rule
    the method applies to its own intermediates.
  * fp8 weights are ``uint8`` OCP E4M3 codes. The host generator draws them
    bit-field by bit-field (sign, exponent field, mantissa field), with an
    exponent-field histogram close to that of a half-normal sample spanning
    the E4M3 range, so no float is encoded there. The device generator for
    full-size models (``model_weights_device``) draws float weights and
    encodes them with torch's float8_e4m3fn cast: input synthesis only.
  * token ids are ``int32``.

Seeding: every tensor block has its own ``np.random.default_rng`` keyed by
(config id, seed, block ids...), so any anchor, suffix or layer can be
regenerated alone.

The shapes follow the synthetic configurations of the Quail pages' workload
class: a single-GPU Qwen3-4B-FP8-shaped model (page "Quail: one billion
tokens per minute on one GPU", key-points list: model qwen3-4b-fp8 on one
GPU), AI.IF filters (one model call per row) and joins (one call per row
pair) as described in page "Quail, il motore di inferenza che supera il
miliardo di token al minuto su una H100", second paragraph.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "ModelShape", "QWEN3_4B", "tiny_shape", "bf16_bits_from_f32", "draw_bf16",
    "draw_fp8_codes", "model_weights", "cascade_case", "c0_case", "c1_case",
    "join_case", "filter_case", "c2_case", "c3a_case", "c3b_case", "c4_case",
    "bf16_to_f32", "depth_case", "depth_multijoin_case", "residual_std", "W_STD",
]


# ----------------------------------------------------------------------------
# shapes
# ----------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class ModelShape:
    """Dense decoder shape: RMSNorm, GQA attention with RoPE, SwiGLU MLP."""
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    rope_theta: float = 1.0e6
    rms_eps: float = 1.0e-6
    kv_fp8: bool = False          # anchor KV stored as OCP E4M3 codes
    k_scale: float = 1.0
    v_scale: float = 1.0
    act_fp8: bool = False         # projections read per-token E4M3 activations (W8A8)

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def qkv_dim(self) -> int:
        return self.q_dim + 2 * self.kv_dim


# Qwen3-4B dense shapes (36 layers, hidden 2560, 32 q / 8 kv heads of 128,
# intermediate 9728, vocabulary 151936).
QWEN3_4B = ModelShape(n_layers=36, hidden=2560, n_q_heads=32, n_kv_heads=8,
                      head_dim=128, intermediate=9728, vocab=151936)


def tiny_shape(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=128,
               intermediate=384, vocab=512, **kw) -> ModelShape:
    """A small model with the same structure, for fast parity cases."""
    return ModelShape(n_layers=n_layers, hidden=hidden, n_q_heads=n_q_heads,
                      n_kv_heads=n_kv_heads, head_dim=head_dim,
                      intermediate=intermediate, vocab=vocab, **kw)


# ----------------------------------------------------------------------------
# raw draws
# ----------------------------------------------------------------------------
def _rng(*key) -> np.random.Generator:
    return np.random.default_rng([int(k) & 0xFFFFFFFF for k in key])


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Top 16 bits of float32 values (truncation; input synthesis only)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact; a bit shift)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def draw_bf16(rng: np.random.Generator, shape, std=1.0, mean=0.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if mean != 0.0:
        x += np.float32(mean)
    return bf16_bits_from_f32(x)


# Exponent-field histogram for the fp8 weight codes: roughly the exponents of
# |N(0, 100)| draws, which span the E4M3 range up to 448. Fields 0..15.
_FP8_EXP_P = np.array([0.001, 0.001, 0.001, 0.001, 0.001, 0.001, 0.002,
                       0.008, 0.016, 0.032, 0.063, 0.124, 0.227, 0.322,
                       0.190, 0.010])
_FP8_EXP_P = _FP8_EXP_P / _FP8_EXP_P.sum()
_FP8_EXP_CDF = np.cumsum(_FP8_EXP_P)


# exponent field for each 16-bit uniform draw (inverse CDF as a lookup table)
_FP8_EXP_TABLE = np.minimum(
    np.searchsorted(_FP8_EXP_CDF, (np.arange(1 << 16) + 0.5) / (1 << 16), side="right"),
    15).astype(np.uint8)


def draw_fp8_codes(rng: np.random.Generator, shape) -> np.ndarray:
    """OCP E4M3 codes drawn field by field from one 32-bit draw per code:
    bits 0..15 pick the exponent field through the histogram above, bits
    16..18 the mantissa, bit 19 the sign; never a NaN code (S.1111.111)."""
    n = int(np.prod(shape))
    out = np.empty(n, np.uint8)
    step = 1 << 24
    for i in range(0, n, step):
        bits = rng.integers(0, 1 << 32, size=min(step, n - i), dtype=np.uint32)
        e = _FP8_EXP_TABLE[bits & 0xFFFF]
        m = ((bits >> 16) & 7).astype(np.uint8)
        m = np.where(e == 15, np.minimum(m, 6), m).astype(np.uint8)
        s = ((bits >> 19) & 1).astype(np.uint8)
        out[i:i + len(bits)] = (s << 7) | (e << 3) | m
    return out.reshape(shape)


# RMS of the magnitudes drawn by draw_fp8_codes (about 100); used only to pick
# a per-row scale so that decoded weights have a standard deviation near 0.02.
_FP8_CODE_RMS = 100.0


def _row_scales(rng, n_rows, target_std=0.02):
    base = target_std / _FP8_CODE_RMS
    jitter = 1.0 + 0.1 * rng.random(n_rows, dtype=np.float64)
    return bf16_bits_from_f32((base * jitter).astype(np.float32))


# ----------------------------------------------------------------------------
# model weights (random init)
# ----------------------------------------------------------------------------
_T_EMBED, _T_FINAL, _T_HEAD = 1, 2, 3
_T_ATTN_NORM, _T_MLP_NORM = 10, 11
_T_QKV, _T_O, _T_GU, _T_D = 20, 21, 22, 23


# Standard deviation of the decoded projection weights. The two projections
# that write into the residual stream (attention output and MLP down) are
# scaled by 1 / sqrt(2 * n_layers), the depth-scaled initialisation of GPT-2
# style decoders: each layer then adds a small update to the residual stream,
# so a deep random-init stack stays well conditioned and last-bit rounding
# differences do not grow into percent-level differences at the last layer.
W_STD = 0.02


def residual_std(shape: ModelShape) -> float:
    """Std of the residual-writing projections (O and down)."""
    return W_STD / math.sqrt(2.0 * shape.n_layers)


def layer_weights(shape: ModelShape, seed: int, layer: int) -> dict:
    """One decoder layer: fp8 codes [out, in] + bf16 per-output-row scales.
    Decoded weights have std W_STD (QKV, gate/up) or residual_std(shape)
    (O, down)."""
    H, I = shape.hidden, shape.intermediate
    out = {}
    r = _rng(7, seed, layer, _T_ATTN_NORM)
    out["attn_norm"] = draw_bf16(r, (H,), std=0.1, mean=1.0)
    r = _rng(7, seed, layer, _T_MLP_NORM)
    out["mlp_norm"] = draw_bf16(r, (H,), std=0.1, mean=1.0)
    for name, tid, (n_out, n_in) in (
            ("qkv", _T_QKV, (shape.qkv_dim, H)),
            ("o", _T_O, (H, shape.q_dim)),
            ("gate_up", _T_GU, (2 * I, H)),
            ("down", _T_D, (H, I))):
        r = _rng(7, seed, layer, tid)
        out["w_" + name] = draw_fp8_codes(r, (n_out, n_in))
        std = residual_std(shape) if name in ("o", "down") else W_STD
        out["s_" + name] = _row_scales(r, n_out, std)
    return out


def model_weights(shape: ModelShape, seed: int = 0, with_layers=True) -> dict:
    """Random-init weights: embedding, per-layer weights, final norm, 8-col head.

    ``head8`` is [hidden, 8] bf16 ~ N(0, 0.02); ``embed`` is [vocab, hidden]
    bf16 ~ N(0, 1); norms are 1 + 0.1 N(0, 1) so that a dropped gain shows.
    """
    H = shape.hidden
    w = {}
    w["embed"] = draw_bf16(_rng(7, seed, 0, _T_EMBED), (shape.vocab, H))
    w["final_norm"] = draw_bf16(_rng(7, seed, 0, _T_FINAL), (H,), std=0.1, mean=1.0)
    w["head8"] = draw_bf16(_rng(7, seed, 0, _T_HEAD), (H, 8), std=0.02)
    if with_layers:
        w["layers"] = [layer_weights(shape, seed, l) for l in range(shape.n_layers)]
    return w


def model_weights_device(shape: ModelShape, seed: int = 0, device="cuda") -> dict:
    """Random-init weights drawn directly in device memory with torch's seeded
    generator (for full-size models, whose host generation takes minutes).
    Same keys and formats as ``model_weights`` (bf16 as int16 bits, fp8 as
    uint8 OCP E4M3 codes); values differ. Projection weights follow the recipe
    W ~ N(0, std) with std = W_STD, or residual_std(shape) for the O and down
    projections; per-row scale = bf16(max|W_row| / 448); codes = E4M3 of
    W / scale (clamped to +-448 first), encoded by torch's float8_e4m3fn cast.
    This is input synthesis only (the library's and the oracle's codecs are
    not involved)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(7_000_003 * seed + 11)
    H, I = shape.hidden, shape.intermediate

    def bf16(shape_, std=1.0, mean=0.0):
        x = torch.randn(shape_, generator=g, device=device, dtype=torch.float32) * std + mean
        return x.to(torch.bfloat16).view(torch.int16)

    def fp8_rows(n_out, n_in, std):
        codes = torch.empty((n_out, n_in), dtype=torch.uint8, device=device)
        scales = torch.empty(n_out, dtype=torch.int16, device=device)
        step = max(1, (1 << 26) // n_in)
        for r0 in range(0, n_out, step):
            r1 = min(n_out, r0 + step)
            w = torch.randn((r1 - r0, n_in), generator=g, device=device, dtype=torch.float32) * std
            sc = (w.abs().amax(dim=1) / 448.0).to(torch.bfloat16)
            q = (w / sc.float()[:, None]).clamp_(-448.0, 448.0)
            codes[r0:r1] = q.to(torch.float8_e4m3fn).view(torch.uint8)
            scales[r0:r1] = sc.view(torch.int16)
        return codes, scales

    w = {"embed": bf16((shape.vocab, H)), "final_norm": bf16((H,), 0.1, 1.0),
         "head8": bf16((H, 8), 0.02), "layers": []}
    for _ in range(shape.n_layers):
        lw = {"attn_norm": bf16((H,), 0.1, 1.0), "mlp_norm": bf16((H,), 0.1, 1.0)}
        for name, (n_out, n_in) in (("qkv", (shape.qkv_dim, H)), ("o", (H, shape.q_dim)),
                                     ("gate_up", (2 * I, H)), ("down", (H, I))):
            std = residual_std(shape) if name in ("o", "down") else W_STD
            lw["w_" + name], lw["s_" + name] = fp8_rows(n_out, n_in, std)
        w["layers"].append(lw)
    return w


def weights_to_host(w: dict) -> dict:
    """Host copy (numpy, bf16 as uint16 bits) of device weights."""
    def h(t):
        a = t.cpu().numpy()
        return a.view(np.uint16) if a.dtype == np.int16 else a
    out = {k: h(v) for k, v in w.items() if k != "layers"}
    out["layers"] = [{k: h(v) for k, v in lw.items()} for lw in w["layers"]]
    return out


def full_head(shape: ModelShape, seed: int = 0, vocab=None) -> np.ndarray:
    """A full unembedding [hidden, vocab] (bf16) for head-restriction checks."""
    V = vocab or shape.vocab
    return draw_bf16(_rng(7, seed, 0, 99), (shape.hidden, V), std=0.02)


# ----------------------------------------------------------------------------
# cascade-attention cases (Q/K/V given directly)
# ----------------------------------------------------------------------------
def cascade_case(seed: int, a_len, s_anchor, s_len, hq: int, hkv: int, d: int,
                 dtype: str = "bf16", cfg_id: int = 1) -> dict:
    """Packed Q/K/V for anchors and suffixes.

    a_len     [n_anchors] anchor lengths (tokens)
    s_anchor  [n_suffix] anchor index of each suffix, -1 = no anchor
    s_len     [n_suffix] suffix lengths
    Returns token-major packed arrays: ak, av [sum La, hkv, d]; q [sum Ls, hq, d];
    k, v [sum Ls, hkv, d]; plus int32 offsets. Each anchor's and each
    suffix's block is drawn from its own seeded generator.
    """
    a_len = np.asarray(a_len, dtype=np.int32)
    s_len = np.asarray(s_len, dtype=np.int32)
    s_anchor = np.asarray(s_anchor, dtype=np.int32)
    a_off = np.zeros(len(a_len) + 1, np.int32)
    a_off[1:] = np.cumsum(a_len)
    s_off = np.zeros(len(s_len) + 1, np.int32)
    s_off[1:] = np.cumsum(s_len)
    f32 = dtype == "f32"
    npdt = np.float32 if f32 else np.uint16

    def draw(r, shp):
        x = r.standard_normal(size=shp, dtype=np.float32)
        return x if f32 else bf16_bits_from_f32(x)

    ak = np.empty((int(a_off[-1]), hkv, d), npdt)
    av = np.empty_like(ak)
    for a in range(len(a_len)):
        r = _rng(cfg_id, seed, 1, a)
        ak[a_off[a]:a_off[a + 1]] = draw(r, (a_len[a], hkv, d))
        av[a_off[a]:a_off[a + 1]] = draw(r, (a_len[a], hkv, d))
    q = np.empty((int(s_off[-1]), hq, d), npdt)
    k = np.empty((int(s_off[-1]), hkv, d), npdt)
    v = np.empty_like(k)
    for s in range(len(s_len)):
        r = _rng(cfg_id, seed, 2, s)
        sl = slice(s_off[s], s_off[s + 1])
        q[sl] = draw(r, (s_len[s], hq, d))
        k[sl] = draw(r, (s_len[s], hkv, d))
        v[sl] = draw(r, (s_len[s], hkv, d))
    return dict(a_len=a_len, a_off=a_off, s_anchor=s_anchor, s_len=s_len,
                s_off=s_off, ak=ak, av=av, q=q, k=k, v=v, hq=hq, hkv=hkv, d=d,
                dtype=dtype, sm_scale=1.0 / math.sqrt(d))


def c0_case(seed: int = 0) -> dict:
    """Tiny fp32 cascade layer: 1 anchor x 64 tokens, 8 suffixes x 32 tokens,
    4 q heads / 2 kv heads, head_dim 64 (hidden 256), plus an 8-column head
    W8 [256, 8] ~ N(0, 0.02) applied to the flattened attention output."""
    case = cascade_case(seed, [64], [0] * 8, [32] * 8, hq=4, hkv=2, d=64,
                        dtype="f32", cfg_id=0)
    r = _rng(0, seed, 3, 0)
    case["w8"] = (0.02 * r.standard_normal(size=(256, 8))).astype(np.float32)
    case["true_mask"] = 0x0F
    return case


def c1_lengths(seed: int = 1, n_anchors: int = 256, per_anchor: int = 64,
               la_range=(512, 2048), ls_range=(32, 128)):
    r = _rng(1, seed, 0, 0)
    a_len = r.integers(la_range[0], la_range[1] + 1, size=n_anchors).astype(np.int32)
    s_len = r.integers(ls_range[0], ls_range[1] + 1,
                       size=n_anchors * per_anchor).astype(np.int32)
    s_anchor = np.repeat(np.arange(n_anchors, dtype=np.int32), per_anchor)
    return a_len, s_anchor, s_len


def c1_case(seed: int = 1, n_anchors: int = 256, per_anchor: int = 64,
            la_range=(512, 2048), ls_range=(32, 128)) -> dict:
    """Qwen3-4B-shaped bf16 attention layer: 32 q / 8 kv heads x 128; anchors
    of U{512..2048} tokens, each joined to ``per_anchor`` suffixes of
    U{32..128} tokens; Q/K/V ~ N(0, 1). At full size (256 anchors) the arrays
    hold about 27 GB; use ``c1_device`` for that."""
    a_len, s_anchor, s_len = c1_lengths(seed, n_anchors, per_anchor, la_range, ls_range)
    return cascade_case(seed, a_len, s_anchor, s_len, hq=32, hkv=8, d=128,
                        dtype="bf16", cfg_id=1)


def cascade_device(seed, a_len, s_anchor, s_len, device="cuda", hq=32, hkv=8, d=128,
                   anchor_kv="bf16"):
    """A bf16 cascade-attention case drawn directly in device memory with
    torch's seeded generator (N(0,1) float32 draws converted to bf16); the
    arrays and keys are those of ``cascade_case``. anchor_kv="e4m3" stores
    the anchor K/V as OCP E4M3 codes of the N(0,1) draws (uint8)."""
    import torch
    a_len = np.asarray(a_len, np.int32)
    s_anchor = np.asarray(s_anchor, np.int32)
    s_len = np.asarray(s_len, np.int32)
    a_off = np.zeros(len(a_len) + 1, np.int32)
    a_off[1:] = np.cumsum(a_len)
    s_off = np.zeros(len(s_len) + 1, np.int32)
    s_off[1:] = np.cumsum(s_len)
    g = torch.Generator(device=device)
    g.manual_seed(1_000_003 * seed + 17)

    def draw(shape, dt=None):
        dt = dt or torch.bfloat16
        out = torch.empty(shape, dtype=dt, device=device)
        # draw in chunks to bound the float32 temporary
        flat = out.view(-1)
        step = 1 << 28
        for i in range(0, flat.numel(), step):
            n = min(step, flat.numel() - i)
            flat[i:i + n] = torch.randn(n, generator=g, device=device, dtype=torch.float32).to(dt)
        return out

    TA, TS = int(a_off[-1]), int(s_off[-1])
    if anchor_kv == "e4m3":
        ak = draw((TA, hkv, d), torch.float8_e4m3fn).view(torch.uint8)
        av = draw((TA, hkv, d), torch.float8_e4m3fn).view(torch.uint8)
    else:
        ak = draw((TA, hkv, d)); av = draw((TA, hkv, d))
    q = draw((TS, hq, d)); k = draw((TS, hkv, d)); v = draw((TS, hkv, d))
    return dict(a_len=a_len, a_off=a_off, s_anchor=s_anchor, s_len=s_len,
                s_off=s_off, ak=ak, av=av, q=q, k=k, v=v, hq=hq, hkv=hkv, d=d,
                dtype="bf16", sm_scale=1.0 / math.sqrt(d))


def c1_device(seed: int = 1, device="cuda", n_anchors: int = 256,
              per_anchor: int = 64, la_range=(512, 2048), ls_range=(32, 128)):
    """Full-size C1 drawn directly in device memory (see ``cascade_device``).
    Same lengths as ``c1_case``; values differ (different generator)."""
    a_len, s_anchor, s_len = c1_lengths(seed, n_anchors, per_anchor, la_range, ls_range)
    return cascade_device(seed, a_len, s_anchor, s_len, device)


def stream_lengths(S: int, n_anchors: int = 1024, la: int = 768):
    """Anchor-KV streaming shape of the multi-join configuration: n_anchors
    anchors of la tokens (the resident KV), each read by one suffix of S
    tokens, so the attention intensity grows with S (4*S FLOP per bf16 KV
    byte)."""
    a_len = np.full(n_anchors, la, np.int32)
    s_anchor = np.arange(n_anchors, dtype=np.int32)
    s_len = np.full(n_anchors, S, np.int32)
    return a_len, s_anchor, s_len


# ----------------------------------------------------------------------------
# token workloads for the model path
# ----------------------------------------------------------------------------
def join_case(seed: int, vocab: int, a_len, pair_anchor, s_len, cfg_id: int = 2,
              true_mask: int = 0x0F) -> dict:
    """Anchors (token ids) and pairs (anchor index, suffix token ids).

    pair_anchor[i] = -1 marks a filter row (no anchor). Suffix tokens are drawn
    per pair; ``suffix_row`` lets several pairs share one row's tokens.
    """
    a_len = np.asarray(a_len, np.int32)
    s_len = np.asarray(s_len, np.int32)
    a_off = np.zeros(len(a_len) + 1, np.int32)
    a_off[1:] = np.cumsum(a_len)
    s_off = np.zeros(len(s_len) + 1, np.int32)
    s_off[1:] = np.cumsum(s_len)
    a_tok = np.empty(int(a_off[-1]), np.int32)
    for a in range(len(a_len)):
        a_tok[a_off[a]:a_off[a + 1]] = _rng(cfg_id, seed, 4, a).integers(
            0, vocab, size=a_len[a], dtype=np.int32)
    s_tok = np.empty(int(s_off[-1]), np.int32)
    for s in range(len(s_len)):
        s_tok[s_off[s]:s_off[s + 1]] = _rng(cfg_id, seed, 5, s).integers(
            0, vocab, size=s_len[s], dtype=np.int32)
    return dict(a_len=a_len, a_off=a_off, a_tok=a_tok,
                pair_anchor=np.asarray(pair_anchor, np.int32), s_len=s_len,
                s_off=s_off, s_tok=s_tok, true_mask=true_mask)


def filter_case(seed: int, vocab: int, lengths, cfg_id: int = 3) -> dict:
    lengths = np.asarray(lengths, np.int32)
    return join_case(seed, vocab, [], -np.ones(len(lengths), np.int32), lengths,
                     cfg_id=cfg_id)


def c2_case(seed: int = 2, n_anchors: int = 16, per_anchor: int = 512,
            la: int = 1024, ls: int = 64, vocab: int = QWEN3_4B.vocab) -> dict:
    """One decoder layer workload: n_anchors x per_anchor suffixes."""
    pa = np.repeat(np.arange(n_anchors, dtype=np.int32), per_anchor)
    return join_case(seed, vocab, [la] * n_anchors, pa, [ls] * len(pa), cfg_id=2)


def c3a_lengths(seed: int = 3, n_rows: int = 10000, lo=200, hi=2000):
    """Truncated lognormal lengths: ln L ~ N(ln sqrt(lo*hi), ln(10)/3.92),
    rounded, redrawn until inside [lo, hi]."""
    r = _rng(3, seed, 0, 0)
    mu = math.log(math.sqrt(lo * hi))
    sigma = math.log(10.0) / 3.92
    out = np.empty(0, np.int64)
    while out.size < n_rows:
        x = np.rint(np.exp(r.normal(mu, sigma, size=2 * n_rows)))
        x = x[(x >= lo) & (x <= hi)]
        out = np.concatenate([out, x.astype(np.int64)])
    return out[:n_rows].astype(np.int32)


def c3a_case(seed: int = 3, n_rows: int = 10000, vocab: int = QWEN3_4B.vocab):
    return filter_case(seed, vocab, c3a_lengths(seed, n_rows), cfg_id=3)


def c3b_case(seed: int = 4, n_anchors: int = 64, per_anchor: int = 2048,
             la: int = 1024, ls: int = 64, vocab: int = QWEN3_4B.vocab):
    pa = np.repeat(np.arange(n_anchors, dtype=np.int32), per_anchor)
    return join_case(seed, vocab, [la] * n_anchors, pa, [ls] * len(pa), cfg_id=4)


def c4_case(seed: int = 5, n_anchors: int = 1024, la: int = 768,
            n_rows: int = 5000, frac: float = 0.05, ls_range=(48, 256),
            vocab: int = QWEN3_4B.vocab):
    """Multi-join: each suffix row probes round(frac * n_anchors) distinct
    anchors drawn without replacement. Pairs are listed row by row (the
    anchor-sorted order is the plan builder's job). ``pair_row`` maps a pair to
    its row; the row's tokens are repeated for every pair that uses it."""
    r = _rng(5, seed, 0, 0)
    k = int(round(frac * n_anchors))
    row_len = r.integers(ls_range[0], ls_range[1] + 1, size=n_rows).astype(np.int32)
    pair_anchor, pair_row = [], []
    for row in range(n_rows):
        anchors = r.choice(n_anchors, size=k, replace=False)
        pair_anchor.append(anchors.astype(np.int32))
        pair_row.append(np.full(k, row, np.int32))
    pair_anchor = np.concatenate(pair_anchor)
    pair_row = np.concatenate(pair_row)
    a_len = np.full(n_anchors, la, np.int32)
    a_off = np.zeros(n_anchors + 1, np.int32)
    a_off[1:] = np.cumsum(a_len)
    a_tok = np.empty(int(a_off[-1]), np.int32)
    for a in range(n_anchors):
        a_tok[a_off[a]:a_off[a + 1]] = _rng(5, seed, 4, a).integers(0, vocab, size=la,
                                                                   dtype=np.int32)
    row_off = np.zeros(n_rows + 1, np.int64)
    row_off[1:] = np.cumsum(row_len)
    row_tok = np.empty(int(row_off[-1]), np.int32)
    for row in range(n_rows):
        row_tok[row_off[row]:row_off[row + 1]] = _rng(5, seed, 5, row).integers(
            0, vocab, size=row_len[row], dtype=np.int32)
    return dict(a_len=a_len, a_off=a_off, a_tok=a_tok, pair_anchor=pair_anchor,
                pair_row=pair_row, row_len=row_len, row_off=row_off,
                row_tok=row_tok, true_mask=0x0F)


def depth_case(seed: int, a_len, per_anchor: int, n_filter: int, ls_range=(2, 12),
               filter_range=(4, 24), vocab: int = QWEN3_4B.vocab, cfg_id: int = 8) -> dict:
    """A small join for full-depth parity: every anchor joined to
    ``per_anchor`` suffixes of U{ls_range} tokens, plus ``n_filter`` filter
    rows of U{filter_range} tokens, the pairs listed in a seeded random order
    (sorting them is the plan's job)."""
    r = _rng(cfg_id, seed, 0, 0)
    n_anchors = len(a_len)
    pa = np.concatenate([np.repeat(np.arange(n_anchors), per_anchor),
                         -np.ones(n_filter, np.int64)]).astype(np.int32)
    sl = np.concatenate([r.integers(ls_range[0], ls_range[1] + 1, size=n_anchors * per_anchor),
                         r.integers(filter_range[0], filter_range[1] + 1, size=n_filter)])
    perm = r.permutation(len(pa))
    return join_case(seed, vocab, a_len, pa[perm], sl[perm].astype(np.int32), cfg_id=cfg_id)


def depth_multijoin_case(seed: int, a_len, n_joins: int, per_join: int, ls_range=(2, 12),
                         vocab: int = QWEN3_4B.vocab, cfg_id: int = 9) -> dict:
    """Several joins over one anchor table for full-depth parity: join k has
    ``per_join`` pairs, each naming a seeded random anchor (with repetition,
    across and within joins) and suffix tokens of U{ls_range}. A join_case
    dict plus ``join_offsets`` [n_joins + 1]."""
    r = _rng(cfg_id, seed, 0, 0)
    n = n_joins * per_join
    pa = r.integers(0, len(a_len), size=n).astype(np.int32)
    sl = r.integers(ls_range[0], ls_range[1] + 1, size=n).astype(np.int32)
    case = join_case(seed, vocab, a_len, pa, sl, cfg_id=cfg_id)
    case["join_offsets"] = (np.arange(n_joins + 1) * per_join).astype(np.int32)
    return case


def shared_prefix_case(seed: int, vocab: int, a_len, families, cfg_id: int = 6,
                       true_mask: int = 0x0F) -> dict:
    """Suffixes that come in families sharing a leading token run, as in agent
    traces whose documents repeat a common prefix.

    families: list of (anchor index, shared length, [tail lengths]); each tail
    length gives one pair whose suffix is the family's shared tokens followed
    by its own tokens. Returns a join_case-shaped dict (pairs in family order)
    plus ``family`` [n_pairs] and ``shared_len`` [n_families]. Only seeded
    draws and layout: which pairs the library groups is for it to find.
    """
    pair_anchor, s_len, fam = [], [], []
    for f, (a, shared, tails) in enumerate(families):
        for t in tails:
            pair_anchor.append(a)
            s_len.append(shared + t)
            fam.append(f)
    case = join_case(seed, vocab, a_len, pair_anchor, s_len, cfg_id=cfg_id, true_mask=true_mask)
    s_tok, s_off = case["s_tok"], case["s_off"]
    for f, (a, shared, tails) in enumerate(families):
        head = _rng(cfg_id, seed, 7, f).integers(0, vocab, size=shared, dtype=np.int32)
        for i in np.flatnonzero(np.asarray(fam) == f):
            s_tok[s_off[i]:s_off[i] + shared] = head
    case["family"] = np.asarray(fam, np.int32)
    case["shared_len"] = np.asarray([f[1] for f in families], np.int32)
    return case
