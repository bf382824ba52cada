"""W8A8 projection: E4M3 activations times E4M3 weights.

Test infrastructure (see the package header).

The pages run the projections as FP8 GEMMs ([pt] "Como funciona", the engine
paragraph naming FP8 GEMM kernels; [fa] key points: qwen3-4b-fp8). The
W8A16 reading keeps the activations in bf16; this module is the other
reading: the activations a projection reads are also quantised to E4M3, so
the product can run on the fp8 matrix cores.

Readings where the pages are silent:
  * one scale per token (per row of the activation matrix): s = amax / 448,
    amax = the row's largest magnitude, so the largest element maps to the
    largest E4M3 magnitude; a row of zeros has s = 0 and codes 0; rows with
    0 < amax < 2^-120 are outside the domain (448 / amax overflows float32);
  * the code of x is the E4M3 encoding (round to nearest, ties to even,
    saturating) of x * inv, where inv = 448 / amax and both the division and
    the product are single float32 operations (a quantised code is an integer
    decided by floating point, so the precision of that decision is part of
    the definition);
  * s itself is float32(amax) / 448 in float32;
  * y[m][n] = s[m] * scale_w[n] * sum_k decode(cx[m][k]) * decode(cw[n][k]),
    evaluated here in float64 (every product of two E4M3 values is exact).

Pins (tests/test_oracle_w8a8.py): a row's largest element maps to code
+-448; rows whose values are E4M3 values times a power-of-two scale with
448 * scale as the largest magnitude come back exactly, and their W8A8
product equals the W8A16 product of the same rows; a worked example; every
dequantised value lies within half an E4M3 step of the input; the W8A8
product stays within the bound those steps imply.
"""
from __future__ import annotations

import numpy as np

from . import codecs


def act_quant_e4m3(x):
    """Per-row E4M3 quantisation of an activation matrix (float32 values,
    e.g. decoded bf16). Returns (codes uint8 [M, K], scale float32 [M])."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=1).astype(np.float32)
    safe = np.where(amax > 0, amax, np.float32(1.0)).astype(np.float32)
    inv = (np.float32(448.0) / safe).astype(np.float32)                # one float32 division
    q = (x * inv[:, None]).astype(np.float32)                          # one float32 product
    codes = codecs.e4m3_encode(q.astype(np.float64))
    codes = np.where(amax[:, None] > 0, codes, np.uint8(0)).astype(np.uint8)
    scale = np.where(amax > 0, (amax / np.float32(448.0)).astype(np.float32), np.float32(0.0))
    return codes, scale.astype(np.float32)


def act_dequant(codes, scale):
    """decode(codes) * scale per row (float64)."""
    return codecs.e4m3_decode(codes) * np.asarray(scale, np.float64)[:, None]


def gemm_w8a8(x_codes, x_scale, w_codes, w_scale_bits):
    """y [M, N] = x_scale[m] * scale_w[n] * sum_k decode(x) * decode(w), in
    float64; w_scale_bits are the bf16 bits of the per-row weight scales."""
    xd = codecs.e4m3_decode(x_codes)
    wd = codecs.e4m3_decode(w_codes)
    sw = codecs.bf16_value(w_scale_bits)
    return (xd @ wd.T) * np.asarray(x_scale, np.float64)[:, None] * sw[None, :]
