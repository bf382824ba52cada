"""Pins for oracle/codecs.py: bf16 RNE and OCP E4M3, against torch's casts and
the format's spot values (tests/golden/e4m3_spot.txt)."""
import os

import numpy as np
import pytest
import torch

from oracle import codecs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_spot.txt")


def _f32_sweep(n=200_000, seed=0):
    r = np.random.default_rng(seed)
    bits = r.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    # add exact bf16 midpoints (ties) and their neighbours
    b = r.integers(0, 1 << 16, size=20_000, dtype=np.uint32)
    mid = ((b << 16) | 0x8000).view(np.float32)
    mid = mid[np.isfinite(mid)]
    nb = np.concatenate([mid, np.nextafter(mid, np.float32(np.inf)),
                         np.nextafter(mid, np.float32(-np.inf))])
    return np.concatenate([x, nb, np.float32([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38])])


def test_bf16_round_matches_torch_rne():
    x = _f32_sweep()
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy().astype(np.float64)
    got = codecs.bf16_round(x.astype(np.float64))
    both_inf = np.isinf(ref) & np.isinf(got) & (np.sign(ref) == np.sign(got))
    assert np.all((got == ref) | both_inf)


def test_bf16_bits_roundtrip():
    x = _f32_sweep(20_000, seed=1)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = codecs.bf16_bits(x.astype(np.float64))
    fin = np.isfinite(codecs.bf16_value(ref))
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(codecs.bf16_value(got[fin]), codecs.bf16_value(ref[fin]))


def test_bf16_round_ties_to_even_hand_values():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to 1 (even mantissa)
    assert codecs.bf16_round(1.0 + 2.0 ** -8) == 1.0
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: ties to 1 + 2^-6
    assert codecs.bf16_round(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert codecs.bf16_round(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7
    # float64 input that float32 would double-round: direct rounding keeps it below
    assert codecs.bf16_round(1.0 + 2.0 ** -8 - 2.0 ** -40) == 1.0


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = codecs.e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert nan.sum() == 2 and codecs.E4M3_MAX == 448.0


def test_e4m3_encode_all_bf16_patterns_match_torch_with_clamp():
    bits = np.arange(1 << 16, dtype=np.uint32)
    x = (bits << 16).view(np.float32)
    fin = ~np.isnan(x)
    xt = torch.from_numpy(x[fin].copy()).clamp(-448.0, 448.0)
    ref = xt.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = codecs.e4m3_encode(x[fin].astype(np.float64))
    assert np.array_equal(got, ref)
    nan_codes = codecs.e4m3_encode(x[~fin].astype(np.float64))
    assert np.all((nan_codes & 0x7F) == 0x7F)


def test_e4m3_spot_values_from_format_definition():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                v, c = line.split()[:2]
                rows.append((float(v), int(c, 16)))
    assert len(rows) >= 15
    for v, c in rows:
        assert int(codecs.e4m3_encode(v)) == c, (v, hex(int(codecs.e4m3_encode(v))), hex(c))
        dv = codecs.e4m3_decode(c)
        assert abs(dv) <= 448.0


def test_e4m3_roundtrip_is_idempotent_on_codes():
    vals = codecs.e4m3_decode(np.arange(256, dtype=np.uint8))
    fin = np.isfinite(vals)
    re = codecs.e4m3_encode(vals[fin])
    assert np.array_equal(codecs.e4m3_decode(re), vals[fin])
    # every E4M3 value is a bf16 value (so W8A16 decode into bf16 is exact)
    assert np.array_equal(codecs.bf16_round(vals[fin]), vals[fin])
