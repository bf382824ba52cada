"""Number formats: bf16 round-to-nearest-even and OCP FP8 E4M3.

Test infrastructure (see the package header).

The pages name the model's precision only as "FP8" ([it] second paragraph:
"Qwen3 4B FP8"; [fa] key points: qwen3-4b-fp8). The readings taken:
  * FP8 is OCP E4M3 ("e4m3fn"): 1 sign, 4 exponent bits with bias 7, 3 mantissa
    bits, no infinities, S.1111.111 is NaN, largest finite value 448.
  * Encoding rounds to nearest with ties to the even code and saturates:
    magnitudes above 448 become 448 (the clamp happens before rounding).
  * bf16 is the top half of IEEE binary32: 8 significant bits; rounding is to
    nearest with ties to even.

Pins (tests/test_oracle_codecs.py): bf16 rounding against torch's float32 ->
bfloat16 cast over a float32 sweep; E4M3 decode of all 256 codes against
torch.float8_e4m3fn; E4M3 encode of all 65,536 bf16 bit patterns against
torch's cast after an explicit +-448 clamp; spot values from the format's
definition (tests/golden/e4m3_spot.txt).
"""
from __future__ import annotations

import numpy as np

BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def bf16_round(x) -> np.ndarray:
    """Nearest bf16 value of each element (float64 in, float64 out).

    A finite x = m * 2**e with 0.5 <= |m| < 1 keeps 8 significant bits, so its
    rounding quantum is 2**(e - 8); below the normal range the quantum stays at
    the subnormal step 2**-133. Ties go to even (np.rint). Results beyond the
    largest finite bf16 become +-inf, which is what round-to-nearest-even does
    at the top of the range.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    qexp = np.maximum(e - 8, -133)
    r = np.ldexp(np.rint(np.ldexp(x, -qexp)), qexp)
    r = np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, x), r)
    return np.where(np.isfinite(x), r, x)


def bf16_bits(x) -> np.ndarray:
    """bf16 bit patterns (uint16) of the nearest bf16 values of x."""
    r = bf16_round(x).astype(np.float32)  # exact: every bf16 value is a float32
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def bf16_value(bits) -> np.ndarray:
    """float64 values of bf16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def e4m3_decode(codes) -> np.ndarray:
    """float64 value of each OCP E4M3 code.

    exponent field E = bits 6..3, mantissa m = bits 2..0:
      E == 0 : (-1)^s * (m / 8) * 2**-6          (subnormal)
      E >= 1 : (-1)^s * (1 + m / 8) * 2**(E - 7)
      S.1111.111 : NaN
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    E = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(E == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(E - 7.0))
    out = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


# non-negative finite values in code order (codes 0..126 are increasing)
_E4M3_POS = e4m3_decode(np.arange(127, dtype=np.uint8))
E4M3_MAX = float(_E4M3_POS[-1])  # 448


def e4m3_encode(x) -> np.ndarray:
    """OCP E4M3 code of each value: saturate to +-448, then nearest code,
    ties to the even code. NaN -> 0x7F (with the input's sign bit)."""
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    with np.errstate(invalid="ignore"):
        return _e4m3_encode_abs(np.minimum(np.abs(x), E4M3_MAX), np.isnan(x), neg)


def _e4m3_encode_abs(a, isnan, neg):
    i = np.searchsorted(_E4M3_POS, a, side="left")   # _POS[i-1] < a <= _POS[i]
    i = np.clip(i, 1, 126)
    lo = _E4M3_POS[i - 1]
    hi = _E4M3_POS[i]
    dlo = a - lo
    dhi = hi - a
    even_lo = ((i - 1) % 2) == 0
    code = np.where(dlo < dhi, i - 1,
                    np.where(dhi < dlo, i, np.where(even_lo, i - 1, i)))
    code = code.astype(np.uint8)
    code = np.where(isnan, np.uint8(0x7F), code).astype(np.uint8)
    return (code | (neg.astype(np.uint8) << 7)).astype(np.uint8)


def e4m3_roundtrip(x, scale: float = 1.0) -> np.ndarray:
    """decode(encode(x / scale)) * scale: the value an fp8 KV store keeps."""
    return e4m3_decode(e4m3_encode(np.asarray(x, np.float64) / scale)) * scale
