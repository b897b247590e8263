"""FP8 E4M3 (OCP 8-bit floating point, "E4M3FN") codec for the fp8 K/V cache.

TEST INFRASTRUCTURE (see the package docstring).

The explainer ["PagedAttention Nedir?", section "KV Cache'i Sıkıştırıyor
mu?"] separates paging from KV-cache quantisation, which lowers the
precision of the stored values; the PagedAttention newsletter ["Makale
Bülteni — PagedAttention ve vLLM", section "Kod ve Entegrasyon Haritası"]
names FP8 among the quantisation schemes of the serving stack. The pages
give no format details. Reading taken (the plainest one): the OCP E4M3
format - 1 sign bit,
4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds
subnormals (mantissa/8 * 2^-6); no infinities; S.1111.111 is NaN, so the
largest finite magnitude is 1.75 * 2^8 = 448. A value is stored as
code = E4M3(x * inv_scale) with the product taken in fp32, clamped to
[-448, 448] (saturation: infinities and overflows become +-448), and rounded
to the nearest representable value, ties to the even code. A NaN input
stays NaN: it is stored as the NaN code with the input's sign bit (0x7F or
0xFF), as the format's own conversion keeps it. A code is read back as
value(code) * scale. The scale is one per tensor, or one per KV head (any
array that broadcasts against the values, e.g. [Hkv, 1] for rows
[T, Hkv, D]).

The encoder is written as a search over the 256 codes of the definition,
not as bit manipulation, so that it can be checked by eye.
"""
from __future__ import annotations

import numpy as np

MAX = 448.0
NAN_CODE = 0x7F     # S.1111.111 with S = 0; the sign bit is added for -NaN


def decode(code: int) -> float:
    """Value of an E4M3 code (NaN for S.1111.111)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_CODES = np.arange(256)
_VALUES = np.array([decode(c) for c in _CODES])
_FINITE = ~np.isnan(_VALUES)


def encode_value(x: float) -> int:
    """Nearest finite code to x (x already in [-448, 448]); ties to the code
    with an even mantissa. Zero keeps its sign."""
    if x == 0.0:
        return 0x80 if np.signbit(x) else 0x00
    cands = _CODES[_FINITE]
    vals = _VALUES[_FINITE]
    # only codes of x's sign (so that -0 is never chosen for a negative x
    # over a same-distance positive code)
    same = (vals > 0) if x > 0 else (vals < 0)
    same |= vals == 0
    cands, vals = cands[same], vals[same]
    dist = np.abs(vals - x)
    best = dist.min()
    tied = cands[dist == best]
    if len(tied) > 1:
        even = [c for c in tied if (c & 1) == 0]
        tied = even if even else tied
    c = int(tied[0])
    if decode(c) == 0.0:                     # rounded to zero: keep x's sign
        return 0x80 if x < 0 else 0x00
    return c


def quantize(x, inv_scale) -> np.ndarray:
    """Codes of x (any float array): fp32 product with inv_scale (a number,
    or an array broadcasting against x), clamp to +-448, round to nearest,
    ties to even; a NaN input gives the NaN code with its sign."""
    x32 = np.asarray(x, dtype=np.float32)
    with np.errstate(invalid="ignore"):   # signalling NaNs stay NaN
        prod = x32 * np.asarray(inv_scale, dtype=np.float32)
    nan = np.isnan(prod)
    prod = np.where(nan, np.float32(0.0), prod)
    prod = np.minimum(np.maximum(prod, np.float32(-MAX)), np.float32(MAX))
    # each distinct fp32 bit pattern (so -0 and +0 stay apart) is encoded
    # once by the search above
    bits, inverse = np.unique(np.ascontiguousarray(prod).view(np.uint32),
                              return_inverse=True)
    codes = np.array([encode_value(float(b)) for b in bits.view(np.float32)],
                     dtype=np.uint8)
    out = codes[inverse.reshape(-1)].reshape(prod.shape)
    nan_codes = np.where(np.signbit(np.broadcast_to(x32, prod.shape)),
                         NAN_CODE | 0x80, NAN_CODE).astype(np.uint8)
    return np.where(nan, nan_codes, out).astype(np.uint8)


def dequantize(codes, scale) -> np.ndarray:
    """fp64 values of codes, times scale (a number, or an array broadcasting
    against codes)."""
    return _VALUES[np.asarray(codes, dtype=np.int64)] * np.asarray(
        scale, dtype=np.float64)
