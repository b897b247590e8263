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
[-448, 448] (IEEE maxNum/minNum: a NaN product becomes -448), and rounded to
the nearest representable value, ties to the even code. It is read back as
value(code) * scale.

The encoder is written as a search over the 256 codes of the definition,
not as bit manipulation, so that it can be checked by eye.
"""
from __future__ import annotations

import numpy as np

MAX = 448.0


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


def quantize(x, inv_scale: float) -> np.ndarray:
    """Codes of x (any float array): fp32 product with inv_scale, clamp to
    +-448 (maxNum/minNum), round to nearest, ties to even."""
    prod = np.float32(np.asarray(x, dtype=np.float32)) * np.float32(inv_scale)
    prod = np.fmin(np.fmax(prod, np.float32(-MAX)), np.float32(MAX))
    # each distinct fp32 bit pattern (so -0 and +0 stay apart) is encoded
    # once by the search above
    bits, inverse = np.unique(np.ascontiguousarray(prod).view(np.uint32),
                              return_inverse=True)
    codes = np.array([encode_value(float(b)) for b in bits.view(np.float32)],
                     dtype=np.uint8)
    return codes[inverse.reshape(-1)].reshape(prod.shape)


def dequantize(codes, scale: float) -> np.ndarray:
    """fp64 values of codes, times scale."""
    return _VALUES[np.asarray(codes, dtype=np.int64)] * float(scale)
