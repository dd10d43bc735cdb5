"""Float reference for the FP8 (E4M3) KV cache: encode, decode, quantize.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``): the product path never
imports this module.

mlx-node perf doc, quantization table (FP8 KV cache row): the paged adapter
stores K and V as FP8 with a scale per layer; the flat path does not. The
format is not spelled out beyond "FP8"; the table's other FP8 rows are E4M3,
and our reading is the OCP E4M3 encoding (the "fn" variant):

* 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
* exponent field 0 is subnormal: value = mantissa / 8 * 2^-6;
* no infinities; S.1111.111 (0x7F, 0xFF) is NaN, so the largest finite
  magnitude is 1.110 * 2^8 = 448 (0x7E);
* rounding to nearest, ties to the even code (mantissa LSB 0);
* saturation (our reading of a KV cache that must stay finite): magnitudes
  above 448 encode as +-448.

Per-layer scales: a stored code c represents ``scale * value(c)``; writing x
stores ``encode(float32(x) / float32(scale))`` (the division in float32,
correctly rounded). One scale for K and one for V per layer pool.

Nothing here is parity-unpinned: ``tests/test_oracle_fp8.py`` pins the table
against values the definition fixes, ties, saturation and a brute-force
nearest-value search.
"""

from __future__ import annotations

import numpy as np

__all__ = ["E4M3_MAX", "decode_e4m3", "encode_e4m3", "quantize", "dequantize"]

E4M3_MAX = 448.0


def _code_value(code: int) -> float:
    """Value of one E4M3 code from the bit fields (NaN for S.1111.111)."""
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** -6
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


_TABLE = np.array([_code_value(c) for c in range(256)], dtype=np.float64)


def decode_e4m3(codes):
    """float64 values of uint8 E4M3 codes (NaN for 0x7F and 0xFF)."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


# Non-negative finite codes 0x00..0x7E in increasing value order (the code is
# its own rank): nearest-value search runs on this table.
_POS_VALUES = _TABLE[:0x7F]


def encode_e4m3(x):
    """uint8 E4M3 codes of ``x``: nearest representable value, ties to the even
    code, magnitudes above 448 saturated to 448, the sign kept (so -0.0 and
    small negatives that round to zero give 0x80). NaN gives 0x7F."""
    x = np.asarray(x, dtype=np.float64)
    mag = np.minimum(np.abs(x), E4M3_MAX)
    # hi: first table value >= mag; lo: the one below it.
    hi = np.searchsorted(_POS_VALUES, mag, side="left")
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_hi = _POS_VALUES[hi] - mag
    d_lo = mag - _POS_VALUES[lo]
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    code = np.where(pick_lo & (hi > 0), lo, hi).astype(np.uint8)
    code = np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)


def quantize(x, scale):
    """Codes stored for values ``x`` (float32-representable) under a per-layer
    ``scale``: ``encode(float32(x) / float32(scale))``."""
    q = np.asarray(x, dtype=np.float32) / np.float32(scale)
    return encode_e4m3(q.astype(np.float32))


def dequantize(codes, scale):
    """float64 values ``scale * value(code)`` that attention reads."""
    return np.float64(np.float32(scale)) * decode_e4m3(codes)
