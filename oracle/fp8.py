"""E4M3 codes for the FP8 window KV cache, written from the format's definition.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH (see ``oracle/__init__``).

Source: "Sliding Window and Sparse Attention, from Longformer to CSA2", s7
(the window KV stays FP8) and s10 glossary, E4M3 (1 sign, 4 exponent and 3
mantissa bits).  The pages fix neither the exponent bias nor the special
values nor a scale; the reading taken is the OCP form of E4M3: bias 7, no
infinities, S.1111.111 is NaN, largest finite value 1.75 * 2^8 = 448, and one
fp32 scale per (batch, key/value head) per tensor, a code c standing for
scale * value(c).

Values of the 256 codes (``decode``): exponent field e, mantissa field m,
  e = 0:            (-1)^s * (m / 8) * 2^-6          (subnormals, and +-0)
  e = 1..15:        (-1)^s * (1 + m / 8) * 2^(e - 7)
  e = 15 and m = 7: NaN.
Encoding (``encode``) picks, for a real y, the code whose value is nearest,
ties to the code with even m; |y| >= 448 saturates to +-448; NaN -> 0x7f with
y's sign.  Quantisation (``quantize``) encodes y = x / scale with the
division done in fp32 and correctly rounded (numpy float32 arithmetic).
Everything here works on exact binary values in Python floats, by search
over the code table rather than by bit manipulation.
"""
from __future__ import annotations

import math

import numpy as np

MAX_FINITE = 448.0


def value(code: int) -> float:
    """Real value of one E4M3 code (NaN for S.1111.111)."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 15 and m == 7:
        return math.nan
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_TABLE = np.array([value(c) for c in range(256)], dtype=np.float64)
# the non-negative finite codes in increasing order of value (0x00 .. 0x7e)
_POS_CODES = np.arange(0x00, 0x7F)
_POS_VALUES = _TABLE[_POS_CODES]


def decode(codes) -> np.ndarray:
    """Codes (uint8 array) -> float64 values."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def encode_one(y: float) -> int:
    """Nearest code to y, ties to even mantissa, saturating at 448."""
    if math.isnan(y):
        return 0xFF if math.copysign(1.0, y) < 0 else 0x7F
    sign = 0x80 if math.copysign(1.0, y) < 0 else 0x00
    a = abs(y)
    if a >= MAX_FINITE:
        return sign | 0x7E
    # largest code whose value is <= a, and the next one up
    i = int(np.searchsorted(_POS_VALUES, a, side="right")) - 1
    lo_code, lo = int(_POS_CODES[i]), float(_POS_VALUES[i])
    if lo == a:
        return sign | lo_code
    hi_code, hi = int(_POS_CODES[i + 1]), float(_POS_VALUES[i + 1])
    d_lo, d_hi = a - lo, hi - a
    if d_lo < d_hi:
        pick = lo_code
    elif d_hi < d_lo:
        pick = hi_code
    else:  # a tie: the code with an even mantissa field
        pick = lo_code if (lo_code & 1) == 0 else hi_code
    return sign | pick


def encode(y) -> np.ndarray:
    y = np.asarray(y, dtype=np.float64)
    return np.vectorize(encode_one, otypes=[np.uint8])(y) if y.size else y.astype(np.uint8)


def quantize(x, scale) -> np.ndarray:
    """Codes of x / scale, the division in fp32 (x: values exactly
    representable in fp32, e.g. bf16 or fp32 data; scale broadcastable)."""
    y = np.asarray(x, dtype=np.float32) / np.asarray(scale, dtype=np.float32)
    return encode(y.astype(np.float64))
