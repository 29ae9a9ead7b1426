"""Number codecs used by the oracle (test infrastructure only).

* FP8 E4M3 in the OCP "E4M3FN" form: 1 sign bit, 4 exponent bits (bias 7),
  3 mantissa bits, no infinities, a single NaN pattern per sign (S.1111.111),
  largest finite value 1.75 * 2^8 = 448.  The value 448 is the FP8 range the
  SageAttention2++ review page uses in its scale formulas ("三、技术架构",
  core formulas: delta_P = max|P~|/448, delta_V = colmax|V|/448).
  Encoding rounds to nearest, ties to even, and saturates to +-448
  ("satfinite"), written here from the format definition, bit by bit.
* FP16 rounding is numpy's IEEE binary16 cast (round to nearest even).
* INT8 P^ of the all-INT8 kernel variant: P^ = round(127 P~), nearest even,
  in [0, 127] (P~ <= 1 under the exact running max).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
_E4M3_BIAS = 7
_E4M3_MIN_NORMAL_EXP = 1 - _E4M3_BIAS       # -6
_E4M3_SUBNORMAL_STEP = 2.0 ** (_E4M3_MIN_NORMAL_EXP - 3)   # 2^-9


def e4m3_encode(x) -> np.ndarray:
    """float array -> uint8 E4M3FN codes (RNE, saturate to +-448).

    The sign of zero is kept (-0.0 -> 0x80).  NaN inputs are not supported.
    """
    x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x).astype(np.uint8) << np.uint8(7)
    a = np.abs(x)
    a = np.minimum(a, E4M3_MAX)          # satfinite: anything above 448 -> 448

    code = np.zeros(a.shape, dtype=np.int64)
    # subnormal range (a < 2^-6): value = m * 2^-9, m in 0..7; m == 8 is the
    # smallest normal, which the code numbering makes seamless (code 8).
    sub = a < 2.0 ** _E4M3_MIN_NORMAL_EXP
    code[sub] = np.rint(a[sub] / _E4M3_SUBNORMAL_STEP).astype(np.int64)
    # normal range: a = (1 + m/8) * 2^e, e in -6..8
    nrm = ~sub
    an = a[nrm]
    _, e2 = np.frexp(an)                 # an = f * 2^e2 with f in [0.5, 1)
    e = e2.astype(np.int64) - 1          # an = (2f) * 2^e, 2f in [1, 2)
    mant = np.rint((np.ldexp(an, -e) - 1.0) * 8.0).astype(np.int64)   # 0..8 (exact args)
    carry = mant == 8
    e = e + carry
    mant = np.where(carry, 0, mant)
    c = ((e + _E4M3_BIAS) << 3) | mant
    code[nrm] = np.minimum(c, 0x7E)      # 0x7E = 448; never produce the NaN code
    return code.astype(np.uint8) | sign


def e4m3_decode(code) -> np.ndarray:
    """uint8 E4M3FN codes -> float64 values (0x7F / 0xFF decode to NaN)."""
    c = np.asarray(code, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    val = np.where(e == 0, m * _E4M3_SUBNORMAL_STEP,
                   np.ldexp(1.0 + m / 8.0, (e - _E4M3_BIAS).astype(np.int64)))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return s * val


def e4m3_flip_step(y, rel) -> np.ndarray:
    """For values y >= 0 (as encoded by e4m3_encode), the size of the change of
    the decoded value if y rounded to its other neighbouring code, wherever y
    lies within a relative distance rel (array or scalar) of the rounding
    boundary between two codes; 0 elsewhere.  Used to bound how far O can move
    when an evaluation of y slightly different from the float64 one rounds
    across a boundary."""
    y = np.asarray(y, dtype=np.float64)
    rel = np.asarray(rel, dtype=np.float64)
    c = e4m3_encode(y).astype(np.int64) & 0x7F
    v = e4m3_decode(c.astype(np.uint8))
    vp = e4m3_decode(np.maximum(c - 1, 0).astype(np.uint8))
    vn = e4m3_decode(np.minimum(c + 1, 0x7E).astype(np.uint8))
    tol = rel * y
    near_lo = (c > 0) & (np.abs(y - 0.5 * (vp + v)) <= tol)
    near_hi = (c < 0x7E) & (np.abs(y - 0.5 * (v + vn)) <= tol)
    return np.where(near_hi, vn - v, np.where(near_lo, v - vp, 0.0))


def int8_flip_step(y, rel) -> np.ndarray:
    """For values y in [0, 127] rounded to the nearest integer (ties to even),
    the size of the change of the code (1) if y rounded to its other
    neighbouring integer, wherever y lies within a relative distance rel
    (array or scalar) of a half-integer between two codes in [0, 127]; 0
    elsewhere.  The INT8 counterpart of e4m3_flip_step."""
    y = np.asarray(y, dtype=np.float64)
    rel = np.asarray(rel, dtype=np.float64)
    c = np.clip(np.rint(y), 0.0, 127.0)
    tol = rel * y
    near_lo = (c > 0) & (np.abs(y - (c - 0.5)) <= tol)
    near_hi = (c < 127) & (np.abs(y - (c + 0.5)) <= tol)
    return np.where(near_lo | near_hi, 1.0, 0.0)


def fp16_round(x) -> np.ndarray:
    """Round to IEEE binary16 (nearest even) and return the values as float64."""
    return np.asarray(x).astype(np.float16).astype(np.float64)
