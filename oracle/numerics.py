"""Rounding to bf16 and to OCP e4m3fn, written from the format definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Both formats are handled the same way: a finite binary64 value v with
frexp(v) = (m, ex), 0.5 <= |m| < 1, has its unit in the last place at
2**(ex - p) for a format with p significant bits; subnormals fix the
exponent at the format's minimum.  Dividing by a power of two is exact in
binary64, numpy's rint rounds half to even, so `rint(v / q) * q` is the
round-to-nearest-even result exactly.

bf16: 8 significant bits, minimum normal 2**-126 (smallest quantum 2**-133),
      overflow to +-inf (never reached by this block's values).
e4m3fn (OCP 8-bit float, E4M3 variant "fn": no infinities, one NaN code per
      sign): 4 significant bits, exponent bias 7, minimum normal 2**-6
      (smallest quantum 2**-9), largest finite 448.  Conversion here is
      round-to-nearest-even with saturation to +-448 ("satfinite").
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def _round_sig(v: np.ndarray, sig_bits: int, min_quantum_exp: int) -> np.ndarray:
    v = np.asarray(v, dtype=np.float64)
    _, ex = np.frexp(v)
    qexp = np.maximum(ex - sig_bits, min_quantum_exp)
    q = np.ldexp(1.0, qexp)
    return np.rint(v / q) * q


def bf16_round(v) -> np.ndarray:
    """Round each value (given as float32 or exact float64) to the nearest bf16, ties to even."""
    v = np.asarray(v, dtype=np.float32).astype(np.float64)
    return _round_sig(v, 8, -133)


def round_f64_to(v, dtype: str) -> np.ndarray:
    """Round exact float64 values ONCE to bf16 or fp32 (RNE), with no float32
    step in between (bf16_round above takes float32 inputs); returns float64."""
    if dtype == "bf16":
        return _round_sig(v, 8, -133)
    if dtype == "f32":
        return _round_sig(v, 24, -149)
    raise ValueError(dtype)


def e4m3_round(v) -> np.ndarray:
    """Round float32 values to e4m3fn values (RNE, saturating at +-448); returns float64."""
    v = np.asarray(v, dtype=np.float32).astype(np.float64)
    r = _round_sig(v, 4, -9)
    return np.clip(r, -E4M3_MAX, E4M3_MAX)


def e4m3_decode_table() -> np.ndarray:
    """Value of every e4m3fn code 0..255 (NaN for 0x7F and 0xFF)."""
    out = np.empty(256, dtype=np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            out[c] = np.nan
        elif e == 0:
            out[c] = s * (m / 8.0) * 2.0 ** -6
        else:
            out[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


_DEC = e4m3_decode_table()


def e4m3_decode(codes) -> np.ndarray:
    return _DEC[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(v) -> np.ndarray:
    """float32 values -> e4m3fn codes (uint8) via e4m3_round."""
    r = e4m3_round(v)
    sign = np.signbit(r).astype(np.uint8) << 7
    mag = np.abs(r)
    # the positive finite codes 0x00..0x7E are in increasing value order
    pos = _DEC[:0x7F]
    code = np.searchsorted(pos, mag).astype(np.uint8)
    return code | sign
