"""Decoders from storage formats to float64 (test infrastructure).

Written from the format definitions, independent of any library cast:

* OCP 8-bit float E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa
  bits.  Exponent field 0 encodes subnormals m * 2^-9; fields 1..15 encode
  (1 + m/8) * 2^(e-7); the two patterns S.1111.111 are NaN; there is no
  infinity, so the largest finite magnitude is 1.75 * 2^8 = 448.
* bfloat16: the upper 16 bits of an IEEE binary32; widening appends 16 zero bits.
* float32 values are exact in float64.

A per-token fp32 scale multiplies the decoded fp8 value; the product of a
binary32 scale and a 4-significant-bit code is exact in float64.
"""
from __future__ import annotations

import numpy as np


def _e4m3fn_table() -> np.ndarray:
    tab = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            tab[code] = np.nan
        elif e == 0:
            tab[code] = sign * (m / 8.0) * 2.0 ** (1 - 7)
        else:
            tab[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return tab


E4M3FN = _e4m3fn_table()


def decode_fp8(codes: np.ndarray) -> np.ndarray:
    return E4M3FN[np.asarray(codes, dtype=np.uint8)]


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def decode(raw: np.ndarray, dtype: str, scale=None, token_axes: int = 1) -> np.ndarray:
    """Storage -> float64.  ``scale`` (fp8 only) has the leading token dims of ``raw``."""
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return decode_bf16(raw)
    if dtype == "fp8":
        v = decode_fp8(raw)
        if scale is not None:
            s = np.asarray(scale, dtype=np.float32).astype(np.float64)
            v = v * s.reshape(s.shape + (1,) * (v.ndim - s.ndim))
        return v
    raise ValueError(dtype)
